"""The C ABI used from plain C (tests/c_abi/abi_smoke.c, built by
__graft_entry__.build()): host-side checks without a GPU, and the whole
route -> dispatch -> combine path with hipMalloc'd buffers on a GPU."""
import os
import subprocess

import pytest
import torch

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_smoke")


def _run(*args):
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: run __graft_entry__.build()")
    return subprocess.run([BIN, *args], capture_output=True, text=True, timeout=100)


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only run; the GPU variant covers it")
def test_c_program_host_checks():
    res = _run()
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_smoke ok" in res.stdout


@pytest.mark.gpu
def test_c_program_runs_the_path_on_the_gpu():
    print("[c_abi] abi_smoke gpu", flush=True)
    res = _run("gpu")
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_smoke ok (gpu)" in res.stdout
