"""probes.py's own measurement kernels compile for gfx950 and export their
entry point (no GPU: hipcc cross-compiles; the kernels run only under
probes.py on a GPU)."""
import os
import subprocess

import pytest

import probes
from combine_topk_route_amd import build as b


def test_ceiling_kernels_compile(tmp_path):
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    src = tmp_path / "hbm_ceiling.hip"
    src.write_text(probes.CEILING_SRC)
    out = str(tmp_path / "libhbm_ceiling.so")
    res = subprocess.run(b.command(out, (), str(src)), capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    syms = subprocess.run(["nm", "-D", "--defined-only", out], capture_output=True, text=True)
    assert "ceiling_launch" in syms.stdout


def test_variant_names_and_defines():
    assert probes._slice_variant(probes.LIB_SLICES) == (None, ())
    assert probes._slice_variant(1) == ("recv_slices_1", ("MOE_RECV_SLICES=1",))
    assert probes._store_variant("nt sc1") == ("recv_store_18", ("MOE_RECV_STORE=18",))
    names = {probes._combine_variant(f)[0] for f in probes.COMBINE_STORE_FORMS}
    assert names == {"combine_store_sc1", "combine_store_wb"}
    assert os.path.basename(b.variant_path("x", "liby.so")) == "liby.so"
