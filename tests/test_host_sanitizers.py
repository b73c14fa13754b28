"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the C ABI's
argument checking (no device is touched): the library is rebuilt with the
sanitizers on its host code only, the plain C smoke program is built with
them too, and its host checks must pass with no sanitizer report.  CPU only."""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "combine_topk_route_amd", "csrc", "moe_route.hip")
INC = os.path.join(ROOT, "include")
C_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")

pytestmark = [pytest.mark.skipif(torch.cuda.is_available(), reason="host-only sanitizer run"),
              pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")]

SAN = "address,undefined"


def test_host_side_abi_checks_are_clean_under_asan_ubsan(tmp_path):
    lib = tmp_path / "libmoe_route.so"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hip_cmd = ["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=" + SAN, "-Xarch_host", "-fno-omit-frame-pointer",
               f"-I{INC}", "-o", str(lib), SRC]
    r = subprocess.run(hip_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = tmp_path / "abi_smoke_san"
    clang = os.path.join(rocm, "lib", "llvm", "bin", "clang")  # the runtime hipcc's code expects
    c_cmd = [clang, "-O1", "-g", "-std=c11", "-fsanitize=" + SAN, "-fno-omit-frame-pointer",
             f"-I{INC}", f"-I{rocm}/include", "-D__HIP_PLATFORM_AMD__", "-o", str(exe), C_SRC,
             f"-L{tmp_path}", "-lmoe_route", f"-Wl,-rpath,{tmp_path}", f"-L{rocm}/lib",
             "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(c_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "abi_smoke ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
