"""Build libmoe_route.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m combine_topk_route_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "moe_route.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libmoe_route.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_route.so)")


def command(out: str = LIB, defines: tuple = (), src: str = SRC) -> list[str]:
    """hipcc command line; ``defines`` (e.g. ``("MOE_RECV_SLICES=1",)``) build
    the measurement variants that probes.py compares against the library,
    and ``src`` its own measurement kernels."""
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", f"-I{INCLUDE}", *[f"-D{d}" for d in defines], "-o", out, src,
    ]


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_smoke")


def c_smoke_command() -> list[str]:
    """A plain C program against the C ABI (gcc; links the library and the
    HIP runtime only for hipMalloc/hipMemcpy)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return ["gcc", "-O2", "-std=c11", "-Wall", f"-I{INCLUDE}", f"-I{rocm}/include",
            "-D__HIP_PLATFORM_AMD__", "-o", C_SMOKE_BIN, C_SMOKE_SRC, f"-L{PKG_DIR}",
            "-lmoe_route", "-Wl,-rpath,$ORIGIN/../../combine_topk_route_amd", f"-L{rocm}/lib",
            "-lamdhip64",
            f"-Wl,-rpath,{rocm}/lib"]


def build_c_smoke(verbose: bool = False) -> str:
    cmd = c_smoke_command()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("gcc failed building the C ABI smoke program")
    return C_SMOKE_BIN


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {LIB}")
    os.replace(tmp, LIB)
    build_c_smoke(verbose)
    return LIB


VARIANT_DIR = os.path.join(ROOT, "_build")


def variant_path(name: str, lib: str = "libmoe_route.so") -> str:
    return os.path.join(VARIANT_DIR, name, lib)


def build_variant(name: str, defines: tuple, verbose: bool = False, src: str = SRC,
                  lib: str = "libmoe_route.so") -> str:
    """The library built with measurement ``defines`` (another slice count
    or store form for the recv kernel), or another measurement source, as
    _build/<name>/<lib>, for probes.py only (never loaded by the package)."""
    out = variant_path(name, lib)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = command(out + ".tmp", defines, src)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {out}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
