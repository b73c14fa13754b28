"""Loads libmoe_route.so and declares its C ABI (include/moe_route.h) for ctypes.

torch is imported first on purpose: it brings its own HIP runtime
(libamdhip64.so.7), and the library must bind to that same runtime so the
stream handles and device pointers it receives from torch are valid.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (see module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_route.so")

_c_int, _c_i32, _c_i64, _c_size, _vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/moe_route.h
SIGNATURES = {
    "moe_abi_version": (_c_int, []),
    "moe_strerror": (ctypes.c_char_p, [_c_int]),
    "moe_route_topk": (_c_int, [_vp, _c_i64, _c_i32, _c_i32, _vp, _vp, _vp]),
    "moe_route_topk_grouped": (_c_int, [_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp,
                                        _vp]),
    "moe_dispatch_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32]),
    "moe_dispatch_send": (_c_int, [_vp, _c_i64, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _c_size, _vp]),
    "moe_dispatch_recv": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _vp, _c_i64, _vp]),
    "moe_dispatch": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp,
                              _vp, _vp, _vp, _c_i64, _vp, _c_size, _vp]),
    "moe_dispatch_recv_fp8": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _vp, _vp, _c_i64, _vp]),
    "moe_dispatch_fp8": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _c_i64, _vp, _c_size, _vp]),
    "moe_combine": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i64, _vp, _vp]),
    "moe_dispatch_noalloc": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "moe_route_dispatch": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp,
                                    _c_size, _vp]),
    "moe_route_dispatch_workspace_bytes": (_c_size, [_c_i64, _c_i32, _c_i32]),
    "moe_route_dispatch_fp8": (_c_int, [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                        _c_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _c_i64, _vp, _c_size, _vp]),
}

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_ALIGNMENT = -2
MOE_ERR_CAPACITY = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

_lib = None


def load() -> ctypes.CDLL:
    """Return the loaded library; raise ImportError if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m combine_topk_route_amd.build` "
                "(hipcc --offload-arch=gfx950); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
