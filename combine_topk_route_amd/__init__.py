"""MI355X (gfx950) MoE top-k routing, dispatch and combine.

The hot path runs in hand-written HIP kernels in ``libmoe_route.so`` behind a
C ABI (``include/moe_route.h``); this package is the thin torch binding.
Importing it loads the library and fails loudly if it was not built.
"""
from . import _lib
from .buffers import MoeBuffers  # noqa: F401
from .binding import (  # noqa: F401
    MoeError,
    SendResult,
    moe_abi_version,
    moe_combine,
    moe_dispatch,
    moe_dispatch_fp8,
    moe_dispatch_noalloc,
    moe_dispatch_recv_fp8,
    moe_dispatch_recv,
    moe_dispatch_send,
    moe_dispatch_workspace_bytes,
    moe_route_dispatch,
    moe_route_dispatch_fp8,
    moe_route_dispatch_workspace_bytes,
    moe_route_topk,
    moe_route_topk_grouped,
)

_lib.load()
