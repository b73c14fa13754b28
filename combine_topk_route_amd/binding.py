"""Thin torch binding of libmoe_route.so: argument marshalling only.

Every function has the name of the C entry point it calls, checks tensor
placement / dtype / contiguity, allocates outputs the caller did not pass
(torch is the device-memory and stream provider), and passes raw pointers
plus the launch stream (the current one unless ``stream=`` names another;
anything the binding allocates is allocated on that stream).  All
computation runs in the library's kernels; there is no other path.  A
non-zero status raises ``MoeError``.
"""
from __future__ import annotations

import contextlib
from typing import NamedTuple, Optional

import torch

from . import _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.load().moe_strerror(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != _lib.MOE_OK:
        raise MoeError(fn, status)


# The current stream's raw handle for a device index, without building a
# torch.cuda.Stream object on every call (that costs a few microseconds, which
# is the whole kernel time at decode sizes).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, like: torch.Tensor) -> int:
    """The stream handle to enqueue on: `stream` if given, else the current
    stream of the device that holds `like`."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(like.get_device())
        return torch.cuda.current_stream(like.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on(stream, like: torch.Tensor):
    """Context for the binding's own allocations (outputs the caller did not
    pass, scratch): the launch stream.  torch's caching allocator then hands
    a freed block out again only to later work on that stream, and the fill
    of ``torch.zeros`` runs on it, so both are ordered with the kernels this
    call enqueues there.  ``stream=None`` launches on the current stream,
    which is where torch allocates anyway."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=like.device)
    return torch.cuda.stream(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None,
         device: Optional[int] = None) -> int:
    """Device pointer of `t` after checking placement, dtype, rank and layout.
    `device`: the device index every tensor of the call must be on (the
    first tensor's); the kernels run on that device's stream."""
    try:
        ok = (t.is_cuda and t.dtype is dtype and (ndim is None or t.dim() == ndim)
              and t.is_contiguous() and (device is None or t.get_device() == device))
    except AttributeError:
        ok = False
    if not ok:
        _reject(t, name, dtype, ndim, device)
    return t.data_ptr()


def _reject(t, name: str, dtype: torch.dtype, ndim: Optional[int], device: Optional[int]) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device is not None and t.get_device() != device:
        raise ValueError(f"{name} is on cuda:{t.get_device()}, but this call runs on cuda:{device}")
    raise ValueError(f"{name} must be contiguous")


def _empty(shape, dtype, like: torch.Tensor, stream) -> torch.Tensor:
    with _on(stream, like):
        return torch.empty(shape, dtype=dtype, device=like.device)


def moe_abi_version() -> int:
    return int(_lib.load().moe_abi_version())


def moe_route_topk(logits: torch.Tensor, k: int, topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None, stream=None):
    """Top-k routing: returns (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    lp = _dev(logits, "logits", torch.float32, 2)
    d = logits.get_device()
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, logits, stream)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, logits, stream)
    ip = _dev(topk_idx, "topk_idx", torch.int32, device=d)
    wp = _dev(topk_w, "topk_w", torch.float32, device=d)
    if topk_idx.numel() != T * k or topk_w.numel() != T * k:
        raise ValueError("topk_idx / topk_w must hold T*k elements")
    _check("moe_route_topk", _lib.load().moe_route_topk(lp, T, E, k, ip, wp, _stream(stream, logits)))
    return topk_idx, topk_w


def moe_route_topk_grouped(logits: torch.Tensor, k: int, n_group: int, topk_group: int,
                           topk_idx: Optional[torch.Tensor] = None,
                           topk_w: Optional[torch.Tensor] = None, stream=None):
    """Group-limited top-k routing: returns (topk_idx int32 [T,k], topk_w fp32 [T,k])."""
    lp = _dev(logits, "logits", torch.float32, 2)
    d = logits.get_device()
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, logits, stream)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, logits, stream)
    ip = _dev(topk_idx, "topk_idx", torch.int32, device=d)
    wp = _dev(topk_w, "topk_w", torch.float32, device=d)
    if topk_idx.numel() != T * k or topk_w.numel() != T * k:
        raise ValueError("topk_idx / topk_w must hold T*k elements")
    _check("moe_route_topk_grouped", _lib.load().moe_route_topk_grouped(
        lp, T, E, k, n_group, topk_group, ip, wp, _stream(stream, logits)))
    return topk_idx, topk_w


def moe_dispatch_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(_lib.load().moe_dispatch_workspace_bytes(T, E, k))


class SendResult(NamedTuple):
    expert_counts: torch.Tensor   # int32 [E]
    expert_offsets: torch.Tensor  # int32 [E+1]
    pair_row: torch.Tensor        # int32 [T, k]
    row_token: torch.Tensor       # int32 [T*k]
    rank_offsets: Optional[torch.Tensor]  # int32 [R+1]


def _send_outputs(topk_idx, E, R, expert_counts, expert_offsets, pair_row, row_token,
                  rank_offsets, with_rank_offsets, stream):
    T, k = topk_idx.shape
    if expert_counts is None:
        expert_counts = _empty((E,), torch.int32, topk_idx, stream)
    if expert_offsets is None:
        expert_offsets = _empty((E + 1,), torch.int32, topk_idx, stream)
    if pair_row is None:
        pair_row = _empty((T, k), torch.int32, topk_idx, stream)
    if row_token is None:
        row_token = _empty((T * k,), torch.int32, topk_idx, stream)
    if rank_offsets is None and with_rank_offsets:
        rank_offsets = _empty((R + 1,), torch.int32, topk_idx, stream)
    sizes = [(expert_counts, E), (expert_offsets, E + 1), (pair_row, T * k), (row_token, T * k)]
    if rank_offsets is not None:
        sizes.append((rank_offsets, R + 1))
    for t, n in sizes:
        if t.numel() != n:
            raise ValueError("dispatch output has the wrong number of elements")
    return SendResult(expert_counts, expert_offsets, pair_row, row_token, rank_offsets)


def _workspace(T, E, k, workspace, like, stream):
    """(pointer, bytes, tensor) of the send workspace; allocated here when the
    caller passed none and the launch needs one.  The library checks the size."""
    if workspace is None:
        need = moe_dispatch_workspace_bytes(T, E, k)
        if need == 0:
            return 0, 0, None
        workspace = _empty((need,), torch.uint8, like, stream)
    return (_dev(workspace, "workspace", torch.uint8, device=like.get_device()), workspace.numel(),
            workspace)


def _send_ptrs(out: "SendResult", d: int):
    """Device pointers of the send outputs (rank_offsets may be None)."""
    rp = (_dev(out.rank_offsets, "rank_offsets", torch.int32, device=d)
          if out.rank_offsets is not None else None)
    return (_dev(out.expert_counts, "expert_counts", torch.int32, device=d),
            _dev(out.expert_offsets, "expert_offsets", torch.int32, device=d),
            _dev(out.pair_row, "pair_row", torch.int32, device=d),
            _dev(out.row_token, "row_token", torch.int32, device=d), rp)


def moe_dispatch_send(topk_idx: torch.Tensor, E: int, num_vranks: int = 1, *,
                      expert_counts=None, expert_offsets=None, pair_row=None, row_token=None,
                      rank_offsets=None, with_rank_offsets: bool = True, workspace=None,
                      stream=None) -> SendResult:
    """Counts, offsets and the stable destination row of every (token, j) pair."""
    ip = _dev(topk_idx, "topk_idx", torch.int32, 2)
    d = topk_idx.get_device()
    T, k = topk_idx.shape
    out = _send_outputs(topk_idx, E, num_vranks, expert_counts, expert_offsets, pair_row,
                        row_token, rank_offsets, with_rank_offsets, stream)
    wp, wn, _ = _workspace(T, E, k, workspace, topk_idx, stream)
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_dispatch_send", _lib.load().moe_dispatch_send(
        ip, T, E, k, num_vranks, cp, op, pp, tp, rp, wp, wn, _stream(stream, topk_idx)))
    return out


def moe_dispatch_recv(x: torch.Tensor, pair_row: torch.Tensor, buf: Optional[torch.Tensor] = None,
                      capacity: Optional[int] = None, stream=None) -> torch.Tensor:
    """Scatter bf16 token rows into the expert-major buffer [capacity, H]."""
    xp = _dev(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    k = pair_row.shape[1] if pair_row.dim() == 2 else 0
    if pair_row.dim() != 2 or pair_row.shape[0] != T:
        raise ValueError("pair_row must be [T, k]")
    if buf is None:
        buf = _empty((T * k if capacity is None else capacity, H), torch.bfloat16, x, stream)
    if capacity is None:
        capacity = buf.shape[0]
    if buf.dim() != 2 or buf.shape[1] != H or buf.shape[0] < capacity:
        raise ValueError("buf must be [>= capacity, H]")
    d = x.get_device()
    _check("moe_dispatch_recv", _lib.load().moe_dispatch_recv(
        xp, _dev(pair_row, "pair_row", torch.int32, device=d), T, H, k,
        _dev(buf, "buf", torch.bfloat16, device=d), capacity, _stream(stream, x)))
    return buf


def moe_dispatch(topk_idx: torch.Tensor, x: torch.Tensor, E: int, num_vranks: int = 1, *,
                 buf=None, capacity=None, expert_counts=None, expert_offsets=None, pair_row=None,
                 row_token=None, rank_offsets=None, with_rank_offsets: bool = True,
                 workspace=None, stream=None):
    """Send then receive on one stream; returns (SendResult, buf)."""
    ip = _dev(topk_idx, "topk_idx", torch.int32, 2)
    d = topk_idx.get_device()
    xp = _dev(x, "x", torch.bfloat16, 2, device=d)
    T, k = topk_idx.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and topk_idx disagree on T")
    out = _send_outputs(topk_idx, E, num_vranks, expert_counts, expert_offsets, pair_row,
                        row_token, rank_offsets, with_rank_offsets, stream)
    if buf is None:
        buf = _empty((T * k if capacity is None else capacity, H), torch.bfloat16, x, stream)
    if capacity is None:
        capacity = buf.shape[0]
    if buf.dim() != 2 or buf.shape[1] != H or buf.shape[0] < capacity:
        raise ValueError("buf must be [>= capacity, H]")
    wp, wn, _ = _workspace(T, E, k, workspace, topk_idx, stream)
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_dispatch", _lib.load().moe_dispatch(
        ip, xp, T, E, k, H, num_vranks, cp, op, pp, tp, rp,
        _dev(buf, "buf", torch.bfloat16, device=d), capacity, wp, wn, _stream(stream, x)))
    return out, buf


def moe_dispatch_noalloc(topk_idx: torch.Tensor, x: torch.Tensor, E: int, num_vranks: int, *,
                         buf: torch.Tensor, expert_counts: torch.Tensor,
                         expert_offsets: torch.Tensor, pair_row: torch.Tensor,
                         row_token: torch.Tensor, rank_offsets: Optional[torch.Tensor] = None,
                         capacity: Optional[int] = None, stream=None):
    """moe_dispatch for callers that cannot allocate: every output is the
    caller's, and the send scratch is the library's own per-device array, so
    neither this function nor the library allocates anything.  Calls that
    overlap on one device race on that array.  Returns (SendResult, buf)."""
    ip = _dev(topk_idx, "topk_idx", torch.int32, 2)
    d = topk_idx.get_device()
    xp = _dev(x, "x", torch.bfloat16, 2, device=d)
    T, k = topk_idx.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and topk_idx disagree on T")
    out = SendResult(expert_counts, expert_offsets, pair_row, row_token, rank_offsets)
    sizes = [(expert_counts, E), (expert_offsets, E + 1), (pair_row, T * k), (row_token, T * k)]
    if rank_offsets is not None:
        sizes.append((rank_offsets, num_vranks + 1))
    for t, n in sizes:
        if t.numel() != n:
            raise ValueError("dispatch output has the wrong number of elements")
    if capacity is None:
        capacity = buf.shape[0]
    if buf.dim() != 2 or buf.shape[1] != H or buf.shape[0] < capacity:
        raise ValueError("buf must be [>= capacity, H]")
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_dispatch_noalloc", _lib.load().moe_dispatch_noalloc(
        ip, xp, T, E, k, H, num_vranks, cp, op, pp, tp, rp,
        _dev(buf, "buf", torch.bfloat16, device=d), capacity, _stream(stream, x)))
    return out, buf


def moe_route_dispatch_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(_lib.load().moe_route_dispatch_workspace_bytes(T, E, k))


def moe_route_dispatch(logits: torch.Tensor, x: torch.Tensor, k: int, num_vranks: int = 1, *,
                       n_group: int = 1, topk_group: int = 1, topk_idx=None, topk_w=None,
                       buf=None, capacity=None, expert_counts=None, expert_offsets=None,
                       pair_row=None, row_token=None, rank_offsets=None,
                       with_rank_offsets: bool = True, workspace=None, stream=None):
    """Route, send and receive in one call; returns (topk_idx, topk_w,
    SendResult, buf).  ``n_group`` / ``topk_group`` select group-limited
    routing as in moe_route_topk_grouped.  ``workspace`` (uint8, at least
    moe_route_dispatch_workspace_bytes bytes) must start zeroed the first time
    it is used; it is allocated zeroed here when not given.  Keep one
    workspace per stream and do not pass it to the other dispatch calls."""
    lp = _dev(logits, "logits", torch.float32, 2)
    d = logits.get_device()
    xp = _dev(x, "x", torch.bfloat16, 2, device=d)
    T, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and logits disagree on T")
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, logits, stream)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, logits, stream)
    if topk_idx.shape != (T, k) or topk_w.shape != (T, k):
        raise ValueError("topk_idx / topk_w must be [T, k]")
    ip = _dev(topk_idx, "topk_idx", torch.int32, device=d)
    wp = _dev(topk_w, "topk_w", torch.float32, device=d)
    out = _send_outputs(topk_idx, E, num_vranks, expert_counts, expert_offsets, pair_row,
                        row_token, rank_offsets, with_rank_offsets, stream)
    if buf is None:
        buf = _empty((T * k if capacity is None else capacity, H), torch.bfloat16, x, stream)
    if capacity is None:
        capacity = buf.shape[0]
    if buf.dim() != 2 or buf.shape[1] != H or buf.shape[0] < capacity:
        raise ValueError("buf must be [>= capacity, H]")
    if workspace is None:
        with _on(stream, logits):  # zero-filled on the launch stream
            workspace = torch.zeros((max(1, moe_route_dispatch_workspace_bytes(T, E, k)),),
                                    dtype=torch.uint8, device=logits.device)
    wsp = _dev(workspace, "workspace", torch.uint8, device=d)
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_route_dispatch", _lib.load().moe_route_dispatch(
        lp, xp, T, E, k, n_group, topk_group, H, num_vranks, ip, wp, cp, op, pp, tp, rp,
        _dev(buf, "buf", torch.bfloat16, device=d), capacity, wsp, workspace.numel(),
        _stream(stream, logits)))
    return topk_idx, topk_w, out, buf


def _fp8_bufs(x, T, k, buf_q, buf_scale, capacity, stream):
    H = x.shape[1]
    rows = T * k if capacity is None else capacity
    if buf_q is None:
        buf_q = _empty((rows, H), torch.uint8, x, stream)
    if buf_scale is None:
        buf_scale = _empty((rows, H // 128 if H % 128 == 0 else 0), torch.float32, x, stream)
    if capacity is None:
        capacity = buf_q.shape[0]
    if buf_q.dim() != 2 or buf_q.shape[1] != H or buf_q.shape[0] < capacity:
        raise ValueError("buf_q must be [>= capacity, H] uint8")
    if buf_scale.dim() != 2 or buf_scale.shape[0] < capacity or buf_scale.shape[1] != H // 128:
        raise ValueError("buf_scale must be [>= capacity, H // 128] float32")
    return buf_q, buf_scale, capacity


def moe_dispatch_recv_fp8(x: torch.Tensor, pair_row: torch.Tensor, buf_q=None, buf_scale=None,
                          capacity: Optional[int] = None, stream=None):
    """Scatter block-scaled fp8 (E4M3) token rows: returns (buf_q uint8
    [capacity, H], buf_scale fp32 [capacity, H/128])."""
    xp = _dev(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    if pair_row.dim() != 2 or pair_row.shape[0] != T:
        raise ValueError("pair_row must be [T, k]")
    k = pair_row.shape[1]
    buf_q, buf_scale, capacity = _fp8_bufs(x, T, k, buf_q, buf_scale, capacity, stream)
    d = x.get_device()
    _check("moe_dispatch_recv_fp8", _lib.load().moe_dispatch_recv_fp8(
        xp, _dev(pair_row, "pair_row", torch.int32, device=d), T, H, k,
        _dev(buf_q, "buf_q", torch.uint8, device=d),
        _dev(buf_scale, "buf_scale", torch.float32, device=d), capacity, _stream(stream, x)))
    return buf_q, buf_scale


def moe_dispatch_fp8(topk_idx: torch.Tensor, x: torch.Tensor, E: int, num_vranks: int = 1, *,
                     buf_q=None, buf_scale=None, capacity=None, expert_counts=None,
                     expert_offsets=None, pair_row=None, row_token=None, rank_offsets=None,
                     with_rank_offsets: bool = True, workspace=None, stream=None):
    """Send then fp8 receive on one stream; returns (SendResult, buf_q, buf_scale)."""
    ip = _dev(topk_idx, "topk_idx", torch.int32, 2)
    d = topk_idx.get_device()
    xp = _dev(x, "x", torch.bfloat16, 2, device=d)
    T, k = topk_idx.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and topk_idx disagree on T")
    out = _send_outputs(topk_idx, E, num_vranks, expert_counts, expert_offsets, pair_row,
                        row_token, rank_offsets, with_rank_offsets, stream)
    buf_q, buf_scale, capacity = _fp8_bufs(x, T, k, buf_q, buf_scale, capacity, stream)
    wp, wn, _ = _workspace(T, E, k, workspace, topk_idx, stream)
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_dispatch_fp8", _lib.load().moe_dispatch_fp8(
        ip, xp, T, E, k, H, num_vranks, cp, op, pp, tp, rp,
        _dev(buf_q, "buf_q", torch.uint8, device=d),
        _dev(buf_scale, "buf_scale", torch.float32, device=d), capacity, wp, wn,
        _stream(stream, x)))
    return out, buf_q, buf_scale


def moe_route_dispatch_fp8(logits: torch.Tensor, x: torch.Tensor, k: int, num_vranks: int = 1, *,
                           n_group: int = 1, topk_group: int = 1, topk_idx=None, topk_w=None,
                           buf_q=None, buf_scale=None, capacity=None, expert_counts=None,
                           expert_offsets=None, pair_row=None, row_token=None,
                           rank_offsets=None, with_rank_offsets: bool = True, workspace=None,
                           stream=None):
    """Route, send and block-scaled fp8 receive in one call; returns
    (topk_idx, topk_w, SendResult, buf_q, buf_scale).  The workspace rules
    are moe_route_dispatch's."""
    lp = _dev(logits, "logits", torch.float32, 2)
    d = logits.get_device()
    xp = _dev(x, "x", torch.bfloat16, 2, device=d)
    T, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x and logits disagree on T")
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, logits, stream)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, logits, stream)
    if topk_idx.shape != (T, k) or topk_w.shape != (T, k):
        raise ValueError("topk_idx / topk_w must be [T, k]")
    ip = _dev(topk_idx, "topk_idx", torch.int32, device=d)
    wp = _dev(topk_w, "topk_w", torch.float32, device=d)
    out = _send_outputs(topk_idx, E, num_vranks, expert_counts, expert_offsets, pair_row,
                        row_token, rank_offsets, with_rank_offsets, stream)
    buf_q, buf_scale, capacity = _fp8_bufs(x, T, k, buf_q, buf_scale, capacity, stream)
    if workspace is None:
        with _on(stream, logits):  # zero-filled on the launch stream
            workspace = torch.zeros((max(1, moe_route_dispatch_workspace_bytes(T, E, k)),),
                                    dtype=torch.uint8, device=logits.device)
    wsp = _dev(workspace, "workspace", torch.uint8, device=d)
    cp, op, pp, tp, rp = _send_ptrs(out, d)
    _check("moe_route_dispatch_fp8", _lib.load().moe_route_dispatch_fp8(
        lp, xp, T, E, k, n_group, topk_group, H, num_vranks, ip, wp, cp, op, pp, tp, rp,
        _dev(buf_q, "buf_q", torch.uint8, device=d),
        _dev(buf_scale, "buf_scale", torch.float32, device=d), capacity, wsp, workspace.numel(),
        _stream(stream, logits)))
    return topk_idx, topk_w, out, buf_q, buf_scale


def moe_combine(y: torch.Tensor, pair_row: torch.Tensor, topk_w: torch.Tensor,
                out: Optional[torch.Tensor] = None, capacity: Optional[int] = None,
                stream=None) -> torch.Tensor:
    """Router-weighted sum of each token's k expert rows: bf16 [T, H]."""
    yp = _dev(y, "y", torch.bfloat16, 2)
    if pair_row.dim() != 2:
        raise ValueError("pair_row must be [T, k]")
    T, k = pair_row.shape
    H = y.shape[1]
    if topk_w.shape != pair_row.shape:
        raise ValueError("topk_w must match pair_row's shape")
    if capacity is None:
        capacity = y.shape[0]
    if capacity > y.shape[0]:
        raise ValueError("capacity exceeds y's rows")
    if out is None:
        out = _empty((T, H), torch.bfloat16, y, stream)
    if out.shape != (T, H):
        raise ValueError("out must be [T, H]")
    d = y.get_device()
    _check("moe_combine", _lib.load().moe_combine(
        yp, _dev(pair_row, "pair_row", torch.int32, device=d),
        _dev(topk_w, "topk_w", torch.float32, device=d), T, H, k, capacity,
        _dev(out, "out", torch.bfloat16, device=d), _stream(stream, y)))
    return out
