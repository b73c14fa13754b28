"""Reusable device buffers for the route -> dispatch -> combine chain.

The dispatch/combine buffers are allocated once and reused across layers
("Efficient and portable mixture-of-experts communication", section "Portable
Kernels"; "Enabling trillion-parameter models on AWS EFA", section "Send and
Receive Buffers": sized for the worst case, so no token is dropped).  This
class holds one set for up to ``max_tokens`` tokens and calls the same
library entry points with them, so a step allocates nothing and can be
captured into a HIP graph.  It does no computation of its own.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from . import binding as _b


class MoeBuffers:
    """Preallocated outputs and workspace for batches of up to ``max_tokens``.

    ``num_vranks`` virtual ranks own ``E // num_vranks`` experts each; the
    dispatch buffer has capacity ``max_tokens * k`` rows (no drops).  Methods
    return views of the buffers sized to the batch; the views are overwritten
    by the next call.
    """

    def __init__(self, max_tokens: int, hidden: int, num_experts: int, k: int,
                 num_vranks: int = 1, device: Optional[torch.device] = None,
                 fp8: bool = False):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        self.max_tokens, self.H, self.E, self.k, self.R = max_tokens, hidden, num_experts, k, num_vranks
        self.device_index = dev.index if dev.index is not None else torch.cuda.current_device()
        cap = max_tokens * k
        i32, f32 = torch.int32, torch.float32
        self.topk_idx = torch.empty((max_tokens, k), dtype=i32, device=dev)
        self.topk_w = torch.empty((max_tokens, k), dtype=f32, device=dev)
        self.expert_counts = torch.empty((num_experts,), dtype=i32, device=dev)
        self.expert_offsets = torch.empty((num_experts + 1,), dtype=i32, device=dev)
        self.rank_offsets = torch.empty((num_vranks + 1,), dtype=i32, device=dev)
        self.pair_row = torch.empty((max_tokens, k), dtype=i32, device=dev)
        self.row_token = torch.empty((cap,), dtype=i32, device=dev)
        ws = _b.moe_dispatch_workspace_bytes(max_tokens, num_experts, k)
        self.workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
        # route_dispatch's own workspace: it starts zeroed and every call
        # leaves it zeroed.
        rws = _b.moe_route_dispatch_workspace_bytes(max_tokens, num_experts, k)
        self.route_workspace = torch.zeros((max(rws, 1),), dtype=torch.uint8, device=dev)
        self.buf = torch.empty((cap, hidden), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((max_tokens, hidden), dtype=torch.bfloat16, device=dev)
        self.buf_q = self.buf_scale = None
        if fp8:
            self.buf_q = torch.empty((cap, hidden), dtype=torch.uint8, device=dev)
            self.buf_scale = torch.empty((cap, hidden // 128), dtype=f32, device=dev)
        self._views = None

    def _t(self, T: int) -> int:
        if not 0 <= T <= self.max_tokens:
            raise ValueError(f"batch of {T} tokens exceeds max_tokens={self.max_tokens}")
        return T

    def _v(self, T: int) -> "_Views":
        """The buffers' views for a batch of T tokens, kept for the most recent
        T: slicing a tensor costs about a microsecond of host time, as much as
        a decode-sized kernel."""
        v = self._views
        if v is None or v.T != T:
            v = self._views = _Views(self, self._t(T))
        return v

    def _send(self, T):
        return self._v(T).send

    def route(self, logits: torch.Tensor, n_group: int = 1, topk_group: int = 1, stream=None):
        v = self._v(logits.shape[0])
        idx, w = v.topk_idx, v.topk_w
        if n_group == 1:
            return _b.moe_route_topk(logits, self.k, topk_idx=idx, topk_w=w, stream=stream)
        return _b.moe_route_topk_grouped(logits, self.k, n_group, topk_group, topk_idx=idx,
                                         topk_w=w, stream=stream)

    def dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor, stream=None):
        """Send + receive; returns (SendResult, buf [T*k, H])."""
        v = self._v(x.shape[0])
        s = v.send
        _b.moe_dispatch(topk_idx, x, self.E, self.R, buf=v.buf,
                        expert_counts=s.expert_counts, expert_offsets=s.expert_offsets,
                        pair_row=s.pair_row, row_token=s.row_token, rank_offsets=s.rank_offsets,
                        workspace=self.workspace, stream=stream)
        return s, v.buf

    def route_dispatch(self, logits: torch.Tensor, x: torch.Tensor, n_group: int = 1,
                       topk_group: int = 1, stream=None):
        """Route + send + receive in one call; returns (topk_idx, topk_w,
        SendResult, buf [T*k, H]).  Only ``logits`` and ``x`` are checked per
        call: the outputs are this object's own buffers, whose pointers the
        views keep."""
        T = x.shape[0]
        v = self._v(T)
        d = self.device_index
        lp = _b._dev(logits, "logits", torch.float32, 2, device=d)
        xp = _b._dev(x, "x", torch.bfloat16, 2, device=d)
        if logits.shape[0] != T or logits.shape[1] != self.E or x.shape[1] != self.H:
            raise ValueError(f"logits must be [T, {self.E}] and x [T, {self.H}]")
        _b._check("moe_route_dispatch", _lib.load().moe_route_dispatch(
            lp, xp, T, self.E, self.k, n_group, topk_group, self.H, self.R, *v.route_dispatch_args,
            _b._stream(stream, x)))
        return v.topk_idx, v.topk_w, v.send, v.buf

    def dispatch_fp8(self, topk_idx: torch.Tensor, x: torch.Tensor, stream=None):
        """Send + fp8 receive; returns (SendResult, codes [T*k, H], scales [T*k, H/128])."""
        if self.buf_q is None:
            raise ValueError("constructed without fp8=True")
        T = self._t(x.shape[0])
        s = self._send(T)
        _b.moe_dispatch_fp8(topk_idx, x, self.E, self.R, buf_q=self.buf_q[: T * self.k],
                            buf_scale=self.buf_scale[: T * self.k],
                            expert_counts=s.expert_counts, expert_offsets=s.expert_offsets,
                            pair_row=s.pair_row, row_token=s.row_token,
                            rank_offsets=s.rank_offsets, workspace=self.workspace,
                            stream=stream)
        return s, self.buf_q[: T * self.k], self.buf_scale[: T * self.k]

    def route_dispatch_fp8(self, logits: torch.Tensor, x: torch.Tensor, n_group: int = 1,
                           topk_group: int = 1, stream=None):
        """Route + send + fp8 receive in one call; returns (topk_idx, topk_w,
        SendResult, codes [T*k, H], scales [T*k, H/128])."""
        if self.buf_q is None:
            raise ValueError("constructed without fp8=True")
        T = x.shape[0]
        v = self._v(T)
        d = self.device_index
        lp = _b._dev(logits, "logits", torch.float32, 2, device=d)
        xp = _b._dev(x, "x", torch.bfloat16, 2, device=d)
        if logits.shape[0] != T or logits.shape[1] != self.E or x.shape[1] != self.H:
            raise ValueError(f"logits must be [T, {self.E}] and x [T, {self.H}]")
        _b._check("moe_route_dispatch_fp8", _lib.load().moe_route_dispatch_fp8(
            lp, xp, T, self.E, self.k, n_group, topk_group, self.H, self.R,
            *v.route_dispatch_fp8_args, _b._stream(stream, x)))
        return v.topk_idx, v.topk_w, v.send, v.buf_q, v.buf_scale

    def combine(self, y: torch.Tensor, pair_row: torch.Tensor, topk_w: torch.Tensor,
                stream=None) -> torch.Tensor:
        v = self._v(pair_row.shape[0])
        if pair_row is not v.send.pair_row or topk_w is not v.topk_w:
            return _b.moe_combine(y, pair_row, topk_w, out=v.out, stream=stream)
        # This object's own routing views: only y is checked per call.
        yp = _b._dev(y, "y", torch.bfloat16, 2, device=self.device_index)
        if y.shape[1] != self.H:
            raise ValueError(f"y must be [capacity, {self.H}]")
        _b._check("moe_combine", _lib.load().moe_combine(
            yp, v.pair_row_ptr, v.topk_w_ptr, v.T, self.H, self.k, y.shape[0], v.out_ptr,
            _b._stream(stream, y)))
        return v.out


class _Views:
    """MoeBuffers' tensors cut to a batch of T tokens, and their device
    pointers in the order the C entry points take them."""

    def __init__(self, b: MoeBuffers, T: int):
        self.T = T
        self.topk_idx, self.topk_w = b.topk_idx[:T], b.topk_w[:T]
        self.buf = b.buf[: T * b.k]
        self.out = b.out[:T]
        self.send = _b.SendResult(b.expert_counts, b.expert_offsets, b.pair_row[:T],
                                  b.row_token[: T * b.k], b.rank_offsets)
        s = self.send
        self.route_dispatch_args = (
            self.topk_idx.data_ptr(), self.topk_w.data_ptr(), s.expert_counts.data_ptr(),
            s.expert_offsets.data_ptr(), s.pair_row.data_ptr(), s.row_token.data_ptr(),
            s.rank_offsets.data_ptr(), self.buf.data_ptr(), T * b.k,
            b.route_workspace.data_ptr(), b.route_workspace.numel())
        self.buf_q = self.buf_scale = self.route_dispatch_fp8_args = None
        if b.buf_q is not None:
            self.buf_q, self.buf_scale = b.buf_q[: T * b.k], b.buf_scale[: T * b.k]
            self.route_dispatch_fp8_args = (
                self.route_dispatch_args[:7]
                + (self.buf_q.data_ptr(), self.buf_scale.data_ptr())
                + self.route_dispatch_args[8:])
        self.pair_row_ptr = s.pair_row.data_ptr()
        self.topk_w_ptr = self.topk_w.data_ptr()
        self.out_ptr = self.out.data_ptr()
