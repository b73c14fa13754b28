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
        # route_dispatch's own workspace: its leading arrival counter starts at
        # zero and every call leaves it at zero.
        rws = _b.moe_route_dispatch_workspace_bytes(max_tokens, num_experts, k)
        self.route_workspace = torch.zeros((max(rws, 1),), dtype=torch.uint8, device=dev)
        self.buf = torch.empty((cap, hidden), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((max_tokens, hidden), dtype=torch.bfloat16, device=dev)
        self.buf_q = self.buf_scale = None
        if fp8:
            self.buf_q = torch.empty((cap, hidden), dtype=torch.uint8, device=dev)
            self.buf_scale = torch.empty((cap, hidden // 128), dtype=f32, device=dev)

    def _t(self, T: int) -> int:
        if not 0 <= T <= self.max_tokens:
            raise ValueError(f"batch of {T} tokens exceeds max_tokens={self.max_tokens}")
        return T

    def _send(self, T):
        return _b.SendResult(self.expert_counts, self.expert_offsets, self.pair_row[:T],
                             self.row_token[: T * self.k], self.rank_offsets)

    def route(self, logits: torch.Tensor, n_group: int = 1, topk_group: int = 1, stream=None):
        T = self._t(logits.shape[0])
        idx, w = self.topk_idx[:T], self.topk_w[:T]
        if n_group == 1:
            return _b.moe_route_topk(logits, self.k, topk_idx=idx, topk_w=w, stream=stream)
        return _b.moe_route_topk_grouped(logits, self.k, n_group, topk_group, topk_idx=idx,
                                         topk_w=w, stream=stream)

    def dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor, stream=None):
        """Send + receive; returns (SendResult, buf [T*k, H])."""
        T = self._t(x.shape[0])
        s = self._send(T)
        _b.moe_dispatch(topk_idx, x, self.E, self.R, buf=self.buf[: T * self.k],
                        expert_counts=s.expert_counts, expert_offsets=s.expert_offsets,
                        pair_row=s.pair_row, row_token=s.row_token, rank_offsets=s.rank_offsets,
                        workspace=self.workspace, stream=stream)
        return s, self.buf[: T * self.k]

    def route_dispatch(self, logits: torch.Tensor, x: torch.Tensor, n_group: int = 1,
                       topk_group: int = 1, stream=None):
        """Route + send + receive in one call; returns (topk_idx, topk_w,
        SendResult, buf [T*k, H])."""
        T = self._t(x.shape[0])
        s = self._send(T)
        _b.moe_route_dispatch(logits, x, self.k, self.R, n_group=n_group, topk_group=topk_group,
                              topk_idx=self.topk_idx[:T],
                              topk_w=self.topk_w[:T], buf=self.buf[: T * self.k],
                              expert_counts=s.expert_counts, expert_offsets=s.expert_offsets,
                              pair_row=s.pair_row, row_token=s.row_token,
                              rank_offsets=s.rank_offsets, workspace=self.route_workspace,
                              stream=stream)
        return self.topk_idx[:T], self.topk_w[:T], s, self.buf[: T * self.k]

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

    def combine(self, y: torch.Tensor, pair_row: torch.Tensor, topk_w: torch.Tensor,
                stream=None) -> torch.Tensor:
        T = self._t(pair_row.shape[0])
        return _b.moe_combine(y, pair_row, topk_w, out=self.out[:T], stream=stream)
