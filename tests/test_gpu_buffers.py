"""MoeBuffers: preallocated buffers give the same results as the plain
calls, allocate nothing per step, serve batches smaller than max_tokens, and
can be captured into a HIP graph."""
import numpy as np
import pytest
import torch

import workloads
from gpuhelp import assert_step_matches_oracle, dev_bf16, dev_f32, host_bf16

pytestmark = pytest.mark.gpu


def test_buffers_match_plain_calls_and_do_not_allocate():
    import combine_topk_route_amd as m

    cfg = workloads.CONFIGS["kimi_k2"]
    mb = m.MoeBuffers(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, fp8=True)
    for T in (cfg.T, 1000, 1):
        wl = workloads.make(cfg, seed=T, T=T)
        print(f"[buffers] kimi_k2 T={T}", flush=True)
        logits, x, y = dev_f32(wl.logits), dev_bf16(wl.x), dev_bf16(wl.y)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        idx, w = mb.route(logits)
        send, buf = mb.dispatch(idx, x)
        out = mb.combine(y, send.pair_row, w)
        s8, q, sc = mb.dispatch_fp8(idx, x)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        r_idx, r_w = m.moe_route_topk(logits, cfg.k)
        r_send, r_buf = m.moe_dispatch(r_idx, x, cfg.E, cfg.R)
        r_out = m.moe_combine(y, r_send.pair_row, r_w)
        _, r_q, r_sc = m.moe_dispatch_fp8(r_idx, x, cfg.E, cfg.R)
        torch.cuda.synchronize()
        assert torch.equal(idx, r_idx) and torch.equal(w, r_w)
        for a, b in zip(send, r_send):
            assert torch.equal(a, b)
        assert np.array_equal(host_bf16(buf), host_bf16(r_buf))
        assert np.array_equal(host_bf16(out), host_bf16(r_out))
        assert torch.equal(q, r_q) and torch.equal(sc, r_sc)
        # The one-call forms (combine on the object's own routing views takes
        # the path that checks only y) allocate nothing either.
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        idx2, w2, send2, buf2 = mb.route_dispatch(logits, x)
        out2 = mb.combine(y, send2.pair_row, w2)
        i8, w8, s8b, q2, sc2 = mb.route_dispatch_fp8(logits, x)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(idx2, r_idx) and torch.equal(w2, r_w)
        for a, b in zip(send2, r_send):
            assert torch.equal(a, b)
        assert np.array_equal(host_bf16(buf2), host_bf16(r_buf))
        assert np.array_equal(host_bf16(out2), host_bf16(r_out))
        assert torch.equal(i8, r_idx) and torch.equal(q2, r_q) and torch.equal(sc2, r_sc)
        assert int(mb.route_workspace.count_nonzero().item()) == 0
    with pytest.raises(ValueError):
        mb.route(torch.zeros((cfg.T + 1, cfg.E), device="cuda"))


def test_buffers_in_a_graph_with_a_smaller_batch():
    """A batch smaller than max_tokens captured into a HIP graph: every
    replay, and a replay on new inputs, matches the oracle (routing,
    dispatch and combine on the kernel's own weights) and the eager run."""
    import combine_topk_route_amd as m

    cfg = workloads.CONFIGS["dsv3_decode"]
    mb = m.MoeBuffers(256, cfg.H, cfg.E, cfg.k, cfg.R)
    wl = workloads.make(cfg, seed=11)
    wl2 = workloads.make(cfg, seed=12, with_y=False)
    logits, x, y = dev_f32(wl.logits), dev_bf16(wl.x), dev_bf16(wl.y)
    print("[buffers] graph capture, T=128 of max 256", flush=True)

    def step():
        idx, w = mb.route(logits)
        send, buf = mb.dispatch(idx, x)
        return idx, w, send, buf, mb.combine(y, send.pair_row, w)

    res = step()
    eager = host_bf16(res[4]).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        mb.out.fill_(0)
        mb.buf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(res[4]), eager)
        assert_step_matches_oracle(wl.logits, wl.x, cfg.k, cfg.E, cfg.R, *res[:4], y_bits=wl.y,
                                   out=res[4])
    logits.copy_(dev_f32(wl2.logits))
    x.copy_(dev_bf16(wl2.x))
    g.replay()
    torch.cuda.synchronize()
    assert_step_matches_oracle(wl2.logits, wl2.x, cfg.k, cfg.E, cfg.R, *res[:4], y_bits=wl.y,
                               out=res[4])
