"""Send, recv and combine on different HIP streams joined by events (the
send/recv split exists so other work can run between them), and the
block-loop path of the row kernels (more row units than one launch holds)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import dev_bf16, dev_f32, dev_i32, host, host_bf16

pytestmark = pytest.mark.gpu


def test_send_recv_combine_on_separate_streams():
    import combine_topk_route_amd as m

    wl = workloads.make("mixtral", seed=5)
    cfg = wl.cfg
    print("[streams] mixtral on three streams", flush=True)
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    logits = dev_f32(wl.logits)
    x = dev_bf16(wl.x)
    y = dev_bf16(wl.y)
    torch.cuda.synchronize()
    idx, w = m.moe_route_topk(logits, cfg.k, stream=s1)
    send = m.moe_dispatch_send(idx, cfg.E, cfg.R, stream=s1)
    e1 = torch.cuda.Event()
    e1.record(s1)
    s2.wait_event(e1)
    buf = m.moe_dispatch_recv(x, send.pair_row, stream=s2)
    s3.wait_event(e1)
    out = m.moe_combine(y, send.pair_row, w, stream=s3)
    torch.cuda.synchronize()
    r_idx, _, r_w32 = oracle.route_topk(wl.logits, cfg.k)
    pr, rt = oracle.dispatch_slots(r_idx, cfg.E)
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host_bf16(buf), wl.x[rt])
    ref = oracle.combine(wl.y, pr, host(w))
    assert np.array_equal(host_bf16(out), ref)


def test_row_kernels_loop_when_units_exceed_one_launch():
    # H = 8 gives one 16-byte chunk per row, so units = T; T above 2^21
    # makes the recv and combine grids loop over their units.
    import combine_topk_route_amd as m

    T, H, k = (1 << 21) + 4099, 8, 1
    print(f"[streams] block-loop path T={T} H={H} k={k}", flush=True)
    rng = np.random.default_rng(8)
    x = rng.integers(0, 2**16, (T, H)).astype(np.uint16)
    x[((x >> 7) & 0xFF) == 0xFF] &= 0x807F
    pr = rng.permutation(T).reshape(T, k).astype(np.int32)
    buf = m.moe_dispatch_recv(dev_bf16(x), dev_i32(pr))
    w = np.ones((T, k), np.float32)
    out = m.moe_combine(buf, dev_i32(pr), dev_f32(w))
    torch.cuda.synchronize()
    hb = host_bf16(buf)
    expect = np.empty_like(x)
    expect[pr[:, 0]] = x
    assert np.array_equal(hb, expect)
    # k = 1 with weight 1: out = x except -0 -> +0
    assert np.array_equal(host_bf16(out), np.where(x == 0x8000, np.uint16(0), x))


@pytest.mark.parametrize("sizes", [(300, 333), (100, 200)])
def test_route_dispatch_on_two_streams_at_once(sizes):
    """Two batches through moe_route_dispatch on two streams at the same time,
    each with its own workspace: at 300 and 333 tokens one route + send launch
    each, so two arrival counters are live together; at 100 and 200 tokens
    routing, then one send + recv launch each.  Both match the oracle, and
    both workspaces are back at zero."""
    import combine_topk_route_amd as m

    print(f"[streams] route_dispatch, two streams, T={sizes}", flush=True)
    E, k, R, H = 256, 8, 32, 256
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = []
    for i, T in enumerate(sizes):
        rng = np.random.default_rng(40 + i)
        lg = rng.standard_normal((T, E)).astype(np.float32)
        xb = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
        ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                         device="cuda")
        cases.append((lg, xb, dev_f32(lg), dev_bf16(xb), ws))
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        for (lg, xb, logits, x, ws), st in zip(cases, streams):
            results.append(m.moe_route_dispatch(logits, x, k, R, workspace=ws, stream=st))
    torch.cuda.synchronize()
    for i, (lg, xb, logits, x, ws) in enumerate(cases):
        idx, w, send, buf = results[-2 + i]
        r_idx, _, _ = oracle.route_topk(lg, k)
        pr, rt = oracle.dispatch_slots(r_idx, E)
        assert np.array_equal(host(idx), r_idx)
        assert np.array_equal(host(send.pair_row), pr)
        assert np.array_equal(host_bf16(buf), xb[rt])
        assert int(ws.count_nonzero().item()) == 0


def test_binding_allocates_on_the_launch_stream():
    """Called with ``stream=`` a side stream and no outputs or workspace, the
    binding allocates them (and zero-fills moe_route_dispatch's workspace) on
    that stream.  The side stream is kept busy first, and work on the current
    stream right after each call allocates and fills blocks of the same size;
    the results must still match the oracle."""
    import combine_topk_route_amd as m
    from gpuhelp import DEV, assert_step_matches_oracle

    T, E, k, R, H = 4096, 256, 8, 32, 512
    rng = np.random.default_rng(21)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xb = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    logits, x = dev_f32(lg), dev_bf16(xb)
    side = torch.cuda.Stream()
    busy = torch.ones((1 << 26,), device=DEV)
    ws_send = m.moe_dispatch_workspace_bytes(T, E, k)
    ws_route = m.moe_route_dispatch_workspace_bytes(T, E, k)
    assert ws_send > 0 and ws_route > 0
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[streams] binding allocations on a side stream, rep {rep}", flush=True)
        with torch.cuda.stream(side):
            busy.mul_(1.0)
        idx, w = m.moe_route_topk(logits, k, stream=side)
        send = m.moe_dispatch_send(idx, E, R, stream=side)
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV)
                for n in (ws_send, ws_route, T * k * 4)]
        buf = m.moe_dispatch_recv(x, send.pair_row, stream=side)
        torch.cuda.synchronize()
        assert_step_matches_oracle(lg, xb, k, E, R, idx, w, send, buf)
        del junk
        with torch.cuda.stream(side):
            busy.mul_(1.0)
        idx2, w2, send2, buf2 = m.moe_route_dispatch(logits, x, k, R, stream=side)
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device=DEV)
                for n in (ws_send, ws_route, T * k * 4)]
        torch.cuda.synchronize()
        assert_step_matches_oracle(lg, xb, k, E, R, idx2, w2, send2, buf2)
        del junk, idx, w, send, buf, idx2, w2, send2, buf2
