"""moe_route_dispatch (route + send + recv in one call; small batches route
and send in one launch) against the separate calls and the oracle: every
output bit-identical, the workspace back at zero after every call, and
graph replays equal to eager calls."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import DEV, assert_step_matches_oracle, dev_bf16, dev_f32, host, host_bf16

pytestmark = pytest.mark.gpu


def _m():
    import combine_topk_route_amd as m

    return m


def _separate(m, logits, x, k, E, R):
    idx, w = m.moe_route_topk(logits, k)
    send, buf = m.moe_dispatch(idx, x, E, R)
    return idx, w, send, buf


def _same(a, b):
    ia, wa, sa, ba = a
    ib, wb, sb, bb = b
    assert torch.equal(ia, ib)
    assert torch.equal(wa.view(torch.int32), wb.view(torch.int32))
    for u, v in zip(sa, sb):
        assert torch.equal(u, v)
    assert torch.equal(ba.view(torch.int16), bb.view(torch.int16))


def _inputs(T, E, H, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    return logits, x


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_route_dispatch_matches_separate_calls_and_oracle(name):
    m = _m()
    wl = workloads.make(name, seed=3, with_y=False)
    cfg = wl.cfg
    print(f"\n[route_dispatch] {name} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    logits, x = dev_f32(wl.logits), dev_bf16(wl.x)
    got = m.moe_route_dispatch(logits, x, cfg.k, cfg.R)
    ref = _separate(m, logits, x, cfg.k, cfg.E, cfg.R)
    torch.cuda.synchronize()
    _same(got, ref)
    r_idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
    r_pr, r_rt = oracle.dispatch_slots(r_idx, cfg.E)
    assert np.array_equal(host(got[0]), r_idx)
    assert np.array_equal(host(got[2].pair_row), r_pr)
    assert np.array_equal(host(got[2].row_token), r_rt)
    rows = np.random.default_rng(1).choice(cfg.P, min(cfg.P, 512), replace=False)
    assert np.array_equal(host_bf16(got[3][torch.from_numpy(rows).to(DEV)]), wl.x[r_rt[rows]])


@pytest.mark.parametrize("T,E,k,R", [
    (1, 8, 2, 1), (5, 8, 8, 2), (7, 256, 8, 32),       # ragged single blocks
    (256, 256, 8, 32),      # P = 2048: one launch, 8-wave send
    (257, 256, 8, 32),      # P = 2056: one launch, 16-wave send, ragged last block
    (512, 512, 8, 64),      # P = 4096 at the 16-wave send's largest E
    (300, 1024, 8, 8),      # E > 512: one launch, 8-wave send in two steps
    (513, 256, 8, 32),      # P = 4104: separate launches
    (2049, 8, 2, 8),        # T above the one-wave-per-token routing
    (3000, 64, 1, 4),
])
def test_route_dispatch_shapes(T, E, k, R):
    m = _m()
    print(f"[route_dispatch] T={T} E={E} k={k} R={R}", flush=True)
    lg, xb = _inputs(T, E, 64, T * 7 + E)
    logits, x = dev_f32(lg), dev_bf16(xb)
    got = m.moe_route_dispatch(logits, x, k, R)
    ref = _separate(m, logits, x, k, E, R)
    torch.cuda.synchronize()
    _same(got, ref)
    r_idx, _, _ = oracle.route_topk(lg, k)
    assert np.array_equal(host(got[0]), r_idx)


def test_workspace_returns_to_zero_across_calls():
    """One workspace reused by calls of varying size on one stream: route and
    send in one launch (arrival counter), and separate launches where the
    routing kernel counts into the histogram matrix and recv clears it
    (one wave per token below 2049 tokens, lane groups above).  Repeated
    sizes would count twice if a clear were missed.  Each call matches the
    separate calls, and the whole workspace is zero after each."""
    m = _m()
    E, k, R, H = 256, 8, 32, 64
    wsb = m.moe_route_dispatch_workspace_bytes(8192, E, k)
    ws = torch.zeros((wsb,), dtype=torch.uint8, device=DEV)
    for i, T in enumerate([128, 300, 4096, 4096, 64, 600, 600, 8192, 1, 511, 2000, 2000, 3001,
                           200]):
        lg, xb = _inputs(T, E, H, 100 + i)
        logits, x = dev_f32(lg), dev_bf16(xb)
        got = m.moe_route_dispatch(logits, x, k, R, workspace=ws)
        ref = _separate(m, logits, x, k, E, R)
        torch.cuda.synchronize()
        _same(got, ref)
        assert int(ws.count_nonzero().item()) == 0, T


@pytest.mark.parametrize("E,k,R", [(64, 8, 8), (127, 4, 1), (128, 8, 16), (1024, 8, 32)])
def test_workspace_zero_around_the_counting_threshold(E, k, R):
    """Multi-block sends on both sides of the expert count from which the
    routing kernel counts the histogram itself (below it the histogram
    kernel fills the matrix, and the rank kernel zeroes it either way):
    repeated calls of two sizes on one workspace."""
    m = _m()
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(4096, E, k),), dtype=torch.uint8,
                     device=DEV)
    for i, T in enumerate([4096, 4096, 1500, 1500, 4096]):
        print(f"[route_dispatch] workspace E={E} T={T} k={k}", flush=True)
        lg, xb = _inputs(T, E, 64, 7 * E + i)
        logits, x = dev_f32(lg), dev_bf16(xb)
        got = m.moe_route_dispatch(logits, x, k, R, workspace=ws)
        ref = _separate(m, logits, x, k, E, R)
        torch.cuda.synchronize()
        _same(got, ref)
        assert int(ws.count_nonzero().item()) == 0, (E, T)


@pytest.mark.parametrize("T,E,k,R", [(3000, 8, 1, 8), (4096, 8, 1, 1)])
def test_route_dispatch_single_block_send_above_one_wave_routing(T, E, k, R):
    """T above 2048 with T*k <= 4096: lane-group routing without counting,
    then the single-block send."""
    m = _m()
    print(f"[route_dispatch] T={T} E={E} k={k} R={R}", flush=True)
    lg, xb = _inputs(T, E, 64, T + E)
    logits, x = dev_f32(lg), dev_bf16(xb)
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                     device=DEV)
    for _ in range(2):
        got = m.moe_route_dispatch(logits, x, k, R, workspace=ws)
        ref = _separate(m, logits, x, k, E, R)
        torch.cuda.synchronize()
        _same(got, ref)
        assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("T,G,TG", [(200, 1, 1), (300, 1, 1), (4096, 1, 1), (4096, 8, 4)])
def test_route_dispatch_graph_replays(T, G, TG):
    """The call captured once into a HIP graph and replayed three times, with
    eager work and a synchronisation between replays, then once more on new
    inputs: every replay matches the oracle (indices, counts, offsets, rows
    and dispatched bytes bit-exact, weights within 2^-20) and the eager
    result, and leaves the workspace zero (200 tokens: routing, then send +
    recv in one launch; 300: route and send in one launch; 4096: the counting
    route and the rank kernel that clears the matrix, with plain and with
    group-limited routing)."""
    m = _m()
    E, k, R, H = 256, 8, 32, 128
    lg, xb = _inputs(T, E, H, 5)
    logits, x = dev_f32(lg), dev_bf16(xb)
    bufs = m.MoeBuffers(T, H, E, k, R)
    res = bufs.route_dispatch(logits, x, G, TG)
    eager = [t.clone() for t in (res[0], bufs.buf[: T * k])]
    torch.cuda.synchronize()
    groups = dict(n_group=G, topk_group=TG) if TG < G else {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bufs.route_dispatch(logits, x, G, TG)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bufs.route_dispatch(logits, x, G, TG)
    for rep in range(3):
        bufs.topk_idx.fill_(-1)
        bufs.buf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[route_dispatch] graph T={T} groups {TG}/{G}: replay {rep}", flush=True)
        assert torch.equal(bufs.topk_idx[:T], eager[0])
        assert torch.equal(bufs.buf[: T * k].view(torch.int16), eager[1].view(torch.int16))
        assert_step_matches_oracle(lg, xb, k, E, R, res[0], res[1], res[2], res[3], **groups)
        assert int(bufs.route_workspace.count_nonzero().item()) == 0
    lg2, xb2 = _inputs(T, E, H, 6)  # new inputs, same graph
    logits.copy_(dev_f32(lg2))
    x.copy_(dev_bf16(xb2))
    g.replay()
    torch.cuda.synchronize()
    assert_step_matches_oracle(lg2, xb2, k, E, R, res[0], res[1], res[2], res[3], **groups)
    assert int(bufs.route_workspace.count_nonzero().item()) == 0


@pytest.mark.parametrize("T,E,k,G,TG,R", [
    (128, 256, 8, 8, 4, 32),     # DeepSeek-V3 shape, decode-sized: one launch
    (300, 384, 8, 8, 4, 48),     # 16-wave single-block send in the same launch
    (4096, 256, 8, 8, 4, 32),    # separate launches
    (77, 384, 8, 48, 6, 48),     # many small groups
])
def test_grouped_route_dispatch_matches_separate_calls(T, E, k, G, TG, R):
    m = _m()
    print(f"[route_dispatch] grouped T={T} E={E} k={k} groups {TG}/{G}", flush=True)
    lg, xb = _inputs(T, E, 64, T + 11 * E)
    logits, x = dev_f32(lg), dev_bf16(xb)
    got = m.moe_route_dispatch(logits, x, k, R, n_group=G, topk_group=TG)
    idx, w = m.moe_route_topk_grouped(logits, k, G, TG)
    send, buf = m.moe_dispatch(idx, x, E, R)
    torch.cuda.synchronize()
    _same(got, (idx, w, send, buf))
    r_idx, _, _ = oracle.route_topk_grouped(lg, k, G, TG)
    assert np.array_equal(host(got[0]), r_idx)


@pytest.mark.parametrize("T,E,k,R", [
    (2049, 8, 3, 8),     # 48 pairs per 16-token tile: tiles straddle histogram rows
    (5003, 100, 5, 4),   # odd E, ragged last tile
    (2100, 127, 16, 1),  # the largest E below the threshold, k = 16: 256 pairs per tile
    (9000, 2, 2, 2),
    (5000, 1, 1, 1),     # one expert: every pair in one bin
    (3000, 12, 7, 4),
    (1100, 64, 4, 8),    # below 2049 tokens: the lane-group kernel routes these too
    (1025, 8, 8, 1),     # P = 8200, ragged last tile
])
def test_route_dispatch_counts_few_experts_in_lds(T, E, k, R):
    """E < 128 with a multi-block send: the lane-group routing kernel counts
    each 16-token tile's pairs in LDS and adds them to the histogram matrix.
    Against the separate calls and the oracle, twice on one workspace, which
    is zero after each call."""
    m = _m()
    print(f"[route_dispatch] lds counting T={T} E={E} k={k} R={R}", flush=True)
    lg, xb = _inputs(T, E, 64, T * 3 + E + k)
    logits, x = dev_f32(lg), dev_bf16(xb)
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                     device=DEV)
    ref = _separate(m, logits, x, k, E, R)
    for _ in range(2):
        got = m.moe_route_dispatch(logits, x, k, R, workspace=ws)
        torch.cuda.synchronize()
        _same(got, ref)
        assert int(ws.count_nonzero().item()) == 0
    r_idx, _, _ = oracle.route_topk(lg, k)
    assert np.array_equal(host(got[0]), r_idx)
    pr, _ = oracle.dispatch_slots(r_idx, E)
    assert np.array_equal(host(got[2].pair_row), pr)
