"""GPU edge cases: ties, degenerate shapes, ragged tiles, path switches,
canaries, determinism, and the identity-expert round trip."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import (DEV, assert_out_close, assert_weights_close, dev_bf16, dev_f32, dev_i32,
                     host, host_bf16)

pytestmark = pytest.mark.gpu


def _m():
    import combine_topk_route_amd as m

    return m


def _rand_bf16(shape, seed):
    rng = np.random.default_rng(seed)
    return workloads.bf16_from_f32(rng.standard_normal(shape).astype(np.float32))


ROUTE_WAVE_MAX_TOKENS = 2048   # larger batches switch to the lane-group routing kernel


def _route_check(logits, k):
    """Routing of ``logits`` against the oracle, as given (a small batch:
    one wave per token) and tiled past 2048 tokens with a ragged tail (the
    lane-group kernel, whose lanes per token depend on T, E and k)."""
    m = _m()
    T = logits.shape[0]
    big_T = ROUTE_WAVE_MAX_TOKENS + 53 + T % 7
    big = np.tile(logits, (-(-big_T // T), 1))[:big_T]
    out = None
    for lg in ([logits, big] if T <= ROUTE_WAVE_MAX_TOKENS else [logits]):
        print(f"[edges] route T={lg.shape[0]} E={lg.shape[1]} k={k}", flush=True)
        idx, w = m.moe_route_topk(dev_f32(lg), k)
        torch.cuda.synchronize()
        r_idx, r_w, _ = oracle.route_topk(lg, k)
        assert np.array_equal(host(idx), r_idx)
        assert_weights_close(host(w), r_w)
        if out is None:
            out = host(idx), host(w)
    return out


# ------------------------------------------------------------------ routing

def test_route_ties_and_signed_zeros():
    E = 256
    logits = np.random.default_rng(1).standard_normal((64, E)).astype(np.float32)
    logits[0] = 0.25                               # all equal
    logits[1, :] = -3.0
    logits[1, 100:120] = 2.0                        # 20 equal values straddle k = 8
    logits[2, :] = -1.0
    logits[2, 7], logits[2, 3] = 0.0, -0.0          # +0 / -0 tie
    logits[3] = np.round(logits[3] * 2) / 2         # many half-integer ties
    logits[4, ::3] = 1.5                            # ties spread over all lanes
    idx, w = _route_check(logits, 8)
    assert idx[0].tolist() == list(range(8))
    assert idx[1].tolist() == list(range(100, 108))
    assert idx[2, :2].tolist() == [3, 7]


@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (5, 8, 8), (33, 1, 1), (7, 2, 2), (100, 64, 32),
                                   (129, 1024, 32), (70, 1000, 7), (3, 65, 3), (257, 384, 8)])
def test_route_shapes(T, E, k):
    logits = np.random.default_rng(T * E + k).standard_normal((T, E)).astype(np.float32)
    _route_check(logits, k)


@pytest.mark.parametrize("T,E,k", [(40, 500, 8), (40, 700, 12), (64, 256, 20), (9, 40, 32),
                                   (31, 200, 5)])
def test_route_lane_group_shapes(T, E, k):
    """Shapes that switch the lanes per token (16, 32, 64), the experts per
    lane and the 16-byte loads (E % 4 != 0 turns them off)."""
    logits = np.random.default_rng(T + E * k).standard_normal((T, E)).astype(np.float32)
    _route_check(logits, k)


@pytest.mark.parametrize("T,E,k", [
    (16384, 256, 8),     # 16 lanes per token, 16 experts per lane, 16-byte loads
    (16390, 384, 8),     # 16 lanes, 24 experts per lane, ragged last wave
    (8200, 512, 8),      # 32 lanes, 16 experts per lane
    (8200, 640, 6),      # 32 lanes, 24 per lane (20 used)
    (16400, 130, 4),     # 16 lanes, 16 per lane (9 used), scalar loads (E % 4 != 0)
    (16384, 200, 17),    # k > 16: 32 lanes, lane g < k reports winner g
])
def test_route_large_batches(T, E, k):
    """Batch sizes at which the routing kernel uses its fewest lanes per
    token (16 or 32) and most experts per lane, with Zipf-skewed logits so
    that winners crowd into a few lanes."""
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits += np.log(np.arange(1, E + 1, dtype=np.float64) ** -1.1)[rng.permutation(E)].astype(
        np.float32)
    _route_check(logits, k)


def test_route_winners_crowded_into_one_lane():
    """Many winners held by one lane of a token (consecutive experts), with
    ties among them: the lane's cache of best candidates empties and is
    refilled during the k rounds."""
    rng = np.random.default_rng(11)
    E = 256
    logits = rng.standard_normal((48, E)).astype(np.float32)
    for t in range(48):
        lo = (t % 16) * 16                       # the experts of one lane
        logits[t, lo:lo + 16] = 5.0 + rng.integers(0, 4, 16).astype(np.float32)
    logits[0, 0:16] = 7.0                        # one lane, all equal
    logits[1, 16:32] = np.float32(-0.0)          # signed zeros, rest below
    logits[1, :16] = -4.0
    logits[1, 32:] = -4.0
    for k in (8, 16, 20, 32):
        idx, _ = _route_check(logits, k)
        assert idx[0, :min(k, 16)].tolist() == list(range(min(k, 16)))


def test_route_wide_logit_range():
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((200, 256)) * 20).astype(np.float32)
    _route_check(logits, 8)


def test_route_logits_further_apart_than_the_fp32_range():
    """Finite logits whose differences overflow fp32 (the winners' weights
    then include exact zeros): weights stay finite and match the float64
    oracle; indices are exact.  Both routing kernels (as given and tiled)."""
    rng = np.random.default_rng(6)
    fmax = np.float32(3.4e38)
    logits = rng.standard_normal((64, 256)).astype(np.float32)
    logits[0, 3], logits[0, 200] = fmax, -fmax            # k-th winner far below the first
    logits[1, :] = -fmax
    logits[1, 17] = fmax                                  # every other expert overflows
    logits[2, :8] = np.float32(2e38)
    logits[2, 8:] = np.float32(-2e38)                     # eight equal winners, the rest at -2e38
    logits[3, ::2] = np.float32(1e38)
    logits[3, 1::2] = np.float32(-3e38)
    logits[4, 5] = np.float32(3.3e38)
    logits[4, 6] = np.float32(-1e38)                      # 4.3e38 below the first
    idx, w = _route_check(logits, 8)
    assert np.all(np.isfinite(w))
    assert w[1, 0] == 1.0 and np.all(w[1, 1:] == 0.0)


@pytest.mark.parametrize("T,E,k,G,TG", [(3000, 256, 8, 8, 4), (2500, 384, 8, 8, 4),
                                        (100, 256, 8, 8, 4)])
def test_route_logits_only_4_byte_aligned(T, E, k, G, TG):
    """Logits one float into their buffer: the lane-group kernel loads them
    one float at a time, and group-limited routing falls back to the wave
    kernel.  Plain routing equals the aligned call bit for bit; every result
    matches the oracle; the one-call path (which counts the send histogram
    in the routing kernel here) matches too."""
    m = _m()
    rng = np.random.default_rng(T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    flat = torch.empty(T * E + 1, dtype=torch.float32, device=DEV)
    mis = flat[1:].view(T, E)
    mis.copy_(torch.from_numpy(lg))
    assert mis.data_ptr() % 16 == 4
    al = dev_f32(lg)
    print(f"[edges] 4-byte aligned logits T={T} E={E} k={k} groups {TG}/{G}", flush=True)
    a_idx, a_w = m.moe_route_topk(mis, k)
    b_idx, b_w = m.moe_route_topk(al, k)
    g_idx, g_w = m.moe_route_topk_grouped(mis, k, G, TG)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_w.view(torch.int32), b_w.view(torch.int32))
    r_idx, r_w, _ = oracle.route_topk(lg, k)
    assert np.array_equal(host(a_idx), r_idx)
    assert_weights_close(host(a_w), r_w)
    r_idx, r_w, _ = oracle.route_topk_grouped(lg, k, G, TG)
    assert np.array_equal(host(g_idx), r_idx)
    assert_weights_close(host(g_w), r_w)
    x = dev_bf16(workloads.bf16_from_f32(rng.standard_normal((T, 64)).astype(np.float32)))
    idx, w, send, buf = m.moe_route_dispatch(mis, x, k, 8)
    torch.cuda.synchronize()
    assert torch.equal(idx, b_idx) and torch.equal(w.view(torch.int32), b_w.view(torch.int32))
    pr, rt = oracle.dispatch_slots(host(b_idx), E)
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host(send.row_token), rt)


# ------------------------------------------------------------------ dispatch send

def _send_check(idx, E, R):
    m = _m()
    T, k = idx.shape
    print(f"[edges] send T={T} k={k} E={E} R={R} (P={T * k})", flush=True)
    res = m.moe_dispatch_send(dev_i32(idx), E, R)
    torch.cuda.synchronize()
    counts = oracle.expert_counts(idx, E)
    off = oracle.expert_offsets(counts)
    pr, rt = oracle.dispatch_slots(idx, E)
    assert np.array_equal(host(res.expert_counts), counts)
    assert np.array_equal(host(res.expert_offsets), off)
    assert np.array_equal(host(res.rank_offsets), oracle.rank_offsets(off, R))
    assert np.array_equal(host(res.pair_row), pr)
    assert np.array_equal(host(res.row_token), rt)
    return res


@pytest.mark.parametrize("T,k,E,R", [
    (1, 1, 1, 1),          # one pair
    (16, 2, 8, 1),
    (256, 8, 256, 32),     # P = 2048: largest one-step 8-wave block
    (2049, 1, 64, 4),      # P = 2049: 16-wave single block, ragged wave ranges
    (300, 8, 512, 16),     # P = 2400: 16-wave block at its largest E
    (400, 8, 1024, 8),     # P = 3200, E > 512: 8-wave block in two steps
    (512, 8, 256, 32),     # P = 4096: largest single-block case
    (513, 8, 256, 32),     # P = 4104: first multi-block case, ragged last block
    (3001, 3, 7, 7),       # odd sizes, small E
    (4096, 8, 1024, 8),    # E = 1024: few blocks with big chunks
    (20000, 8, 384, 48),
    (65536, 8, 256, 32),   # many blocks
])
def test_send_random_routes(T, k, E, R):
    rng = np.random.default_rng(T + E)
    idx = np.argsort(rng.standard_normal((T, E)), axis=1)[:, :k].astype(np.int32)
    _send_check(idx, E, R)


def test_send_all_tokens_one_expert_and_duplicates():
    # all pairs to one expert (the hottest possible skew), and repeated experts
    # within a token (dispatch does not need k distinct experts)
    _send_check(np.full((3000, 4), 5, np.int32), 64, 8)
    _send_check(np.full((300, 2), 0, np.int32), 8, 1)
    rng = np.random.default_rng(3)
    _send_check(rng.integers(0, 16, (5000, 8)).astype(np.int32), 16, 4)
    _send_check(rng.integers(0, 3, (700, 5)).astype(np.int32), 300, 3)   # mostly empty experts


def test_send_drops_out_of_range_experts():
    m = _m()
    idx = np.array([[0, 9], [-1, 1], [1, 1]], np.int32)   # 9 and -1 are outside [0, 4)
    res = m.moe_dispatch_send(dev_i32(idx), 4, 1)
    torch.cuda.synchronize()
    assert host(res.expert_counts).tolist() == [1, 3, 0, 0]
    assert host(res.expert_offsets).tolist() == [0, 1, 4, 4, 4]
    pr = host(res.pair_row)
    assert pr.tolist() == [[0, -1], [-1, 1], [2, 3]]
    assert host(res.row_token)[:4].tolist() == [0, 1, 2, 2]


@pytest.mark.parametrize("T,k,E,R,H", [
    (1, 1, 1, 1, 8), (3, 2, 4, 1, 64), (16, 2, 8, 1, 256), (128, 8, 256, 32, 7168),
    (256, 8, 256, 32, 1032), (300, 6, 40, 8, 8200), (2048, 1, 7, 7, 64), (683, 3, 1000, 8, 136),
])
def test_dispatch_in_one_launch_matches_send_then_recv(T, k, E, R, H):
    """moe_dispatch runs send and recv in one launch for T*k <= 2048 and
    k <= 8 (block 0 sends; the other blocks find their rows from topk_idx).
    Against moe_dispatch_send then moe_dispatch_recv, with out-of-range
    experts (dropped), repeated experts inside a token, spare capacity and
    canary rows: every output and every buffer byte identical."""
    m = _m()
    print(f"[edges] dispatch one launch T={T} k={k} E={E} R={R} H={H}", flush=True)
    rng = np.random.default_rng(T * 7 + k * 3 + E)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    drop = rng.random((T, k)) < 0.05
    idx[drop] = rng.choice(np.array([-1, E, E + 5, -(2 ** 31)], np.int32), int(drop.sum()))
    if T > 2:
        idx[1, :] = idx[0, 0] if idx[0, 0] >= 0 else 0   # one expert repeated inside a token
    x = _rand_bf16((T, H), T + H)
    cap = T * k + 5
    canary = np.uint16(0x7FA5)
    bufs = []
    for one_call in (True, False):
        buf = dev_bf16(np.full((cap, H), canary, np.uint16))
        if one_call:
            res, _ = m.moe_dispatch(dev_i32(idx), dev_bf16(x), E, R, buf=buf, capacity=cap)
        else:
            res = m.moe_dispatch_send(dev_i32(idx), E, R)
            m.moe_dispatch_recv(dev_bf16(x), res.pair_row, buf=buf, capacity=cap)
        torch.cuda.synchronize()
        bufs.append((res, host_bf16(buf)))
    (a, ba), (b, bb) = bufs
    n_valid = int(host(a.expert_offsets)[E])   # row_token past this is left untouched
    for name in ("expert_counts", "expert_offsets", "pair_row", "rank_offsets"):
        assert np.array_equal(host(getattr(a, name)), host(getattr(b, name))), name
    assert np.array_equal(host(a.row_token)[:n_valid], host(b.row_token)[:n_valid])
    assert n_valid == int((idx >= 0).sum() - ((idx >= E).sum()))
    assert np.array_equal(ba, bb)
    assert (ba[n_valid:] == canary).all()


# ------------------------------------------------------------------ recv / combine

@pytest.mark.parametrize("T,H,k", [(1, 8, 1), (3, 8, 2), (37, 296, 3), (1000, 4096, 2),
                                   (129, 7168, 8), (5, 520, 10), (64, 1024, 32), (300, 64, 4),
                                   (3, 1 << 20, 2), (2, 1 << 20, 8)])   # the widest rows allowed
def test_recv_and_combine_ragged_shapes(T, H, k):
    m = _m()
    print(f"[edges] recv/combine T={T} H={H} k={k}", flush=True)
    rng = np.random.default_rng(T * H + k)
    P = T * k
    cap = P + 3
    pr = rng.permutation(P).reshape(T, k)
    x = _rand_bf16((T, H), seed=T + 1)
    buf = torch.full((cap, H), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    m.moe_dispatch_recv(dev_bf16(x), dev_i32(pr), buf=buf)
    y = _rand_bf16((cap, H), seed=T + 2)
    w = rng.random((T, k)).astype(np.float32)
    out = m.moe_combine(dev_bf16(y), dev_i32(pr), dev_f32(w))
    torch.cuda.synchronize()
    fill = np.full((cap, H), 0x1234, np.uint16)
    assert np.array_equal(host_bf16(buf), oracle.dispatch_rows(x, pr, cap, fill))
    ref = oracle.combine(y, pr, w)
    assert assert_out_close(host_bf16(out), ref) == 0


def test_combine_zero_and_negative_zero_rows():
    m = _m()
    T, H, k = 4, 64, 3
    y = np.zeros((T * k, H), np.uint16)
    y[1::2] = 0x8000                                 # -0.0 rows
    pr = np.arange(T * k).reshape(T, k)
    w = np.full((T, k), 0.5, np.float32)
    w[0] = -0.5
    out = host_bf16(m.moe_combine(dev_bf16(y), dev_i32(pr), dev_f32(w)))
    torch.cuda.synchronize()
    assert np.array_equal(out, oracle.combine(y, pr, w))


def test_combine_rounding_edges():
    # values around bf16 rounding ties, subnormals, large magnitudes
    m = _m()
    T, H, k = 8, 128, 2
    rng = np.random.default_rng(11)
    y = rng.integers(0, 2**16, (T * k, H)).astype(np.uint16)
    exp = (y >> 7) & 0xFF
    y[exp == 0xFF] &= 0x807F                          # no inf/nan inputs
    pr = rng.permutation(T * k).reshape(T, k)
    w = np.array([[1.0, 2.0**-8], [0.5, 0.5], [1.0, 1.0], [1.0, -1.0], [2.0**-30, 2.0**-30],
                  [3.0, 1.0 / 3.0], [1.0 + 2.0**-8, 1.0], [2.0**40, 2.0**-40]], np.float32)
    out = m.moe_combine(dev_bf16(y), dev_i32(pr), dev_f32(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(out), oracle.combine(y, pr, w))


# ------------------------------------------------------------------ whole path

def test_identity_experts_round_trip_and_determinism():
    """route -> dispatch -> combine with y = the dispatch buffer returns x bit
    for bit, except that -0.0 comes back as +0.0 (the accumulator starts at
    +0.0); two runs give identical bytes."""
    m = _m()
    for name in ["tiny", "mixtral", "dsv3_decode", "dsv3_prefill", "kimi_k2"]:
        wl = workloads.make(name, seed=1, with_y=False)
        cfg = wl.cfg
        print(f"[edges] identity round trip {name}", flush=True)
        x = dev_bf16(wl.x)
        logits = dev_f32(wl.logits)
        outs = []
        for _ in range(2):
            idx, w = m.moe_route_topk(logits, cfg.k)
            send, buf = m.moe_dispatch(idx, x, cfg.E, cfg.R)
            out = m.moe_combine(buf, send.pair_row, w)
            torch.cuda.synchronize()
            outs.append([t.view(torch.int16) if t.dtype == torch.bfloat16 else t
                         for t in (idx, w, send.pair_row, buf, out)])
        expect = np.where(wl.x == 0x8000, np.uint16(0), wl.x)
        assert np.array_equal(host_bf16(outs[0][4].view(torch.bfloat16)), expect), name
        for a, b in zip(outs[0], outs[1]):  # bytes compared on the device
            assert torch.equal(a, b), name
        del outs, buf, out, x
        torch.cuda.empty_cache()


def test_empty_batch_is_a_no_op():
    m = _m()
    logits = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    idx, w = m.moe_route_topk(logits, 2)
    assert idx.shape == (0, 2)
    send, buf = m.moe_dispatch(idx, torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), 8, 2)
    out = m.moe_combine(buf, send.pair_row, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_capacity_errors_raise():
    m = _m()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    pr = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.moe_dispatch_recv(x, pr, buf=torch.zeros((7, 64), dtype=torch.bfloat16, device=DEV))
    assert ei.value.status == -3


def test_dirty_route_dispatch_workspace_stays_in_bounds():
    """A moe_route_dispatch workspace that was not zeroed (against the
    documented contract) gives wrong routing tables but no access out of
    bounds: every pair_row entry is -1 or below T*k, and the canary entries
    of row_token and rows of buf past T*k are untouched.  Zeroed again, the
    same workspace gives the oracle's results."""
    m = _m()
    from gpuhelp import assert_step_matches_oracle

    T, E, k, R, H = 4096, 256, 8, 32, 64
    P = T * k
    rng = np.random.default_rng(31)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xb = _rand_bf16((T, H), 32)
    logits, x = dev_f32(lg), dev_bf16(xb)
    nws = m.moe_route_dispatch_workspace_bytes(T, E, k)
    ws = torch.zeros((nws,), dtype=torch.uint8, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    pair_row = torch.empty((T, k), dtype=torch.int32, device=DEV)
    row_token = torch.full((P + 64,), -7, dtype=torch.int32, device=DEV)
    rank_off = torch.empty((R + 1,), dtype=torch.int32, device=DEV)
    buf = torch.full((P + 4, H), 0x3C5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    # Small counts shift rows a little (collisions inside [0, P)); large ones
    # push most rows past P.  Values stay small enough that no sum overflows.
    for hi in (4, 1 << 15):
        dirty = rng.integers(0, hi, size=nws // 4, dtype=np.int32)
        ws.copy_(dev_i32(dirty).view(torch.uint8))
        print(f"[edges] dirty route_dispatch workspace, counts below {hi}", flush=True)
        m.moe_route_dispatch(logits, x, k, R, topk_idx=idx, topk_w=w, expert_counts=counts,
                             expert_offsets=offsets, pair_row=pair_row,
                             row_token=row_token[:P], rank_offsets=rank_off, buf=buf,
                             capacity=P + 4, workspace=ws)
        torch.cuda.synchronize()
        pr = host(pair_row)
        assert ((pr >= -1) & (pr < P)).all()
        assert (host(row_token)[P:] == -7).all()
        assert (host_bf16(buf)[P:] == 0x3C5A).all()
    ws.zero_()
    m.moe_route_dispatch(logits, x, k, R, topk_idx=idx, topk_w=w, expert_counts=counts,
                         expert_offsets=offsets, pair_row=pair_row, row_token=row_token[:P],
                         rank_offsets=rank_off, buf=buf, capacity=P + 4, workspace=ws)
    torch.cuda.synchronize()
    assert_step_matches_oracle(lg, xb, k, E, R, idx, w,
                               (counts, offsets, pair_row, row_token[:P], rank_off), buf)
    assert int(ws.count_nonzero().item()) == 0


SC1_MIN_BYTES = 256 << 20   # combine bytes above which output rows take the sc1 stores


@pytest.mark.parametrize("T,H,k", [
    (2675, 7168, 6), (2674, 7168, 6),     # combine_kernel: just above / below the threshold
    (10923, 4096, 2), (10922, 4096, 2),   # the fixed-k kernel at k = 2
    (6554, 4096, 4), (6553, 4096, 4),     # and at k = 4
])
def test_combine_on_both_sides_of_the_store_threshold(T, H, k):
    """moe_combine stores its output rows with the sc1 cache policy when it
    moves more than 256 MiB (2TkH + 2TH bytes) and with write-back stores
    below; both forms of every kernel shape against the oracle on every
    token, with spare capacity."""
    m = _m()
    nbytes = 2 * T * H * (k + 1)
    above = nbytes > SC1_MIN_BYTES
    print(f"[edges] combine T={T} H={H} k={k} bytes={nbytes} sc1={above}", flush=True)
    rng = np.random.default_rng(T * 31 + k)
    P = T * k
    cap = P + 5
    pr = rng.permutation(cap)[:P].reshape(T, k).astype(np.int32)
    y = _rand_bf16((cap, H), T + k)
    w = rng.random((T, k)).astype(np.float32)
    out = host_bf16(m.moe_combine(dev_bf16(y), dev_i32(pr), dev_f32(w)))
    torch.cuda.synchronize()
    for t0 in range(0, T, 1024):
        t1 = min(T, t0 + 1024)
        ref = oracle.combine_tokens(y, pr, w, np.arange(t0, t1))
        assert np.array_equal(out[t0:t1], ref), f"tokens [{t0}, {t1}) differ"


def _combine_skipping(y, pr, w, cap):
    """The combine contract with skipped terms, from the oracle's own
    arithmetic: a term whose row lies outside [0, cap) leaves acc as it is."""
    T, k = pr.shape
    acc = np.zeros((T, y.shape[1]), np.float32)
    for j in range(k):
        ok = (pr[:, j] >= 0) & (pr[:, j] < cap)
        rows = oracle.bf16_to_f32(y[np.where(ok, pr[:, j], 0)])
        acc = np.where(ok[:, None], oracle.fmaf(w[:, j][:, None], rows, acc), acc)
    return oracle.f32_to_bf16_rne(acc)


@pytest.mark.parametrize("T,H,k", [(37, 256, 8), (129, 1024, 3), (300, 512, 2), (64, 7168, 1),
                                   (50, 640, 4), (5, 136, 12)])
def test_combine_skips_terms_outside_the_buffer(T, H, k):
    """Rows -1, -2^31, capacity, capacity + 7 and 2^31 - 1 in pair_row are
    skipped terms (every combine kernel: fixed k = 1, 2, 4, 8 and any other
    k); the rest of each token's chain is the oracle's."""
    m = _m()
    print(f"[edges] combine skipped terms T={T} H={H} k={k}", flush=True)
    rng = np.random.default_rng(T * 7 + H + k)
    P = T * k
    cap = P + 2
    pr = rng.permutation(cap)[:P].reshape(T, k).astype(np.int64)
    bad = rng.random((T, k)) < 0.15
    pr[bad] = rng.choice(np.array([-1, -(2 ** 31), cap, cap + 7, 2 ** 31 - 1]), int(bad.sum()))
    pr[0, :] = -1                       # a token with every term skipped: +0
    pr = pr.astype(np.int32)
    y = _rand_bf16((cap, H), T + H)
    w = rng.random((T, k)).astype(np.float32)
    out = host_bf16(m.moe_combine(dev_bf16(y), dev_i32(pr), dev_f32(w), capacity=cap))
    torch.cuda.synchronize()
    ref = _combine_skipping(y, pr.astype(np.int64), w, cap)
    assert (ref[0] == 0).all()
    assert np.array_equal(out, ref)
