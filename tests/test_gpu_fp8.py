"""GPU parity for block-scaled fp8 dispatch: E4M3 codes and fp32 scales must
be bit-exact with the oracle (the division x/scale and the rounding to E4M3
are taken in fp32 on both sides)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import DEV, dev_bf16, dev_i32, host

pytestmark = pytest.mark.gpu


def _fp8_check(x_bits, pr, cap=None, label=""):
    import combine_topk_route_amd as m

    T, H = x_bits.shape
    k = pr.shape[1]
    cap = T * k + 3 if cap is None else cap
    print(f"[fp8] {label} T={T} H={H} k={k} capacity={cap}", flush=True)
    bq = torch.full((cap, H), 0x5A, dtype=torch.uint8, device=DEV)
    bs = torch.full((cap, H // 128), -2.0, dtype=torch.float32, device=DEV)
    m.moe_dispatch_recv_fp8(dev_bf16(x_bits), dev_i32(pr), buf_q=bq, buf_scale=bs)
    torch.cuda.synchronize()
    rq, rs = oracle.dispatch_rows_fp8(x_bits, pr, cap, np.full((cap, H), 0x5A, np.uint8),
                                      np.full((cap, H // 128), -2.0, np.float32))
    gq, gs = host(bq), host(bs)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_fp8_dispatch_parity_on_configs(name):
    wl = workloads.make(name, seed=0, with_y=False)
    cfg = wl.cfg
    idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
    pr, _ = oracle.dispatch_slots(idx, cfg.E)
    _fp8_check(wl.x, pr, label=name)


@pytest.mark.parametrize("T,H,k", [(1, 128, 1), (3, 384, 3), (37, 640, 10), (64, 1024, 32),
                                   (129, 7168, 8), (5, 4224, 2), (300, 128, 4)])
def test_fp8_dispatch_ragged_shapes(T, H, k):
    rng = np.random.default_rng(T * H + k)
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    pr = rng.permutation(T * k).reshape(T, k)
    _fp8_check(x, pr, label="ragged")


def test_fp8_special_values():
    rng = np.random.default_rng(77)
    T, H = 8, 1024
    f = rng.standard_normal((T, H)).astype(np.float32)
    f[0, :128] = 0.0                                   # zero block -> scale 1, codes 0
    f[0, 128:256] = -0.0                               # -0 block -> codes 0x80
    f[1, :128] = rng.standard_normal(128) * 1e30       # huge magnitudes
    f[1, 128:256] = rng.standard_normal(128) * 1e-30   # tiny magnitudes
    f[2, :128] = 1e-38 * rng.standard_normal(128)      # bf16 subnormals
    f[3, :128] = 1.0
    f[3, 1:64] = 1.0625                                # x/scale = 1.0625*448/amax: E4M3 ties
    f[3, 0] = 448.0                                    # amax 448 -> scale exactly 1
    f[4, :128] = np.where(np.arange(128) % 2, 3e4, -1e-3)  # wide range inside one block
    f[5] = np.linspace(-7, 7, H)
    x = workloads.bf16_from_f32(f)
    x[6, :128] = 0x0001                                # smallest positive bf16 subnormal
    x[7, :128] = 0x7F7F                                # largest finite bf16
    pr = np.arange(T).reshape(T, 1)
    _fp8_check(x, pr, label="special")


def test_fp8_chain_matches_oracle():
    import combine_topk_route_amd as m

    wl = workloads.make("kimi_k2", seed=2, with_y=False)
    cfg = wl.cfg
    print("[fp8] chain kimi_k2 route -> moe_dispatch_fp8", flush=True)
    from gpuhelp import dev_f32
    idx, w = m.moe_route_topk(dev_f32(wl.logits), cfg.k)
    send, bq, bs = m.moe_dispatch_fp8(idx, dev_bf16(wl.x), cfg.E, cfg.R)
    torch.cuda.synchronize()
    r_idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
    pr, rt = oracle.dispatch_slots(r_idx, cfg.E)
    assert np.array_equal(host(send.pair_row), pr)
    rq, rs = oracle.dispatch_rows_fp8(wl.x, pr, cfg.P)
    assert np.array_equal(host(bs).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(bq), rq)


@pytest.mark.parametrize("T,E,k,R,H,G,TG", [
    (16, 8, 2, 1, 256, 1, 1),          # one launch for route + send
    (128, 256, 8, 32, 7168, 1, 1),     # DSv3 decode shape: routing, then send + fp8 recv in one launch
    (128, 256, 8, 32, 7168, 8, 4),     # the same with group-limited routing
    (300, 384, 8, 48, 1024, 8, 4),     # group-limited, 16-wave single-block send
    (3000, 64, 4, 8, 512, 1, 1),       # lane-group routing, histogram kernel (E < 128)
    (4096, 256, 8, 32, 2048, 1, 1),    # routing that counts the send histogram
])
def test_route_dispatch_fp8_matches_the_separate_calls(T, E, k, R, H, G, TG):
    """moe_route_dispatch_fp8 against routing then moe_dispatch_fp8: indices
    and weights, every send output, codes and scales bit-identical; the
    codes also against the oracle on the oracle's routing; the workspace is
    zero after two calls."""
    import combine_topk_route_amd as m

    print(f"[fp8] route_dispatch_fp8 T={T} E={E} k={k} H={H} groups {TG}/{G}", flush=True)
    rng = np.random.default_rng(T + E + H)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    lg, xd = torch.from_numpy(logits).to(DEV), dev_bf16(x)
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                     device=DEV)
    for _ in range(2):
        idx, w, send, q, s = m.moe_route_dispatch_fp8(lg, xd, k, R, n_group=G, topk_group=TG,
                                                      workspace=ws)
    if TG < G:
        idx2, w2 = m.moe_route_topk_grouped(lg, k, G, TG)
    else:
        idx2, w2 = m.moe_route_topk(lg, k)
    send2, q2, s2 = m.moe_dispatch_fp8(idx2, xd, E, R)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    for a, b in zip(send, send2):
        assert torch.equal(a, b)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    assert int(ws.count_nonzero().item()) == 0
    r_idx = (oracle.route_topk_grouped(logits, k, G, TG) if TG < G else oracle.route_topk(logits, k))[0]
    assert np.array_equal(host(idx), r_idx)
    pr, _ = oracle.dispatch_slots(r_idx, E)
    rq, rs = oracle.dispatch_rows_fp8(x, pr, T * k)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("T,k,E,R,H,drops", [
    (1, 1, 1, 1, 128, False), (3, 2, 4, 1, 128, True), (16, 2, 8, 1, 256, False),
    (128, 8, 256, 32, 7168, False), (128, 8, 256, 32, 7168, True), (256, 8, 256, 32, 4096, True),
    (300, 6, 40, 8, 8320, True), (2048, 1, 7, 7, 128, False), (682, 3, 1000, 8, 640, True),
    (683, 3, 1000, 8, 640, True),   # one pair past the one-launch limit
])
def test_fp8_dispatch_in_one_launch_matches_send_then_recv(T, k, E, R, H, drops):
    """moe_dispatch_fp8 sends and quantises in one launch for T*k <= 2048 and
    k <= 8 (block 0 sends; the other blocks quantise 4096-element units and
    find their rows from topk_idx).  Against moe_dispatch_send then
    moe_dispatch_recv_fp8: every send output, code and scale identical, with
    out-of-range experts (dropped), a repeated expert inside a token, rows
    cut inside a unit, spare capacity and canary rows; every referenced row
    holds the oracle's quantisation of its token, and without drops the rows
    are the oracle's."""
    import combine_topk_route_amd as m

    print(f"[fp8] dispatch one launch T={T} k={k} E={E} R={R} H={H} drops={drops}", flush=True)
    rng = np.random.default_rng(T * 11 + k * 5 + E + H)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    if drops:
        drop = rng.random((T, k)) < 0.05
        idx[drop] = rng.choice(np.array([-1, E, E + 5, -(2 ** 31)], np.int32), int(drop.sum()))
        if T > 2:
            idx[1, :] = idx[0, 0] if idx[0, 0] >= 0 else 0   # one expert repeated inside a token
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    cap = T * k + 5
    out = []
    for one_call in (True, False):
        bq = torch.full((cap, H), 0x5A, dtype=torch.uint8, device=DEV)
        bs = torch.full((cap, H // 128), -2.0, dtype=torch.float32, device=DEV)
        if one_call:
            res, _, _ = m.moe_dispatch_fp8(dev_i32(idx), dev_bf16(x), E, R, buf_q=bq, buf_scale=bs,
                                           capacity=cap)
        else:
            res = m.moe_dispatch_send(dev_i32(idx), E, R)
            m.moe_dispatch_recv_fp8(dev_bf16(x), res.pair_row, buf_q=bq, buf_scale=bs, capacity=cap)
        torch.cuda.synchronize()
        out.append((res, host(bq), host(bs)))
    (a, qa, sa), (b, qb, sb) = out
    n_valid = int(host(a.expert_offsets)[E])
    for name in ("expert_counts", "expert_offsets", "pair_row", "rank_offsets"):
        assert np.array_equal(host(getattr(a, name)), host(getattr(b, name))), name
    assert np.array_equal(host(a.row_token)[:n_valid], host(b.row_token)[:n_valid])
    assert np.array_equal(qa, qb)
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    rq, rs = oracle.quantize_rows(x)
    pr = host(a.pair_row)
    t_of, j_of = np.nonzero(pr >= 0)
    assert len(t_of) == n_valid == int(((idx >= 0) & (idx < E)).sum())
    rows = pr[t_of, j_of]
    assert np.array_equal(qa[rows], rq[t_of])
    assert np.array_equal(sa[rows].view(np.uint32), rs[t_of].view(np.uint32))
    assert (qa[n_valid:] == 0x5A).all() and (sa[n_valid:] == -2.0).all()
    if not drops:
        r_pr, _ = oracle.dispatch_slots(idx, E)
        assert np.array_equal(pr, r_pr)
        eq, es = oracle.dispatch_rows_fp8(x, r_pr, cap, np.full((cap, H), 0x5A, np.uint8),
                                          np.full((cap, H // 128), -2.0, np.float32))
        assert np.array_equal(qa, eq) and np.array_equal(sa.view(np.uint32), es.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "dsv3_decode"])
def test_fp8_one_call_on_the_small_workloads(name):
    """moe_route_dispatch_fp8 on the seeded workloads whose T*k <= 2048
    (routing, then send + fp8 recv in one launch), against the oracle:
    indices, slots, codes and scales bit-exact, weights within 2^-20."""
    import combine_topk_route_amd as m
    from gpuhelp import assert_weights_close, dev_f32

    wl = workloads.make(name, seed=4, with_y=False)
    cfg = wl.cfg
    assert cfg.T * cfg.k <= 2048
    print(f"[fp8] one call {name} T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H}", flush=True)
    idx, w, send, q, s = m.moe_route_dispatch_fp8(dev_f32(wl.logits), dev_bf16(wl.x), cfg.k, cfg.R)
    torch.cuda.synchronize()
    r_idx, r_w, _ = oracle.route_topk(wl.logits, cfg.k)
    assert np.array_equal(host(idx), r_idx)
    assert_weights_close(host(w), r_w)
    pr, rt = oracle.dispatch_slots(r_idx, cfg.E)
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host(send.row_token), rt)
    rq, rs = oracle.dispatch_rows_fp8(wl.x, pr, cfg.P)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
