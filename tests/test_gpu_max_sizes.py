"""The entry points at the largest sizes they accept, on the GPU.

* Pairs at the limit: T*k = 2^31 - 2 (T = 2^30 - 1 tokens, k = 2, E = 4).
  Routing runs far past 2^32 lanes, so the routing kernel's waves loop over
  token tiles; send runs 64 blocks of 2^25 pairs; recv and combine run
  2^30 row units through their capped grids.
* The one-call path (route, send, recv) at T*k = 2^31 - 32 with E = 128,
  where the routing kernel counts the send histogram, and with E = 8 at
  T = 2^24 + 37, where it counts per tile in LDS past its 2^20-block grid.
* Group-limited routing with 64*T past 2^32 (one wave per token, looping).
* Row offsets past 2^31 16-byte units (H = 8192, T = 2^21 + 3): recv,
  combine and the fp8 recv address bytes beyond 2^35.

The oracle cannot run 10^9 tokens, so each check is one of two kinds.
(1) The definition itself, evaluated on the device with torch comparisons,
chunk by chunk, on every output: the selection is the top k with ties to the
lower index; every pair's row is its expert's offset plus the number of
earlier pairs of that expert; every dispatched row is its token's row.
(2) The oracle on a seeded sample of tokens that includes both ends, for the
weights and the combine and fp8 arithmetic.  Outputs are pre-filled with
values the kernels never write (-1, NaN), so a token no wave reached fails.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from gpuhelp import DEV, assert_weights_close, host, host_bf16

pytestmark = pytest.mark.gpu

# Every torch op of the checks touches at most EL elements: the largest
# tensors here hold 2^33, past what single library launches are sized for.
EL = 1 << 27


def _step(width):
    return max(1, EL // width)


def _randn(shape, g, dtype=torch.float32):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    n = _step(shape[1])
    for r0 in range(0, shape[0], n):
        t[r0:r0 + n].normal_(generator=g)
    return t


def _full(shape, value, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    n = _step(shape[1])
    for r0 in range(0, shape[0], n):
        t[r0:r0 + n].fill_(value)
    return t


@pytest.fixture(autouse=True)
def _free_memory():
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(msg):
    print(f"\n[max] {msg}", flush=True)


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    ends = np.r_[np.arange(64), np.arange(T - 4096, T)]
    return np.unique(np.r_[ends, rng.integers(0, T, n)]).astype(np.int64)


def _before(la, a, lb, b):
    """Expert a (logit la) ranks before expert b: larger logit, or equal
    logits (+0 == -0) and the lower index."""
    return (la > lb) | ((la == lb) & (a < b))


def _check_topk_rows(logits, idx, allowed=None):
    """idx[t] lists the k best experts of token t in ranking order, over the
    experts that ``allowed`` (bool [n, E]; None: all) admits."""
    n, E = logits.shape
    k = idx.shape[1]
    ar = torch.arange(E, device=DEV)
    li = idx.long()
    assert bool(((li >= 0) & (li < E)).all()), "expert index out of range (or token not routed)"
    lsel = logits.gather(1, li)
    for j in range(1, k):
        assert bool(_before(lsel[:, j - 1], li[:, j - 1], lsel[:, j], li[:, j]).all()), \
            f"winners {j - 1} and {j} out of order"
    last_l, last_i = lsel[:, k - 1:k], li[:, k - 1:k]
    chosen = torch.zeros((n, E), dtype=torch.bool, device=DEV)
    chosen.scatter_(1, li, True)
    ok = chosen | _before(last_l, last_i, logits, ar)
    if allowed is not None:
        assert bool((chosen <= allowed).all()), "winner outside the kept groups"
        ok = ok | ~allowed
    assert bool(ok.all()), "an expert left out ranks before a winner"


def _check_slots(idx_flat, E, k, send):
    """Every pair's row is offsets[e] + (earlier pairs of expert e); every
    row's token is the token of the pair that lands on it."""
    P = idx_flat.numel()
    counts = torch.zeros(E, dtype=torch.int64, device=DEV)
    for p0 in range(0, P, EL):
        counts += torch.bincount(idx_flat[p0:p0 + EL].long(), minlength=E)
    assert torch.equal(send.expert_counts.long(), counts)
    off = torch.zeros(E + 1, dtype=torch.int64, device=DEV)
    off[1:] = torch.cumsum(counts, 0)
    assert torch.equal(send.expert_offsets.long(), off)
    seen = off[:E].clone()  # expert e's next row
    pr = send.pair_row.view(-1)
    experts = torch.arange(E, device=DEV)
    for p0 in range(0, P, EL):
        e_c = idx_flat[p0:p0 + EL].long()
        pr_c = pr[p0:p0 + EL].long()
        n = e_c.numel()
        # a stable sort keeps each expert's pairs in ascending p; a pair's
        # rank among its expert's pairs in this chunk is its sorted position
        # minus the expert's first sorted position
        sorted_e, order = torch.sort(e_c, stable=True)
        first = torch.searchsorted(sorted_e, experts)
        want = torch.empty_like(pr_c)
        want[order] = seen[sorted_e] + torch.arange(n, device=DEV) - first[sorted_e]
        seen += torch.bincount(e_c, minlength=E)
        assert torch.equal(pr_c, want), f"pair rows differ in pairs [{p0}, {p0 + n})"
        tok = torch.arange(p0, p0 + pr_c.numel(), device=DEV) // k
        assert torch.equal(send.row_token[pr_c].long(), tok), "row_token differs"
    assert torch.equal(seen, off[1:])


def _check_rows(buf, x, row_token):
    """Row r of buf is a bit copy of x[row_token[r]]."""
    P, H = buf.shape[0], x.shape[1]
    n = _step(H)
    for r0 in range(0, row_token.numel(), n):
        rows = row_token[r0:r0 + n].long()
        assert torch.equal(buf[r0:r0 + n].view(torch.int16), x[rows].view(torch.int16)), \
            f"dispatched rows differ in [{r0}, {r0 + rows.numel()})"


def test_pairs_at_the_int32_limit():
    import combine_topk_route_amd as m

    T, E, k, R, H = (1 << 30) - 1, 4, 2, 2, 8
    P = T * k
    assert P == (1 << 31) - 2
    _say(f"route T={T} E={E} k={k}")
    g = torch.Generator(device=DEV).manual_seed(31)
    logits = _randn((T, E), g)
    n = _step(E)
    for t0 in range(0, T, n):  # exact ties in every seventh token
        lc = logits[t0:t0 + n]
        lc[1::7] = torch.round(lc[1::7] * 2) / 2
    idx = _full((T, k), -1, torch.int32)
    w = _full((T, k), float("nan"), torch.float32)
    m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    for t0 in range(0, T, n):
        _check_topk_rows(logits[t0:t0 + n], idx[t0:t0 + n])
        ws = w[t0:t0 + n]
        assert bool(torch.isfinite(ws).all())
        assert bool(((ws.sum(1, dtype=torch.float64) - 1).abs() <= 2.0**-18).all())
    s = _sample(T, 8192, 1)
    lg = host(logits[torch.from_numpy(s).to(DEV)])
    r_idx, r_w, _ = oracle.route_topk(lg, k)
    st = torch.from_numpy(s).to(DEV)
    assert np.array_equal(host(idx[st]), r_idx)
    assert_weights_close(host(w[st]), r_w)
    del logits

    _say(f"send P={P} E={E} R={R}")
    send = m.moe_dispatch_send(idx, E, R)
    torch.cuda.synchronize()
    _check_slots(idx.view(-1), E, k, send)
    assert torch.equal(send.rank_offsets.long(), send.expert_offsets.long()[::E // R])

    _say(f"recv + combine T={T} H={H}")
    x = _randn((T, H), g, torch.bfloat16)
    buf = m.moe_dispatch_recv(x, send.pair_row)
    torch.cuda.synchronize()
    _check_rows(buf, x, send.row_token)
    out = _full((T, H), -1, torch.int16).view(torch.bfloat16)  # a NaN pattern combine never writes
    m.moe_combine(buf, send.pair_row, w, out=out)
    torch.cuda.synchronize()
    pr_s = host(send.pair_row[st]).astype(np.int64)
    y_s = host_bf16(buf[torch.from_numpy(pr_s.reshape(-1)).to(DEV)])
    local = np.arange(pr_s.size, dtype=np.int64).reshape(pr_s.shape)
    ref = oracle.combine(y_s, local, host(w[st]))
    assert np.array_equal(host_bf16(out[st]), ref)
    n = _step(H)
    for t0 in range(0, T, n):
        assert not bool((out[t0:t0 + n].view(torch.int16) == -1).all(1).any()), \
            f"a token in [{t0}, {t0 + n}) was not combined"


def test_one_call_path_at_the_pair_limit():
    """moe_route_dispatch with T*k = 2^31 - 32 and E = 128: the routing kernel
    counts the send histogram itself (rows of 2^25 pairs), the rank kernel
    reads and clears it; the workspace is zero again afterwards."""
    import combine_topk_route_amd as m

    T, E, k, R, H = (1 << 26) - 1, 128, 32, 32, 8
    _say(f"route_dispatch T={T} E={E} k={k} R={R} H={H}")
    g = torch.Generator(device=DEV).manual_seed(32)
    logits = _randn((T, E), g)
    x = _randn((T, H), g, torch.bfloat16)
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                     device=DEV)
    idx = _full((T, k), -1, torch.int32)
    w = _full((T, k), float("nan"), torch.float32)
    idx, w, send, buf = m.moe_route_dispatch(logits, x, k, R, topk_idx=idx, topk_w=w,
                                             workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0
    n = _step(E)
    for t0 in range(0, T, n):
        _check_topk_rows(logits[t0:t0 + n], idx[t0:t0 + n])
        assert bool(torch.isfinite(w[t0:t0 + n]).all())
    s = _sample(T, 2048, 4)
    st = torch.from_numpy(s).to(DEV)
    r_idx, r_w, _ = oracle.route_topk(host(logits[st]), k)
    assert np.array_equal(host(idx[st]), r_idx)
    assert_weights_close(host(w[st]), r_w)
    del logits
    _check_slots(idx.view(-1), E, k, send)
    assert torch.equal(send.rank_offsets.long(), send.expert_offsets.long()[::E // R])
    _check_rows(buf, x, send.row_token)


def test_lds_counting_route_past_its_grid():
    """moe_route_dispatch with E = 8, where the routing kernel counts each
    16-token tile's pairs in LDS, at T = 2^24 + 37: its 2^20 blocks take a
    second tile where there is one (the last one ragged), tiles straddle
    histogram rows, and the rank kernel reads and clears the matrix.  Two
    calls on one workspace, which is zero after each."""
    import combine_topk_route_amd as m

    T, E, k, R, H = (1 << 24) + 37, 8, 2, 2, 8
    _say(f"route_dispatch (LDS counting) T={T} E={E} k={k} R={R} H={H}")
    g = torch.Generator(device=DEV).manual_seed(24)
    logits = _randn((T, E), g)
    x = _randn((T, H), g, torch.bfloat16)
    ws = torch.zeros((m.moe_route_dispatch_workspace_bytes(T, E, k),), dtype=torch.uint8,
                     device=DEV)
    idx = _full((T, k), -1, torch.int32)
    w = _full((T, k), float("nan"), torch.float32)
    for _ in range(2):
        idx, w, send, buf = m.moe_route_dispatch(logits, x, k, R, topk_idx=idx, topk_w=w,
                                                 workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0
    n = _step(E)
    for t0 in range(0, T, n):
        _check_topk_rows(logits[t0:t0 + n], idx[t0:t0 + n])
        assert bool(torch.isfinite(w[t0:t0 + n]).all())
    s = _sample(T, 2048, 5)
    st = torch.from_numpy(s).to(DEV)
    r_idx, r_w, _ = oracle.route_topk(host(logits[st]), k)
    assert np.array_equal(host(idx[st]), r_idx)
    assert_weights_close(host(w[st]), r_w)
    del logits
    _check_slots(idx.view(-1), E, k, send)
    assert torch.equal(send.rank_offsets.long(), send.expert_offsets.long()[::E // R])
    _check_rows(buf, x, send.row_token)


def test_grouped_routing_past_the_32_bit_grid():
    import combine_topk_route_amd as m

    T, E, k, G, TG = (1 << 26) + 1001, 16, 4, 8, 3  # k > kept groups: the rule bites
    _say(f"grouped route T={T} E={E} k={k} groups {TG}/{G}")
    g = torch.Generator(device=DEV).manual_seed(26)
    logits = _randn((T, E), g)
    n = _step(E)
    for t0 in range(0, T, n):  # ties between experts and between groups
        lc = logits[t0:t0 + n]
        lc[::5] = torch.round(lc[::5])
    idx = _full((T, k), -1, torch.int32)
    w = _full((T, k), float("nan"), torch.float32)
    m.moe_route_topk_grouped(logits, k, G, TG, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    gs = E // G
    gar = torch.arange(G, device=DEV)
    for t0 in range(0, T, n):
        lc = logits[t0:t0 + n]
        score = lc.view(-1, G, gs).amax(2)  # a group's score is its largest logit
        # groups ranked before group h
        ahead = _before(score[:, :, None], gar[:, None], score[:, None, :], gar[None, :]).sum(1)
        kept = (ahead < TG).repeat_interleave(gs, dim=1)
        _check_topk_rows(lc, idx[t0:t0 + n], allowed=kept)
        assert bool(torch.isfinite(w[t0:t0 + n]).all())
    s = _sample(T, 8192, 2)
    st = torch.from_numpy(s).to(DEV)
    r_idx, r_w, _ = oracle.route_topk_grouped(host(logits[st]), k, G, TG)
    assert np.array_equal(host(idx[st]), r_idx)
    assert_weights_close(host(w[st]), r_w)


def test_row_offsets_past_2_31_units():
    import combine_topk_route_amd as m

    T, E, k, H = (1 << 21) + 3, 2, 1, 8192
    assert T * (H // 8) > 1 << 31
    _say(f"dispatch T={T} E={E} k={k} H={H}")
    g = torch.Generator(device=DEV).manual_seed(21)
    logits = _randn((T, E), g)
    idx, w = m.moe_route_topk(logits, k)
    x = _randn((T, H), g, torch.bfloat16)
    send, buf = m.moe_dispatch(idx, x, E, 1)
    torch.cuda.synchronize()
    assert bool((w == 1.0).all())  # k = 1: the one weight is exactly 1
    _check_slots(idx.view(-1), E, k, send)
    _check_rows(buf, x, send.row_token)

    _say(f"combine T={T} H={H}")
    out = m.moe_combine(buf, send.pair_row, w)
    torch.cuda.synchronize()
    # k = 1, weight 1: fma(1, y, +0) returns y, with -0 becoming +0.
    step = _step(H)
    for t0 in range(0, T, step):
        pr = send.pair_row[t0:t0 + step, 0].long()
        want = buf[pr].view(torch.int16)
        want = torch.where(want == -32768, torch.zeros_like(want), want)
        assert torch.equal(out[t0:t0 + step].view(torch.int16), want), \
            f"combine differs in tokens [{t0}, {t0 + pr.numel()})"
    s = _sample(T, 256, 3)
    st = torch.from_numpy(s).to(DEV)
    pr_s = host(send.pair_row[st]).astype(np.int64)
    y_s = host_bf16(buf[torch.from_numpy(pr_s.reshape(-1)).to(DEV)])
    local = np.arange(pr_s.size, dtype=np.int64).reshape(pr_s.shape)
    assert np.array_equal(host_bf16(out[st]), oracle.combine(y_s, local, host(w[st])))
    del out, buf

    _say(f"fp8 recv T={T} H={H}")
    q, sc = m.moe_dispatch_recv_fp8(x, send.pair_row)
    torch.cuda.synchronize()
    rq, rs = quant.quantize_rows(host_bf16(x[st]))
    rows = torch.from_numpy(pr_s[:, 0]).to(DEV)
    assert np.array_equal(host(q[rows]), rq)
    assert np.array_equal(host(sc[rows]).view(np.uint32), rs.view(np.uint32))
