"""Pins for the oracle's dispatch (counts, offsets, slots, rows) and combine."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_idx(T, k, E, seed, distinct=True, zipf=None):
    rng = np.random.default_rng(seed)
    if distinct:
        scores = rng.standard_normal((T, E))
        if zipf:
            scores += -zipf * np.log(np.arange(1, E + 1))[rng.permutation(E)]
        return np.argsort(-scores, axis=1)[:, :k].astype(np.int32)
    return rng.integers(0, E, (T, k)).astype(np.int32)


# ---------------------------------------------------------------- counts/offsets

@pytest.mark.parametrize("T,k,E,distinct", [(1, 1, 1, True), (16, 2, 8, True), (33, 3, 5, False),
                                            (200, 8, 64, True), (257, 4, 7, False)])
def test_counts_offsets_slots_against_brute_force(T, k, E, distinct):
    idx = _random_idx(T, k, E, seed=T * 7 + k, distinct=distinct)
    counts = oracle.expert_counts(idx, E)
    brute = [sum(1 for t in range(T) for j in range(k) if idx[t, j] == e) for e in range(E)]
    assert counts.tolist() == brute
    assert counts.sum() == T * k
    off = oracle.expert_offsets(counts)
    assert off[0] == 0 and off[-1] == T * k
    assert np.array_equal(np.diff(off), counts)
    pr, rt = oracle.dispatch_slots(idx, E)
    pr2, rt2 = oracle.dispatch_slots_sequential(idx, E)
    assert np.array_equal(pr, pr2) and np.array_equal(rt, rt2)


def test_slots_are_a_stable_permutation():
    for name, cfg in workloads.CONFIGS.items():
        wl = workloads.make(cfg, with_y=False)
        idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
        counts = oracle.expert_counts(idx, cfg.E)
        off = oracle.expert_offsets(counts)
        pr, rt = oracle.dispatch_slots(idx, cfg.E)
        P = cfg.P
        # every (token, j) pair lands on exactly one row: a bijection onto [0, P)
        assert np.array_equal(np.sort(pr.ravel()), np.arange(P)), name
        # each row records the token it holds
        assert np.array_equal(rt[pr], np.repeat(np.arange(cfg.T), cfg.k).reshape(cfg.T, cfg.k)), name
        # rows fall inside their expert's segment
        e = idx.astype(np.int64)
        assert ((pr >= off[e]) & (pr < off[e + 1])).all(), name
        # inside a segment the tokens strictly increase (k distinct experts per token)
        for ex in range(cfg.E):
            seg = rt[off[ex]:off[ex + 1]]
            assert (np.diff(seg) > 0).all(), (name, ex)


def test_rank_offsets_follow_contiguous_expert_ownership():
    counts = np.array([3, 0, 2, 5, 1, 0, 0, 4], dtype=np.int64)
    off = oracle.expert_offsets(counts)
    assert off.tolist() == [0, 3, 3, 5, 10, 11, 11, 11, 15]
    assert oracle.rank_offsets(off, 4).tolist() == [0, 3, 10, 11, 15]
    assert oracle.rank_offsets(off, 1).tolist() == [0, 15]
    assert oracle.rank_offsets(off, 8).tolist() == off.tolist()
    with pytest.raises(ValueError):
        oracle.rank_offsets(off, 3)


def test_counts_match_the_pages_worked_arithmetic():
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        idx = _random_idx(c["tokens"], c["k"], c["E"], seed=c["tokens"])
        counts = oracle.expert_counts(idx, c["E"])
        if "mean_tokens_per_expert" in c:
            assert counts.sum() / c["E"] == c["mean_tokens_per_expert"]
        if "max_distinct_experts" in c:
            assert np.count_nonzero(counts) <= c["max_distinct_experts"]
            assert c["tokens"] * c["k"] == c["max_distinct_experts"]
        if "mean_pairs_per_rank" in c:
            R = c["R"]
            off = oracle.expert_offsets(counts)
            ro = oracle.rank_offsets(off, R)
            assert np.diff(ro).sum() / R == c["mean_pairs_per_rank"]
            assert c["E"] // R == c["local_experts_per_rank"]


# ---------------------------------------------------------------- dispatch rows

def test_dispatch_rows_are_bit_copies_and_canaries_survive():
    wl = workloads.make("tiny")
    cfg = wl.cfg
    idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
    pr, rt = oracle.dispatch_slots(idx, cfg.E)
    cap = cfg.P + 4
    fill = np.full((cap, cfg.H), 0xBEEF, np.uint16)
    buf = oracle.dispatch_rows(wl.x, pr, cap, fill)
    assert np.array_equal(buf[: cfg.P], wl.x[rt])
    assert (buf[cfg.P:] == 0xBEEF).all()
    with pytest.raises(ValueError):
        oracle.dispatch_rows(wl.x, pr, cfg.P - 1)


# ---------------------------------------------------------------- combine

def test_combine_matches_exact_rational_fma_chain():
    wl = workloads.make("tiny")
    cfg = wl.cfg
    idx, _, w32 = oracle.route_topk(wl.logits, cfg.k)
    pr, _ = oracle.dispatch_slots(idx, cfg.E)
    got = oracle.combine(wl.y, pr, w32)
    ref = oracle.combine_exact(wl.y, pr, w32)
    assert np.array_equal(got, ref)


def test_combine_exact_on_adversarial_weights():
    # weights chosen so partial sums often land on fp32 midpoints
    rng = np.random.default_rng(3)
    T, H, k = 6, 64, 5
    y = workloads.bf16_from_f32(rng.standard_normal((T * k, H)).astype(np.float32))
    w = (1.0 + rng.integers(1, 2**23, (T, k)) * 2.0**-23).astype(np.float32)
    w *= np.float32(2.0) ** rng.integers(-30, 2, (T, k)).astype(np.float32)
    pr = rng.permutation(T * k).reshape(T, k)
    assert np.array_equal(oracle.combine(y, pr, w), oracle.combine_exact(y, pr, w))


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3_decode"])
def test_identity_experts_return_the_input(name):
    # y = dispatched x with normalised weights: the weighted average of k copies
    # of x[t] is x[t]; fp32 error (< 2^-20 relative) is far below half a bf16
    # ulp, so the bf16 result is x[t] bit for bit, except that -0.0 comes back
    # as +0.0 because the accumulator starts at +0.0.
    cfg = workloads.CONFIGS[name]
    T = min(cfg.T, 256)
    wl = workloads.make(cfg, T=T, with_y=False)
    idx, _, w32 = oracle.route_topk(wl.logits, cfg.k)
    pr, _ = oracle.dispatch_slots(idx, cfg.E)
    x = wl.x.copy()
    x[:3, :5] = 0x8000                       # plant some -0.0 inputs
    buf = oracle.dispatch_rows(x, pr, T * cfg.k)
    expect = np.where(x == 0x8000, np.uint16(0), x)
    assert np.array_equal(oracle.combine(buf, pr, w32), expect)


def test_combine_k1_copies_and_scaling_and_zero():
    rng = np.random.default_rng(4)
    T, H = 8, 32
    y = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    pr = rng.permutation(T).reshape(T, 1)
    one = np.ones((T, 1), np.float32)
    assert np.array_equal(oracle.combine(y, pr, one), y[pr[:, 0]])
    # scaling every weight by a power of two scales the result exactly
    k = 3
    y3 = workloads.bf16_from_f32(rng.standard_normal((T * k, H)).astype(np.float32))
    pr3 = rng.permutation(T * k).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    a = oracle.bf16_to_f32(oracle.combine(y3, pr3, w))
    b = oracle.bf16_to_f32(oracle.combine(y3, pr3, w * np.float32(4.0)))
    assert np.array_equal(b, a * np.float32(4.0))
    # zero rows give +0.0
    z = oracle.combine(np.zeros((T * k, H), np.uint16), pr3, w)
    assert (z == 0).all()


def test_combine_against_float64_weighted_sum():
    # the fp32 chain stays within a bf16 ulp of the exact weighted sum
    # wherever there is no heavy cancellation
    wl = workloads.make("mixtral", T=64)
    cfg = wl.cfg
    idx, w64, w32 = oracle.route_topk(wl.logits, cfg.k)
    pr, _ = oracle.dispatch_slots(idx, cfg.E)
    got = oracle.bf16_to_f32(oracle.combine(wl.y, pr, w32)).astype(np.float64)
    yf = oracle.bf16_to_f32(wl.y).astype(np.float64)
    exact = sum(w32[:, j, None].astype(np.float64) * yf[pr[:, j]] for j in range(cfg.k))
    mag = sum(np.abs(w32[:, j, None].astype(np.float64) * yf[pr[:, j]]) for j in range(cfg.k))
    assert (np.abs(got - exact) <= 2.0**-8 * np.abs(exact) + 2.0**-22 * mag).all()
