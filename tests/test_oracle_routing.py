"""Pins for the oracle's top-k routing (no GPU).

Each check is independent of the oracle's own code: exhaustive subset
search, hand-worked rational weights, closed forms and invariants.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


def _sets(idx):
    return [tuple(sorted(int(e) for e in row)) for row in idx]


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (8, 4), (10, 3), (7, 7)])
def test_route_matches_exhaustive_search(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    logits = rng.standard_normal((40, E)).astype(np.float32)
    # plant exact ties, some straddling the k-th place, and signed zeros
    logits[0] = 0.5
    logits[1, : E // 2] = 1.25
    logits[2, 0], logits[2, -1] = -0.0, 0.0
    logits[2, 1:-1] = -1.0
    logits[3] = np.round(logits[3])          # many small-integer ties
    logits[4] = np.float32(0.0)
    logits[4, ::2] = np.float32(-0.0)
    idx, w, _ = oracle.route_topk(logits, k)
    assert _sets(idx) == oracle.route_topk_bruteforce(logits, k)


def test_route_tiny_workload_matches_exhaustive_search():
    wl = workloads.make("tiny")
    idx, _, _ = oracle.route_topk(wl.logits, wl.cfg.k)
    assert _sets(idx) == oracle.route_topk_bruteforce(wl.logits, wl.cfg.k)


def test_route_rational_weights_worked_by_hand():
    # logits = ln(n): the softmax is proportional to n, so the renormalised
    # weights of the chosen experts are n_j / sum(n_chosen).
    n = [3, 1, 4, 1, 5, 9, 2, 6]
    logits = np.log(np.array([n], dtype=np.float64)).astype(np.float32)
    idx, w, _ = oracle.route_topk(logits, 3)
    # 9 (expert 5), 6 (expert 7), 5 (expert 4): 9/20, 6/20, 5/20
    assert idx.tolist() == [[5, 7, 4]]
    assert np.allclose(w, [[0.45, 0.30, 0.25]], rtol=1e-6, atol=0)
    # ties between the two experts with n = 1 go to the lower index
    idx, w, _ = oracle.route_topk(logits, 8)
    assert idx.tolist() == [[5, 7, 4, 2, 0, 6, 1, 3]]
    assert np.allclose(w, [[9 / 31, 6 / 31, 5 / 31, 4 / 31, 3 / 31, 2 / 31, 1 / 31, 1 / 31]],
                       rtol=1e-6, atol=0)


def test_route_closed_forms():
    # all-equal logits: the first k experts, weight 1/k
    for E, k in [(8, 2), (256, 8), (384, 8), (16, 16)]:
        idx, w, w32 = oracle.route_topk(np.full((3, E), 0.75, np.float32), k)
        assert (idx == np.arange(k)).all()
        assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-16)
    # k = 1: weight exactly 1
    rng = np.random.default_rng(5)
    _, w, w32 = oracle.route_topk(rng.standard_normal((50, 16)).astype(np.float32), 1)
    assert (w == 1.0).all() and (w32 == 1.0).all()
    # k = 2 with logits (a, b, -inf-ish): w0 = e^a / (e^a + e^b)
    logits = np.array([[2.0, 0.5, -30.0, -30.0], [0.0, -1.0, -5.0, -7.0]], np.float32)
    _, w, _ = oracle.route_topk(logits, 2)
    assert math.isclose(w[0, 0], math.exp(2.0) / (math.exp(2.0) + math.exp(0.5)), rel_tol=1e-14)
    assert math.isclose(w[1, 1], math.exp(-1.0) / (1.0 + math.exp(-1.0)), rel_tol=1e-14)


def test_route_closed_forms_past_the_fp32_range():
    # logits further apart than FLT_MAX: e^(a - m) underflows to exactly 0 in
    # float64, so the top logit takes weight 1, and equal winners split it
    fmax = float(np.finfo(np.float32).max)
    logits = np.full((3, 8), -fmax, np.float32)
    logits[0, 5] = fmax
    logits[1, 2] = logits[1, 6] = np.float32(2e38)
    logits[1, [0, 1, 3]] = np.float32(-2e38)
    logits[2, :] = np.float32(-3e38)
    logits[2, 4] = np.float32(1e38)
    logits[2, 1] = np.float32(0.5)
    idx, w, w32 = oracle.route_topk(logits, 3)
    assert idx.tolist() == [[5, 0, 1], [2, 6, 0], [4, 1, 0]]
    assert w[0].tolist() == [1.0, 0.0, 0.0] and w[1].tolist() == [0.5, 0.5, 0.0]
    assert w[2].tolist() == [1.0, 0.0, 0.0] and np.all(np.isfinite(w32))


def test_route_invariants_on_all_configs():
    for name, cfg in workloads.CONFIGS.items():
        T = min(cfg.T, 1024)
        wl = workloads.make(cfg, T=T, with_y=False)
        idx, w, w32 = oracle.route_topk(wl.logits, cfg.k)
        # k different experts per token
        assert all(len(set(r)) == cfg.k for r in idx.tolist()), name
        # weights sum to one and do not increase along j
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14), name
        assert (np.diff(w, axis=1) <= 0).all(), name
        # the chosen logits dominate every unchosen logit
        chosen = np.take_along_axis(wl.logits, idx, axis=1)
        mask = np.ones_like(wl.logits, dtype=bool)
        np.put_along_axis(mask, idx, False, axis=1)
        rest = np.where(mask, wl.logits, -np.inf).max(axis=1)
        assert (chosen.min(axis=1) >= rest).all(), name
        # w32 is w rounded to fp32
        assert np.array_equal(w32, w.astype(np.float32))


def test_route_is_permutation_equivariant():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((64, 32)).astype(np.float32)
    perm = rng.permutation(32)
    idx, w, _ = oracle.route_topk(logits, 6)
    idx_p, w_p, _ = oracle.route_topk(logits[:, perm], 6)
    assert np.array_equal(perm[idx_p], idx)
    assert np.allclose(w_p, w, rtol=1e-15, atol=0)


def test_route_shift_invariance_exact():
    # dyadic logits and a dyadic shift: every shifted value is exact in fp32
    rng = np.random.default_rng(10)
    logits = (rng.integers(-64, 64, (32, 24)) / 8.0).astype(np.float32)
    idx, w, _ = oracle.route_topk(logits, 5)
    idx2, w2, _ = oracle.route_topk(logits + np.float32(3.5), 5)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w, w2, rtol=1e-14, atol=0)


def test_route_signed_zero_tie_goes_to_lower_index():
    logits = np.full((2, 6), -1.0, np.float32)
    logits[0, 3], logits[0, 1] = 0.0, -0.0
    logits[1, 3], logits[1, 1] = -0.0, 0.0
    idx, w, _ = oracle.route_topk(logits, 2)
    assert idx.tolist() == [[1, 3], [1, 3]]
    assert np.allclose(w, 0.5, rtol=0, atol=1e-16)


def test_route_rejects_non_finite_and_bad_k():
    with pytest.raises(ValueError):
        oracle.route_topk(np.array([[0.0, np.nan]], np.float32), 1)
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((1, 4), np.float32), 5)


def test_kimi_hot_expert_share_is_about_thirty_percent():
    wl = workloads.make("kimi_k2", with_y=False)
    idx, _, _ = oracle.route_topk(wl.logits, wl.cfg.k)
    share = (idx == wl.hot_expert).any(axis=1).mean()
    assert 0.25 <= share <= 0.35


def test_decode_config_is_skewed():
    wl = workloads.make("dsv3_decode", with_y=False)
    idx, _, _ = oracle.route_topk(wl.logits, wl.cfg.k)
    c = oracle.expert_counts(idx, wl.cfg.E)
    assert c.max() > 0.8 * wl.cfg.T           # one expert takes most tokens
    assert (c == 0).sum() > wl.cfg.E // 2      # most experts get nothing
