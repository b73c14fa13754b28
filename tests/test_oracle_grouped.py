"""Pins for group-limited routing: the pages' special case (all groups kept
is plain top-k), a hand-worked case, the group-selection characterisation,
and exhaustive search inside the kept groups."""
import itertools

import numpy as np
import pytest

import oracle
import workloads


def test_all_groups_kept_is_plain_routing():
    # "Mixtral routing is a special case of DeepSeek routing where the top-K
    # group is the group of all experts" (multi-node DeepSeek page, MoE Router)
    for name in ["tiny", "dsv3_decode", "kimi_k2"]:
        wl = workloads.make(name, T=256, with_y=False)
        c = wl.cfg
        for G in [1, 2, 4, 8]:
            if c.E % G:
                continue
            a = oracle.route_topk(wl.logits, c.k)
            b = oracle.route_topk_grouped(wl.logits, c.k, G, G)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), (name, G)


def test_hand_worked_group_limit():
    logits = np.array([[5.0, 0.0, 4.9, 4.8, 1.0, 1.0, 1.0, 1.0]], np.float32)
    # groups of 2: maxima 5, 4.9, 1, 1
    idx, w, _ = oracle.route_topk_grouped(logits, 2, 4, 1)
    assert idx.tolist() == [[0, 1]]                  # only group 0 may be used
    assert np.allclose(w, [[np.exp(5) / (np.exp(5) + 1), 1 / (np.exp(5) + 1)]], rtol=1e-14)
    idx, _, _ = oracle.route_topk_grouped(logits, 3, 4, 2)
    assert idx.tolist() == [[0, 2, 3]]
    idx, _, _ = oracle.route_topk_grouped(logits, 3, 4, 3)   # groups 2 and 3 tie: lower wins
    assert idx.tolist() == [[0, 2, 3]]
    idx, _, _ = oracle.route_topk_grouped(logits, 6, 4, 3)
    assert idx.tolist() == [[0, 2, 3, 4, 5, 1]]


def _kept_groups(idx, gs):
    return [set(int(e) // gs for e in row) for row in idx]


@pytest.mark.parametrize("E,G,TG,k", [(8, 4, 2, 2), (12, 3, 2, 3), (16, 8, 3, 4), (10, 5, 2, 4),
                                      (9, 3, 1, 3)])
def test_grouped_against_exhaustive_search(E, G, TG, k):
    rng = np.random.default_rng(E * 100 + G * 10 + TG)
    logits = rng.standard_normal((60, E)).astype(np.float32)
    logits[0] = 1.0                                     # every group ties
    logits[1] = np.round(logits[1])                     # many ties
    logits[2, :] = -1.0
    logits[2, 0], logits[2, E - 1] = -0.0, 0.0          # +0 / -0
    idx, w, _ = oracle.route_topk_grouped(logits, k, G, TG)
    gs = E // G
    for t in range(logits.shape[0]):
        gmax = logits[t].reshape(G, gs).max(axis=1).astype(np.float64)
        # the kept groups: each beats (or ties with a higher index than) every dropped group
        best = sorted(range(G), key=lambda g: (-gmax[g], g))[:TG]
        assert _kept_groups(idx[t:t + 1], gs)[0] <= set(best)
        for g in best:
            for h in set(range(G)) - set(best):
                assert gmax[g] > gmax[h] or (gmax[g] == gmax[h] and g < h)
        # inside the kept groups: exhaustive k-subset with the largest sum
        allowed = [e for e in range(E) if e // gs in best]
        cand = None
        for sub in itertools.combinations(allowed, k):
            key = (-sum(float(logits[t, e]) for e in sub), sub)
            if cand is None or key < cand:
                cand = key
        assert tuple(sorted(int(e) for e in idx[t])) == cand[1]
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)


def test_grouped_rejects_bad_shapes():
    x = np.zeros((1, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.route_topk_grouped(x, 2, 3, 1)     # E % n_group != 0
    with pytest.raises(ValueError):
        oracle.route_topk_grouped(x, 3, 4, 1)     # kept groups hold fewer than k experts
    with pytest.raises(ValueError):
        oracle.route_topk_grouped(x, 2, 4, 5)
