"""A seeded sweep of random shapes through the one-call path
(moe_route_dispatch, then moe_combine) against the oracle: batch sizes on
both sides of every launch-plan switch (one launch for route and send, the
single-block and multi-block sends, one wave per token and lane groups, the
routing kernel counting the send histogram with global atomics, per tile in
LDS, or not at all), expert counts from 1 to
1024, odd widths, plain and group-limited routing.  One workspace serves
every call and must be all zeros after each.  Bars: indices, counts,
offsets, slots and rows bit-exact; weights within 2^-20; combine of the
dispatched rows (identity experts) bit-identical to the oracle's fma chain
on the kernel's own weights."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import DEV, assert_weights_close, dev_bf16, dev_f32, host, host_bf16

pytestmark = pytest.mark.gpu

E_CHOICES = [1, 2, 3, 8, 16, 40, 64, 100, 127, 128, 129, 256, 384, 500, 513, 768, 1000, 1024]
T_CHOICES = [1, 7, 64, 129, 255, 256, 511, 512, 513, 1000, 2047, 2048, 2049, 3000, 4097, 6000]
H_CHOICES = [8, 64, 136, 520, 1024]
MAX_ELEMS = 1 << 22   # T * k * H per case, so the oracle's combine stays quick


def _cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice(E_CHOICES))
        k = int(rng.integers(1, min(32, E) + 1))
        T = int(rng.choice(T_CHOICES))
        H = int(rng.choice(H_CHOICES))
        if T * k * H > MAX_ELEMS:
            continue
        divisors = [r for r in range(1, E + 1) if E % r == 0]
        R = int(rng.choice(divisors))
        n_group = topk_group = 1
        if rng.random() < 0.25:
            groups = [g for g in range(2, 65) if E % g == 0]
            if groups:
                n_group = int(rng.choice(groups))
                need = -(-k // (E // n_group))
                topk_group = int(rng.integers(need, n_group + 1))
        out.append((T, E, k, R, H, n_group, topk_group))
    return out


# Large batches that the draw above rarely reaches: lane-group routing that
# counts the send histogram (E >= 128), multi-step waves in the rank kernel
# (E = 1024, k = 32: 16 blocks of 16384 pairs), and the per-tile LDS counts
# below 128 experts.
EXTRA = [(4097, 256, 8, 32, 8, 1, 1), (6000, 384, 8, 48, 8, 1, 1), (4097, 1024, 8, 32, 8, 1, 1),
         (3000, 128, 16, 16, 64, 1, 1), (6000, 513, 5, 27, 8, 1, 1),
         (8192, 1024, 32, 32, 8, 1, 1), (5000, 100, 8, 4, 8, 1, 1),
         (4500, 256, 8, 32, 8, 8, 4)]
CASES = _cases() + EXTRA
WS_BYTES = 64 * 1024 + 256   # the largest workspace any case needs (checked below)


@pytest.fixture(scope="module")
def workspace():
    return torch.zeros((WS_BYTES,), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("case", CASES, ids=[
    f"T{c[0]}-E{c[1]}-k{c[2]}-R{c[3]}-H{c[4]}-g{c[5]}.{c[6]}" for c in CASES])
def test_random_shape_through_the_one_call_path(case, workspace):
    import combine_topk_route_amd as m

    T, E, k, R, H, G, TG = case
    print(f"\n[random] T={T} E={E} k={k} R={R} H={H} groups {TG}/{G}", flush=True)
    assert m.moe_route_dispatch_workspace_bytes(T, E, k) <= WS_BYTES
    rng = np.random.default_rng(T * 131 + E * 7 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if rng.random() < 0.3:   # coarse logits: many exact ties
        logits = np.round(logits * 2) / 2
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))

    idx, w, send, buf = m.moe_route_dispatch(dev_f32(logits), dev_bf16(x), k, R, n_group=G,
                                             topk_group=TG, workspace=workspace)
    out = m.moe_combine(buf, send.pair_row, w)
    torch.cuda.synchronize()
    assert int(workspace.count_nonzero().item()) == 0

    if TG < G:
        r_idx, r_w, _ = oracle.route_topk_grouped(logits, k, G, TG)
    else:
        r_idx, r_w, _ = oracle.route_topk(logits, k)
    assert np.array_equal(host(idx), r_idx)
    assert_weights_close(host(w), r_w)

    counts = oracle.expert_counts(r_idx, E)
    off = oracle.expert_offsets(counts)
    pr, rt = oracle.dispatch_slots(r_idx, E)
    assert np.array_equal(host(send.expert_counts), counts)
    assert np.array_equal(host(send.expert_offsets), off)
    assert np.array_equal(host(send.rank_offsets), oracle.rank_offsets(off, R))
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host(send.row_token), rt)

    buf_bits = host_bf16(buf)
    assert np.array_equal(buf_bits, oracle.dispatch_rows(x, pr, T * k))
    w32 = host(w).astype(np.float32)
    assert np.array_equal(host_bf16(out), oracle.combine(buf_bits, pr, w32))


FP8_CASES = CASES[::3]


@pytest.mark.parametrize("case", FP8_CASES, ids=[
    f"T{c[0]}-E{c[1]}-k{c[2]}-R{c[3]}-g{c[5]}.{c[6]}" for c in FP8_CASES])
def test_random_shape_through_the_fp8_one_call_path(case, workspace):
    """moe_route_dispatch_fp8 on every third shape (rows widened to a
    multiple of 128): indices, slots, E4M3 codes and fp32 scales bit-exact
    against the oracle; the shared workspace is zero after each call."""
    import combine_topk_route_amd as m

    T, E, k, R, H, G, TG = case
    H = 128 * max(1, -(-H // 128))
    print(f"\n[random fp8] T={T} E={E} k={k} R={R} H={H} groups {TG}/{G}", flush=True)
    rng = np.random.default_rng(T * 17 + E * 5 + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = workloads.bf16_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    idx, w, send, q, s = m.moe_route_dispatch_fp8(dev_f32(logits), dev_bf16(x), k, R,
                                                  n_group=G, topk_group=TG, workspace=workspace)
    torch.cuda.synchronize()
    assert int(workspace.count_nonzero().item()) == 0
    if TG < G:
        r_idx, r_w, _ = oracle.route_topk_grouped(logits, k, G, TG)
    else:
        r_idx, r_w, _ = oracle.route_topk(logits, k)
    assert np.array_equal(host(idx), r_idx)
    assert_weights_close(host(w), r_w)
    pr, rt = oracle.dispatch_slots(r_idx, E)
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host(send.row_token), rt)
    rq, rs = oracle.dispatch_rows_fp8(x, pr, T * k)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
