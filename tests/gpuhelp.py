"""Helpers shared by the GPU tests: host <-> device moves of bf16 bit arrays
and the tolerances the parity tests use."""
import numpy as np
import torch

DEV = torch.device("cuda:0")

# Routing weights: the kernel's fp32 weights against the float64 oracle's
# renormalised softmax.  The kernel forms only the k winners' numerators
# exp(l - l_max) (the E-term denominator cancels) and divides each by their
# compensated sum.  Rounding budget (units of u = 2^-24): numerator <= 3u
# (expf 2u, the fma that carries the exact difference u), counted twice
# (numerator and sum), sum ~u, division u: below 8u, so 16u = 2^-20
# relative, plus an absolute floor for fp32 underflow.
W_REL = 2.0**-20
W_ABS = 2.0**-126

# Combine: per element |gpu - ref| <= 2^-7 |ref|; +-0 must match as zero.
OUT_REL = 2.0**-7


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_bf16(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.cpu().numpy()


def bf16_vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_weights_close(gpu_w, ref_w):
    g = np.asarray(gpu_w, np.float64)
    r = np.asarray(ref_w, np.float64)
    err = np.abs(g - r)
    bad = err > W_REL * np.abs(r) + W_ABS
    assert not bad.any(), (
        f"{bad.sum()} weights out of tolerance; worst rel err "
        f"{(err / np.maximum(np.abs(r), 1e-300)).max():.3e}")
    return float((err / np.maximum(np.abs(r), 1e-300)).max())


def assert_out_close(gpu_bits, ref_bits, extra_abs=None):
    """Combine outputs: within 2^-7 relative per element (plus ``extra_abs``,
    an optional per-element absolute allowance); returns the count of
    elements that are not bit-identical."""
    g = bf16_vals(gpu_bits).astype(np.float64)
    r = bf16_vals(ref_bits).astype(np.float64)
    tol = OUT_REL * np.abs(r)
    if extra_abs is not None:
        tol = tol + extra_abs
    bad = ~(np.abs(g - r) <= tol)
    assert not bad.any(), f"{bad.sum()} of {bad.size} combine elements out of tolerance"
    return int(np.count_nonzero(np.asarray(gpu_bits) != np.asarray(ref_bits)))


def assert_step_matches_oracle(logits, x_bits, k, E, R, idx, w, send, buf, y_bits=None,
                               out=None, n_group=None, topk_group=None):
    """One route -> dispatch (-> combine) step against the oracle: indices,
    counts, offsets, rank offsets, pair_row, row_token and the dispatched rows
    bit-exact; weights within 2^-20; and, given y and out, combine
    bit-identical to the oracle's on the kernel's own fp32 weights.  ``send``
    holds (expert_counts, expert_offsets, pair_row, row_token, rank_offsets)
    device tensors; ``buf`` needs at least T*k rows."""
    import oracle

    T = logits.shape[0]
    if n_group is None:
        r_idx, r_w, _ = oracle.route_topk(logits, k)
    else:
        r_idx, r_w, _ = oracle.route_topk_grouped(logits, k, n_group, topk_group)
    assert np.array_equal(host(idx)[:T], r_idx), "indices differ from the oracle"
    assert_weights_close(host(w)[:T], r_w)
    counts = oracle.expert_counts(r_idx, E)
    off = oracle.expert_offsets(counts)
    pr, rt = oracle.dispatch_slots(r_idx, E)
    counts_g, off_g, pr_g, rt_g, rank_g = send
    assert np.array_equal(host(counts_g), counts), "expert_counts differ"
    assert np.array_equal(host(off_g), off), "expert_offsets differ"
    assert np.array_equal(host(rank_g), oracle.rank_offsets(off, R)), "rank_offsets differ"
    assert np.array_equal(host(pr_g).reshape(-1, k)[:T], pr), "pair_row differs"
    assert np.array_equal(host(rt_g)[: T * k], rt), "row_token differs"
    assert np.array_equal(host_bf16(buf)[: T * k], oracle.dispatch_rows(x_bits, pr, T * k)), \
        "dispatched rows differ"
    if out is not None:
        ref = oracle.combine(y_bits, pr, host(w)[:T].astype(np.float32))
        assert np.array_equal(host_bf16(out)[:T], ref), "combine differs from the oracle"
