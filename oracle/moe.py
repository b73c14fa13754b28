"""Plain, slow, obviously-correct CPU definitions of MoE top-k routing,
dispatch and combine.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module.  It shares no code with the HIP path and never calls it.

What the method computes, and where the pages state it
------------------------------------------------------
* Routing.  A small linear router gives each token a probability
  distribution over the experts; the K highest-scoring experts are chosen, and
  the token's output is the weighted average of their outputs with the
  router's weights ("Efficient and portable mixture-of-experts communication",
  section "Introduction").  DeepSeek-V3 sends every token to 8 *different*
  routed experts and sums their results with weights ("Lower latency and
  higher throughput with multi-node DeepSeek deployment", section "Expert
  parallelism").  The Mixtral router is the special case of DeepSeek routing
  whose top-K group is all experts (same page, section "MoE Router"); that
  special case is what ``route_topk`` defines.
* Dispatch.  The sender counts the tokens bound for each expert
  ("Efficient and portable mixture-of-experts communication", section
  "Dispatch"; "Enabling trillion-parameter models on AWS EFA", section
  "Dispatch and Combine": per-expert counts by atomic accumulation, then a
  prefix sum of the counts gives the offsets at which tokens are packed
  contiguously per peer, section "Send and Receive Buffers").  Buffers are
  sized for the worst case, so no token is ever dropped.  The receiver
  stores the tokens of each expert contiguously for the grouped GEMM and
  records, per row, which token it holds.
* Combine.  The receiver reads each token's K expert rows, uses the routing
  table to pick the buffer and the weight of each, and writes the weighted
  sum into caller-allocated tensors ("Efficient and portable
  mixture-of-experts communication", section "Combine"); accumulation happens
  on the receiving side only ("Enabling trillion-parameter models on AWS
  EFA", section "Evaluation").

Readings taken where the pages are silent
-----------------------------------------
R1  Selection is made on the fp32 logits.  Softmax is strictly increasing,
    so this equals selection on the exact probabilities; it avoids letting
    the rounding of ``exp`` decide the index set.
R2  Ties go to the lower expert index; +0.0 and -0.0 are equal.  Logits are
    finite (NaN/inf are outside the contract).
R3  The K outputs of a token are in descending-weight order, ties to the
    lower index.  This fixes the order combine accumulates in.
R4  Weights are the selected softmax probabilities renormalised to sum to 1
    (computed here in float64; the full-softmax denominator cancels).
R5  Expert ``e`` belongs to virtual rank ``e // (E // R)`` (contiguous).
R6  Within one expert, rows are ordered by ascending flat pair index
    ``p = t*K + j`` (stable counting sort); the pages' own receive order is
    non-deterministic.
R7  The dispatch buffer is packed: expert ``e`` owns rows
    ``[offsets[e], offsets[e+1])``; capacity must be at least ``T*K``.
R8  Combine: ``acc = +0.0f``; for j in 0..K-1 ``acc = fmaf(w[t,j],
    y[row], acc)`` in fp32 with one rounding per step; the result is rounded
    once to bf16, round-to-nearest-even.

Precision: routing weights in float64 (the pages fix no precision for
them); combine in fp32 with an fp32 FMA chain (the fp32 accumulation in K
order and single bf16 rounding that the combine contract states).
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

# ----------------------------------------------------------------------------
# bf16 <-> fp32 bit conversions (bf16 is carried as raw uint16 storage)
# ----------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 value is the upper 16 bits of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, round-to-nearest, ties to even; NaN stays NaN (quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return r


# ----------------------------------------------------------------------------
# fp32 fused multiply-add, correctly rounded (round-to-nearest-even)
# ----------------------------------------------------------------------------


def fmaf(a, b, c) -> np.ndarray:
    """Vectorised fp32 ``fma(a, b, c)`` with a single rounding.

    The product of two fp32 values is exact in float64 (24+24 < 53 bits).  The
    float64 sum ``s = p + c`` is rounded once; TwoSum recovers its exact error
    ``err``.  Rounding ``s`` to fp32 then gives the correctly rounded result,
    except when ``s`` is exactly halfway between two fp32 neighbours and
    ``err`` is non-zero: the exact value then lies strictly on the side of the
    midpoint that ``err`` points to.  Finite results only.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    r = s.astype(np.float32)
    rb = r.astype(np.float64)
    toward = np.where(s > rb, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    other = np.nextafter(r, toward)
    mid = (rb + other.astype(np.float64)) * 0.5
    fix = (rb != s) & (s == mid) & (err != 0)
    if np.any(fix):
        hi = np.maximum(r, other)
        lo = np.minimum(r, other)
        r = np.where(fix, np.where(err > 0, hi, lo), r).astype(np.float32)
    return r


def _round_fraction_to_f32(x: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32 (finite range)."""
    if x == 0:
        return np.float32(0.0)
    guess = np.float32(float(x))
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = None
    for cnd in cands:
        d = abs(Fraction(float(cnd)) - x)
        key = (d, int(np.array(cnd, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cnd)
    return np.float32(best[1])


def fmaf_exact(a: float, b: float, c: float) -> np.float32:
    """Scalar fp32 fma in exact rational arithmetic (reference for ``fmaf``)."""
    a, b, c = np.float32(a), np.float32(b), np.float32(c)
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if exact == 0:
        prod_neg = bool(np.signbit(a)) != bool(np.signbit(b))
        prod_zero = (a == 0) or (b == 0)
        neg = prod_zero and prod_neg and bool(np.signbit(c)) and c == 0
        return np.float32(-0.0) if neg else np.float32(0.0)
    return _round_fraction_to_f32(exact)


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------


def route_topk(logits: np.ndarray, k: int):
    """Top-k routing of every token (readings R1-R4).

    Returns ``idx`` int32 [T, k] (descending weight, ties to the lower index),
    ``w`` float64 [T, k] (renormalised softmax weights) and ``w32`` (``w``
    rounded to fp32, round-to-nearest-even).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    l64 = logits.astype(np.float64)
    # Selection: order experts by descending logit; a stable sort keeps the
    # lower index first among equal keys.  Adding +0.0 folds -0.0 into +0.0.
    key = -l64 + 0.0
    order = np.argsort(key, axis=1, kind="stable")
    idx = order[:, :k]
    # Softmax over all E experts (float64), then renormalise the k selected.
    m = l64.max(axis=1, keepdims=True)
    z = np.exp(l64 - m)
    p = z / z.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(p, idx, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    # The full-softmax denominator cancels: the same weights follow from the
    # selected numerators alone.  The two routes must agree.
    zsel = np.take_along_axis(z, idx, axis=1)
    w_alt = zsel / zsel.sum(axis=1, keepdims=True)
    if T and not np.allclose(w, w_alt, rtol=1e-13, atol=0.0):
        raise AssertionError("softmax renormalisation forms disagree")
    return idx.astype(np.int32), w, w.astype(np.float32)


def route_topk_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int):
    """Group-limited top-k routing (readings G1-G3).

    The pages call Mixtral routing the special case of DeepSeek routing in
    which the top-K group is the group of all experts ("Lower latency and
    higher throughput with multi-node DeepSeek deployment", section "MoE
    Router"); the group rule itself is not on the pages.  Reading: experts
    form ``n_group`` contiguous groups of E / n_group (G1); a group's score is
    its largest logit (G2); the ``topk_group`` best groups are kept, equal
    scores to the lower group index, and top-k runs over the kept experts
    with the usual ties and weights (G3: the full-E softmax renormalised over
    the k chosen).  ``topk_group == n_group`` is plain ``route_topk``.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if n_group < 1 or E % n_group:
        raise ValueError("E must be a multiple of n_group")
    gs = E // n_group
    if not 1 <= topk_group <= n_group or topk_group * gs < k:
        raise ValueError("need 1 <= topk_group <= n_group and topk_group * E/n_group >= k")
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    gmax = logits.astype(np.float64).reshape(T, n_group, gs).max(axis=2)
    gorder = np.argsort(-gmax + 0.0, axis=1, kind="stable")[:, :topk_group]
    keep = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep, gorder, True, axis=1)
    keep_e = np.repeat(keep, gs, axis=1)
    l64 = logits.astype(np.float64)
    key = np.where(keep_e, -l64 + 0.0, np.inf)
    idx = np.argsort(key, axis=1, kind="stable")[:, :k]
    m = l64.max(axis=1, keepdims=True)
    z = np.exp(l64 - m)
    p = z / z.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(p, idx, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w, w.astype(np.float32)


def route_topk_bruteforce(logits: np.ndarray, k: int):
    """Exhaustive top-k for tiny E: the k-subset with the largest exact logit
    sum; among equal sums, the lexicographically smallest sorted index tuple
    (which equals "ties to the lower index").  Returns the chosen sets as
    sorted int tuples, one per token.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    out = []
    for t in range(T):
        vals = [Fraction(float(v)) for v in logits[t]]
        best = None
        for sub in itertools.combinations(range(E), k):
            s = sum(vals[e] for e in sub)
            key = (-s, sub)
            if best is None or key < best:
                best = key
        out.append(best[1])
    return out


# ----------------------------------------------------------------------------
# Dispatch
# ----------------------------------------------------------------------------


def _check_idx(idx: np.ndarray, E: int) -> np.ndarray:
    idx = np.asarray(idx)
    if idx.ndim != 2:
        raise ValueError("idx must be [T, k]")
    if idx.size and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert index out of range")
    return idx.astype(np.int64)


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, j) pairs routed to each expert."""
    idx = _check_idx(idx, E)
    return np.bincount(idx.ravel(), minlength=E).astype(np.int64)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum of the counts, with the total appended (E+1)."""
    counts = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def rank_offsets(offsets: np.ndarray, R: int) -> np.ndarray:
    """Row offset of each virtual rank's segment (R+1): experts are assigned
    to ranks contiguously (reading R5)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    if R < 1 or E % R:
        raise ValueError("E must be a multiple of R")
    return offsets[:: E // R].copy()


def dispatch_slots(idx: np.ndarray, E: int):
    """Destination row of every pair and the token held by every row.

    Rows are expert-major; inside an expert, pairs keep ascending flat index
    ``p = t*k + j`` (reading R6).  Returns ``pair_row`` int64 [T, k] and
    ``row_token`` int64 [T*k].
    """
    idx = _check_idx(idx, E)
    T, k = idx.shape
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")        # row r holds pair order[r]
    pair_row = np.empty(flat.size, dtype=np.int64)
    pair_row[order] = np.arange(flat.size, dtype=np.int64)
    row_token = order // k if k else order
    return pair_row.reshape(T, k), row_token.astype(np.int64)


def dispatch_slots_sequential(idx: np.ndarray, E: int):
    """The same result as ``dispatch_slots`` by a one-pass counting sort in
    pure Python (for small inputs): walk pairs in ascending order, give each
    the next free slot of its expert."""
    idx = _check_idx(idx, E)
    T, k = idx.shape
    counts = [0] * E
    for e in idx.ravel().tolist():
        counts[e] += 1
    start = [0] * E
    acc = 0
    for e in range(E):
        start[e] = acc
        acc += counts[e]
    used = [0] * E
    pair_row = np.empty((T, k), dtype=np.int64)
    row_token = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            r = start[e] + used[e]
            used[e] += 1
            pair_row[t, j] = r
            row_token[r] = t
    return pair_row, row_token


def dispatch_rows(x_bits: np.ndarray, pair_row: np.ndarray, capacity: int,
                  fill: np.ndarray | None = None) -> np.ndarray:
    """Expert-major buffer: row ``pair_row[t, j]`` is a bit copy of ``x[t]``.
    Rows at or past ``T*k`` keep ``fill`` (zeros if not given)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    pair_row = np.asarray(pair_row, dtype=np.int64)
    k = pair_row.shape[1] if pair_row.ndim == 2 else 0
    if capacity < T * k:
        raise ValueError("capacity below T*k: the method never drops a token")
    if fill is None:
        buf = np.zeros((capacity, H), dtype=np.uint16)
    else:
        buf = np.array(fill, dtype=np.uint16, copy=True)
        assert buf.shape == (capacity, H)
    for j in range(k):
        buf[pair_row[:, j]] = x_bits
    return buf


# ----------------------------------------------------------------------------
# Combine
# ----------------------------------------------------------------------------


def combine_tokens(y_bits: np.ndarray, pair_row: np.ndarray, w32: np.ndarray,
                   tokens: np.ndarray) -> np.ndarray:
    """Combine for the listed tokens only (reading R8); bf16 bits [len, H]."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    pair_row = np.asarray(pair_row, dtype=np.int64)
    w32 = np.asarray(w32, dtype=np.float32)
    tokens = np.asarray(tokens, dtype=np.int64)
    H = y_bits.shape[1]
    k = pair_row.shape[1]
    acc = np.zeros((tokens.size, H), dtype=np.float32)   # +0.0f
    for j in range(k):
        rows = bf16_to_f32(y_bits[pair_row[tokens, j]])
        acc = fmaf(w32[tokens, j][:, None], rows, acc)
    return f32_to_bf16_rne(acc)


def combine(y_bits: np.ndarray, pair_row: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """Weighted sum of every token's k expert rows; bf16 bits [T, H]."""
    T = np.asarray(pair_row).shape[0]
    return combine_tokens(y_bits, pair_row, w32, np.arange(T))


def combine_exact(y_bits: np.ndarray, pair_row: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """Combine with every fma step done in exact rational arithmetic (tiny
    inputs only): the reference that ``combine``'s vectorised fma is checked
    against."""
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    pair_row = np.asarray(pair_row, dtype=np.int64)
    T, k = pair_row.shape
    H = y_bits.shape[1]
    out = np.empty((T, H), dtype=np.float32)
    yf = bf16_to_f32(y_bits)
    for t in range(T):
        for h in range(H):
            acc = np.float32(0.0)
            for j in range(k):
                acc = fmaf_exact(w32[t, j], yf[pair_row[t, j], h], acc)
            out[t, h] = acc
    return f32_to_bf16_rne(out)
