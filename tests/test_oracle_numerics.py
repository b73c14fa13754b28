"""Pins for the oracle's numeric helpers: bf16 rounding and fp32 fma.

These check the oracle against things other than itself: hand-worked bit
patterns, torch's CPU bf16 conversion, glibc's ``fmaf`` and exact rational
arithmetic.
"""
import ctypes
import ctypes.util

import numpy as np
import torch

import oracle


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_hand_worked_patterns():
    cases = {
        0x3F800000: 0x3F80,  # 1.0 exact
        0x3F808000: 0x3F80,  # exactly halfway, lower neighbour even -> down
        0x3F818000: 0x3F82,  # exactly halfway, lower neighbour odd -> up
        0x3F808001: 0x3F81,  # just above halfway -> up
        0x3F807FFF: 0x3F80,  # just below halfway -> down
        0x80000000: 0x8000,  # -0.0 keeps its sign
        0x00000000: 0x0000,
        0x7F7FFFFF: 0x7F80,  # fp32 max rounds past bf16 max -> +inf
        0x7F7F7FFF: 0x7F7F,  # bf16 max finite stays
        0xFF800000: 0xFF80,  # -inf
        0x00000001: 0x0000,  # smallest subnormal rounds to +0
        0x00008000: 0x0000,  # halfway subnormal, even -> down
        0x00018000: 0x0002,  # halfway subnormal, odd -> up
        0x807FFFFF: 0x8080,  # largest negative subnormal rounds up in magnitude
    }
    got = oracle.f32_to_bf16_rne(_f32(list(cases)))
    assert got.tolist() == list(cases.values())


def test_bf16_rne_nan_stays_nan():
    got = oracle.f32_to_bf16_rne(_f32([0x7FC00000, 0x7F800001, 0xFFFFFFFF]))
    back = oracle.bf16_to_f32(got)
    assert np.isnan(back).all()


def test_bf16_rne_matches_torch_cpu():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    a = bits.view(np.float32)
    a = a[np.isfinite(a)]
    a = np.concatenate([a, rng.standard_normal(200_000).astype(np.float32)])
    ours = oracle.f32_to_bf16_rne(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_widening_is_exact_roundtrip():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    keep = ~np.isnan(f)
    assert np.array_equal(oracle.f32_to_bf16_rne(f[keep]), b[keep])
    assert np.array_equal(f.view(np.uint32) & 0xFFFF, np.zeros(65536, np.uint32))


# ---------------------------------------------------------------- fp32 fma

def _libm_fmaf():
    name = ctypes.util.find_library("m") or "libm.so.6"
    lib = ctypes.CDLL(name)
    f = lib.fmaf
    f.restype = ctypes.c_float
    f.argtypes = [ctypes.c_float] * 3
    return f


def _near_midpoint_triples(n, seed):
    """Triples whose fp64 sum lands on or next to an fp32 midpoint."""
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(n).astype(np.float32)
    ulp = (np.nextafter(np.abs(c), np.float32(np.inf)) - np.abs(c)).astype(np.float64)
    a = (1.0 + rng.integers(1, 2**23, n) * 2.0**-23).astype(np.float32)
    b = ((ulp / 2) / a.astype(np.float64)).astype(np.float32)
    b *= np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    return a, b, c


def test_fmaf_double_rounding_case_by_hand():
    # a*b = 2^-24 - 2^-70 exactly; c = 1 + 2^-23 (odd last bit).  The float64
    # sum rounds onto the fp32 midpoint c + 2^-24; the exact value is below
    # it, so the correct fp32 result is c itself (a naive double rounding would
    # go to the even neighbour 1 + 2^-22).
    a = np.float32(1 + 2.0**-23)
    b = np.float32(2.0**-24 * (1 - 2.0**-23))
    c = np.float32(1 + 2.0**-23)
    assert float(a) * float(b) + float(c) == 1 + 2.0**-23 + 2.0**-24
    assert oracle.fmaf(a, b, c) == c
    assert oracle.fmaf_exact(a, b, c) == c
    assert np.float32(float(a) * float(b) + float(c)) != c


def test_fmaf_matches_exact_rationals():
    a, b, c = _near_midpoint_triples(3000, seed=7)
    rng = np.random.default_rng(8)
    a2, b2, c2 = (rng.standard_normal(2000).astype(np.float32) for _ in range(3))
    a, b, c = (np.concatenate(v) for v in ((a, a2), (b, b2), (c, c2)))
    got = oracle.fmaf(a, b, c)
    ref = np.array([oracle.fmaf_exact(x, y, z) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fmaf_matches_glibc_fmaf():
    f = _libm_fmaf()
    a, b, c = _near_midpoint_triples(20000, seed=11)
    rng = np.random.default_rng(12)
    # wide exponent spread, including results near the subnormal range
    a2 = (rng.standard_normal(20000) * 2.0 ** rng.integers(-60, 60, 20000)).astype(np.float32)
    b2 = (rng.standard_normal(20000) * 2.0 ** rng.integers(-60, 60, 20000)).astype(np.float32)
    c2 = (rng.standard_normal(20000) * 2.0 ** rng.integers(-120, 100, 20000)).astype(np.float32)
    a, b, c = (np.concatenate(v) for v in ((a, a2), (b, b2), (c, c2)))
    got = oracle.fmaf(a, b, c)
    ref = np.array([f(float(x), float(y), float(z)) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the near-midpoint set really exercises the fix-up path
    s = a[:20000].astype(np.float64) * b[:20000] + c[:20000]
    assert np.count_nonzero(np.float32(s) != got[:20000]) > 0


def test_fmaf_signed_zero():
    z = oracle.fmaf(np.float32(-1.0), np.float32(0.0), np.float32(0.0))
    assert z == 0 and not np.signbit(z)
    z = oracle.fmaf(np.float32(-1.0), np.float32(0.0), np.float32(-0.0))
    assert z == 0 and np.signbit(z)
    assert not np.signbit(oracle.fmaf_exact(-1.0, 0.0, 0.0))
    assert np.signbit(oracle.fmaf_exact(-1.0, 0.0, -0.0))
