"""CPU oracle for block-scaled fp8 dispatch.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module.  It shares no code with the HIP path.

What the pages fix: activations are quantised to fp8 on the fly with one
scale per 128-element block ("Lower latency and higher throughput with
multi-node DeepSeek deployment", section "Quantization"), and dispatch ships
the fp8 tokens together with their block scale factors ("Efficient and
portable mixture-of-experts communication", section "Dispatch"; "Enabling
trillion-parameter models on AWS EFA", section "Evaluation": fp8 block-scaled
dispatch, bf16 combine).

Readings taken where the pages are silent:
Q1  The fp8 format is OCP E4M3 ("e4m3fn": 4 exponent bits, bias 7, 3 mantissa
    bits, no infinities, largest finite 448, NaN = S.1111.111).
Q2  Block b of a token row holds elements [128 b, 128 b + 128); H must be a
    multiple of 128.
Q3  scale = amax / 448 in fp32 (one rounding), amax = max |x| over the block;
    a block of zeros gets scale 1.0.
Q4  code = E4M3(x / scale): fp32 division (one rounding), then round to the
    nearest E4M3 value, ties to the even code, saturating at +-448.
Q5  Scales are stored as fp32, [capacity, H / 128], next to the fp8 rows
    [capacity, H]; the rows go where the bf16 dispatch would put them.
"""
from __future__ import annotations

import numpy as np

from .moe import bf16_to_f32

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of every E4M3 code (float32; NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man * 2.0 ** -9
    nor = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    val = np.where(exp == 0, sub, nor) * sign
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return val.astype(np.float32)


_POS_CODES = np.arange(0x7F, dtype=np.uint8)           # 0x00 .. 0x7E: 0 .. 448
_POS_VALUES = e4m3_decode(_POS_CODES).astype(np.float64)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each float32, ties to the even code, saturating
    at +-448 (reading Q4).  The sign of zero is kept."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, _POS_VALUES.size - 1)
    lo = np.clip(hi - 1, 0, None)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, (code & 0x80) | 0x7F, code).astype(np.uint8)
    return code


def quantize_rows(x_bits: np.ndarray):
    """Block-scaled fp8 of bf16 rows [T, H] -> (codes uint8 [T, H],
    scales float32 [T, H / 128]) (readings Q2-Q4)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    if H % BLOCK:
        raise ValueError("H must be a multiple of 128")
    xf = bf16_to_f32(x_bits).reshape(T, H // BLOCK, BLOCK)
    amax = np.abs(xf).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((xf / scale[:, :, None]).astype(np.float32))
    return q.reshape(T, H), scale


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float32 values code * scale (for error checks)."""
    q = np.asarray(q, dtype=np.uint8)
    T, H = q.shape
    vals = e4m3_decode(q).reshape(T, H // BLOCK, BLOCK).astype(np.float64)
    return (vals * np.asarray(scale, np.float64)[:, :, None]).reshape(T, H)


def dispatch_rows_fp8(x_bits: np.ndarray, pair_row: np.ndarray, capacity: int,
                      fill_q: np.ndarray | None = None, fill_s: np.ndarray | None = None):
    """fp8 expert-major buffer: row ``pair_row[t, j]`` holds the block-scaled
    fp8 codes of ``x[t]`` and its scales.  Rows at or past ``T*k`` keep the
    fills (zeros if not given)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    pair_row = np.asarray(pair_row, dtype=np.int64)
    k = pair_row.shape[1]
    if capacity < T * k:
        raise ValueError("capacity below T*k: the method never drops a token")
    q, s = quantize_rows(x_bits)
    buf_q = np.zeros((capacity, H), np.uint8) if fill_q is None else np.array(fill_q, np.uint8)
    buf_s = (np.zeros((capacity, H // BLOCK), np.float32) if fill_s is None
             else np.array(fill_s, np.float32))
    for j in range(k):
        buf_q[pair_row[:, j]] = q
        buf_s[pair_row[:, j]] = s
    return buf_q, buf_s
