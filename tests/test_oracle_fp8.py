"""Pins for the fp8 (OCP E4M3) block-scaled dispatch oracle: hand-decoded
codes, the round trip over every code, torch's float8_e4m3fn conversion
inside the representable range, ties to even, saturation, and the block
invariants of the scale."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def test_decode_hand_worked_codes():
    cases = {0x00: 0.0, 0x01: 2.0**-9, 0x07: 7 * 2.0**-9, 0x08: 2.0**-6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x79: 288.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    got = oracle.e4m3_decode(np.array(list(cases), np.uint8))
    assert got.tolist() == list(cases.values())
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    z = oracle.e4m3_decode(np.array([0x80], np.uint8))
    assert z[0] == 0 and np.signbit(z[0])


def test_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    keep = (codes & 0x7F) != 0x7F
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes[keep])), codes[keep])


def test_encode_matches_torch_inside_the_range():
    rng = np.random.default_rng(21)
    v = (rng.standard_normal(1_000_000) * 2.0 ** rng.integers(-14, 9, 1_000_000)).astype(np.float32)
    grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)       # every tie, exact in fp32
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(0))]).astype(np.float32)
    v = v[np.abs(v) <= 464.0]                                   # torch does not saturate past it
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_ties_go_to_even_and_saturation():
    enc = lambda xs: oracle.e4m3_encode(np.array(xs, np.float32)).tolist()
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39)
    assert enc([1.0625, 1.1875, 2.0**-10, 1.5 * 2.0**-10, 2.5 * 2.0**-9]) == [0x38, 0x3A, 0x00, 0x01, 0x02]
    assert enc([448.0, 464.0, 470.0, 1e6, 3e38, -500.0]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert enc([-0.0, -2.0**-11, 0.0]) == [0x80, 0x80, 0x00]


def test_block_quantization_invariants():
    wl = workloads.make("dsv3_decode", with_y=False)
    x = wl.x.copy()
    x[0, :128] = 0                      # a zero block
    x[1, 128:256] = 0x8000              # a block of -0.0
    q, s = oracle.quantize_rows(x)
    T, H = x.shape
    assert q.shape == (T, H) and s.shape == (T, H // 128)
    assert s[0, 0] == 1.0 and (q[0, :128] == 0).all()
    assert s[1, 1] == 1.0 and (q[1, 128:256] == 0x80).all()
    xf = oracle.bf16_to_f32(x).reshape(T, H // 128, 128).astype(np.float64)
    amax = np.abs(xf).max(axis=2)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448.0)))
    # the largest element of every non-zero block lands on +-448
    qb = q.reshape(T, H // 128, 128)
    top = np.take_along_axis(qb, np.abs(xf).argmax(axis=2)[:, :, None], axis=2)[:, :, 0]
    assert ((top[nz] & 0x7F) == 0x7E).all()
    # dequantised error: half an E4M3 ulp (2^-4 relative) in the normal
    # range, 2^-10 * scale below it
    deq = oracle.dequantize_rows(q, s).reshape(T, H // 128, 128)
    rel = np.abs(deq - xf) / s[:, :, None].astype(np.float64)
    assert (rel <= np.maximum(2.0**-4 * np.abs(xf) / s[:, :, None], 2.0**-10) * (1 + 1e-6)).all()


def test_fp8_dispatch_rows_follow_pair_row():
    wl = workloads.make("tiny", with_y=False)
    cfg = wl.cfg
    idx, _, _ = oracle.route_topk(wl.logits, cfg.k)
    pr, rt = oracle.dispatch_slots(idx, cfg.E)
    cap = cfg.P + 2
    bq, bs = oracle.dispatch_rows_fp8(wl.x, pr, cap, np.full((cap, cfg.H), 0x5A, np.uint8),
                                      np.full((cap, cfg.H // 128), -1.0, np.float32))
    q, s = oracle.quantize_rows(wl.x)
    assert np.array_equal(bq[: cfg.P], q[rt]) and np.array_equal(bs[: cfg.P], s[rt])
    assert (bq[cfg.P:] == 0x5A).all() and (bs[cfg.P:] == -1.0).all()
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.zeros((2, 100), np.uint16))
