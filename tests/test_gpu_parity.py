"""GPU parity: the HIP path against the CPU oracle on all five seeded configs,
at their full sizes, through the C ABI (the same launches bench.py times).

Every input comes from ``workloads``; every expected value from ``oracle``.
Indices, counts, offsets, rows and dispatched bytes must be bit-exact; routing
weights within 2^-20 relative; combine within 2^-7 relative (same inputs:
expected bit-exact, and the count of differing elements is reported).
Combine is compared on every token of every config; the oracle runs over
chunks of tokens to bound host memory.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import (DEV, assert_out_close, assert_weights_close, bf16_vals, dev_bf16, dev_f32,
                     dev_i32, host, host_bf16)

pytestmark = pytest.mark.gpu

CHUNK = 1024          # tokens per oracle combine call


@pytest.fixture(scope="module", params=list(workloads.CONFIGS))
def case(request):
    import combine_topk_route_amd as m  # noqa: F401  (fail loudly if not built)

    name = request.param
    print(f"\n[parity] config {name}: generating inputs", flush=True)
    wl = workloads.make(name, seed=0)
    cfg = wl.cfg
    idx, w64, w32 = oracle.route_topk(wl.logits, cfg.k)
    counts = oracle.expert_counts(idx, cfg.E)
    offsets = oracle.expert_offsets(counts)
    pair_row, row_token = oracle.dispatch_slots(idx, cfg.E)
    d = dict(wl=wl, cfg=cfg, idx=idx, w64=w64, w32=w32, counts=counts, offsets=offsets,
             rank_offsets=oracle.rank_offsets(offsets, cfg.R), pair_row=pair_row,
             row_token=row_token)
    yield d
    d.clear()
    torch.cuda.empty_cache()


def test_route_parity(case):
    import combine_topk_route_amd as m

    cfg, wl = case["cfg"], case["wl"]
    print(f"[parity] {cfg.name}: moe_route_topk T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    idx, w = m.moe_route_topk(dev_f32(wl.logits), cfg.k)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), case["idx"])
    worst = assert_weights_close(host(w), case["w64"])
    print(f"[parity] {cfg.name}: indices bit-exact, worst weight rel err {worst:.2e}", flush=True)


def test_send_parity(case):
    import combine_topk_route_amd as m

    cfg = case["cfg"]
    print(f"[parity] {cfg.name}: moe_dispatch_send P={cfg.P}", flush=True)
    res = m.moe_dispatch_send(dev_i32(case["idx"]), cfg.E, cfg.R)
    torch.cuda.synchronize()
    assert np.array_equal(host(res.expert_counts), case["counts"])
    assert np.array_equal(host(res.expert_offsets), case["offsets"])
    assert np.array_equal(host(res.rank_offsets), case["rank_offsets"])
    assert np.array_equal(host(res.pair_row), case["pair_row"])
    assert np.array_equal(host(res.row_token), case["row_token"])


def test_recv_parity_with_canaries(case):
    import combine_topk_route_amd as m

    cfg, wl = case["cfg"], case["wl"]
    cap = cfg.P + 4
    print(f"[parity] {cfg.name}: moe_dispatch_recv H={cfg.H} capacity={cap}", flush=True)
    buf = torch.full((cap, cfg.H), 0, dtype=torch.int16, device=DEV)
    buf.fill_(0x3C5A)  # canary bf16 pattern
    buf = buf.view(torch.bfloat16)
    m.moe_dispatch_recv(dev_bf16(wl.x), dev_i32(case["pair_row"]), buf=buf)
    torch.cuda.synchronize()
    got = host_bf16(buf)
    fill = np.full((cap, cfg.H), 0x3C5A, np.uint16)
    ref = oracle.dispatch_rows(wl.x, case["pair_row"], cap, fill)
    assert np.array_equal(got, ref)
    del got, ref


def _token_chunks(cfg):
    for t0 in range(0, cfg.T, CHUNK):
        yield np.arange(t0, min(cfg.T, t0 + CHUNK))


def test_combine_parity(case):
    import combine_topk_route_amd as m

    cfg, wl = case["cfg"], case["wl"]
    print(f"[parity] {cfg.name}: moe_combine T={cfg.T} H={cfg.H} k={cfg.k}", flush=True)
    out = m.moe_combine(dev_bf16(wl.y), dev_i32(case["pair_row"]), dev_f32(case["w32"]))
    torch.cuda.synchronize()
    got_all = host_bf16(out)
    ndiff = 0
    for tokens in _token_chunks(cfg):
        ref = oracle.combine_tokens(wl.y, case["pair_row"], case["w32"], tokens)
        ndiff += assert_out_close(got_all[tokens], ref)
    print(f"[parity] {cfg.name}: combine checked all {cfg.T} tokens, {ndiff} elements "
          f"not bit-identical", flush=True)
    assert ndiff == 0


def test_chain_parity(case):
    """route -> dispatch -> combine entirely on the GPU, against the oracle's
    chain.  Indices and rows are bit-exact; the weights differ from the
    oracle's within 2^-20, so combine gets an extra absolute allowance of
    2^-19 * sum_j w_j |y_j| on top of 2^-7 relative."""
    import combine_topk_route_amd as m

    cfg, wl = case["cfg"], case["wl"]
    print(f"[parity] {cfg.name}: chained route/dispatch/combine", flush=True)
    x = dev_bf16(wl.x)
    idx, w = m.moe_route_topk(dev_f32(wl.logits), cfg.k)
    send, buf = m.moe_dispatch(idx, x, cfg.E, cfg.R)
    out = m.moe_combine(dev_bf16(wl.y), send.pair_row, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), case["idx"])
    assert np.array_equal(host(send.pair_row), case["pair_row"])
    assert np.array_equal(host(send.row_token), case["row_token"])
    # dispatched rows: every row r holds x[row_token[r]]
    assert np.array_equal(host_bf16(buf), wl.x[case["row_token"]])
    got_all = host_bf16(out)
    yv = bf16_vals(wl.y)
    ndiff = 0
    for tokens in _token_chunks(cfg):
        ref = oracle.combine_tokens(wl.y, case["pair_row"], case["w32"], tokens)
        mag = sum(case["w64"][tokens, j, None] * np.abs(yv[case["pair_row"][tokens, j]])
                  for j in range(cfg.k))
        ndiff += assert_out_close(got_all[tokens], ref, extra_abs=2.0**-19 * mag)
    print(f"[parity] {cfg.name}: chain ok over all {cfg.T} tokens, {ndiff} combine elements "
          f"not bit-identical", flush=True)
