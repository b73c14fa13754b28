"""More seeds: the whole bf16 path (route, send, recv, combine) against the
oracle on every config at further seeds, with the same bars as the main
parity suite (bit-exact indices, counts, offsets, rows; weights within
2^-20; combine on identical inputs bit-identical)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import (assert_out_close, assert_weights_close, dev_bf16, dev_f32, dev_i32, host,
                     host_bf16)

pytestmark = pytest.mark.gpu

CASES = [(n, s) for n in ["tiny", "mixtral", "dsv3_decode", "kimi_k2"] for s in (1, 2, 3)]
CASES += [("dsv3_prefill", 7)]


@pytest.mark.parametrize("name,seed", CASES)
def test_whole_path_at_more_seeds(name, seed):
    import combine_topk_route_amd as m

    wl = workloads.make(name, seed=seed)
    cfg = wl.cfg
    print(f"[seeds] {name} seed={seed}", flush=True)
    idx, w = m.moe_route_topk(dev_f32(wl.logits), cfg.k)
    torch.cuda.synchronize()
    r_idx, r_w, r_w32 = oracle.route_topk(wl.logits, cfg.k)
    assert np.array_equal(host(idx), r_idx)
    assert_weights_close(host(w), r_w)

    send, buf = m.moe_dispatch(dev_i32(r_idx), dev_bf16(wl.x), cfg.E, cfg.R)
    out = m.moe_combine(dev_bf16(wl.y), send.pair_row, dev_f32(r_w32))
    torch.cuda.synchronize()
    counts = oracle.expert_counts(r_idx, cfg.E)
    off = oracle.expert_offsets(counts)
    pr, rt = oracle.dispatch_slots(r_idx, cfg.E)
    assert np.array_equal(host(send.expert_counts), counts)
    assert np.array_equal(host(send.expert_offsets), off)
    assert np.array_equal(host(send.rank_offsets), oracle.rank_offsets(off, cfg.R))
    assert np.array_equal(host(send.pair_row), pr)
    assert np.array_equal(host(send.row_token), rt)
    assert np.array_equal(host_bf16(buf), wl.x[rt])
    got = host_bf16(out)
    for t0 in range(0, cfg.T, 1024):  # every token, the oracle in chunks
        tokens = np.arange(t0, min(cfg.T, t0 + 1024))
        ref = oracle.combine_tokens(wl.y, pr, r_w32, tokens)
        assert assert_out_close(got[tokens], ref) == 0
