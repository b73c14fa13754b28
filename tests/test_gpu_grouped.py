"""GPU parity for group-limited routing against the oracle.

Batches up to 2048 tokens route one wave per token; larger ones take the
lane-group kernel wherever each group is 1, 2, 4, 8 or 16 whole lanes of
16-byte loads, and the wave kernel otherwise.  Every shape below runs as
given and tiled past 2048 tokens, so both kernels see it."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpuhelp import assert_weights_close, dev_f32, host

pytestmark = pytest.mark.gpu


ROUTE_WAVE_MAX_TOKENS = 2048   # larger batches can take the lane-group kernel


def _check(logits, k, G, TG, label):
    import combine_topk_route_amd as m

    T = logits.shape[0]
    big_T = ROUTE_WAVE_MAX_TOKENS + 53 + T % 7
    big = np.tile(logits, (-(-big_T // T), 1))[:big_T]
    for lg in ([logits, big] if T <= ROUTE_WAVE_MAX_TOKENS else [logits]):
        print(f"[grouped] {label} T={lg.shape[0]} E={lg.shape[1]} k={k} G={G} TG={TG}",
              flush=True)
        idx, w = m.moe_route_topk_grouped(dev_f32(lg), k, G, TG)
        torch.cuda.synchronize()
        r_idx, r_w, _ = oracle.route_topk_grouped(lg, k, G, TG)
        assert np.array_equal(host(idx), r_idx)
        assert_weights_close(host(w), r_w)


@pytest.mark.parametrize("name,G,TG", [("dsv3_prefill", 8, 4), ("dsv3_decode", 8, 4),
                                       ("kimi_k2", 8, 4), ("kimi_k2", 48, 6), ("mixtral", 4, 2),
                                       ("tiny", 2, 1), ("dsv3_prefill", 8, 8)])
def test_grouped_parity_on_configs(name, G, TG):
    wl = workloads.make(name, seed=0, with_y=False)
    _check(wl.logits, wl.cfg.k, G, TG, name)


# Past 2048 tokens: lanes per group 8 (256/8/3), 16 (1024/4/2), 1 (256/64/8),
# 2 (128/8/3 and 256/32/1), 4 (512/16/5, 1024/16/4 with k = 32, and 96/3/2,
# whose last four lanes hold no expert); the rest keep the wave kernel.
@pytest.mark.parametrize("E,k,G,TG", [(320, 8, 64, 2), (1024, 32, 16, 4), (64, 6, 64, 6),
                                      (12, 3, 3, 1), (100, 5, 4, 3), (256, 8, 32, 1),
                                      (256, 8, 8, 3), (1024, 32, 4, 2), (256, 8, 64, 8),
                                      (128, 6, 8, 3), (512, 16, 16, 5), (96, 4, 3, 2),
                                      (64, 20, 4, 2)])
def test_grouped_shapes_and_ties(E, k, G, TG):
    rng = np.random.default_rng(E + G)
    logits = rng.standard_normal((200, E)).astype(np.float32)
    logits[0] = 0.5                                   # every group ties
    logits[1] = np.round(logits[1] * 2) / 2           # many ties
    logits[2, :] = -1.0
    logits[2, 0], logits[2, E - 1] = -0.0, 0.0
    _check(logits, k, G, TG, "shapes")


def test_keeping_every_group_equals_plain_routing():
    import combine_topk_route_amd as m

    wl = workloads.make("kimi_k2", seed=4, with_y=False)
    lg = dev_f32(wl.logits)
    a = m.moe_route_topk(lg, 8)
    b = m.moe_route_topk_grouped(lg, 8, 48, 48)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
