"""HIP-graph capture of the whole path: launches are sized from T*k only, so
one captured graph serves any routing.  Every replay, with eager work and
synchronisations between replays, is checked against the oracle (indices,
counts, offsets, rows and dispatched bytes bit-exact, weights within 2^-20,
combine bit-identical on the kernel's weights) and against the eager run."""
import numpy as np
import pytest
import torch

import workloads
from gpuhelp import DEV, assert_step_matches_oracle, dev_bf16, dev_f32, host, host_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "mixtral", "dsv3_decode"])
def test_graph_replays_match_eager(name):
    import combine_topk_route_amd as m

    cfg = workloads.CONFIGS[name]
    wl = workloads.make(cfg, seed=3)
    wl2 = workloads.make(cfg, seed=4, with_y=False)
    print(f"[graph] {name}: capture route/dispatch/combine", flush=True)
    T, H, E, k, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.R
    P = T * k
    logits = dev_f32(wl.logits)
    x = dev_bf16(wl.x)
    y = dev_bf16(wl.y)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    pair_row = torch.empty((T, k), dtype=torch.int32, device=DEV)
    row_token = torch.empty((P,), dtype=torch.int32, device=DEV)
    rank_off = torch.empty((R + 1,), dtype=torch.int32, device=DEV)
    ws = torch.empty((max(1, m.moe_dispatch_workspace_bytes(T, E, k)),), dtype=torch.uint8,
                     device=DEV)
    buf = torch.empty((P, H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    outs = (idx, w, counts, offsets, pair_row, row_token, rank_off, buf, out)

    def step(st):
        m.moe_route_topk(logits, k, topk_idx=idx, topk_w=w, stream=st)
        m.moe_dispatch(idx, x, E, R, expert_counts=counts, expert_offsets=offsets,
                       pair_row=pair_row, row_token=row_token, rank_offsets=rank_off,
                       buf=buf, workspace=ws, stream=st)
        m.moe_combine(y, pair_row, w, out=out, stream=st)

    def snapshot():
        return [host_bf16(t) if t.dtype == torch.bfloat16 else host(t) for t in outs]

    def check_oracle(w_in):
        assert_step_matches_oracle(w_in.logits, w_in.x, k, E, R, idx, w,
                                   (counts, offsets, pair_row, row_token, rank_off), buf,
                                   y_bits=wl.y, out=out)

    main = torch.cuda.current_stream()
    step(main)
    torch.cuda.synchronize()
    eager = snapshot()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        step(side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), f"replay {rep} differs from eager"
        check_oracle(wl)

    # new routing inputs, same graph: the replay must equal a fresh eager run
    logits.copy_(dev_f32(wl2.logits))
    x.copy_(dev_bf16(wl2.x))
    g.replay()
    torch.cuda.synchronize()
    got = snapshot()
    check_oracle(wl2)
    step(main)
    torch.cuda.synchronize()
    for a, b in zip(got, snapshot()):
        assert np.array_equal(a, b), "replay on new inputs differs from eager"
