"""moe_dispatch_noalloc (the dispatch entry point for callers that cannot
allocate) against moe_dispatch with a caller workspace, and against the
oracle, on two calls in a row (the second smaller, with another E, so stale
scratch from the first would show), then a batch small enough to need no
scratch.  Nothing may be allocated by the calls."""
import numpy as np
import pytest
import torch

import oracle
from gpuhelp import DEV, dev_bf16, dev_i32, host, host_bf16

pytestmark = pytest.mark.gpu

# (T, E, k, H, R): the first uses the whole 64 KiB matrix (64 blocks x 256
# experts); the second 6 blocks x 384 experts; the third T*k <= 2048.
CALLS = [(8192, 256, 8, 256, 32), (1000, 384, 6, 512, 48), (200, 64, 4, 128, 8)]


def _outputs(T, E, k, H, R):
    P = T * k
    return dict(
        expert_counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
        expert_offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
        pair_row=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
        row_token=torch.full((P,), -7, dtype=torch.int32, device=DEV),
        rank_offsets=torch.full((R + 1,), -7, dtype=torch.int32, device=DEV),
        buf=torch.zeros((P, H), dtype=torch.bfloat16, device=DEV),
    )


def test_noalloc_dispatch_matches_workspace_dispatch_and_oracle():
    import combine_topk_route_amd as m

    rng = np.random.default_rng(11)
    for T, E, k, H, R in CALLS:
        print(f"[noalloc] T={T} E={E} k={k} H={H} R={R}", flush=True)
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        x_bits = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
        x_bits[(x_bits & 0x7F80) == 0x7F80] = 0x3F80  # no NaN/inf patterns in the copy
        d_idx, d_x = dev_i32(idx), dev_bf16(x_bits)
        got = _outputs(T, E, k, H, R)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        m.moe_dispatch_noalloc(d_idx, d_x, E, R, **got)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before, "the no-alloc call allocated"
        ref = _outputs(T, E, k, H, R)
        buf = ref.pop("buf")
        r_send, r_buf = m.moe_dispatch(d_idx, d_x, E, R, buf=buf, **ref)
        torch.cuda.synchronize()
        for name, t in zip(("expert_counts", "expert_offsets", "pair_row", "row_token",
                            "rank_offsets"), r_send):
            assert torch.equal(got[name], t), f"{name} differs from moe_dispatch"
        assert torch.equal(got["buf"].view(torch.int16), r_buf.view(torch.int16))
        counts = oracle.expert_counts(idx, E)
        off = oracle.expert_offsets(counts)
        pr, rt = oracle.dispatch_slots(idx, E)
        assert np.array_equal(host(got["expert_counts"]), counts)
        assert np.array_equal(host(got["expert_offsets"]), off)
        assert np.array_equal(host(got["rank_offsets"]), oracle.rank_offsets(off, R))
        assert np.array_equal(host(got["pair_row"]), pr)
        assert np.array_equal(host(got["row_token"]), rt)
        assert np.array_equal(host_bf16(got["buf"]), oracle.dispatch_rows(x_bits, pr, T * k))


def test_noalloc_dispatch_in_a_graph():
    """The use the entry point is for: captured into a HIP graph (after one
    eager call, which looks up the device's scratch array), replayed three
    times with eager work between replays and once more on new inputs,
    allocating nothing; every replay matches the oracle."""
    import combine_topk_route_amd as m

    T, E, k, H, R = 4096, 256, 8, 128, 32
    rng = np.random.default_rng(12)

    def inputs():
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        xb = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
        xb[(xb & 0x7F80) == 0x7F80] = 0x3F80
        return idx, xb

    idx, xb = inputs()
    d_idx, d_x = dev_i32(idx), dev_bf16(xb)
    got = _outputs(T, E, k, H, R)
    main = torch.cuda.current_stream()
    m.moe_dispatch_noalloc(d_idx, d_x, E, R, **got)
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        m.moe_dispatch_noalloc(d_idx, d_x, E, R, stream=side, **got)
    main.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_dispatch_noalloc(d_idx, d_x, E, R, stream=torch.cuda.current_stream(), **got)
    torch.cuda.synchronize()

    def check(idx_, xb_):
        pr, rt = oracle.dispatch_slots(idx_, E)
        counts = oracle.expert_counts(idx_, E)
        off = oracle.expert_offsets(counts)
        assert np.array_equal(host(got["expert_counts"]), counts)
        assert np.array_equal(host(got["expert_offsets"]), off)
        assert np.array_equal(host(got["rank_offsets"]), oracle.rank_offsets(off, R))
        assert np.array_equal(host(got["pair_row"]), pr)
        assert np.array_equal(host(got["row_token"]), rt)
        assert np.array_equal(host_bf16(got["buf"]), oracle.dispatch_rows(xb_, pr, T * k))

    before = torch.cuda.memory_allocated()
    for rep in range(3):
        print(f"[noalloc] graph replay {rep}", flush=True)
        for name, t in got.items():
            (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(idx, xb)
    idx2, xb2 = inputs()
    d_idx.copy_(dev_i32(idx2))
    d_x.copy_(dev_bf16(xb2))
    g.replay()
    torch.cuda.synchronize()
    check(idx2, xb2)
    assert torch.cuda.memory_allocated() == before
