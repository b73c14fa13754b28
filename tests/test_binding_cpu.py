"""The binding's own argument checks, which reject bad tensors before any
call into the library (so they run without a GPU)."""
import pytest
import torch

import combine_topk_route_amd as m


def test_host_tensors_are_rejected():
    logits = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        m.moe_route_topk(logits, 2)
    with pytest.raises(ValueError, match="device"):
        m.moe_dispatch_send(torch.zeros((4, 2), dtype=torch.int32), 8)
    with pytest.raises(ValueError, match="device"):
        m.moe_dispatch_recv(torch.zeros((4, 8), dtype=torch.bfloat16),
                            torch.zeros((4, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="device"):
        m.moe_combine(torch.zeros((8, 8), dtype=torch.bfloat16), torch.zeros((4, 2), dtype=torch.int32),
                      torch.zeros((4, 2), dtype=torch.float32))


def test_non_tensors_are_rejected():
    with pytest.raises(TypeError, match="torch.Tensor"):
        m.moe_route_topk([[0.0] * 8] * 4, 2)


def test_abi_version_matches_the_header():
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "include", "moe_route.h")) as f:
        version = int(re.search(r"#define MOE_ABI_VERSION (\d+)", f.read()).group(1))
    assert m.moe_abi_version() == version
