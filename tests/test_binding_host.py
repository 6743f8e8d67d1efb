"""The Python binding on the CPU: every call refuses host tensors before any
pointer reaches the library (there is no CPU path)."""
import numpy as np
import pytest
import torch

import combine_moe_get_dispatch_amd as moe


def test_layout_refuses_host_tensors():
    idx = torch.zeros((4, 2), dtype=torch.int64)
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_get_dispatch_layout(idx, 8, 2, 1)


def test_dispatch_and_combine_refuse_host_tensors():
    lay = moe.allocate_layout(4, 2, 8, 2, 1, device="cpu")
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_dispatch(x, lay)
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_dispatch_static(x, lay, torch.ones(1))
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_combine(torch.zeros((lay.recv_capacity, 64), dtype=torch.bfloat16), lay)
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_combine_fused(torch.zeros((lay.recv_capacity, 64), dtype=torch.bfloat16), lay)
    with pytest.raises(ValueError, match="HIP device"):
        moe.moe_dispatch_prequantized(torch.zeros((4, 32), dtype=torch.uint8), None, lay)


def test_layout_sizes_follow_the_capacity_bound():
    lay = moe.allocate_layout(100, 4, 16, 4, 8, device="cpu")
    assert lay.recv_capacity == 100 * 4 + 16 * 7
    assert tuple(lay.token_row.shape) == (100, 4) and tuple(lay.recv_src.shape) == (lay.recv_capacity,)
    assert tuple(lay.is_token_in_rank.shape) == (100, 4) and tuple(lay.expert_offsets.shape) == (17,)
    with pytest.raises(ValueError):
        moe.allocate_layout(-1, 4, 16, 4, 8, device="cpu")
