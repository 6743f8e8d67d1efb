"""The Python binding on the CPU: every call refuses host tensors before any
pointer reaches the library (there is no CPU path)."""
import dataclasses

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


def test_layouts_are_checked_when_made():
    """Every tensor of a layout is checked against its sizes when the layout
    is made, and the fields cannot be reassigned afterwards."""
    lay = moe.allocate_layout(64, 4, 16, 4, 2, device="cpu")
    bad_fields = [
        ("token_row", lay.token_row[:-1]),
        ("token_row", lay.token_row.to(torch.int64)),
        ("recv_src", lay.recv_src[:-1]),
        ("is_token_in_rank", torch.empty((4, 64), dtype=torch.int32).t()),   # right shape, not contiguous
        ("expert_offsets", lay.expert_offsets[:-1]),
        ("num_tokens_per_rank", torch.empty(5, dtype=torch.int32)),
        ("num_tokens_per_expert", torch.empty(16, dtype=torch.int64)),
        ("num_recv_tokens_per_expert", torch.empty(15, dtype=torch.int32)),
        ("error_flag", torch.empty(2, dtype=torch.int32)),
        ("workspace", torch.empty(8, dtype=torch.int32)),
        ("recv_src", torch.empty(lay.recv_capacity, dtype=torch.int32, device="meta")),  # another device
    ]
    for field, bad in bad_fields:
        with pytest.raises((ValueError, TypeError)):
            dataclasses.replace(lay, **{field: bad})
    with pytest.raises((ValueError, TypeError)):
        dataclasses.replace(lay, num_tokens=63)
    with pytest.raises(dataclasses.FrozenInstanceError):
        lay.token_row = lay.token_row.clone()
    ok = dataclasses.replace(lay, token_row=lay.token_row.clone())
    assert ok.token_row.shape == (64, 4)
