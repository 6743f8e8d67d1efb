"""Dynamic quantisation (per token, per 128-element group, MX per 32-element
block) against plain torch arithmetic on the GPU, a check that shares
nothing with the oracle.

CANN page "aclnnMoeDistributeDispatchV2", Formula Case 3: the row's scale is
the destination maximum (127 for int8, 448 for e4m3fn, 57344 for e5m2)
divided by the row's largest magnitude, each code is the cast of the fp32
product of the element and that scale, and the stored scale is the
reciprocal of it.  Torch computes the same with IEEE fp32 division and
multiplication (`torch.div` of two tensors; `scalar / tensor` multiplies by
a reciprocal instead and is not used), round-half-even then clamp for int8,
and its own float8 casts (round-half-even; no product exceeds the maximum by
more than its rounding, so no cast overflows).  Every valid row's codes and
scale must be bit-equal.  Rows whose maximum is zero are left to the oracle
tests (torch's 0 * inf is NaN).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe
    from gpu_util import DEV

MODES = [(2, 127.0, torch.int8), (0x12, 448.0, torch.float8_e4m3fn), (0x22, 57344.0, torch.float8_e5m2)]


@pytest.mark.parametrize("quant,dst_max,dtype", MODES, ids=["int8", "e4m3fn", "e5m2"])
def test_per_token_codes_equal_torch_arithmetic(quant, dst_max, dtype):
    T, H, E, R, K = 2048, 7168, 64, 8, 4
    print(f"[torch crosscheck] quant={quant:#x} T={T} H={H}", flush=True)
    rng = np.random.default_rng(quant)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    idx[rng.random((T, K)) < 0.05] = -1
    g = torch.Generator(device=DEV)
    g.manual_seed(quant)
    x = (torch.randn((T, H), device=DEV, generator=g) * 2.0).to(torch.bfloat16)
    x[::97] *= 1e-30           # tiny rows: scales near the top of the fp32 range
    lay = moe.moe_get_dispatch_layout(torch.from_numpy(idx).to(DEV), E, R, 1)
    rx, rs, _ = moe.moe_dispatch(x, lay, None, quant)

    xf = x.float()
    m = xf.abs().amax(dim=1, keepdim=True)
    assert bool((m > 0).all())
    ds = torch.div(torch.full_like(m, dst_max), m)
    assert bool(torch.isfinite(ds).all())
    prod = xf * ds
    if dtype == torch.int8:
        q = torch.round(prod).clamp_(-127.0, 127.0).to(torch.int8)
    else:
        q = prod.to(dtype)
    s = torch.div(torch.ones_like(ds), ds)[:, 0]

    tr = lay.token_row.long()
    valid = tr >= 0
    tok = torch.arange(T, device=DEV)[:, None].expand(T, K)[valid]
    rows = tr[valid]
    assert torch.equal(rx[rows].view(torch.uint8), q[tok].view(torch.uint8))
    assert torch.equal(rs[rows].view(torch.int32), s[tok].view(torch.int32))
    torch.cuda.synchronize()


def _routed(T, E, K, seed, H):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    idx[rng.random((T, K)) < 0.05] = -1
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.randn((T, H), device=DEV, generator=g)
    x[:, ::50] *= 40.0         # outliers, so that blocks and groups differ in range
    return torch.from_numpy(idx).to(DEV), x.to(torch.bfloat16)


def _valid_rows(lay, T, K):
    tr = lay.token_row.long()
    valid = tr >= 0
    return torch.arange(T, device=DEV)[:, None].expand(T, K)[valid], tr[valid]


@pytest.mark.parametrize("quant,emax,dst_max,dtype", [(4, 8, 448.0, torch.float8_e4m3fn),
                                                      (0x24, 15, 57344.0, torch.float8_e5m2)],
                         ids=["mxfp8_e4m3", "mxfp8_e5m2"])
def test_mx_codes_equal_torch_arithmetic(quant, emax, dst_max, dtype):
    """CANN page, Formula Case 5, in torch: per 32-element block the shared
    exponent is floor(log2 max|x|) - emax (frexp gives it exactly), at least
    -127; the stored byte is that exponent + 127; codes are the cast of x
    times 2^-exponent (ldexp, exact), clamped to the largest finite value
    first.  An all-zero block has exponent -127."""
    T, H, E, R, K = 1024, 7168, 64, 8, 4
    idx, x = _routed(T, E, K, quant, H)
    lay = moe.moe_get_dispatch_layout(idx, E, R, 1)
    rx, rs, _ = moe.moe_dispatch(x, lay, None, quant)

    xb = x.float().view(T, H // 32, 32)
    amax = xb.abs().amax(dim=2, keepdim=True)
    _, e = torch.frexp(amax)                       # amax = m * 2^e, m in [0.5, 1)
    se = torch.where(amax > 0, (e - 1 - emax).clamp(min=-127), torch.full_like(e, -127))
    v = torch.ldexp(xb, (-se).float())
    q = v.clamp(-dst_max, dst_max).to(dtype).view(T, H)
    sb = (se + 127).to(torch.uint8).view(T, H // 32)

    tok, rows = _valid_rows(lay, T, K)
    assert torch.equal(rx[rows].view(torch.uint8), q[tok].view(torch.uint8))
    assert torch.equal(rs[rows], sb[tok])
    torch.cuda.synchronize()


@pytest.mark.parametrize("quant,dst_max,dtype", [(0x13, 448.0, torch.float8_e4m3fn),
                                                 (0x23, 57344.0, torch.float8_e5m2)],
                         ids=["group_e4m3fn", "group_e5m2"])
def test_per_group_codes_equal_torch_arithmetic(quant, dst_max, dtype):
    """CANN page, Formula Case 4: Case 3's formula over each 128-element
    group of the row, one fp32 scale per group."""
    T, H, E, R, K = 1024, 7168, 64, 8, 4
    idx, x = _routed(T, E, K, quant, H)
    lay = moe.moe_get_dispatch_layout(idx, E, R, 1)
    rx, rs, _ = moe.moe_dispatch(x, lay, None, quant)

    xg = x.float().view(T, H // 128, 128)
    m = xg.abs().amax(dim=2, keepdim=True)
    assert bool((m > 0).all())
    ds = torch.div(torch.full_like(m, dst_max), m)
    q = (xg * ds).to(dtype).view(T, H)
    s = torch.div(torch.ones_like(ds), ds).view(T, H // 128)

    tok, rows = _valid_rows(lay, T, K)
    assert torch.equal(rx[rows].view(torch.uint8), q[tok].view(torch.uint8))
    assert torch.equal(rs[rows].view(torch.int32), s[tok].view(torch.int32))
    torch.cuda.synchronize()
