"""End to end, the way a MoE layer uses the library: layout, dispatch, one
matrix product per expert over that expert's row segment [expert_offsets[e],
expert_offsets[e + 1]) of the receive buffer, combine -- against a dense
reference computed on the CPU, token by token, from the routing alone.

The expert products run in fp32 with torch (not this library) and are
rounded to bf16, as an expert's output would be; the reference rounds the
same products the same way, so the comparison holds each token's combine to
the combine bound.  Both the two-call layout + dispatch and the one-launch
form are used, with and without alignment padding.
"""
import numpy as np
import pytest
import torch

from combine_moe_get_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe
    from gpu_util import DEV, bf16_dev, bf16_host_bits


@pytest.mark.parametrize("one_launch,a", [(False, 1), (False, 16), (True, 1), (True, 8)])
def test_moe_layer_against_dense_reference(one_launch, a):
    rng = np.random.default_rng(61 + a + one_launch)
    T, H, E, R, K = 200, 256, 16, 4, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = np.argsort(-logits, axis=1)[:, :K].astype(np.int64)
    idx[rng.random((T, K)) < 0.1] = -1
    top = np.take_along_axis(logits, np.maximum(idx, 0), axis=1)
    wts = np.exp(top - top.max(axis=1, keepdims=True))
    wts = (wts / wts.sum(axis=1, keepdims=True)).astype(np.float32)
    wts[idx < 0] = 0.0
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w_experts = (rng.standard_normal((E, H, H)) / np.sqrt(H)).astype(np.float32)

    x = bf16_dev(x_bits)
    idx_d, w_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(wts).to(DEV)
    if one_launch:
        lay, rx, _, _ = moe.moe_layout_and_dispatch(idx_d, x, E, R, a)
    else:
        lay = moe.moe_get_dispatch_layout(idx_d, E, R, a)
        rx, _, _ = moe.moe_dispatch(x, lay)
    off = lay.expert_offsets.cpu().numpy()
    y = torch.zeros_like(rx)
    wex = torch.from_numpy(w_experts).to(DEV)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:   # padding rows are expert input too; combine never reads them
            y[lo:hi] = (rx[lo:hi].float() @ wex[e]).to(torch.bfloat16)
    out = moe.moe_combine(y, lay, w_d)
    g = W.bf16_bits_to_f32(bf16_host_bits(out)).astype(np.float64)

    # dense reference: every (token, k) through its expert, rounded to bf16,
    # weighted and summed in fp64
    xf = torch.from_numpy(W.bf16_bits_to_f32(x_bits))
    ref = np.zeros((T, H))
    bound = np.zeros((T, H))
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if e < 0:
                continue
            ye = (xf[t:t + 1] @ torch.from_numpy(w_experts[e])).to(torch.bfloat16).float().numpy()[0]
            ref[t] += float(wts[t, k]) * ye.astype(np.float64)
            bound[t] += abs(float(wts[t, k])) * np.abs(ye)
    # the expert products on the GPU and the CPU may round differently to
    # bf16 (one ulp, 2^-8 relative, of each product), then the combine bound
    tol = 2.0 ** -7 * bound + 2.0 ** -8 * np.abs(ref) + (K + 1) * 2.0 ** -24 * bound
    assert (np.abs(g - ref) <= tol).all(), float(np.max(np.abs(g - ref) - tol))
    torch.cuda.synchronize()
