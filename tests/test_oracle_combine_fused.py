"""Pins for the combine epilogues (shared-expert add, residual add, RMS
normalisation; Modular MAX EPBatchManager, ep_combine() fused shared-expert
mode; CANN aclnnMoeDistributeDispatchV2 Description, the
CombineAddRmsNorm companion).

  * identity experts with the token itself as shared output: out = x (sum w + 1)
  * a residual equal to minus the routed sum cancels it exactly
  * RMS normalisation: constant rows, a hand-worked row, scale invariance with
    eps = 0, gamma applied per channel, brute force with math.fsum / sqrt
"""
import math

import numpy as np
import pytest

from combine_moe_get_dispatch_amd import workloads as W
from test_oracle_quant import bf16


def _setup(orc, T=40, K=4, E=8, H=64, seed=0):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    lay = orc.layout(idx, E, 2, 2)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    rx, _, _ = orc.dispatch(x, lay.token_row, lay.recv_capacity)
    w = rng.random((T, K)).astype(np.float32)
    return rng, idx, lay, x, rx, w


def test_shared_expert_add_closed_form(orc):
    _, idx, lay, x, rx, w = _setup(orc)
    out, _ = orc.combine_fused(rx, lay.token_row, w, shared=x)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    wsum = np.where(idx >= 0, w.astype(np.float64), 0).sum(axis=1)
    np.testing.assert_allclose(out, xf * (wsum + 1)[:, None], rtol=1e-13, atol=0)


def test_residual_cancels_routed_sum(orc):
    rng = np.random.default_rng(3)
    T, H, E = 20, 96, 5
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = orc.layout(idx, E, 1, 1)
    rx, _, _ = orc.dispatch(x, lay.token_row, lay.recv_capacity)
    neg = x ^ np.uint16(0x8000)
    out, _ = orc.combine_fused(rx, lay.token_row, np.ones((T, 1), np.float32), residual=neg)
    assert (out == 0).all()
    out2, _ = orc.combine_fused(rx, lay.token_row, np.ones((T, 1), np.float32), shared=x, residual=neg)
    np.testing.assert_array_equal(out2, W.bf16_bits_to_f32(x).astype(np.float64))


def test_rmsnorm_constant_and_hand_worked_rows(orc):
    H = 32
    y = np.zeros((2, H), np.float32)
    y[0, :] = -3.0                       # constant row: norm = sign * gamma when eps = 0
    y[1, 0], y[1, 1] = 3.0, 4.0          # mean of squares 25/32: rms = 5 / sqrt(32)
    yb = bf16(y)
    rows = np.array([[0], [1]], np.int32)
    gamma = bf16(np.linspace(0.5, 2.0, H).astype(np.float32))
    g = W.bf16_bits_to_f32(gamma).astype(np.float64)
    _, norm = orc.combine_fused(yb, rows, None, gamma=gamma, eps=0.0, with_norm=True)
    np.testing.assert_allclose(norm[0], -g, rtol=1e-15)
    rms = 5.0 / math.sqrt(32.0)
    np.testing.assert_allclose(norm[1, :2], np.array([3.0, 4.0]) / rms * g[:2], rtol=1e-15)
    assert (norm[1, 2:] == 0).all()


def test_rmsnorm_scale_invariance_and_eps(orc):
    rng, idx, lay, x, rx, w = _setup(orc, seed=5)
    gamma = bf16(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    _, n1 = orc.combine_fused(rx, lay.token_row, w, gamma=gamma, eps=0.0, with_norm=True)
    _, n2 = orc.combine_fused(rx, lay.token_row, w * np.float32(4.0), gamma=gamma, eps=0.0, with_norm=True)
    live = (idx >= 0).any(axis=1)
    np.testing.assert_allclose(n1[live], n2[live], rtol=1e-12)
    _, n3 = orc.combine_fused(rx, lay.token_row, w, gamma=gamma, eps=1e6, with_norm=True)
    assert (np.abs(n3[live]) < np.abs(n1[live]) + 1e-30).all()


@pytest.mark.parametrize("seed", range(3))
def test_brute_force(orc, seed):
    rng, idx, lay, x, rx, w = _setup(orc, T=6, K=3, H=32, seed=seed + 10)
    sh = W.random_bf16_rows(6, 32, seed + 20)
    res = W.random_bf16_rows(6, 32, seed + 30)
    gamma = W.random_bf16_rows(1, 32, seed + 40)[0]
    eps = 1e-5
    out, norm = orc.combine_fused(rx, lay.token_row, w, sh, res, gamma, eps, with_norm=True)
    y = W.bf16_bits_to_f32(rx).astype(float)
    shf, rf, gf = (W.bf16_bits_to_f32(a).astype(float) for a in (sh, res, gamma))
    for t in range(6):
        s = []
        for h in range(32):
            terms = [float(w[t, k]) * y[lay.token_row[t, k], h] for k in range(3) if lay.token_row[t, k] >= 0]
            s.append(math.fsum(terms + [shf[t, h], rf[t, h]]))
        rms = math.sqrt(math.fsum(v * v for v in s) / 32 + eps)
        for h in range(32):
            assert abs(out[t, h] - s[h]) <= 1e-14 * (abs(s[h]) + 1)
            assert abs(norm[t, h] - s[h] / rms * gf[h]) <= 1e-12 * (abs(s[h] / rms * gf[h]) + 1e-12)
