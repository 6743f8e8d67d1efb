"""Pins for the oracle's combine (weighted sum of each token's expert rows).

  * identity experts: combine(dispatch(x)) = x * sum_k w[t, k]
  * a single expert with weight 1 returns x bit for bit
  * brute force with exactly rounded sums (math.fsum) on small inputs, with
    rows, tokens and hidden sizes all different so a transposed or
    mis-indexed operand cannot pass
  * no weights means weight 1; a token with no valid entry gives 0.
"""
import math

import numpy as np
import pytest

from combine_moe_get_dispatch_amd import workloads as W


def test_identity_experts_give_x_times_weight_sum(orc):
    w = W.WORKLOADS[0]
    inp = W.generate(w)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rx, _, _ = orc.dispatch(inp.x_bits, lay.token_row, lay.recv_capacity)
    out = orc.combine(rx, lay.token_row, inp.topk_weights)
    x = W.bf16_bits_to_f32(inp.x_bits).astype(np.float64)
    wsum = np.where(inp.topk_idx >= 0, inp.topk_weights.astype(np.float64), 0).sum(axis=1)
    np.testing.assert_allclose(out, x * wsum[:, None], rtol=1e-13, atol=0)


def test_identity_experts_with_drops_and_alignment(orc):
    w = W.WORKLOADS[3]
    inp = W.generate(w, num_tokens=64)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rx, _, _ = orc.dispatch(inp.x_bits, lay.token_row, lay.recv_capacity)
    out = orc.combine(rx, lay.token_row, inp.topk_weights)
    x = W.bf16_bits_to_f32(inp.x_bits).astype(np.float64)
    wsum = np.where(inp.topk_idx >= 0, inp.topk_weights.astype(np.float64), 0).sum(axis=1)
    np.testing.assert_allclose(out, x * wsum[:, None], rtol=1e-13, atol=0)


def test_single_expert_weight_one_is_exact(orc):
    rng = np.random.default_rng(2)
    T, H, E = 20, 96, 5
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay = orc.layout(idx, E, 1, 3)
    rx, _, _ = orc.dispatch(x, lay.token_row, lay.recv_capacity)
    out = orc.combine(rx, lay.token_row, np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(out, W.bf16_bits_to_f32(x).astype(np.float64))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_fsum(orc, seed):
    rng = np.random.default_rng(seed)
    T, K, H = 7, 3, 64
    cap = 23
    y = W.random_bf16_rows(cap, H, seed)
    rows = rng.integers(-1, cap, size=(T, K)).astype(np.int32)
    wts = rng.standard_normal((T, K)).astype(np.float32)
    out = orc.combine(y, rows, wts)
    yf = W.bf16_bits_to_f32(y)
    for t in range(T):
        for h in range(H):
            terms = [float(wts[t, k]) * float(yf[rows[t, k], h]) for k in range(K) if rows[t, k] >= 0]
            exact = math.fsum(terms)
            bound = 4 * 2.0 ** -53 * sum(abs(v) for v in terms)
            assert abs(out[t, h] - exact) <= bound


def test_no_weights_means_plain_sum(orc):
    rng = np.random.default_rng(9)
    y = W.random_bf16_rows(10, 32, 4)
    rows = np.array([[0, 3], [9, -1], [-1, -1]], np.int32)
    out = orc.combine(y, rows, None)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    np.testing.assert_array_equal(out[0], yf[0] + yf[3])
    np.testing.assert_array_equal(out[1], yf[9])
    np.testing.assert_array_equal(out[2], np.zeros(32))


def test_rows_outside_capacity_are_ignored(orc):
    y = W.random_bf16_rows(4, 32, 5)
    rows = np.array([[1, 4], [-1, 7]], np.int32)
    out = orc.combine(y, rows, np.ones((2, 2), np.float32))
    np.testing.assert_array_equal(out[0], W.bf16_bits_to_f32(y)[1].astype(np.float64))
    assert (out[1] == 0).all()
