"""Pins for per-group dynamic FP8 quantisation (CANN aclnnMoeDistributeDispatchV2,
Formula Case 4 = Case 3 per group of 128) and static int8 quantisation
(Formula Case 2).

Per-group: groups whose maximum is the destination's largest value have scale
exactly 1 and give the element casts, wherever in the group the maximum
lies; groups are independent (different
magnitudes in neighbouring groups give their own power-of-two scales); a
partial last group; a zero group next to normal groups; the fp32 formula in
exact rationals.
Static: scale 1 on integer rows gives the saturated integers; half-way ties;
per-channel power-of-two scales; per-channel scales are applied by channel.
"""
from fractions import Fraction

import numpy as np
import pytest

from combine_moe_get_dispatch_amd import workloads as W
from test_oracle_quant import bf16, fp32_round


def cast(orc, fmt):
    return orc.cast_to_fp8_e4m3fn if fmt == "e4m3" else orc.cast_to_fp8_e5m2


VMAX = {"e4m3": 448.0, "e5m2": 57344.0}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pergroup_groups_are_independent(orc, fmt):
    # three groups of 128 with maxima vmax*2^3, vmax*2^-5, vmax: scales 2^3, 2^-5, 1
    rng = np.random.default_rng(31)
    vmax = VMAX[fmt]
    v = W.bf16_bits_to_f32(bf16(rng.uniform(-vmax, vmax, (2, 384)).astype(np.float32)))
    v[:, [0, 128, 256]] = vmax
    x = v.copy()
    x[:, :128] *= np.float32(8.0)
    x[:, 128:256] *= np.float32(2.0 ** -5)
    q, s = orc.quant_fp8_pergroup_rows(bf16(x), fmt)
    np.testing.assert_array_equal(q, cast(orc, fmt)(v))
    np.testing.assert_array_equal(s, np.tile(np.array([8.0, 2.0 ** -5, 1.0], np.float32), (2, 1)))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pergroup_maximum_at_every_position(orc, fmt):
    # row p holds the destination's largest value at position p of group 0
    # and at position 127 - p of group 1 (every other element smaller), so
    # each group's maximum is met at every index, the first and last
    # included: every scale is exactly 1 and the codes are the element casts
    rng = np.random.default_rng(34)
    vmax = VMAX[fmt]
    v = W.bf16_bits_to_f32(bf16(rng.uniform(-vmax / 2, vmax / 2, (128, 256)).astype(np.float32)))
    p = np.arange(128)
    v[p, p] = -vmax
    v[p, 255 - p] = vmax
    q, s = orc.quant_fp8_pergroup_rows(bf16(v), fmt)
    assert (s == 1.0).all()
    np.testing.assert_array_equal(q, cast(orc, fmt)(v))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pergroup_partial_last_group_and_zero_group(orc, fmt):
    # H = 160: groups [0,128) and [128,160); the first group is all zero
    rng = np.random.default_rng(32)
    vmax = VMAX[fmt]
    x = np.zeros((1, 160), np.float32)
    tail = W.bf16_bits_to_f32(bf16(rng.uniform(-vmax, vmax, 32).astype(np.float32)))
    tail[7] = -vmax
    x[0, 128:] = tail
    q, s = orc.quant_fp8_pergroup_rows(bf16(x), fmt)
    assert s.shape == (1, 2)
    assert s[0].tolist() == [0.0, 1.0]
    assert (q[0, :128] == 0).all()
    np.testing.assert_array_equal(q[0, 128:], cast(orc, fmt)(tail))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pergroup_exact_rational_evaluation(orc, fmt):
    rng = np.random.default_rng(33)
    x = bf16(rng.standard_normal((2, 256)).astype(np.float32) * np.float32(3.0))
    q, s = orc.quant_fp8_pergroup_rows(x, fmt)
    xf = W.bf16_bits_to_f32(x)
    for t in range(2):
        for g in range(2):
            xs = [Fraction(float(v)) for v in xf[t, 128 * g:128 * (g + 1)]]
            ds = fp32_round(Fraction(int(VMAX[fmt])) / max(abs(v) for v in xs))
            prods = np.array([float(fp32_round(v * ds)) for v in xs], np.float32)
            np.testing.assert_array_equal(q[t, 128 * g:128 * (g + 1)], cast(orc, fmt)(prods))
            assert s[t, g] == np.float32(float(fp32_round(1 / ds)))


@pytest.mark.parametrize("quant,fmt", [(0x13, "e4m3"), (0x23, "e5m2")])
def test_dispatch_pergroup_rows(orc, quant, fmt):
    w = W.Workload("t", 30, 416, 12, 3, 4, 4, quant, drop_prob=0.2, seed_index=17)
    inp = W.generate(w)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rx, rs, _ = orc.dispatch(inp.x_bits, lay.token_row, lay.recv_capacity, inp.topk_weights, quant)
    assert rs.shape == (lay.recv_capacity, 4)        # ceil(416 / 128)
    tq, ts = orc.quant_fp8_pergroup_rows(inp.x_bits, fmt)
    for t in range(w.num_tokens):
        for k in range(w.num_topk):
            r = lay.token_row[t, k]
            if r >= 0:
                np.testing.assert_array_equal(rx[r], tq[t])
                np.testing.assert_array_equal(rs[r], ts[t])


# ----------------------------------------------------------------------------- static int8

def test_static_scale_one_integer_rows_saturate(orc):
    rng = np.random.default_rng(34)
    v = rng.integers(-300, 301, size=(4, 64)).astype(np.float32)   # integers up to 256 are exact in bf16
    v[v > 256] = 256
    v[v < -256] = -256
    q = orc.quant_static_int8_rows(bf16(v), np.array([1.0], np.float32))
    np.testing.assert_array_equal(q, np.clip(v, -128, 127).astype(np.int8))


def test_static_ties_and_bounds(orc):
    x = np.zeros((1, 32), np.float32)
    x[0, :10] = [2.5, 3.5, -2.5, -3.5, 0.5, 127.5, -128.5, 126.5, -0.5, 1.5]
    q = orc.quant_static_int8_rows(bf16(x), np.array([1.0], np.float32))
    assert q[0, :10].tolist() == [2, 4, -2, -4, 0, 127, -128, 126, 0, 2]


def test_static_per_channel_scales_are_applied_by_channel(orc):
    H = 64
    rng = np.random.default_rng(35)
    x = rng.integers(-15, 16, size=(3, H)).astype(np.float32)
    j = rng.integers(-3, 4, size=H)
    scales = np.exp2(j).astype(np.float32)                       # x * 2^j exact in fp32
    q = orc.quant_static_int8_rows(bf16(x), scales)
    expect = np.clip(np.round(x * scales), -128, 127)           # numpy round: half to even
    np.testing.assert_array_equal(q, expect.astype(np.int8))
    q_rev = orc.quant_static_int8_rows(bf16(x), scales[::-1].copy())
    assert not np.array_equal(q, q_rev)


def test_dispatch_static_rows(orc):
    w = W.Workload("t", 25, 128, 8, 2, 3, 2, 0, drop_prob=0.1, seed_index=18)
    inp = W.generate(w)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    scales = np.full(128, 40.0, np.float32)
    rx, rw = orc.dispatch_static(inp.x_bits, lay.token_row, lay.recv_capacity, scales,
                                 inp.topk_weights, with_weights=True)
    tq = orc.quant_static_int8_rows(inp.x_bits, scales)
    assert (np.abs(tq.astype(int)) == 128).any() or (tq == 127).any()   # saturation exercised
    for t in range(w.num_tokens):
        for k in range(w.num_topk):
            r = lay.token_row[t, k]
            if r >= 0:
                np.testing.assert_array_equal(rx[r], tq[t])
                assert rw[r] == inp.topk_weights[t, k]


@pytest.mark.parametrize("n,code", [(1, 0), (128, 0), (64, -1), (0, -1), (129, -1)])
def test_static_rules(orc, n, code):
    assert orc.check_static_args(8, 128, 2, 100, n) == code


@pytest.mark.parametrize("q,code", [(0x13, 0), (0x23, 0), (0x03, -1), (0x33, -1)])
def test_pergroup_mode_rules(orc, q, code):
    assert orc.check_rows_args(16, 1024, 4, 1000, q) == code


# ----------------------------------------------------------------------------- static int8, (E, H) scales

def _routing(T, K, E, seed, drop=0.0):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    if drop > 0:
        idx[rng.random((T, K)) < drop] = -1
    return idx


def test_static_expert_uniform_rows_reduce_to_the_shared_shapes(orc):
    """Every expert holding the same scale row is the (H,) shape, and every
    expert holding one constant is the (1,) shape (both pinned above)."""
    w = W.Workload("t", 40, 256, 16, 4, 4, 3, 0, drop_prob=0.15, x_sigma=20.0, seed_index=19)
    inp = W.generate(w)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rng = np.random.default_rng(36)
    per_channel = rng.uniform(0.25, 4.0, size=256).astype(np.float32)
    for shared in (per_channel, np.array([3.0], np.float32)):
        table = np.broadcast_to(shared, (w.num_experts, 256)).astype(np.float32)
        ex, ew = orc.dispatch_static_expert(inp.x_bits, inp.topk_idx, lay.token_row, lay.recv_capacity,
                                            table, inp.topk_weights, with_weights=True)
        sx, sw = orc.dispatch_static(inp.x_bits, lay.token_row, lay.recv_capacity, shared,
                                     inp.topk_weights, with_weights=True)
        np.testing.assert_array_equal(ex, sx)
        np.testing.assert_array_equal(ew, sw)


def test_static_expert_each_copy_uses_its_experts_row(orc):
    """Integer-valued x and power-of-two scales 2^j[e, h]: each product is
    exact, so the code is the product rounded half to even and saturated
    (closed form).  Each copy must follow the scale row of the expert it is
    sent to, so copies of one token differ across experts."""
    T, H, K, E = 48, 64, 4, 8
    rng = np.random.default_rng(37)
    x = rng.integers(-40, 41, size=(T, H)).astype(np.float32)
    x[:, :4] = [0.5, -0.5, 1.5, -2.5]                             # half-way ties after scale 1
    j = rng.integers(-3, 4, size=(E, H))
    j[:, :4] = 0
    scales = np.exp2(j).astype(np.float32)
    idx = _routing(T, K, E, 38, drop=0.1)
    lay = orc.layout(idx, E, 2, 2)
    rx, _ = orc.dispatch_static_expert(bf16(x), idx, lay.token_row, lay.recv_capacity, scales)
    differ = 0
    for t in range(T):
        rows = []
        for k in range(K):
            r = lay.token_row[t, k]
            if r < 0:
                continue
            e = idx[t, k]
            expect = np.clip(np.round(x[t].astype(np.float64) * np.exp2(j[e])), -128, 127)
            np.testing.assert_array_equal(rx[r], expect.astype(np.int8), err_msg=f"t={t} k={k} e={e}")
            rows.append(rx[r])
        differ += sum(not np.array_equal(a, b) for a in rows for b in rows) > 0
    assert differ > T // 2
    assert (rx[:, :4] == [0, 0, 2, -2]).all(axis=1)[lay.recv_src >= 0].all()
    assert (np.abs(rx.astype(int)) >= 127).any()                  # saturation exercised


def test_static_expert_rows_not_named_stay_untouched(orc):
    T, H, K, E = 20, 32, 3, 6
    idx = _routing(T, K, E, 39, drop=0.3)
    lay = orc.layout(idx, E, 3, 4)
    x = bf16(np.random.default_rng(40).normal(size=(T, H)).astype(np.float32))
    scales = np.full((E, H), 50.0, np.float32)
    init = np.full((lay.recv_capacity, H), 77, np.int8)
    rx, _ = orc.dispatch_static_expert(x, idx, lay.token_row, lay.recv_capacity, scales, recv_x=init.copy())
    unused = lay.recv_src < 0
    assert unused.any()
    np.testing.assert_array_equal(rx[unused], init[unused])


@pytest.mark.parametrize("E,code", [(1, 0), (512, 0), (0, -1), (513, -1)])
def test_static_expert_rules(orc, E, code):
    assert orc.check_static_expert_args(8, 128, 2, E, 100) == code
    assert orc.check_static_expert_args(8, 100, 2, 4, 100) == -1     # H not a multiple of 32
