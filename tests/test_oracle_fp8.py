"""Pins for the oracle's 8-bit float destinations beyond MXFP8 e4m3 and for the
pass-through of pre-quantised rows.

e5m2 cast: every finite code round-trips through the format definition;
  every finite bf16 value and random fp32 values against torch's
  float8_e5m2 cast after clamping to +-57344; saturation.
MXFP8 e5m2 (CANN aclnnMoeDistributeDispatchV2, Formula Case 5, emax 15):
  hand-worked block, block exponent against frexp, block maximum lands in the
  top binade, reconstruction bound.
Per-token FP8 (Formula Case 3 with dstTypeMax = 448 or 57344): rows whose
  scale is exactly 1 or a power of two give the element casts, wherever in
  the row the maximum lies; the fp32
  formula re-evaluated in exact rationals; invariants.
Pre-quantised rows: copied byte for byte to the layout rows.
"""
import numpy as np
import pytest

from combine_moe_get_dispatch_amd import workloads as W
from test_oracle_quant import bf16, e4m3fn_value, fp32_round, row32
from fractions import Fraction


def e5m2_value(code: int) -> float:
    """Value of a finite e5m2 code from the format definition: sign, 5-bit
    exponent with bias 15, 2-bit mantissa; exponent field 0 is subnormal
    (m * 2^-16); field 31 is infinity / NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    assert e != 31
    return s * (m * 2.0 ** -16 if e == 0 else (1 + m / 4) * 2.0 ** (e - 15))


FINITE_E5M2 = [c for c in range(256) if ((c >> 2) & 0x1F) != 31]


def test_e5m2_every_finite_code_round_trips(orc):
    vals = np.array([e5m2_value(c) for c in FINITE_E5M2], np.float32)
    np.testing.assert_array_equal(orc.cast_to_fp8_e5m2(vals), np.array(FINITE_E5M2, np.uint8))
    assert e5m2_value(0x7B) == 57344.0


def _torch_e5m2(v):
    import torch
    return torch.from_numpy(np.clip(v, -57344.0, 57344.0)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_all_bf16_values_vs_torch(orc):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    v = W.bf16_bits_to_f32(b)
    np.testing.assert_array_equal(orc.cast_to_fp8_e5m2(v), _torch_e5m2(v))


def test_e5m2_random_fp32_vs_torch(orc):
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-20, 17, 1 << 20))).astype(np.float32)
    np.testing.assert_array_equal(orc.cast_to_fp8_e5m2(v), _torch_e5m2(v))


def test_e5m2_saturates(orc):
    got = orc.cast_to_fp8_e5m2(np.array([57344, 61439, 61440, 1e9, np.inf, -7e4], np.float32))
    assert got.tolist() == [0x7B] * 5 + [0xFB]


# ----------------------------------------------------------------------------- MX e5m2

def test_mx_e5m2_hand_worked_block(orc):
    # block max 3: floor(log2 3) = 1, sharedExp = 1 - emax(15) = -14, byte 113.
    # x / 2^-14: 3 -> 49152 = 1.5*2^15 -> (30<<2)|2 = 0x7A; 1 -> 2^14 -> 29<<2 = 0x74;
    # -0.5 -> -(2^13) -> 0x80 | (28<<2) = 0xF0; 2^-12 -> 4 = 2^2 -> 17<<2 = 0x44.
    q, s = orc.quant_mx_e5m2_rows(row32([3.0, 1.0, -0.5, 2.0 ** -12]))
    assert s[0].tolist() == [113]
    assert q[0, :4].tolist() == [0x7A, 0x74, 0xF0, 0x44]
    assert (q[0, 4:] == 0).all()


def test_mx_e5m2_invariants(orc):
    inp = W.generate(W.WORKLOADS[3], num_tokens=256)
    q, s = orc.quant_mx_e5m2_rows(inp.x_bits)
    T, H = q.shape
    x = W.bf16_bits_to_f32(inp.x_bits).astype(np.float64).reshape(T, H // 32, 32)
    m = np.abs(x).max(axis=2)
    _, e = np.frexp(m)
    se = np.where(m > 0, np.maximum(e - 1 - 15, -127), -127)
    np.testing.assert_array_equal(s.astype(np.int64), se + 127)
    amax = np.argmax(np.abs(x), axis=2)
    top = np.take_along_axis(q.reshape(T, H // 32, 32), amax[..., None], axis=2)[..., 0]
    assert (((top & 0x7F) >> 2) == 30).all()
    lut = np.array([e5m2_value(c) if c in FINITE_E5M2 else np.nan for c in range(256)])
    v = x / np.exp2(se)[..., None]
    dec = lut[q].reshape(v.shape)
    ebin = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    sat = np.abs(v) > 57344
    err = np.abs(v - dec)
    assert (err[~sat] <= np.exp2(ebin - 3)[~sat]).all()
    assert (err[sat] <= 8192).all()


# ----------------------------------------------------------------------------- per-token FP8

@pytest.mark.parametrize("fmt,vmax,value", [("e4m3", 448.0, e4m3fn_value), ("e5m2", 57344.0, e5m2_value)])
def test_pertoken_fp8_scale_one_rows(orc, fmt, vmax, value):
    # max |x| = dstTypeMax: dynamicScales = 1 exactly, so codes are the element casts
    codes = [c for c in range(256) if (fmt == "e4m3" and (c & 0x7F) != 0x7F) or
             (fmt == "e5m2" and c in FINITE_E5M2)]
    vals = np.array([value(c) for c in codes], np.float32)
    H = (len(vals) + 31) // 32 * 32 + 32
    row = np.zeros(H, np.float32)
    row[:len(vals)] = vals
    row[-1] = vmax
    q, s = orc.quant_fp8_pertoken_rows(bf16(row[None, :]), fmt)
    assert s[0] == 1.0
    assert q[0, :len(codes)].tolist() == codes
    assert q[0, -1] == (0x7E if fmt == "e4m3" else 0x7B)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("j", [-40, -3, 2, 30])
def test_pertoken_fp8_power_of_two_rows(orc, fmt, j):
    # x = v * 2^j with max |v| = dstTypeMax: dynamicScales = 2^-j exactly, codes = cast(v)
    vmax = 448.0 if fmt == "e4m3" else 57344.0
    rng = np.random.default_rng(abs(j) + 7)
    v = W.bf16_bits_to_f32(bf16(rng.uniform(-vmax, vmax, (3, 64)).astype(np.float32)))
    v[:, 5] = vmax
    q, s = orc.quant_fp8_pertoken_rows(bf16(v * np.float32(2.0 ** j)), fmt)
    cast = orc.cast_to_fp8_e4m3fn if fmt == "e4m3" else orc.cast_to_fp8_e5m2
    np.testing.assert_array_equal(q, cast(v))
    np.testing.assert_array_equal(s, np.full(3, 2.0 ** j, np.float32))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pertoken_fp8_exact_rational_evaluation(orc, fmt):
    """dynamicScales and the product rounded to fp32 in exact rationals, then
    the element cast (itself pinned against torch)."""
    vmax = 448 if fmt == "e4m3" else 57344
    rng = np.random.default_rng(21)
    x = bf16(rng.standard_normal((4, 64)).astype(np.float32) * np.float32(5.0))
    q, s = orc.quant_fp8_pertoken_rows(x, fmt)
    xf = W.bf16_bits_to_f32(x)
    cast = orc.cast_to_fp8_e4m3fn if fmt == "e4m3" else orc.cast_to_fp8_e5m2
    for t in range(4):
        xs = [Fraction(float(v)) for v in xf[t]]
        ds = fp32_round(Fraction(vmax) / max(abs(v) for v in xs))
        prods = np.array([float(fp32_round(v * ds)) for v in xs], np.float32)
        np.testing.assert_array_equal(q[t], cast(prods))
        assert s[t] == np.float32(float(fp32_round(1 / ds)))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pertoken_fp8_invariants_and_degenerate_rows(orc, fmt):
    inp = W.generate(W.WORKLOADS[2], num_tokens=128)
    q, s = orc.quant_fp8_pertoken_rows(inp.x_bits, fmt)
    top = 0x7E if fmt == "e4m3" else 0x7B
    assert ((q & 0x7F).max(axis=1) == top).all()
    value = e4m3fn_value if fmt == "e4m3" else e5m2_value
    lut = np.array([value(c) if ((fmt == "e4m3" and (c & 0x7F) != 0x7F) or
                                 (fmt == "e5m2" and c in FINITE_E5M2)) else np.nan for c in range(256)])
    x = W.bf16_bits_to_f32(inp.x_bits).astype(np.float64)
    dec = lut[q] * s[:, None].astype(np.float64)
    rel_ulp = 2.0 ** -3 if fmt == "e4m3" else 2.0 ** -2
    sub = (2.0 ** -6 if fmt == "e4m3" else 2.0 ** -14) * s[:, None]
    assert (np.abs(x - dec) <= (0.5 * rel_ulp * np.abs(x) + sub) * (1 + 2.0 ** -20)).all()
    z = np.zeros((2, 64), np.float32)
    z[1, 3] = 2.0 ** -126
    qz, sz = orc.quant_fp8_pertoken_rows(bf16(z), fmt)
    assert (qz == 0).all() and sz.tolist() == [0.0, 0.0]


@pytest.mark.parametrize("quant", [0x12, 0x22, 0x24])
def test_dispatch_new_modes_are_per_token_results(orc, quant):
    w = W.Workload("t", 40, 96, 12, 3, 4, 4, quant, drop_prob=0.2, seed_index=13)
    inp = W.generate(w)
    lay = orc.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rx, rs, _ = orc.dispatch(inp.x_bits, lay.token_row, lay.recv_capacity, inp.topk_weights, quant)
    if quant == 0x24:
        tq, ts = orc.quant_mx_e5m2_rows(inp.x_bits)
    else:
        tq, ts = orc.quant_fp8_pertoken_rows(inp.x_bits, "e4m3" if quant == 0x12 else "e5m2")
    for t in range(w.num_tokens):
        for k in range(w.num_topk):
            r = lay.token_row[t, k]
            if r >= 0:
                np.testing.assert_array_equal(rx[r], tq[t])
                np.testing.assert_array_equal(rs[r], ts[t])


# ----------------------------------------------------------------------------- pre-quantised rows

@pytest.mark.parametrize("row_bytes,scale_bytes", [(3584, 224), (7168, 224), (16, 0), (64, 3)])
def test_dispatch_prequantized_copies_rows(orc, row_bytes, scale_bytes):
    rng = np.random.default_rng(row_bytes + scale_bytes)
    T, K, E = 30, 3, 8
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    lay = orc.layout(idx, E, 2, 4)
    cap = lay.recv_capacity
    data = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
    sc = rng.integers(0, 256, size=(T, scale_bytes), dtype=np.uint8) if scale_bytes else None
    rd0 = np.full((cap, row_bytes), 0xA5, np.uint8)
    rs0 = np.full((cap, scale_bytes), 0x5A, np.uint8) if scale_bytes else None
    rd, rs, _ = orc.dispatch_prequantized(data, sc, lay.token_row, cap, recv_data=rd0.copy(),
                                          recv_scales=None if rs0 is None else rs0.copy())
    used = lay.recv_src >= 0
    src_t = lay.recv_src[used] // K
    np.testing.assert_array_equal(rd[used], data[src_t])
    np.testing.assert_array_equal(rd[~used], rd0[~used])
    if scale_bytes:
        np.testing.assert_array_equal(rs[used], sc[src_t])
        np.testing.assert_array_equal(rs[~used], rs0[~used])


@pytest.mark.parametrize("args,code", [
    ((4, 16, 1, 2, 10), 0), ((4, 8, 1, 2, 10), -1), ((4, 24, 1, 2, 10), -1), ((4, 32784, 0, 2, 10), -1),
    ((4, 32768, 4096, 2, 10), 0), ((4, 32, 4097, 2, 10), -1), ((4, 32, -1, 2, 10), -1),
    ((4, 32, 1, 0, 10), -1), ((4, 32, 1, 17, 10), -1), ((-1, 32, 1, 2, 10), -1), ((0, 32, 1, 2, 0), 0),
])
def test_prequantized_rules(orc, args, code):
    assert orc.check_prequant_args(*args) == code


@pytest.mark.parametrize("q,code", [(0x12, 0), (0x22, 0), (0x24, 0), (0x14, -1), (0x32, -1), (0x02, 0), (0x42, -1)])
def test_new_quant_mode_rules(orc, q, code):
    assert orc.check_rows_args(16, 1024, 4, 1000, q) == code


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_pertoken_fp8_row_maximum_at_every_position(orc, fmt):
    # row p holds +-dstTypeMax at position p and smaller values elsewhere, so
    # the row maximum is met at every index, the last included: every scale is
    # exactly 1 and the codes are the element casts
    vmax = {"e4m3": 448.0, "e5m2": 57344.0}[fmt]
    cast = orc.cast_to_fp8_e4m3fn if fmt == "e4m3" else orc.cast_to_fp8_e5m2
    rng = np.random.default_rng(36)
    H = 64
    v = W.bf16_bits_to_f32(bf16(rng.uniform(-vmax / 2, vmax / 2, (H, H)).astype(np.float32)))
    p = np.arange(H)
    v[p, p] = np.where(p % 2 == 0, vmax, -vmax)
    q, s = orc.quant_fp8_pertoken_rows(bf16(v), fmt)
    np.testing.assert_array_equal(s, np.ones(H, np.float32))
    np.testing.assert_array_equal(q, cast(v))
