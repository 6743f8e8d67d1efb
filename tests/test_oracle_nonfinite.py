"""Pins for non-finite inputs.  The pages do not cover NaN or infinity; the
readings (IEEE fp32 arithmetic carried through, each cast given a defined
result) are:
  * Max(Abs(x)) ignores NaN elements (IEEE maxNum, as C's fmaxf);
  * CastToInt8(NaN) = 0; static int8 saturates +-inf to 127 / -128;
  * CastToFp8(NaN) = the NaN code 0x7F (either sign); +-inf saturate like any
    value above the format's largest finite one;
  * a row or group whose maximum is +inf: dynamicScales = dstTypeMax / inf = 0,
    scale 1 / 0 = +inf, finite elements give signed zeros, infinite ones NaN;
  * an MX block whose maximum is +inf: sharedExp = +inf, e8m0 byte 0xFF (the
    format's NaN), elements divided by 2^+inf.
Each pin states the expected codes directly, or relates a row with NaN to the
same row with that element replaced by 0 (which the finite pins cover)."""
import numpy as np
import pytest

PINF, NINF, QNAN, NQNAN, SNAN = 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81


def f32_bits(v):
    return np.frombuffer(np.float32(v).tobytes(), np.uint32)[0]


def row(H, vals, fill=None, seed=0):
    """bf16 bit row: seeded finite values (|x| < 4), then the given (index, bits) pairs."""
    rng = np.random.default_rng(seed)
    from combine_moe_get_dispatch_amd import workloads as W
    r = W.f32_to_bf16_bits(rng.uniform(-4, 4, H).astype(np.float32)) if fill is None else np.full(H, fill, np.uint16)
    for i, b in vals:
        r[i] = b
    return r


@pytest.mark.parametrize("fmt,maxcode", [("e4m3", 0x7E), ("e5m2", 0x7B)])
def test_fp8_casts_of_nan_and_infinity(orc, fmt, maxcode):
    cast = orc.cast_to_fp8_e4m3fn if fmt == "e4m3" else orc.cast_to_fp8_e5m2
    v = np.array([np.nan, -np.nan, np.inf, -np.inf], np.float32)
    v[1] = np.frombuffer(np.uint32(0xFFC00000).tobytes(), np.float32)[0]       # negative quiet NaN
    assert cast(v).tolist() == [0x7F, 0x7F, maxcode, 0x80 | maxcode]


def test_int8_per_token_nan_element_takes_no_part(orc):
    H = 64
    base = row(H, [(5, 0)], seed=1)                       # element 5 = +0
    with_nan = base.copy()
    with_nan[5] = QNAN
    q0, s0 = orc.quant_int8_rows(base[None])
    q1, s1 = orc.quant_int8_rows(with_nan[None])
    assert q1[0, 5] == 0
    np.testing.assert_array_equal(q1, q0)
    assert f32_bits(s1[0]) == f32_bits(s0[0])
    with_nan[7] = NQNAN
    q2, _ = orc.quant_int8_rows(with_nan[None])
    assert q2[0, 7] == 0


def test_int8_per_token_row_with_infinity(orc):
    for inf in (PINF, NINF):
        r = row(64, [(3, inf), (9, QNAN)], seed=2)
        q, s = orc.quant_int8_rows(r[None])
        assert (q == 0).all()
        assert f32_bits(s[0]) == 0x7F800000                 # 1 / (127 / inf) = +inf


def test_int8_per_token_all_nan_row_is_degenerate(orc):
    q, s = orc.quant_int8_rows(np.full((1, 32), QNAN, np.uint16))
    assert (q == 0).all() and f32_bits(s[0]) == 0           # maximum 0: codes 0, scale 0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_per_token_row_with_infinity(orc, fmt):
    r = row(64, [(3, PINF), (4, NINF), (9, QNAN)], seed=3)
    q, s = orc.quant_fp8_pertoken_rows(r[None], fmt)
    x = (r.astype(np.uint32) << 16).view(np.float32)
    finite = np.isfinite(x)
    expect = np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8)   # x * 0 keeps the sign
    np.testing.assert_array_equal(q[0, finite], expect[finite])
    assert q[0, 3] == 0x7F and q[0, 4] == 0x7F and q[0, 9] == 0x7F
    assert f32_bits(s[0]) == 0x7F800000


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_per_token_nan_element_takes_no_part(orc, fmt):
    base = row(96, [(11, 0)], seed=4)
    with_nan = base.copy()
    with_nan[11] = SNAN
    q0, s0 = orc.quant_fp8_pertoken_rows(base[None], fmt)
    q1, s1 = orc.quant_fp8_pertoken_rows(with_nan[None], fmt)
    assert q1[0, 11] == 0x7F
    keep = np.arange(96) != 11
    np.testing.assert_array_equal(q1[0, keep], q0[0, keep])
    assert f32_bits(s1[0]) == f32_bits(s0[0])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_per_group_infinity_stays_in_its_group(orc, fmt):
    base = row(256, [], seed=5)
    r = base.copy()
    r[130] = PINF                                            # second group of 128
    r[10] = QNAN                                             # first group: NaN only
    q, s = orc.quant_fp8_pergroup_rows(r[None], fmt)
    qb, sb = orc.quant_fp8_pergroup_rows(base[None], fmt)
    assert f32_bits(s[0, 1]) == 0x7F800000
    x = (r.astype(np.uint32) << 16).view(np.float32)
    g2 = slice(128, 256)
    expect = np.where(np.signbit(x[g2]), 0x80, 0x00).astype(np.uint8)
    expect[130 - 128] = 0x7F
    np.testing.assert_array_equal(q[0, g2], expect)
    assert q[0, 10] == 0x7F
    keep = np.arange(128) != 10
    base0 = base.copy()
    base0[10] = 0
    qz, sz = orc.quant_fp8_pergroup_rows(base0[None], fmt)
    np.testing.assert_array_equal(q[0, :128][keep], qz[0, :128][keep])
    assert f32_bits(s[0, 0]) == f32_bits(sz[0, 0])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mx_block_with_infinity(orc, fmt):
    quant = orc.quant_mxfp8_rows if fmt == "e4m3" else orc.quant_mx_e5m2_rows
    base = row(128, [], seed=6)
    r = base.copy()
    r[40] = NINF                                            # block 1
    r[41] = QNAN
    r[70] = QNAN                                            # block 2: NaN, finite maximum
    q, s = quant(r[None])
    qb, sb = quant(base[None])
    assert s[0, 1] == 0xFF
    x = (r.astype(np.uint32) << 16).view(np.float32)
    b1 = slice(32, 64)
    expect = np.where(np.signbit(x[b1]), 0x80, 0x00).astype(np.uint8)
    expect[8] = 0x7F
    expect[9] = 0x7F
    np.testing.assert_array_equal(q[0, b1], expect)
    assert q[0, 70] == 0x7F
    base2 = base.copy()
    base2[70] = 0
    q2, s2 = quant(base2[None])
    assert s[0, 2] == s2[0, 2]
    keep = [j for j in range(64, 96) if j != 70]
    np.testing.assert_array_equal(q[0, keep], q2[0, keep])
    for blk in (0, 3):                                      # other blocks as without the specials
        assert s[0, blk] == sb[0, blk]
        np.testing.assert_array_equal(q[0, 32 * blk:32 * blk + 32], qb[0, 32 * blk:32 * blk + 32])


def test_static_int8_nan_and_infinity(orc):
    r = np.zeros(32, np.uint16)
    r[:5] = [QNAN, NQNAN, PINF, NINF, SNAN]
    for scales in (np.array([3.0], np.float32), np.full(32, 0.5, np.float32)):
        q = orc.quant_static_int8_rows(r[None], scales)
        assert q[0, :5].tolist() == [0, 0, 127, -128, 0]
        assert (q[0, 5:] == 0).all()


def test_static_int8_non_finite_scales(orc):
    """Scales are the caller's data and may be non-finite too: x * inf
    saturates by the sign of the product, 0 * inf and anything * NaN is NaN
    (code 0), and a finite product that overflows fp32 saturates as well."""
    from combine_moe_get_dispatch_amd import workloads as W
    x = W.f32_to_bf16_bits(np.array([1.0, -1.0, 0.0, 2.0, -0.0, 3.0, 2.0, -2.0], np.float32))
    s = np.array([np.inf, np.inf, np.inf, np.nan, -np.inf, -np.inf, 3e38, 3e38], np.float32)
    q = orc.quant_static_int8_rows(x[None], s)
    assert q[0].tolist() == [127, -128, 0, 0, 0, -128, 127, -128]
    for one in (np.inf, -np.inf, np.nan):
        q1 = orc.quant_static_int8_rows(x[None], np.array([one], np.float32))
        expect = [0 if (np.isnan(one) or v == 0) else (127 if v * one > 0 else -128)
                  for v in (1.0, -1.0, 0.0, 2.0, -0.0, 3.0, 2.0, -2.0)]
        assert q1[0].tolist() == expect
