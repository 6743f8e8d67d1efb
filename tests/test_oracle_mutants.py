"""The oracle's pins catch plausible mistakes.

Each mutant below is the oracle's C source with one plausible mistake planted
(an off-by-one, a wrong bias, sign or constant, a dropped term, a transposed
index, a wrong rounding or rank map), compiled into a library of its own.
The pin tests (tests/test_oracle_*.py: brute force, hand-worked example,
invariants, closed forms, exhaustive encoder checks, library casts) then run
against that library in a subprocess, the files of the mutant's own area
first, and must fail with an ordinary test failure.  The unmutated source,
built and run the same way, must pass.  Every mutant keeps all memory
accesses in bounds, so a failure is a pin catching it, not a crash.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

LAYOUT = ["tests/test_oracle_layout.py", "tests/test_oracle_rules.py"]
CODECS = ["tests/test_oracle_quant.py", "tests/test_oracle_fp8.py", "tests/test_oracle_group_static.py",
          "tests/test_oracle_mx_exhaustive.py", "tests/test_oracle_nonfinite.py"]
COMBINE = ["tests/test_oracle_combine.py", "tests/test_oracle_combine_fused.py"]
ALL = LAYOUT + CODECS + COMBINE

# (name, area files, text in the source (must occur exactly once), replacement)
MUTANTS = [
    # layout
    ("dropped id counted as an error", LAYOUT,
     "if (e < -1 || e >= E) {", "if (e < 0 || e >= E) {"),
    ("rank map e % R instead of e / L", LAYOUT,
     "itr[(int64_t)t * R + e / L] = 1;", "itr[(int64_t)t * R + e % R] = 1;"),
    ("tokens per rank counts entries", LAYOUT,
     "itr[(int64_t)t * R + e / L] = 1;", "itr[(int64_t)t * R + e / L] += 1;"),
    ("alignment dropped", LAYOUT,
     "nrtpe[e] = ((ntpe[e] + a - 1) / a) * a;", "nrtpe[e] = ntpe[e];"),
    ("offsets from unaligned counts", LAYOUT,
     "off[e + 1] = off[e] + nrtpe[e];", "off[e + 1] = off[e] + ntpe[e];"),
    ("rows in descending entry order", LAYOUT,
     "for (int64_t i = 0; i < M; ++i) {\n        int e = eid[i];\n        if (e < 0) {",
     "for (int64_t i = M - 1; i >= 0; --i) {\n        int e = eid[i];\n        if (e < 0) {"),
    ("recv_src holds the token, not the entry", LAYOUT,
     "recv_src[row] = (int32_t)i;", "recv_src[row] = (int32_t)(i / K);"),
    ("padding rows not marked", LAYOUT,
     "for (int64_t row = 0; row < cap; ++row)\n        recv_src[row] = -1;",
     "for (int64_t row = 0; row < cap; ++row)\n        recv_src[row] = 0;"),
    # element codecs
    ("e4m3 exponent bias 8", CODECS,
     "(uint8_t)(sign | (uint8_t)(((exponent + 7) << 3) | (int)m))",
     "(uint8_t)(sign | (uint8_t)(((exponent + 8) << 3) | (int)m))"),
    ("e4m3 subnormals truncated", CODECS,
     "double q = nearbyint(a * 512.0);", "double q = floor(a * 512.0);"),
    ("e4m3 mantissa truncated", CODECS,
     "double m = nearbyint((2.0 * f - 1.0) * 8.0);", "double m = floor((2.0 * f - 1.0) * 8.0);"),
    ("e4m3 mantissa carry lost", CODECS,
     "if (m == 8.0) {", "if (m > 8.0) {"),
    ("e4m3 negative zero loses its sign", CODECS,
     "uint8_t sign = signbit(v) ? 0x80 : 0x00;\n    double a = fabs(v);\n    if (a > 448.0)",
     "uint8_t sign = v < 0 ? 0x80 : 0x00;\n    double a = fabs(v);\n    if (a > 448.0)"),
    ("e5m2 exponent bias 16", CODECS,
     "(uint8_t)(sign | (uint8_t)(((exponent + 15) << 2) | (int)m))",
     "(uint8_t)(sign | (uint8_t)(((exponent + 16) << 2) | (int)m))"),
    ("e5m2 saturates above the largest finite value", CODECS,
     "if (a > 57344.0)\n        a = 57344.0;", "if (a > 61440.0)\n        a = 61440.0;"),
    ("e4m3 emax 7", CODECS,
     "return fmt == FMT_E5M2 ? 15 : 8;", "return fmt == FMT_E5M2 ? 15 : 7;"),
    ("int8 dstTypeMax 128", CODECS,
     "const float dstTypeMax = 127.0f;", "const float dstTypeMax = 128.0f;"),
    ("int8 row maximum skips the last element", CODECS,
     "for (int h = 0; h < H; ++h) {\n        float xFp32 = bf16_to_f32(x[h]);\n        float ab = fabsf(xFp32);",
     "for (int h = 0; h < H - 1; ++h) {\n        float xFp32 = bf16_to_f32(x[h]);\n        float ab = fabsf(xFp32);"),
    ("MX block maximum skips the last element", CODECS,
     "for (int j = 0; j < 32; ++j) {\n            double ab", "for (int j = 0; j < 31; ++j) {\n            double ab"),
    ("per-token FP8 maximum skips the last element", CODECS,
     "for (int h = 0; h < H; ++h) {\n        float ab = fabsf(bf16_to_f32(x[h]));",
     "for (int h = 0; h < H - 1; ++h) {\n        float ab = fabsf(bf16_to_f32(x[h]));"),
    ("int8 codes truncated", CODECS,
     "float q = rintf(prod);", "float q = truncf(prod);"),
    ("int8 scale as max / 127", CODECS,
     "    *scale_out = 1.0f / dynamicScales;\n}\n\n/* [CANN] Formula Case 5",
     "    *scale_out = maxabs / 127.0f;\n}\n\n/* [CANN] Formula Case 5"),
    ("MX block maximum of x, not |x|", CODECS,
     "double ab = fabs((double)bf16_to_f32(xb[j]));", "double ab = (double)bf16_to_f32(xb[j]);"),
    ("MX shared exponent clamped at -126", CODECS,
     "if (sharedExp < -127)\n                sharedExp = -127;",
     "if (sharedExp < -126)\n                sharedExp = -126;"),
    ("MX scale byte stores the negated exponent", CODECS,
     "scales_out[blk] = (uint8_t)(sharedExp + 127);", "scales_out[blk] = (uint8_t)(127 - sharedExp);"),
    ("per-token FP8 e4m3 maximum 240", CODECS,
     "return fmt == FMT_E5M2 ? 57344.0 : 448.0;", "return fmt == FMT_E5M2 ? 57344.0 : 240.0;"),
    ("per-group maximum skips the group's last element", CODECS,
     "for (int h = g0; h < g0 + n; ++h) {\n            float ab",
     "for (int h = g0; h < g0 + n - 1; ++h) {\n            float ab"),
    ("static int8 saturates at -127", CODECS,
     "if (r < -128.0f)\n            r = -128.0f;", "if (r < -127.0f)\n            r = -127.0f;"),
    ("e4m3 NaN encoded as the largest finite value", CODECS,
     "    if (isnan(v))\n        return 0x7F;\n    uint8_t sign = signbit(v) ? 0x80 : 0x00;\n    double a = fabs(v);\n    if (a > 448.0)",
     "    if (isnan(v))\n        return 0x7E;\n    uint8_t sign = signbit(v) ? 0x80 : 0x00;\n    double a = fabs(v);\n    if (a > 448.0)"),
    ("MX block with an infinite maximum stores byte 254", CODECS,
     "            scales_out[blk] = 0xFF;", "            scales_out[blk] = 0xFE;"),
    ("per-token int8 NaN code -128", CODECS,
     "quantOut[h] = isnan(q) ? 0 : (int8_t)q;", "quantOut[h] = isnan(q) ? -128 : (int8_t)q;"),
    ("per-expert static scales taken by k, not by expert", CODECS,
     "quant_static_int8_row(x + (int64_t)t * H, H, scales + e * H, H,",
     "quant_static_int8_row(x + (int64_t)t * H, H, scales + (int64_t)k * H, H,"),
    ("per-expert static scales of the token's first expert", CODECS,
     "quant_static_int8_row(x + (int64_t)t * H, H, scales + e * H, H,",
     "quant_static_int8_row(x + (int64_t)t * H, H, scales + (topk_idx[(int64_t)t * K] >= 0 && topk_idx[(int64_t)t * K] < E ? topk_idx[(int64_t)t * K] : e) * H, H,"),
    ("static per-channel scales reversed", CODECS,
     "scales[num_scales == 1 ? 0 : h]", "scales[num_scales == 1 ? 0 : H - 1 - h]"),
    ("FP8 destination formats swapped", CODECS,
     "const int fmt = (quant_mode >> 4) == 2 ? FMT_E5M2 : FMT_E4M3FN;",
     "const int fmt = (quant_mode >> 4) == 1 ? FMT_E5M2 : FMT_E4M3FN;"),
    # argument rules
    ("top-k limit 17 in the layout rules", LAYOUT,
     "if (T < 0 || K < 1 || K > 16 || E < 1 || E > 512 || R < 1 || R > E || E % R != 0 ||",
     "if (T < 0 || K < 1 || K > 17 || E < 1 || E > 512 || R < 1 || R > E || E % R != 0 ||"),
    ("hidden sizes in multiples of 16", LAYOUT,
     "H % 32 != 0 || cap < 0 ||", "H % 16 != 0 || cap < 0 ||"),
    # combine
    ("combine product rounded to fp32", COMBINE,
     "o[h] += w * (double)bf16_to_f32(yr[h]);", "o[h] += (double)((float)w * bf16_to_f32(yr[h]));"),
    ("RMS mean over H - 1 elements", COMBINE,
     "const double rms = sqrt(ss / H + eps);", "const double rms = sqrt(ss / (H - 1) + eps);"),
    ("combine weight index transposed", COMBINE,
     "double w = topk_weights ? (double)topk_weights[(int64_t)t * K + k] : 1.0;",
     "double w = topk_weights ? (double)topk_weights[(int64_t)k * T + t] : 1.0;"),
    ("combine without weights sums nothing", COMBINE,
     "double w = topk_weights ? (double)topk_weights[(int64_t)t * K + k] : 1.0;",
     "double w = topk_weights ? (double)topk_weights[(int64_t)t * K + k] : 0.0;"),
    ("combine weight dropped", COMBINE,
     "o[h] += w * (double)bf16_to_f32(yr[h]);", "o[h] += (double)bf16_to_f32(yr[h]);"),
    ("residual add dropped", COMBINE,
     "if (residual)\n                o[h] += (double)bf16_to_f32(residual[(int64_t)t * H + h]);",
     "if (0)\n                o[h] += (double)bf16_to_f32(residual[(int64_t)t * H + h]);"),
    ("RMS eps outside the square root", COMBINE,
     "const double rms = sqrt(ss / H + eps);", "const double rms = sqrt(ss / H) + eps;"),
    ("RMS norm gamma dropped", COMBINE,
     "norm[(int64_t)t * H + h] = o[h] / rms * (double)bf16_to_f32(gamma[h]);",
     "norm[(int64_t)t * H + h] = o[h] / rms;"),
]


def _build(text: str, out: str) -> None:
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-x", "c", "-", "-o", out, "-lm"], input=text, text=True,
                   check=True, capture_output=True)


def _run_pins(lib_path: str, files):
    env = dict(os.environ, MOE_ORACLE_LIB_OVERRIDE=lib_path, OMP_NUM_THREADS="2")
    order = list(dict.fromkeys(files + ALL))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *order], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_mutants_are_unique_substitutions():
    src = open(SRC).read()
    for name, _, old, new in MUTANTS:
        assert src.count(old) == 1, name
        assert old != new, name


@pytest.mark.slow
def test_pins_catch_every_mutant(tmp_path):
    src = open(SRC).read()
    jobs = [("unmutated", ALL, src)]
    for name, files, old, new in MUTANTS:
        jobs.append((name, files, src.replace(old, new)))
    paths = []
    for i, (name, files, text) in enumerate(jobs):
        p = str(tmp_path / f"mutant_{i}.so")
        _build(text, p)
        paths.append(p)

    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda j: _run_pins(paths[j], jobs[j][1]), range(len(jobs))))

    rc0, out0 = results[0]
    assert rc0 == 0, f"the unmutated oracle fails its pins:\n{out0}"
    survivors = [jobs[i][0] for i in range(1, len(jobs)) if results[i][0] == 0]
    crashed = [(jobs[i][0], results[i][0]) for i in range(1, len(jobs)) if results[i][0] not in (0, 1)]
    assert not survivors, f"mutants no pin catches: {survivors}"
    assert not crashed, f"mutants that crashed instead of failing a pin: {crashed}"
