"""bench.py's host-side parts on the CPU: the one-GPU refusal, the
algorithmic byte counts, the counter-file key and the CPU baseline leg."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from combine_moe_get_dispatch_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_algorithmic_bytes():
    # x read once + each valid row written and read once + out written + index traffic
    T, H, K, R, E = 4096, 7168, 8, 8, 256
    V = T * K
    sb = bench.stage_bytes(T, H, K, R, E, V, V, 0)
    assert sb["dispatch"] == 2 * T * H + 4 * T * K + 2 * V * H == 528_613_376
    assert sb["combine"] == 2 * V * H + 8 * T * K + 2 * T * H == 528_744_448
    assert sum(sb.values()) == 528_613_376 + 528_744_448 + sb["layout"]
    # the fused epilogue adds shared + residual reads, the normalised row and gamma
    sf = bench.stage_bytes(T, H, K, R, E, V, V, 0, epilogue=True)
    assert sf["combine"] - sb["combine"] == 3 * 2 * T * H + 2 * H


def test_counter_key_ignores_comments_and_layout():
    a = "int f(int x) { return x + 1; } // one\n"
    b = "/* header */\nint  f(int x)\n{\n    return x + 1;   // other comment\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("+ 1", "+ 2"))
    for stage in ("dispatch", "combine", "layout"):
        t = bench.counter_traffic("bf16_4096x7168_e256_top8", stage)
        assert t is None or t > 0


def test_cpu_baseline_leg_reports_both_thread_counts():
    w = W.WORKLOADS[0]
    inp = W.generate(w)
    res = bench.cpu_baseline(inp, w, w.quant_mode, 0.2,
                             lambda v, c: bench.stage_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_ranks,
                                                            w.num_experts, v, c, w.quant_mode))
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["value"] > 0
    assert res["cores"] >= 1 and res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0


def test_static_per_expert_bytes_count_ids_and_the_scale_table():
    T, H, K, R, E = 8192, 7168, 8, 16, 256
    V = T * K
    base = bench.stage_bytes(T, H, K, R, E, V, V, 0, static=True)
    per_expert = bench.stage_bytes(T, H, K, R, E, V, V, 0, static=True, static_per_expert=True)
    assert per_expert["dispatch"] - base["dispatch"] == 8 * T * K + 4 * E * H
    assert per_expert["combine"] == base["combine"] and per_expert["layout"] == base["layout"]
