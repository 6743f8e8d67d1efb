"""Seeded synthetic workloads for MoE token dispatch / combine.

This module only draws inputs: token activations ``x`` (bf16 bit patterns),
router decisions ``topk_idx`` (int64, ``-1`` = no expert) and router weights
``topk_weights`` (fp32).  It contains none of the dispatch / combine
arithmetic, so both the CPU oracle and the HIP path can be fed from it.

Shapes and laws follow the five workloads the library is measured on (the
token counts, hidden sizes, expert counts, top-k and alignment mirror the
ranges in the sgl-kernel-npu "Normal Mode API" page, Constraints section, and
the expert-parallel shapes of the CANN aclnnMoeDistributeDispatchV2 page,
Constraint 7).  No public dataset is involved: every value is drawn from
numpy's PCG64 generator with a fixed seed per workload (x and the
routing from two independent streams).

Recipe (also listed in the design notes):
  * x ~ N(0, sigma) in fp32, rounded to bf16 with round-half-even;
    the "outlier" law multiplies an i.i.d. Bernoulli(p) element mask by a
    factor before rounding.
  * "uniform" routing: logits ~ N(0,1) of shape [T, E]; topk_idx = the K
    largest logits in descending order (a uniformly random distinct subset);
    topk_weights = softmax of those K logits in fp32.
  * "zipf" routing: expert popularity p_e ~ (pi(e)+1)^-s for a seeded
    permutation pi; K distinct experts per token by Gumbel-top-k over log p
    (sampling without replacement); weights = softmax of K fresh N(0,1)
    logits.
  * "firstk" routing (the degenerate extreme of skew): every token picks
    experts 0..K-1 in order, weights = softmax of K N(0,1) logits.  Each of
    those K experts receives every token, so dispatch writes K streams of
    consecutive rows: the same bytes as uniform routing in address order.
  * "drop" fraction: after routing, each (t, k) entry is set to -1 with that
    probability and its weight to 0.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20261202

QUANT_NONE = 0
QUANT_INT8_PER_TOKEN = 2
QUANT_MXFP8_E4M3 = 4
QUANT_FP8_E4M3_PER_TOKEN = 0x12
QUANT_FP8_E5M2_PER_TOKEN = 0x22
QUANT_MXFP8_E5M2 = 0x24
QUANT_FP8_E4M3_PER_GROUP = 0x13
QUANT_FP8_E5M2_PER_GROUP = 0x23
QUANT_NAMES = {QUANT_FP8_E4M3_PER_GROUP: "FP8 e4m3 per-group(128)",
               QUANT_FP8_E5M2_PER_GROUP: "FP8 e5m2 per-group(128)",QUANT_NONE: "bf16", QUANT_INT8_PER_TOKEN: "int8 per-token",
               QUANT_MXFP8_E4M3: "MXFP8 e4m3", QUANT_FP8_E4M3_PER_TOKEN: "FP8 e4m3 per-token",
               QUANT_FP8_E5M2_PER_TOKEN: "FP8 e5m2 per-token", QUANT_MXFP8_E5M2: "MXFP8 e5m2"}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    num_ranks: int
    num_topk: int
    expert_alignment: int
    quant_mode: int
    routing: str = "uniform"        # "uniform" | "zipf"
    zipf_s: float = 0.0
    drop_prob: float = 0.0
    x_sigma: float = 1.0
    outlier_prob: float = 0.0
    outlier_scale: float = 1.0
    seed_index: int = 0
    prequant: str = ""              # "" | "mxfp8" | "mxfp4": pre-quantised (data, scale) input
    static_scale: float = 0.0       # > 0: static int8 quantisation with this one coefficient
    static_per_expert: bool = False  # with static_scale: one scale row per expert (expert_scales)
    epilogue: str = ""              # "" | "shared_residual_rmsnorm": combine epilogues

    def describe(self) -> str:
        q = QUANT_NAMES[self.quant_mode]
        if self.prequant:
            q = f"pre-quantised {self.prequant.upper()} pass-through"
        if self.static_scale > 0:
            q = f"static int8 (scale {self.static_scale:g})"
        if self.static_per_expert:
            q = f"static int8, one scale row per expert (around {self.static_scale:g})"
        if self.epilogue:
            q += ", combine + shared expert + residual + RMSNorm"
        return (f"{self.num_tokens} tokens x hidden {self.hidden}, "
                f"{self.num_experts} experts / {self.num_ranks} virtual ranks, "
                f"top-{self.num_topk} {self.routing}, alignment {self.expert_alignment}, {q}")


# The five measured workloads.  WORKLOADS[1] is the headline case.
WORKLOADS = [
    Workload("tiny_128x1024_e16_top2", 128, 1024, 16, 4, 2, 1, QUANT_NONE, seed_index=0),
    Workload("bf16_4096x7168_e256_top8", 4096, 7168, 256, 8, 8, 1, QUANT_NONE, seed_index=1),
    Workload("int8_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128,
             QUANT_INT8_PER_TOKEN, routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2),
    Workload("mxfp8_8192x4096_e128_top8_drop", 8192, 4096, 128, 8, 8, 32,
             QUANT_MXFP8_E4M3, drop_prob=0.1, outlier_prob=0.01, outlier_scale=50.0,
             seed_index=3),
    Workload("bf16_32768x7168_e512_top16", 32768, 7168, 512, 64, 16, 128, QUANT_NONE,
             seed_index=4),
]
# Further rows: the other 8-bit destinations the pages allow and the
# pre-quantised tuple input, on the shapes of the measured workloads.
NEXT_WORKLOADS = [
    # a decode-sized batch at the headline's expert shape (one-workgroup layout)
    Workload("bf16_128x7168_e256_top8_decode", 128, 7168, 256, 8, 8, 1, QUANT_NONE, seed_index=1),
    Workload("fp8e4m3_128x7168_e256_top8_decode", 128, 7168, 256, 8, 8, 1,
             QUANT_FP8_E4M3_PER_TOKEN, seed_index=1),
    Workload("fp8e4m3_pertoken_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128,
             QUANT_FP8_E4M3_PER_TOKEN, routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2),
    Workload("fp8e5m2_pertoken_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128,
             QUANT_FP8_E5M2_PER_TOKEN, routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2),
    Workload("mxfp8e5m2_8192x4096_e128_top8_drop", 8192, 4096, 128, 8, 8, 32, QUANT_MXFP8_E5M2,
             drop_prob=0.1, outlier_prob=0.01, outlier_scale=50.0, seed_index=3),
    Workload("bf16_4096x7168_e256_top8_shared_addrmsnorm", 4096, 7168, 256, 8, 8, 1, QUANT_NONE,
             seed_index=1, epilogue="shared_residual_rmsnorm"),
    Workload("fp8e4m3_pergroup_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128,
             QUANT_FP8_E4M3_PER_GROUP, routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2),
    Workload("int8_static_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128, QUANT_NONE,
             routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2, static_scale=127.0 / 12.0),
    Workload("mxfp8_prequant_8192x7168_e256_top8", 8192, 7168, 256, 8, 8, 1, QUANT_NONE,
             seed_index=5, prequant="mxfp8"),
    Workload("mxfp4_prequant_8192x7168_e256_top8", 8192, 7168, 256, 8, 8, 1, QUANT_NONE,
             seed_index=6, prequant="mxfp4"),
    Workload("int8_static_expert_8192x7168_e256_top8_zipf", 8192, 7168, 256, 16, 8, 128, QUANT_NONE,
             routing="zipf", zipf_s=1.1, x_sigma=2.0, seed_index=2, static_scale=127.0 / 12.0,
             static_per_expert=True),
    # the headline's shape and bytes with every token routed to experts 0..7:
    # dispatch's rows are then written in address order (8 streams)
    Workload("bf16_4096x7168_e256_top8_firstk", 4096, 7168, 256, 8, 8, 1, QUANT_NONE,
             routing="firstk", seed_index=1),
]
BY_NAME = {w.name: w for w in WORKLOADS + NEXT_WORKLOADS}


def prequant_row_bytes(w: Workload):
    """(data bytes, scale bytes) per token of a pre-quantised workload."""
    return (w.hidden if w.prequant == "mxfp8" else w.hidden // 2), w.hidden // 32


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-half-even) and return the uint16 bit
    patterns.  Uses torch's CPU cast, the library routine for this rounding."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def _softmax_f32(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=-1, keepdims=True, dtype=np.float32)).astype(np.float32)


def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, largest first."""
    part = np.argpartition(-scores, k - 1, axis=1)[:, :k]
    vals = np.take_along_axis(scores, part, axis=1)
    order = np.argsort(-vals, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def make_x(rng: np.random.Generator, T: int, H: int, sigma: float,
           outlier_prob: float = 0.0, outlier_scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal((T, H), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if outlier_prob > 0.0:
        mask = rng.random((T, H), dtype=np.float32) < outlier_prob
        x[mask] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def make_routing(rng: np.random.Generator, T: int, E: int, K: int, routing: str,
                 zipf_s: float = 0.0, drop_prob: float = 0.0):
    if routing == "uniform":
        logits = rng.standard_normal((T, E), dtype=np.float32)
        idx = _topk_desc(logits, K)
        w = _softmax_f32(np.take_along_axis(logits, idx, axis=1))
    elif routing == "zipf":
        perm = rng.permutation(E)
        logp = -zipf_s * np.log(perm.astype(np.float64) + 1.0)
        g = rng.gumbel(size=(T, E))
        idx = _topk_desc(logp[None, :] + g, K)
        w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    elif routing == "firstk":
        idx = np.broadcast_to(np.arange(K), (T, K))
        w = _softmax_f32(rng.standard_normal((T, K), dtype=np.float32))
    else:
        raise ValueError(f"unknown routing law {routing!r}")
    idx = idx.astype(np.int64)
    w = np.ascontiguousarray(w, dtype=np.float32)
    if drop_prob > 0.0:
        drop = rng.random((T, K)) < drop_prob
        idx[drop] = -1
        w[drop] = 0.0
    return np.ascontiguousarray(idx), w


@dataclasses.dataclass
class Inputs:
    workload: Workload
    x_bits: np.ndarray          # uint16 [T, H] bf16 bit patterns
    topk_idx: np.ndarray        # int64 [T, K]
    topk_weights: np.ndarray    # float32 [T, K]


def _rng(w: Workload, stream: int, seed_offset: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([BASE_SEED, w.seed_index, seed_offset, stream]))


def generate_routing(w: Workload, num_tokens: Optional[int] = None, seed_offset: int = 0):
    """(topk_idx, topk_weights) of workload ``w``; the same draw as ``generate``."""
    T = w.num_tokens if num_tokens is None else num_tokens
    return make_routing(_rng(w, 1, seed_offset), T, w.num_experts, w.num_topk, w.routing,
                        w.zipf_s, w.drop_prob)


def generate(w: Workload, num_tokens: Optional[int] = None, seed_offset: int = 0) -> Inputs:
    """Draw the inputs of workload ``w``.  ``num_tokens`` overrides T (a
    smaller draw is not a prefix of the full one).  x and the routing come
    from independent streams."""
    T = w.num_tokens if num_tokens is None else num_tokens
    x = make_x(_rng(w, 0, seed_offset), T, w.hidden, w.x_sigma, w.outlier_prob, w.outlier_scale)
    idx, wt = generate_routing(w, T, seed_offset)
    return Inputs(w, x, idx, wt)


def generate_prequant(w: Workload, num_tokens: Optional[int] = None):
    """(data uint8 [T, row_bytes], scales uint8 [T, H/32], topk_idx,
    topk_weights) of a pre-quantised workload.  The data bytes are uniform
    (dispatch moves them without reading their values); scale bytes are
    e8m0 exponents 2^-27..2^12 (bytes 100..139)."""
    T = w.num_tokens if num_tokens is None else num_tokens
    rb, sb = prequant_row_bytes(w)
    rng = _rng(w, 0, 0)
    data = rng.integers(0, 256, size=(T, rb), dtype=np.uint8)
    scales = rng.integers(100, 140, size=(T, sb), dtype=np.uint8)
    idx, wt = generate_routing(w, T)
    return data, scales, idx, wt


def expert_scales(w: Workload) -> np.ndarray:
    """fp32 [E, H] static scale rows of a per-expert static workload: the
    workload's coefficient times independent uniform factors in [0.5, 2)."""
    rng = _rng(w, 2, 0)
    u = rng.uniform(0.5, 2.0, size=(w.num_experts, w.hidden)).astype(np.float32)
    return np.ascontiguousarray(u * np.float32(w.static_scale), dtype=np.float32)


def random_bf16_rows(rows: int, hidden: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    """Independent bf16 rows (used as arbitrary expert outputs for combine)."""
    rng = np.random.Generator(np.random.PCG64([BASE_SEED, 99, seed, 2]))
    return make_x(rng, rows, hidden, sigma)
