"""Benchmark: MoE dispatch + combine on one MI355X.

One step = moe_get_dispatch_layout -> moe_dispatch -> moe_combine on one HIP
stream, over the whole batch (identity experts: the combine input is the
receive buffer itself for bf16, or its bf16 dequantisation -- made once,
outside the timed region -- for int8 / MXFP8).  Inputs are resident in HBM
before timing starts.  W untimed warm-up steps, then exactly K timed steps
bracketed by torch.cuda.synchronize().

Stage durations come from HIP events recorded, inside the timed region, on
the stream the kernels run on: around the dominant kernel (dispatch or
combine, found in one untimed step after the warm-up) on every Nth step, and
around all three stages on every other such step (--event-every; at least 10
samples of the dominant kernel from 10 steps on).  The events are created
with hipEventDisableSystemFence, so a record does not flush caches to system
scope; recording them on a sample of steps, and only the marks needed, keeps
their cost (~1-2 us of GPU time per mark) out of the headline.

Cold-cache legs follow the timed region (--cold-reps): each stage alone,
after 1 GiB of unrelated device traffic (a fill, then separately a read),
reported as `cold_cache` beside the back-to-back figures.

Prints ONE JSON line.  `value` = effective HBM GB/s = algorithmic bytes per
step * K / elapsed; algorithmic bytes count x read once, each valid expanded
row written once and read once, the output written once, and the index
traffic (padding rows are never touched and not counted).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
KERNEL_SOURCES = {
    "dispatch": ["dispatch.hip", "element_codecs.h", "device_common.h", "launch.h"],
    "combine": ["combine.hip", "device_common.h", "launch.h"],
    "layout": ["layout.hip", "device_common.h", "launch.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_4096x7168_e256_top8")
    p.add_argument("--tokens", type=int, default=0,
                   help="draw the workload with this many tokens instead of its own T (0 = its own)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU time budget for the oracle baseline (0 = skip)")
    p.add_argument("--event-every", type=int, default=0,
                   help="record timing events on every Nth timed step (0 = every max(1, steps // 10)th "
                        "step: at least 10 samples of the dominant kernel from 10 steps on; every "
                        "other such step times all three stages)")
    p.add_argument("--cold-reps", type=int, default=10,
                   help="after timing, repetitions of the cold-cache legs: each stage timed alone "
                        "after 1 GiB of device traffic (a fill, or a read) has evicted L2 and the "
                        "memory-side cache (0 = skip)")
    p.add_argument("--graph", action="store_true",
                   help="time replays of one captured HIP graph of the step instead of eager launches "
                        "(stage times then come from an eager pass with events before it)")
    p.add_argument("--one-launch", action="store_true",
                   help="lay out and dispatch with moe_layout_and_dispatch, one launch (bf16 or "
                        "per-token workloads whose batch it takes); the layout stage's time is then "
                        "that launch and the dispatch stage's is empty")
    p.add_argument("--no-check", action="store_true", help="skip the post-run sanity check")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, run 3 torch copies of 256 MiB: a kernel of known traffic "
                        "that hardware byte counters (FETCH_SIZE / WRITE_SIZE) are scaled against")
    return p.parse_args()


PER_TOKEN_MODES = (0x02, 0x12, 0x22)
PER_GROUP_MODES = (0x13, 0x23)


def stage_bytes(T, H, K, R, E, V, cap, quant, prequant_rows=None, static=False, epilogue=False,
                static_per_expert=False):
    """Algorithmic bytes of each stage (see module docstring).  prequant_rows =
    (data bytes, scale bytes) per token for the pre-quantised pass-through;
    static_per_expert adds the ids (int64 [T, K]) and the [E, H] fp32 scale
    table read once."""
    layout = 8 * T * K + 4 * T * R + 4 * R + 8 * E + 4 * (E + 1) + 4 * T * K + 4 * cap + 4
    if prequant_rows is not None:
        rb, sb = prequant_rows
        dispatch = T * (rb + sb) + 4 * T * K + V * (rb + sb)
    elif static_per_expert:
        dispatch = 2 * T * H + 4 * T * K + 8 * T * K + 4 * E * H + V * H
    elif static:
        dispatch = 2 * T * H + 4 * T * K + V * H
    else:
        s_q = 2 if quant == 0 else 1
        if quant == 0:
            sigma = 0
        elif quant in PER_TOKEN_MODES:
            sigma = 4
        elif quant in PER_GROUP_MODES:
            sigma = 4 * ((H + 127) // 128)
        else:
            sigma = H // 32
        dispatch = 2 * T * H + 4 * T * K + V * (H * s_q + sigma)
    combine = 2 * V * H + 8 * T * K + 2 * T * H
    if epilogue:   # shared row + residual row read, normalised row written, gamma read
        combine += 3 * 2 * T * H + 2 * H
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (string literals kept)."""
    import re
    text = re.sub(r'//[^\n]*|/\*.*?\*/', " ", text, flags=re.S)
    return re.sub(r"\s+", "", text)


def kernel_source_sha(stage: str) -> str:
    """First 16 hex digits of sha256 over the code of the kernel's source
    files; edits to comments or layout leave it unchanged."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "combine_moe_get_dispatch_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter
    summary (profiles/<stage>_<workload>_counters.txt), or None when there is
    none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_sha(stage):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_stage_us(workload: str, stage: str):
    """Average kernel time of one call of `stage` over the timed steps, from
    the committed rocprofv3 kernel statistics of this workload
    (profiles/<workload>_kernel_stats.txt), or None when there are none or
    the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get(f"source_sha256_{stage}") != kernel_source_sha(stage):
        return None
    try:
        return float(kv[f"stage_timed_avg_us_{stage}"])
    except (KeyError, ValueError):
        return None


class StageEvents:
    """Timing events on torch's current stream.  Uses HIP events created with
    hipEventDisableSystemFence through the HIP runtime torch already loaded;
    falls back to torch.cuda.Event if that is not possible."""

    def __init__(self, torch):
        self.torch = torch
        self.hip = None
        self._created = []  # HIP events to destroy in close()
        try:
            path = [l.split()[-1] for l in open("/proc/self/maps").read().split("\n")
                    if "libamdhip64" in l][0]
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0:
                self.hip = hip
                self.kind = "hipEventDisableSystemFence"
                self._created.append(e)
        except (IndexError, OSError, AttributeError):
            self.hip = None
        if self.hip is None:
            self.kind = "torch.cuda.Event"

    def new(self):
        if self.hip is None:
            return self.torch.cuda.Event(enable_timing=True)
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self._created.append(e)
        return e

    def close(self):
        """Destroy the HIP events this timer created (after their last use)."""
        if self.hip is not None:
            for e in self._created:
                self.hip.hipEventDestroy(e)
        self._created = []

    def record(self, ev):
        if self.hip is None:
            ev.record()
        else:
            s = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
            rc = self.hip.hipEventRecord(ev, s)
            if rc != 0:
                raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_us(self, a, b):
        if self.hip is None:
            return a.elapsed_time(b) * 1e3
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value * 1e3


def cpu_baseline(inp, w, quant, budget_s, bytes_fn, prequant=None):
    """The oracle, as it is, on the same workload, repeated until the time
    budget is used (at least once)."""
    import numpy as np
    import oracle
    E, R, a = w.num_experts, w.num_ranks, w.expert_alignment
    if w.epilogue:
        from combine_moe_get_dispatch_amd import workloads as W
        epi = (W.random_bf16_rows(w.num_tokens, w.hidden, 21), W.random_bf16_rows(w.num_tokens, w.hidden, 22),
               np.full(w.hidden, 0x3F80, np.uint16))
    V = int((inp.topk_idx >= 0).sum())
    if w.static_per_expert:
        from combine_moe_get_dispatch_amd import workloads as W
        expert_scales = W.expert_scales(w)

    def leg(budget):
        reps, total_bytes = 0, 0
        t0 = time.perf_counter()
        while True:
            ol = oracle.layout(inp.topk_idx, E, R, a)
            if prequant is not None:
                oracle.dispatch_prequantized(prequant[0], prequant[1], ol.token_row, ol.recv_capacity)
                y = prequant[2]
            elif w.static_per_expert:
                oracle.dispatch_static_expert(inp.x_bits, inp.topk_idx, ol.token_row, ol.recv_capacity,
                                              expert_scales)
                y = np.zeros((ol.recv_capacity, w.hidden), np.uint16)
            elif w.static_scale > 0:
                oracle.dispatch_static(inp.x_bits, ol.token_row, ol.recv_capacity,
                                       np.array([w.static_scale], np.float32))
                y = np.zeros((ol.recv_capacity, w.hidden), np.uint16)
            else:
                rx, rs, _ = oracle.dispatch(inp.x_bits, ol.token_row, ol.recv_capacity, None, quant)
                y = rx if quant == 0 else np.zeros((ol.recv_capacity, w.hidden), np.uint16)
            if w.epilogue:
                oracle.combine_fused(y, ol.token_row, inp.topk_weights, epi[0], epi[1], epi[2], 1e-6,
                                     with_norm=True)
            else:
                oracle.combine(y, ol.token_row, inp.topk_weights)
            reps += 1
            total_bytes += sum(bytes_fn(V, ol.recv_capacity).values())
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, total_bytes, el

    threads = oracle.num_threads()
    reps, total_bytes, el = leg(budget_s)
    res = {"value": round(total_bytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"full workload ({w.num_tokens} tokens), layout+dispatch+combine, {reps} repetition(s) "
                     f"in {el:.1f} s", "tokens_per_s": round(reps * w.num_tokens / el, 1)}
    # the same oracle on one thread (its layout is sequential in both legs)
    oracle.set_num_threads(1)
    try:
        reps1, bytes1, el1 = leg(budget_s / 2)
    finally:
        oracle.set_num_threads(threads)
    res["single_thread"] = {"value": round(bytes1 / el1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                            "sample": f"{reps1} repetition(s) in {el1:.1f} s"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library runs the path on a single GPU, virtual ranks are expert partitions)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from combine_moe_get_dispatch_amd import build_lib
    if not os.path.exists(build_lib.LIB_PATH):
        build_lib.build(verbose=True)
    import combine_moe_get_dispatch_amd as moe
    from combine_moe_get_dispatch_amd import workloads as W

    w = W.BY_NAME[args.workload]
    if args.tokens > 0:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}@T{args.tokens}", num_tokens=args.tokens)
    T, H, K, E, R, a, quant = (w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                               w.expert_alignment, w.quant_mode)
    dev = torch.device("cuda", 0)
    prequant_rows = W.prequant_row_bytes(w) if w.prequant else None
    if w.prequant:
        data_h, scales_h, idx_h, wt_h = W.generate_prequant(w)
        inp = W.Inputs(w, None, idx_h, wt_h)
    else:
        inp = W.generate(w)
    V = int((inp.topk_idx >= 0).sum())

    idx = torch.from_numpy(inp.topk_idx).to(dev)
    wt = torch.from_numpy(inp.topk_weights).to(dev)
    lay = moe.allocate_layout(T, K, E, R, a, device=dev)
    cap = lay.recv_capacity
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    moe.moe_get_dispatch_layout(idx, E, R, a, out=lay)
    cpu_y = None
    if w.prequant:
        data = torch.from_numpy(data_h).to(dev)
        scales = torch.from_numpy(scales_h).to(dev)
        rd = torch.empty((cap, data.shape[1]), dtype=torch.uint8, device=dev)
        rsc = torch.empty((cap, scales.shape[1]), dtype=torch.uint8, device=dev)
        # expert output stand-in: seeded bf16 rows (combine does not depend on values)
        y_bits = W.random_bf16_rows(cap, H, 5)
        y = torch.from_numpy(y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        cpu_y = (data_h, scales_h, y_bits)

        def run_dispatch():
            moe.moe_dispatch_prequantized(data, scales, lay, None, rd, rsc)
    elif w.static_per_expert:
        x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        rx = torch.empty((cap, H), dtype=torch.int8, device=dev)
        escales = torch.from_numpy(W.expert_scales(w)).to(dev)

        def run_dispatch():
            moe.moe_dispatch_static_per_expert(x, lay, idx, escales, None, recv_x=rx)

        run_dispatch()
        # identity expert: each row divided by its expert's scale row
        row_expert = torch.repeat_interleave(torch.arange(E, device=dev), lay.num_recv_tokens_per_expert.long())
        row_expert = torch.nn.functional.pad(row_expert, (0, cap - row_expert.numel()))
        y = torch.nan_to_num(rx.float() / escales[row_expert], nan=0.0, posinf=0.0,
                             neginf=0.0).to(torch.bfloat16)
        del row_expert
    elif w.static_scale > 0:
        x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        rx = torch.empty((cap, H), dtype=torch.int8, device=dev)
        sscale = torch.tensor([w.static_scale], dtype=torch.float32, device=dev)

        def run_dispatch():
            moe.moe_dispatch_static(x, lay, sscale, None, recv_x=rx)

        run_dispatch()
        y = (rx.float() / w.static_scale).to(torch.bfloat16)   # identity expert
    else:
        x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        rx, rs, _ = moe.allocate_recv(lay, H, quant)

        def run_dispatch():
            moe.moe_dispatch(x, lay, None, quant, recv_x=rx, recv_scales=rs)

        # identity expert output (made once, outside the timed region)
        run_dispatch()
        if quant == 0:
            y = rx
        else:
            codes = rx.float()
            if quant in PER_TOKEN_MODES:
                y = codes * rs[:, None]
            elif quant in PER_GROUP_MODES:
                y = codes * rs.repeat_interleave(128, dim=1)[:, :H]
            else:
                y = (codes.view(cap, H // 32, 32) * torch.exp2(rs.float() - 127.0)[:, :, None]).view(cap, H)
            y = torch.nan_to_num(y, nan=0.0, posinf=0.0, neginf=0.0).to(torch.bfloat16)
    torch.cuda.synchronize()

    if w.epilogue:
        shared = torch.from_numpy(W.random_bf16_rows(T, H, 21).view(np.int16)).to(dev).view(torch.bfloat16)
        residual = torch.from_numpy(W.random_bf16_rows(T, H, 22).view(np.int16)).to(dev).view(torch.bfloat16)
        gamma = torch.ones(H, dtype=torch.bfloat16, device=dev)
        out_norm = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

        def run_combine():
            moe.moe_combine_fused(y, lay, wt, shared, residual, gamma, 1e-6, out=out, out_norm=out_norm)
    else:
        def run_combine():
            moe.moe_combine(y, lay, wt, out=out)

    timer = StageEvents(torch)

    if args.one_launch:
        if (quant not in moe.ONE_LAUNCH_MODES or w.prequant or w.static_scale > 0
                or not moe.moe_layout_and_dispatch_fits(T, H, K, R)):
            raise SystemExit(f"--one-launch takes bf16 or per-token quantised batches of at most 512 "
                             f"tokens, 3072 entries and hidden 8192; {w.name} is not one")

        def run_layout():
            moe.moe_layout_and_dispatch(idx, x, E, R, a, None, quant_mode=quant, out=lay, recv_x=rx,
                                        recv_scales=rs)

        def run_dispatch():
            pass
    else:
        def run_layout():
            moe.moe_get_dispatch_layout(idx, E, R, a, out=lay)

    # a step with optional timing marks: ev[0] before the layout, ev[1] after it,
    # ev[2] after dispatch, ev[3] after combine (None = not recorded)
    def step(ev=None):
        if ev is not None and ev[0] is not None:
            timer.record(ev[0])
        run_layout()
        if ev is not None and ev[1] is not None:
            timer.record(ev[1])
        run_dispatch()
        if ev is not None and ev[2] is not None:
            timer.record(ev[2])
        run_combine()
        if ev is not None and ev[3] is not None:
            timer.record(ev[3])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the dominant row kernel: medians over five more untimed steps with every
    # mark (one step alone can pick the shorter kernel on an outlier launch)
    probes = [[timer.new() for _ in range(4)] for _ in range(5)]
    for pr in probes:
        step(pr)
    torch.cuda.synchronize()
    d_us = sorted(timer.elapsed_us(pr[1], pr[2]) for pr in probes)[2]
    c_us = sorted(timer.elapsed_us(pr[2], pr[3]) for pr in probes)[2]
    dom = "dispatch" if d_us >= c_us else "combine"

    # timed region: exactly K steps.  Every Nth step (at least 10 samples from
    # 10 steps on) records the two marks around the dominant kernel, and every
    # other such step all four marks; each mark costs the GPU ~1-2 us, so
    # fewer of them keep the step close to an unobserved one.
    every = args.event_every if args.event_every > 0 else max(1, args.steps // 10)
    sampled = list(range(0, args.steps, every))
    events = {}
    for n, i in enumerate(sampled):
        if n % 2 == 1 or len(sampled) == 1:
            events[i] = [timer.new() for _ in range(4)]
        elif dom == "dispatch":
            events[i] = [None, timer.new(), timer.new(), None]
        else:
            events[i] = [None, None, timer.new(), timer.new()]
    graph = None
    if args.graph:
        # stage times from an eager pass with events; then the step captured once
        for i in range(args.steps):
            step(events.get(i))
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for i in range(args.steps):
            graph.replay()
    else:
        for i in range(args.steps):
            step(events.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    st = {"layout": [], "dispatch": [], "combine": []}
    for ev in events.values():
        for name, (a_, b_) in (("layout", (0, 1)), ("dispatch", (1, 2)), ("combine", (2, 3))):
            if ev[a_] is not None and ev[b_] is not None:
                st[name].append(timer.elapsed_us(ev[a_], ev[b_]))
    avg_us = {k: float(np.mean(v)) for k, v in st.items() if v}
    med_us = {k: float(np.median(v)) for k, v in st.items() if v}

    sb = stage_bytes(T, H, K, R, E, V, cap, quant, prequant_rows, w.static_scale > 0,
                     bool(w.epilogue), w.static_per_expert)
    step_bytes = sum(sb.values())
    ms_per_step = elapsed / args.steps * 1e3
    gbs = step_bytes * args.steps / elapsed / 1e9
    tokens_per_s = T * args.steps / elapsed

    # cold-cache legs (outside the timed region): before each stage, 1 GiB of
    # unrelated traffic evicts the 4 MB L2s and the 256 MB memory-side cache;
    # each stage is then timed alone and a cold step is the sum of the stage
    # medians.  "fill" writes the 1 GiB (the caches are left holding dirty
    # lines, whose write-back the next stage pays for); "read" reads it (the
    # caches are left holding clean lines: only the stage's own misses count).
    cold = None
    if args.cold_reps > 0:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        flush64 = flush.view(torch.int64)
        stages = [("layout", run_layout), ("dispatch", run_dispatch), ("combine", run_combine)]
        cold = {"reps": args.cold_reps}
        for kind, evict in (("fill", lambda n: flush.fill_(n)), ("read", lambda n: flush64.sum())):
            cev = [[(timer.new(), timer.new()) for _ in stages] for _ in range(args.cold_reps)]
            torch.cuda.synchronize()
            for rep in cev:
                for (name, fn), (e0, e1) in zip(stages, rep):
                    evict(len(name))
                    timer.record(e0)
                    fn()
                    timer.record(e1)
            torch.cuda.synchronize()
            med = {name: float(np.median([timer.elapsed_us(*rep[j]) for rep in cev]))
                   for j, (name, _) in enumerate(stages)}
            cold[kind] = {"stage_median_us": {k: round(v, 2) for k, v in med.items()},
                          "step_us": round(sum(med.values()), 2)}
        del flush, flush64

    achieved = sb[dom] / (avg_us[dom] * 1e-6) / 1e9
    prof_us = profiled_stage_us(w.name, dom)

    if not args.no_check:
        # cheap sanity check after timing: every dispatched row is its token
        src = lay.recv_src.long()
        u = src >= 0
        if w.prequant:
            assert torch.equal(rd[u], data[src[u] // K])
        elif quant == 0 and not w.static_scale > 0:
            assert torch.equal(rx.view(torch.int16)[u], x.view(torch.int16)[src[u] // K])
        assert int(lay.error_flag.item()) == 0

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(inp, w, quant, args.cpu_seconds,
                           lambda v, c: stage_bytes(T, H, K, R, E, v, c, quant, prequant_rows,
                                                    w.static_scale > 0, bool(w.epilogue),
                                                    w.static_per_expert),
                           prequant=cpu_y)

    qname = {0: "bf16", 2: "int8", 4: "mxfp8_e4m3", 0x12: "fp8_e4m3_per_token",
             0x22: "fp8_e5m2_per_token", 0x24: "mxfp8_e5m2", 0x13: "fp8_e4m3_per_group",
             0x23: "fp8_e5m2_per_group"}[quant]
    if w.static_scale > 0:
        qname = "int8_static_per_expert" if w.static_per_expert else "int8_static"
    if w.prequant:
        qname = f"{w.prequant}_prequantized"
    rec = {
        "metric": "dispatch+combine effective HBM GB/s and tokens/s (% of peak) at 4096x7168 top-8",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if qname == "bf16" else f"bf16->{qname}") if not w.prequant else qname,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.describe(), "num_tokens": T, "hidden": H,
                   "num_experts": E, "num_virtual_ranks": R, "top_k": K, "expert_alignment": a,
                   "quant": qname, "valid_entries": V, "recv_capacity": cap,
                   "parallelism": "single GPU (virtual expert ranks)"},
        "tokens_per_s": round(tokens_per_s, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "stage_bytes": sb,
        "stage_avg_us": {k: round(v, 2) for k, v in avg_us.items()},
        "stage_median_us": {k: round(v, 2) for k, v in med_us.items()},
        "stage_achieved_gbs": {k: round(sb[k] / (v * 1e-6) / 1e9, 1) for k, v in avg_us.items() if v > 0},
        "stage_events": {"kind": timer.kind, "every_nth_step": every,
                         "samples": {k: len(v) for k, v in st.items()},
                         "timed_region": "eager pass before the graph replays" if graph is not None
                         else "the timed steps"},
        "launch": ("graph replay" if graph is not None else "eager")
                  + (", layout and dispatch in one launch" if args.one_launch else ""),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(w.name, dom),
                     "algorithmic_bytes_per_launch": sb[dom],
                     "avg_launch_us": round(avg_us[dom], 2),
                     "event_samples": len(st[dom]),
                     "profiled_avg_launch_us": prof_us,
                     "profiled_frac": (round(sb[dom] / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                       if prof_us else None),
                     "profile": f"profiles/{w.name}_kernel_stats.txt" if prof_us else None},
        "cpu_baseline": cpu,
    }
    if cold is not None:
        for kind in ("fill", "read"):
            c = cold[kind]
            c["gbs"] = round(step_bytes / (c["step_us"] * 1e-6) / 1e9, 1)
            c["frac_of_hbm_peak"] = round(c["gbs"] / HBM_PEAK_GBS, 4)
            c["tokens_per_s"] = round(T / (c["step_us"] * 1e-6), 1)
        rec["cold_cache"] = cold
    timer.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
