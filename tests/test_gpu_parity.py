"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: layout, indices, rows, codes and scales bit-exact (whole buffers,
including the sentinel left in rows nobody writes); combine within
|g - r| <= 2^-8 |r| + (K+1) 2^-24 sum|w y| of the fp64 oracle, and, with
identity experts, max relative error <= 1e-2.
"""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from combine_moe_get_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe
    from gpu_util import (DEV, assert_layout_equal, bf16_dev, bf16_host_bits, check_combine,
                          combine_bound, dequant_identity_expert, gpu_layout, layout_to_host,
                          oracle_poisoned, poisoned_recv, recv_to_host)


def run_full_case(x_bits, idx, wts, E, R, a, quant, max_rel_1e2=True):
    T, H = x_bits.shape
    K = idx.shape[1]
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    gl = layout_to_host(lay)
    assert_layout_equal(gl, ol)

    cap = ol.recv_capacity
    orx, ors = oracle_poisoned(cap, H, quant)
    orx, ors, orw = oracle.dispatch(x_bits, ol.token_row, cap, wts, quant, recv_x=orx,
                                    recv_scales=ors, with_weights=True)
    rx, rs, rw = poisoned_recv(lay, H, quant)
    x_dev = bf16_dev(x_bits)
    w_dev = torch.from_numpy(wts).to(DEV)
    moe.moe_dispatch(x_dev, lay, w_dev, quant, recv_x=rx, recv_scales=rs, recv_weights=rw)
    grx = recv_to_host(rx, quant)
    np.testing.assert_array_equal(grx, orx)
    if rs is not None and rs.dtype == torch.float32:
        np.testing.assert_array_equal(rs.cpu().numpy().view(np.uint32), ors.view(np.uint32))
    elif rs is not None:
        np.testing.assert_array_equal(rs.cpu().numpy(), ors)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])
    assert (rw.cpu().numpy()[~used] == -3.0).all()

    # combine with identity experts
    y_bits = dequant_identity_expert(orx, ors, quant)
    y_dev = bf16_dev(y_bits) if quant != 0 else rx
    out = moe.moe_combine(y_dev, lay, w_dev)
    exact = oracle.combine(y_bits, ol.token_row, wts)
    S = combine_bound(y_bits, ol.token_row, wts, K)
    return check_combine(bf16_host_bits(out), exact, S, K, max_rel_1e2=max_rel_1e2)


@pytest.mark.parametrize("w", W.WORKLOADS[:4], ids=[w.name for w in W.WORKLOADS[:4]])
def test_workload_full_parity(w):
    inp = W.generate(w)
    rel = run_full_case(inp.x_bits, inp.topk_idx, inp.topk_weights, w.num_experts, w.num_ranks,
                        w.expert_alignment, w.quant_mode)
    print(f"{w.name}: combine max relative error {rel:.3e}")


DECODE = [w for w in W.NEXT_WORKLOADS if w.name.endswith("_decode")]


@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_workload_full_parity(w):
    """Decode-sized batches (the one-workgroup layout) at the headline's
    expert shape, whole path."""
    inp = W.generate(w)
    run_full_case(inp.x_bits, inp.topk_idx, inp.topk_weights, w.num_experts, w.num_ranks,
                  w.expert_alignment, w.quant_mode)


def test_large_workload_layout_full_rows_sampled():
    """32768 x 7168, 512 experts, top-16: layout compared in full; every
    dispatched row checked on the GPU against its source token; a sample of
    tokens compared with the oracle's rows and combine."""
    w = W.WORKLOADS[4]
    inp = W.generate(w)
    T, H, K = w.num_tokens, w.hidden, w.num_topk
    ol = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    lay = gpu_layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    assert_layout_equal(layout_to_host(lay), ol)
    rx, _, rw = poisoned_recv(lay, H, 0)
    x_dev = bf16_dev(inp.x_bits)
    w_dev = torch.from_numpy(inp.topk_weights).to(DEV)
    moe.moe_dispatch(x_dev, lay, w_dev, 0, recv_x=rx, recv_weights=rw)
    # every valid row equals its token; every other row still holds the sentinel
    src = lay.recv_src.long()
    used = src >= 0
    rows_i16 = rx.view(torch.int16)
    x_i16 = x_dev.view(torch.int16)
    step = 65536
    for lo in range(0, lay.recv_capacity, step):
        s = src[lo:lo + step]
        u = used[lo:lo + step]
        blk = rows_i16[lo:lo + step]
        assert torch.equal(blk[u], x_i16[s[u] // K])
        assert (blk[~u] == -1).all()
    # oracle on a token sample
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(T, 512, replace=False))
    rows = ol.token_row[sample]
    sub_rows = np.arange(rows.size, dtype=np.int32).reshape(rows.shape)
    orx, _, _ = oracle.dispatch(inp.x_bits[sample], sub_rows, rows.size)
    grx = bf16_host_bits(rx[torch.from_numpy(rows.reshape(-1).astype(np.int64)).to(DEV)])
    np.testing.assert_array_equal(grx, orx)
    out = moe.moe_combine(rx, lay, w_dev)
    exact = oracle.combine(orx, sub_rows, inp.topk_weights[sample])
    S = combine_bound(orx, sub_rows, inp.topk_weights[sample], K)
    check_combine(bf16_host_bits(out[torch.from_numpy(sample).to(DEV)]), exact, S, K)


def _routing(rng, T, K, E, dup=False, drop=0.0):
    if dup:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K]
    idx = idx.astype(np.int64)
    if drop:
        idx[rng.random((T, K)) < drop] = -1
    w = rng.random((T, K)).astype(np.float32)
    return np.ascontiguousarray(idx), w


EDGE = [
    # name, T, H, E, R, K, a, quant, dup, drop
    ("ragged_tail", 4161, 96, 64, 8, 6, 5, 0, False, 0.0),
    ("h32", 257, 32, 8, 2, 3, 1, 4, False, 0.1),
    ("h1056_int8", 300, 1056, 32, 4, 4, 16, 2, True, 0.2),
    ("k1_e_eq_r", 513, 256, 16, 16, 1, 1, 0, False, 0.0),
    ("k16_e512", 700, 128, 512, 512, 16, 1, 0, False, 0.0),
    ("max_hidden_mx", 40, 16384, 128, 8, 8, 32, 4, False, 0.0),
    ("max_hidden_int8", 40, 16384, 128, 8, 8, 32, 2, False, 0.0),
    ("align_gt_counts", 50, 64, 16, 4, 2, 256, 0, False, 0.0),
    ("duplicates", 333, 64, 4, 2, 8, 3, 0, True, 0.0),
    ("all_dropped", 64, 64, 8, 2, 4, 4, 0, False, 1.0),
    ("one_token", 1, 7168, 256, 8, 8, 128, 2, False, 0.0),
    ("fp8_e4m3_per_token", 700, 7168, 64, 8, 8, 16, 0x12, False, 0.05),
    ("fp8_e5m2_per_token", 700, 4096, 64, 8, 8, 16, 0x22, True, 0.05),
    ("mxfp8_e5m2", 700, 4096, 128, 8, 8, 32, 0x24, False, 0.1),
    ("mxfp8_e5m2_max_hidden", 40, 16384, 128, 8, 8, 32, 0x24, False, 0.0),
    ("fp8_e4m3_per_token_h96", 257, 96, 8, 2, 3, 1, 0x12, False, 0.1),
    ("fp8_e4m3_per_group", 700, 7168, 64, 8, 8, 16, 0x13, False, 0.05),
    ("fp8_e5m2_per_group", 700, 4096, 64, 8, 8, 16, 0x23, True, 0.05),
    ("fp8_e4m3_per_group_partial", 300, 160, 16, 4, 4, 8, 0x13, False, 0.1),
    ("fp8_e5m2_per_group_max_hidden", 40, 16384, 128, 8, 8, 32, 0x23, False, 0.0),
    # the limits of the one-workgroup layout: T*K <= 3072 and T*R <= 16384
    ("single_layout_max_entries", 384, 64, 256, 8, 8, 1, 0, False, 0.0),
    ("chunked_layout_min_entries", 385, 64, 256, 8, 8, 1, 0, False, 0.0),
    ("single_layout_max_flags", 2048, 32, 64, 8, 1, 2, 0, False, 0.05),
    ("chunked_layout_flags_over", 1024, 32, 512, 32, 2, 1, 0, False, 0.0),
    # count tables of >= 131072 cells: the column-scan launch between count and rank
    ("scan_layout_e512_r512", 8192, 32, 512, 512, 2, 1, 0, False, 0.0),
    ("scan_layout_ragged_a7_drop", 8200, 64, 512, 512, 3, 7, 0, False, 0.2),
    ("scan_layout_e256_r256_k1", 32768, 32, 256, 256, 1, 1, 0, False, 0.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(case):
    name, T, H, E, R, K, a, quant, dup, drop = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    idx, wts = _routing(rng, T, K, E, dup, drop)
    wts[idx < 0] = 0.0
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_full_case(x, idx, wts, E, R, a, quant)


def test_skewed_routing_all_to_one_expert():
    rng = np.random.default_rng(4)
    T, K, E = 6000, 4, 64
    idx = np.zeros((T, K), np.int64)
    idx[:, 1:] = rng.integers(0, E, size=(T, K - 1))
    wts = rng.random((T, K)).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, 64)).astype(np.float32))
    run_full_case(x, idx, wts, E, 4, 7, 0, max_rel_1e2=False)


@pytest.mark.parametrize("T,K,E,R", [(900, 4, 32, 4), (3000, 4, 32, 4), (8192, 2, 512, 512)],
                         ids=["one_workgroup", "chunked", "chunked_scan"])
def test_out_of_range_ids_flagged(T, K, E, R):
    """Ids outside [-1, E) set the error flag and count as dropped, on every
    layout path (bad ids placed in the first and the last chunk)."""
    rng = np.random.default_rng(6 + T)
    idx, wts = _routing(rng, T, K, E)
    idx[5, 1] = E
    idx[T - 3, K - 1] = -9
    ol = oracle.layout(idx, E, R, 8)
    gl = layout_to_host(gpu_layout(idx, E, R, 8))
    assert ol.error_flag == 1
    assert_layout_equal(gl, ol)


@pytest.mark.parametrize("T", [100, 3000], ids=["one_workgroup", "chunked"])
def test_capacity_above_the_bound(T):
    """A caller may size the receive buffer above T*K + E*(a-1): the whole
    layout, rows past the last expert included (recv_src -1), equals the
    oracle's at that capacity, and dispatch and combine run unchanged on it."""
    rng = np.random.default_rng(4242 + T)
    H, K, E, R, a = 256, 4, 16, 4, 8
    idx, wts = _routing(rng, T, K, E, drop=0.1)
    cap = oracle.recv_capacity_bound(T, K, E, a) + 777
    ol = oracle.layout(idx, E, R, a, recv_capacity=cap)
    lay = gpu_layout(idx, E, R, a, cap=cap)
    assert lay.recv_capacity == cap
    gl = layout_to_host(lay)
    assert_layout_equal(gl, ol)
    assert (gl["recv_src"][ol.expert_offsets[-1]:] == -1).all()
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    orx, _ = oracle_poisoned(cap, H, 0)
    orx, _, _ = oracle.dispatch(x_bits, ol.token_row, cap, wts, 0, recv_x=orx, with_weights=True)
    rx, _, rw = poisoned_recv(lay, H, 0)
    w_dev = torch.from_numpy(wts).to(DEV)
    moe.moe_dispatch(bf16_dev(x_bits), lay, w_dev, 0, recv_x=rx, recv_weights=rw)
    np.testing.assert_array_equal(recv_to_host(rx, 0), orx)
    out = moe.moe_combine(rx, lay, w_dev)
    exact = oracle.combine(orx, ol.token_row, wts)
    S = combine_bound(orx, ol.token_row, wts, K)
    check_combine(bf16_host_bits(out), exact, S, K)


def test_zero_tokens():
    idx = np.zeros((0, 4), np.int64)
    ol = oracle.layout(idx, 16, 4, 8)
    lay = gpu_layout(idx, 16, 4, 8)
    assert_layout_equal(layout_to_host(lay), ol)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    rx, rs, rw = moe.moe_dispatch(x, lay, None, 0)
    out = moe.moe_combine(rx, lay, None)
    assert out.shape == (0, 64)


def test_quant_special_rows():
    """Zero rows, subnormal rows, rows whose int8 scale overflows, -0, and
    single outliers, through both quantisers."""
    H, K, E = 256, 2, 4
    rows = []
    rows.append(np.zeros(H, np.float32))
    r = np.zeros(H, np.float32); r[3] = -0.0; r[100] = 2.0 ** -130; rows.append(r)
    rows.append(np.full(H, 2.0 ** -127, np.float32))
    r = np.zeros(H, np.float32); r[7] = 3.0e38; r[8] = -1.0; rows.append(r)
    rng = np.random.default_rng(8)
    r = rng.standard_normal(H).astype(np.float32) * 1e-3; r[200] = 5e4; rows.append(r)
    r = (rng.integers(-127, 128, H)).astype(np.float32); r[0] = 127; rows.append(r)
    x = W.f32_to_bf16_bits(np.stack(rows))
    x[1, 3] = 0x8000
    T = x.shape[0]
    idx = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], axis=1).astype(np.int64)
    wts = np.full((T, K), 0.5, np.float32)
    for quant in (2, 4, 0x12, 0x22, 0x24, 0x13, 0x23):
        run_full_case(x, idx, wts, E, 2, 1, quant, max_rel_1e2=False)


def _nonfinite_rows(H=256):
    """bf16 rows holding NaN and infinities: a NaN with a finite maximum, +inf
    with a NaN, -inf, an all-NaN row, NaN and inf in different 32-blocks and
    128-groups of one row, and a finite control row."""
    rng = np.random.default_rng(12)
    x = W.f32_to_bf16_bits(rng.uniform(-3, 3, (7, H)).astype(np.float32))
    PINF, NINF, QNAN, NQNAN = 0x7F80, 0xFF80, 0x7FC0, 0xFFC1
    x[0, 17] = QNAN
    x[1, 5], x[1, 90] = PINF, QNAN
    x[2, 200] = NINF
    x[3, :] = QNAN
    x[4, 33], x[4, 130], x[4, 131] = PINF, NQNAN, NINF
    x[5, 255] = PINF
    return x


def test_quant_nonfinite_rows():
    """NaN and infinities through every quantiser (dynamic modes, static int8
    with one and per-channel scales, per-expert static -- the static ones
    also with infinite, NaN, zero and huge scales -- the one-launch
    per-token path): codes and scales bit-exact against the oracle's
    readings (NaN elements take no part in a maximum, NaN casts to int8 0 and
    to the FP8 NaN code 0x7F, an infinite maximum gives scale +inf or the e8m0
    byte 0xFF)."""
    x = _nonfinite_rows()
    T, H = x.shape
    K, E, R, a = 2, 4, 2, 1
    idx = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], axis=1).astype(np.int64)
    wts = np.full((T, K), 0.5, np.float32)
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    cap = ol.recv_capacity
    x_dev = bf16_dev(x)
    for quant in (2, 0x12, 0x22, 4, 0x24, 0x13, 0x23):
        print(f"[nonfinite] mode {quant:#x}", flush=True)
        orx, ors = oracle_poisoned(cap, H, quant)
        orx, ors, _ = oracle.dispatch(x, ol.token_row, cap, None, quant, recv_x=orx, recv_scales=ors)
        rx, rs, _ = poisoned_recv(lay, H, quant)
        moe.moe_dispatch(x_dev, lay, None, quant, recv_x=rx, recv_scales=rs)
        np.testing.assert_array_equal(recv_to_host(rx, quant), orx)
        g = rs.cpu().numpy()
        if g.dtype == np.float32:
            np.testing.assert_array_equal(g.view(np.uint32), ors.view(np.uint32))
        else:
            np.testing.assert_array_equal(g, ors)
        if quant in (2, 0x12, 0x22):
            lay1, rx1, rs1, _ = moe.moe_layout_and_dispatch(torch.from_numpy(idx).to(DEV), x_dev, E, R, a,
                                                             quant_mode=quant)
            used = ol.recv_src >= 0
            np.testing.assert_array_equal(recv_to_host(rx1, quant)[used], orx[used])
            np.testing.assert_array_equal(rs1.cpu().numpy().view(np.uint32)[used], ors.view(np.uint32)[used])
    odd = np.linspace(0.5, 40.0, H, dtype=np.float32)
    odd[::5], odd[1::7], odd[2::11], odd[3::13] = np.inf, np.nan, 0.0, 3e38
    odd[4::17] = -np.inf
    for scales in (np.array([3.0], np.float32), np.linspace(0.5, 40.0, H, dtype=np.float32), odd,
                   np.array([np.inf], np.float32), np.array([np.nan], np.float32)):
        print(f"[nonfinite] static {scales.size}", flush=True)
        orx, _ = oracle.dispatch_static(x, ol.token_row, cap, scales, recv_x=np.full((cap, H), 0x55, np.int8))
        rx = torch.full((cap, H), 0x55, dtype=torch.int8, device=DEV)
        moe.moe_dispatch_static(x_dev, lay, torch.from_numpy(scales).to(DEV), recv_x=rx)
        np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    escales = np.random.default_rng(13).uniform(0.5, 40.0, (E, H)).astype(np.float32)
    eodd = escales.copy()
    eodd[0, ::3], eodd[1, 1::4], eodd[2, ::2], eodd[3, 1::5] = np.inf, np.nan, 0.0, -3e38
    for name, es in (("finite", escales), ("non-finite", eodd)):
        print(f"[nonfinite] per-expert static, {name} scales", flush=True)
        orx, _ = oracle.dispatch_static_expert(x, idx, ol.token_row, cap, es,
                                               recv_x=np.full((cap, H), 0x55, np.int8))
        rx = torch.full((cap, H), 0x55, dtype=torch.int8, device=DEV)
        moe.moe_dispatch_static_per_expert(x_dev, lay, torch.from_numpy(idx).to(DEV),
                                           torch.from_numpy(es).to(DEV), recv_x=rx)
        np.testing.assert_array_equal(rx.cpu().numpy(), orx)


def test_combine_random_expert_outputs():
    """Combine alone on arbitrary expert rows (cancellation allowed), with and
    without weights."""
    rng = np.random.default_rng(12)
    T, K, E, H = 2000, 8, 64, 512
    idx, wts = _routing(rng, T, K, E, drop=0.1)
    wts = rng.standard_normal((T, K)).astype(np.float32)
    ol = oracle.layout(idx, E, 8, 4)
    lay = gpu_layout(idx, E, 8, 4)
    y = W.random_bf16_rows(ol.recv_capacity, H, 3)
    y_dev = bf16_dev(y)
    for w in (wts, None):
        out = moe.moe_combine(y_dev, lay, None if w is None else torch.from_numpy(w).to(DEV))
        exact = oracle.combine(y, ol.token_row, w)
        S = combine_bound(y, ol.token_row, w, K)
        check_combine(bf16_host_bits(out), exact, S, K, max_rel_1e2=False)


def test_deterministic_repeat():
    w = W.WORKLOADS[2]
    inp = W.generate(w, num_tokens=2048)
    outs = []
    for _ in range(2):
        lay = gpu_layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
        rx, rs, _ = moe.moe_dispatch(bf16_dev(inp.x_bits), lay, None, 2)
        y = (rx.float() * rs[:, None]).to(torch.bfloat16)
        out = moe.moe_combine(y, lay, torch.from_numpy(inp.topk_weights).to(DEV))
        outs.append((layout_to_host(lay), rx.cpu(), rs.cpu(), out.cpu()))
    a, b = outs
    for k in a[0]:
        np.testing.assert_array_equal(a[0][k], b[0][k])
    used = a[0]["recv_src"] >= 0
    assert torch.equal(a[1][used], b[1][used]) and torch.equal(a[2][used], b[2][used])
    assert torch.equal(a[3].view(torch.int16), b[3].view(torch.int16))


def test_pending_unrelated_hip_error_does_not_fail_calls():
    """A HIP error left pending by an unrelated host-side call (a device
    attribute query for a device that does not exist) must not be reported
    by the library's own launches."""
    import ctypes
    path = [l.split()[-1] for l in open("/proc/self/maps").read().split("\n") if "libamdhip64" in l][0]
    hip = ctypes.CDLL(path)
    v = ctypes.c_int()
    assert hip.hipDeviceGetAttribute(ctypes.byref(v), 0, 9999) != 0     # leaves an error pending
    rng = np.random.default_rng(1)
    idx, wts = _routing(rng, 64, 2, 8)
    lay = gpu_layout(idx, 8, 2, 1)
    x = bf16_dev(W.f32_to_bf16_bits(rng.standard_normal((64, 64)).astype(np.float32)))
    rx, _, _ = moe.moe_dispatch(x, lay, None, 0)
    moe.moe_combine(rx, lay, None)
    torch.cuda.synchronize()
    hip.hipGetLastError()                                               # leave no error behind
    assert_layout_equal(layout_to_host(lay), oracle.layout(idx, 8, 2, 1))


@pytest.mark.parametrize("quant,T", [(0, 300), (2, 300), (4, 300), (0, 2000), (4, 2000), (0, 8192)])
def test_graph_capture_replays_match_eager(quant, T):
    """The three calls allocate nothing and never synchronise, so a step can be
    captured in a HIP graph.  Replay it several times, with eager work and
    synchronisations in between, and check every replay against the eager
    result (layout, rows, scales, combine output).  T = 300 takes the
    one-workgroup layout, T = 2000 the two-launch one, and T = 8192 with
    512 experts over 512 ranks the three-launch one (column scan)."""
    rng = np.random.default_rng(40 + quant + T)
    H, K, E, R, a = (512, 4, 32, 4, 8) if T < 8192 else (64, 2, 512, 512, 1)
    idx, wts = _routing(rng, T, K, E, drop=0.05)
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    idx_d = torch.from_numpy(idx).to(DEV)
    x = bf16_dev(x_bits)
    w = torch.from_numpy(wts).to(DEV)
    lay = moe.allocate_layout(T, K, E, R, a, device=DEV)
    rx, rs, _ = moe.allocate_recv(lay, H, quant)
    y = bf16_dev(W.random_bf16_rows(lay.recv_capacity, H, 7))
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.moe_get_dispatch_layout(idx_d, E, R, a, out=lay)
        moe.moe_dispatch(x, lay, None, quant, recv_x=rx, recv_scales=rs)
        moe.moe_combine(y, lay, w, out=out)

    def snapshot():
        torch.cuda.synchronize()
        used = lay.recv_src >= 0
        return (lay.token_row.clone(), lay.recv_src.clone(), lay.expert_offsets.clone(),
                rx.view(torch.uint8)[used].clone(),
                None if rs is None else (rs.view(torch.int32) if rs.dim() == 1 else rs)[used].clone(),
                out.view(torch.int16).clone())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        for t_ in (lay.token_row, lay.recv_src, lay.expert_offsets, out):
            t_.fill_(7)
        rx.view(torch.uint8).fill_(3)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a_, b_ in zip(ref, got):
            if a_ is not None:
                assert torch.equal(a_, b_)


@pytest.mark.parametrize("E", [64, 300])
def test_graph_capture_static_expert_and_fused_combine(E):
    """A step of layout, per-expert static int8 dispatch (64 experts: 128-
    channel slices; 300: 64-channel slices) and the normalising fused
    combine (shared output, residual, RMSNorm; nontemporal stores) captured
    in a HIP graph and replayed several times with eager work and
    synchronisations in between: every replay equals the eager step."""
    rng = np.random.default_rng(77 + E)
    T, H, K, R, a = 700, 1056, 6, 4, 8
    idx, wts = _routing(rng, T, K, E, drop=0.05)
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x = bf16_dev(x_bits)
    idx_d = torch.from_numpy(idx).to(DEV)
    w = torch.from_numpy(wts).to(DEV)
    scales = torch.from_numpy(rng.uniform(0.5, 40.0, (E, H)).astype(np.float32)).to(DEV)
    lay = moe.allocate_layout(T, K, E, R, a, device=DEV)
    rx = torch.empty((lay.recv_capacity, H), dtype=torch.int8, device=DEV)
    rw = torch.empty((lay.recv_capacity,), dtype=torch.float32, device=DEV)
    y = bf16_dev(W.random_bf16_rows(lay.recv_capacity, H, 8))
    sh = bf16_dev(W.random_bf16_rows(T, H, 9))
    res = bf16_dev(W.random_bf16_rows(T, H, 10))
    gamma = bf16_dev(W.random_bf16_rows(1, H, 11))[0].contiguous()
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    out_n = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.moe_get_dispatch_layout(idx_d, E, R, a, out=lay)
        moe.moe_dispatch_static_per_expert(x, lay, idx_d, scales, w, recv_x=rx, recv_weights=rw)
        moe.moe_combine_fused(y, lay, w, sh, res, gamma, 1e-6, out=out, out_norm=out_n)

    def snapshot():
        torch.cuda.synchronize()
        used = lay.recv_src >= 0
        return (lay.token_row.clone(), rx[used].clone(), rw[used].clone(),
                out.view(torch.int16).clone(), out_n.view(torch.int16).clone())

    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        step()
    torch.cuda.current_stream().wait_stream(s_)
    ref = snapshot()
    # the eager step itself against the oracle (layout rows and codes)
    ol = oracle.layout(idx, E, R, a)
    orx, _ = oracle.dispatch_static_expert(x_bits, idx, ol.token_row, ol.recv_capacity,
                                           scales.cpu().numpy(), wts)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(ref[0].cpu().numpy(), ol.token_row)
    np.testing.assert_array_equal(ref[1].cpu().numpy(), orx[used])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        for t_ in (lay.token_row, out, out_n):
            t_.fill_(7)
        rx.fill_(3)
        rw.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a_, b_ in zip(ref, got):
            assert torch.equal(a_, b_)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "no_scales", "wide_rows_odd_scales"])
def test_dispatch_prequantized_parity(fmt):
    """Pre-quantised (data, scale) rows are copied byte for byte: whole
    receive buffers equal the oracle's, sentinels included.  The last case
    takes 32 KiB rows (two 16-byte vectors per lane) and 5-byte scale rows."""
    rng = np.random.default_rng(zlib.crc32(fmt.encode()))
    T, H, K, E, R, a = 900, 7168, 8, 64, 8, 32
    if fmt == "wide_rows_odd_scales":
        T, H = 200, 16384
    idx, wts = _routing(rng, T, K, E, drop=0.05)
    row_bytes = {"mxfp8": H, "mxfp4": H // 2, "no_scales": H // 2, "wide_rows_odd_scales": 2 * H}[fmt]
    scale_bytes = {"no_scales": 0, "wide_rows_odd_scales": 5}.get(fmt, H // 32)
    data = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
    sc = rng.integers(100, 140, size=(T, scale_bytes), dtype=np.uint8) if scale_bytes else None
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    cap = ol.recv_capacity
    ord0 = np.full((cap, row_bytes), 0xA5, np.uint8)
    ors0 = np.full((cap, scale_bytes), 0x5A, np.uint8) if scale_bytes else None
    ord_, ors, orw = oracle.dispatch_prequantized(data, sc, ol.token_row, cap, wts, ord0,
                                                  ors0, with_weights=True)
    dtype = torch.float8_e4m3fn if fmt == "mxfp8" else torch.uint8
    d_dev = torch.from_numpy(data).to(DEV).view(dtype)
    s_dev = None if sc is None else torch.from_numpy(sc).to(DEV)
    rd = torch.full((cap, row_bytes), 0xA5, dtype=torch.uint8, device=DEV).view(dtype)
    rs = None if sc is None else torch.full((cap, scale_bytes), 0x5A, dtype=torch.uint8, device=DEV)
    rw = torch.full((cap,), -3.0, device=DEV)
    moe.moe_dispatch_prequantized(d_dev, s_dev, lay, torch.from_numpy(wts).to(DEV), rd, rs, rw)
    np.testing.assert_array_equal(rd.view(torch.uint8).cpu().numpy(), ord_)
    if sc is not None:
        np.testing.assert_array_equal(rs.cpu().numpy(), ors)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])


@pytest.mark.parametrize("per_channel,H", [(False, 7168), (True, 7168), (False, 16384), (True, 16384),
                                           (True, 96)])
def test_dispatch_static_parity(per_channel, H):
    """Static int8 (caller scales, saturating): whole receive buffers equal
    the oracle's, sentinels included.  H = 16384 takes two vectors per lane;
    H = 96 a partial wave."""
    rng = np.random.default_rng(77 + per_channel + H)
    T, K, E, R, a = 600, 8, 64, 8, 4
    idx, wts = _routing(rng, T, K, E, drop=0.05)
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    if per_channel:
        scales = rng.uniform(10.0, 80.0, H).astype(np.float32)
    else:
        scales = np.array([45.0], np.float32)
    ol = oracle.layout(idx, E, R, a)
    cap = ol.recv_capacity
    orx, orw = oracle.dispatch_static(x_bits, ol.token_row, cap, scales, wts,
                                      recv_x=np.full((cap, H), 0x55, np.int8), with_weights=True)
    assert (orx == 127).any() and (orx == -128).any()        # saturation exercised
    lay = gpu_layout(idx, E, R, a)
    rx = torch.full((cap, H), 0x55, dtype=torch.int8, device=DEV)
    rw = torch.full((cap,), -3.0, device=DEV)
    moe.moe_dispatch_static(bf16_dev(x_bits), lay, torch.from_numpy(scales).to(DEV),
                            torch.from_numpy(wts).to(DEV), recv_x=rx, recv_weights=rw)
    np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])


STATIC_EXPERT_CASES = [
    # name, T, H, K, E, R, a, dup, drop
    ("t600_h7168_k8", 600, 7168, 8, 64, 8, 4, False, 0.05),
    ("h96_duplicates", 300, 96, 5, 24, 4, 3, True, 0.2),
    ("h16384_k16_e512", 257, 16384, 16, 512, 64, 128, False, 0.0),
    ("h2080_k16_e256", 700, 2080, 16, 256, 16, 8, False, 0.05),
    ("e257_64_channel_slices", 300, 512, 8, 257, 1, 2, False, 0.05),
    ("t1_h7168_e256", 1, 7168, 8, 256, 8, 128, False, 0.0),
    ("h32_k1_one_expert", 77, 32, 1, 1, 1, 1, False, 0.1),
    ("all_dropped", 50, 256, 4, 16, 4, 2, False, 1.0),
]


@pytest.mark.parametrize("case", STATIC_EXPERT_CASES, ids=[c[0] for c in STATIC_EXPERT_CASES])
def test_dispatch_static_per_expert_parity(case):
    """Static int8 with one scale row per expert: whole receive buffers equal
    the oracle's, sentinels included; copies of a token to different experts
    carry different codes."""
    name, T, H, K, E, R, a, dup, drop = case
    print(f"[static-expert] {name}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    idx, wts = _routing(rng, T, K, E, dup=dup, drop=drop)
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    scales = rng.uniform(10.0, 90.0, size=(E, H)).astype(np.float32)
    ol = oracle.layout(idx, E, R, a)
    cap = ol.recv_capacity
    orx, orw = oracle.dispatch_static_expert(x_bits, idx, ol.token_row, cap, scales, wts,
                                             recv_x=np.full((cap, H), 0x55, np.int8), with_weights=True)
    lay = gpu_layout(idx, E, R, a)
    rx = torch.full((cap, H), 0x55, dtype=torch.int8, device=DEV)
    rw = torch.full((cap,), -3.0, device=DEV)
    moe.moe_dispatch_static_per_expert(bf16_dev(x_bits), lay, torch.from_numpy(idx).to(DEV),
                                       torch.from_numpy(scales).to(DEV), torch.from_numpy(wts).to(DEV),
                                       recv_x=rx, recv_weights=rw)
    np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])
    assert (rw.cpu().numpy()[~used] == -3.0).all()
    if drop < 1.0 and K > 1 and E > 1:
        r0, r1 = ol.token_row[:, 0], ol.token_row[:, 1]
        both = (r0 >= 0) & (r1 >= 0) & (idx[:, 0] != idx[:, 1])
        assert any(not np.array_equal(orx[a_], orx[b_]) for a_, b_ in zip(r0[both], r1[both]))


def test_dispatch_static_per_expert_int8_workload_full():
    """The per-token int8 workload's shape (8192 x 7168, 256 experts over 16
    ranks, top-8 Zipf, alignment 128) with per-expert scale rows: every row of
    the receive buffer (98048 x 7168 codes) against the oracle."""
    w = W.BY_NAME["int8_static_expert_8192x7168_e256_top8_zipf"]
    print(f"[static-expert] {w.name}", flush=True)
    inp = W.generate(w)
    scales = W.expert_scales(w)
    ol = oracle.layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    cap = ol.recv_capacity
    orx, orw = oracle.dispatch_static_expert(inp.x_bits, inp.topk_idx, ol.token_row, cap, scales,
                                             inp.topk_weights, recv_x=np.full((cap, w.hidden), 0x55, np.int8),
                                             with_weights=True)
    assert (orx == 127).any() and (orx == -128).any()
    lay = gpu_layout(inp.topk_idx, w.num_experts, w.num_ranks, w.expert_alignment)
    rx = torch.full((cap, w.hidden), 0x55, dtype=torch.int8, device=DEV)
    rw = torch.full((cap,), -3.0, device=DEV)
    moe.moe_dispatch_static_per_expert(bf16_dev(inp.x_bits), lay, torch.from_numpy(inp.topk_idx).to(DEV),
                                       torch.from_numpy(scales).to(DEV),
                                       torch.from_numpy(inp.topk_weights).to(DEV), recv_x=rx, recv_weights=rw)
    np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])


def _tie_and_bound_values():
    """bf16 elements whose products with power-of-two scales land exactly on
    half-way points (k + 0.5 for |k| up to 255), on and around the int8
    bounds, on zero of both signs, below the smallest normal and beyond the
    fp32 range."""
    halves = [k + 0.5 for k in range(-128, 128)]              # ties at scale 1
    ints = list(range(-1024, 1025))                           # ties at scales 1/2 and 1/4
    vals = np.array(halves + ints, np.float32)
    vals = vals[W.bf16_bits_to_f32(W.f32_to_bf16_bits(vals)) == vals]  # keep the bf16 values
    # largest finite, 2^97, smallest normal, smallest subnormal (both signs), -0
    special = np.array([0x7F7F, 0xFF7F, 0x7000, 0xF000, 0x0080, 0x8080, 0x0001, 0x8001, 0x8000],
                       np.uint16)
    return np.concatenate([W.f32_to_bf16_bits(vals), special])


@pytest.mark.parametrize("E", [8, 300])
def test_static_per_expert_ties_and_bounds(E):
    """Per-expert static int8 on products at half-way points (round half to
    even), on and past both saturation bounds, subnormal, zero of both signs
    and overflowing to infinity; every element finite, so the short
    conversion takes every code (E = 8: 128-channel slices, 300: 64-channel
    slices).  The whole receive buffer equals the oracle's."""
    rng = np.random.default_rng(E)
    T, H, K, R, a = 520, 256, 4, 4, 1
    pool = _tie_and_bound_values()
    x_bits = pool[rng.integers(0, pool.size, (T, H))]
    pw2 = np.array([0.25, 0.5, 1.0, 2.0, 4.0, 1.0, 1.0, 1.0], np.float32)
    scales = pw2[rng.integers(0, pw2.size, (E, H))]
    odd = rng.random((E, H))
    scales[odd < 0.04] = np.float32(1.0000001)
    scales[(odd >= 0.04) & (odd < 0.06)] = np.float32(3e38)
    scales[(odd >= 0.06) & (odd < 0.08)] = np.float32(1e-40)
    scales[(odd >= 0.08) & (odd < 0.10)] = np.float32(-0.5)
    idx, _ = _routing(rng, T, K, E, drop=0.05)
    ol = oracle.layout(idx, E, R if E % R == 0 else 1, a)
    cap = ol.recv_capacity
    orx, _ = oracle.dispatch_static_expert(x_bits, idx, ol.token_row, cap, scales,
                                           recv_x=np.full((cap, H), 0x55, np.int8))
    used = ol.recv_src >= 0
    assert (orx[used] == 127).any() and (orx[used] == -128).any() and (orx[used] == 0).any()
    lay = gpu_layout(idx, E, R if E % R == 0 else 1, a)
    rx = torch.full((cap, H), 0x55, dtype=torch.int8, device=DEV)
    print(f"[static-expert ties] E={E}", flush=True)
    moe.moe_dispatch_static_per_expert(bf16_dev(x_bits), lay, torch.from_numpy(idx).to(DEV),
                                       torch.from_numpy(scales).to(DEV), recv_x=rx)
    np.testing.assert_array_equal(rx.cpu().numpy(), orx)


@pytest.mark.parametrize("variant", ["shared", "residual", "shared_residual_norm", "norm_only",
                                     "norm_h16384_k16"])
def test_combine_fused_parity(variant):
    """Combine epilogues against the fp64 oracle.  Sum: the combine bound with
    the two extra terms.  Normalised output: one bf16 rounding (2^-9,
    doubled) plus 2e-4 relative for the fp32 sum of squares and the
    reciprocal square root, plus the sum's own error scaled by gamma / rms."""
    rng = np.random.default_rng(zlib.crc32(variant.encode()))
    T, H, K, E = (64, 16384, 16, 64) if variant == "norm_h16384_k16" else (900, 7168, 8, 64)
    idx, wts = _routing(rng, T, K, E, drop=0.05)
    wts = rng.standard_normal((T, K)).astype(np.float32)
    ol = oracle.layout(idx, E, 8, 4)
    lay = gpu_layout(idx, E, 8, 4)
    y = W.random_bf16_rows(ol.recv_capacity, H, 11)
    sh = W.random_bf16_rows(T, H, 12) if "shared" in variant else None
    res = W.random_bf16_rows(T, H, 13, sigma=2.0) if "residual" in variant else None
    norm = "norm" in variant
    gamma = W.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32)) if norm else None
    eps = 1e-5
    _fused_against_oracle(y, lay, ol, wts, sh, res, gamma, eps, norm, K)


def _fused_against_oracle(y, lay, ol, wts, sh, res, gamma, eps, norm, K):
    dv = lambda a: None if a is None else bf16_dev(a)
    out, out_norm = moe.moe_combine_fused(bf16_dev(y), lay, torch.from_numpy(wts).to(DEV), dv(sh),
                                          dv(res), dv(gamma), eps, with_norm=norm)
    ro, rn = oracle.combine_fused(y, ol.token_row, wts, sh, res, gamma, eps, with_norm=norm)
    absb = lambda a: None if a is None else (a & np.uint16(0x7FFF)).astype(np.uint16)
    S, _ = oracle.combine_fused(absb(y), ol.token_row, np.abs(wts), absb(sh), absb(res))
    g = W.bf16_bits_to_f32(bf16_host_bits(out)).astype(np.float64)
    err_bound = (K + 3) * 2.0 ** -24 * S
    assert (np.abs(g - ro) <= 2.0 ** -8 * np.abs(ro) + err_bound).all()
    if norm:
        gn = W.bf16_bits_to_f32(bf16_host_bits(out_norm)).astype(np.float64)
        rms = np.sqrt((ro ** 2).mean(axis=1, keepdims=True) + eps)
        gam = np.abs(W.bf16_bits_to_f32(gamma).astype(np.float64))[None, :]
        bound = (2.0 ** -8 + 2e-4) * np.abs(rn) + gam / rms * err_bound * 2
        assert (np.abs(gn - rn) <= bound).all(), float(np.max(np.abs(gn - rn) - bound))
    else:
        assert out_norm is None
    return g, (gn if norm else None)


@pytest.mark.parametrize("variant", ["shared_residual_norm", "norm_only"])
@pytest.mark.parametrize("H", [32, 96, 2080])
def test_combine_fused_edges(H, variant):
    """Rows narrower than one wave (H = 32: four lanes of 8 elements; 96: 12)
    and a ragged last wave (2080: 260 lanes), with tokens 0-9 having every
    entry dropped: their sum is empty, so the output is shared + residual, or
    an all-zero row whose normalised form is zero as well."""
    rng = np.random.default_rng(H + len(variant))
    T, K, E = 200, 4, 16
    idx, _ = _routing(rng, T, K, E, drop=0.1)
    idx[:10] = -1
    wts = rng.standard_normal((T, K)).astype(np.float32)
    ol = oracle.layout(idx, E, 4, 1)
    lay = gpu_layout(idx, E, 4, 1)
    y = W.random_bf16_rows(max(ol.recv_capacity, 1), H, 21)[:ol.recv_capacity]
    sh = W.random_bf16_rows(T, H, 22) if "shared" in variant else None
    res = W.random_bf16_rows(T, H, 23, sigma=2.0) if "residual" in variant else None
    gamma = W.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    print(f"[fused edges] H={H} {variant}", flush=True)
    g, gn = _fused_against_oracle(y, lay, ol, wts, sh, res, gamma, 1e-5, True, K)
    if variant == "norm_only":
        assert (g[:10] == 0).all() and (gn[:10] == 0).all()
    else:
        want = (W.bf16_bits_to_f32(sh[:10]).astype(np.float64) + W.bf16_bits_to_f32(res[:10]))
        assert (np.abs(g[:10] - want) <= 2.0 ** -8 * np.abs(want) + 2.0 ** -20 * np.abs(want).max()).all()


@pytest.mark.parametrize("quant", [4, 0x24], ids=["mxfp8_e4m3", "mxfp8_e5m2"])
def test_mx_every_element_and_shared_exponent(quant):
    """MX dispatch on rows that pair every finite bf16 element with every block
    exponent it can meet (8.6 M elements): codes and e8m0 bytes bit-exact
    against the oracle, scatter over 8 experts with a ragged expert size."""
    from mx_exhaustive import exhaustive_mx_rows
    x_bits, _ = exhaustive_mx_rows(1024)
    T, H = x_bits.shape
    E = 8
    idx = np.ascontiguousarray((np.arange(T, dtype=np.int64) * 5 % E)[:, None])
    ol = oracle.layout(idx, E, 2, 4)
    lay = gpu_layout(idx, E, 2, 4)
    assert_layout_equal(layout_to_host(lay), ol)
    cap = ol.recv_capacity
    orx, ors = oracle_poisoned(cap, H, quant)
    orx, ors, _ = oracle.dispatch(x_bits, ol.token_row, cap, None, quant, recv_x=orx, recv_scales=ors)
    rx, rs, _ = poisoned_recv(lay, H, quant)
    moe.moe_dispatch(bf16_dev(x_bits), lay, None, quant, recv_x=rx, recv_scales=rs)
    np.testing.assert_array_equal(recv_to_host(rx, quant), orx)
    np.testing.assert_array_equal(rs.cpu().numpy(), ors)


def test_combine_grid_stride_iterations():
    """The combine kernels take work items beyond their grid cap in later
    iterations.  The small-grid test build (cap 64 workgroups) runs those
    iterations here; its outputs must equal the normal build's bit for bit and
    meet the oracle bound (plain combine, and shared + residual epilogues)."""
    import ctypes
    from combine_moe_get_dispatch_amd import build_lib
    if not os.path.exists(build_lib.SMALL_GRID_LIB_PATH):
        pytest.skip("small-grid test build not present (built by __graft_entry__.build())")
    small = moe.declare_signatures(ctypes.CDLL(build_lib.SMALL_GRID_LIB_PATH))
    rng = np.random.default_rng(77)
    T, H, K, E, R, a = 300, 1056, 5, 24, 4, 3         # 132 vectors: 3 slices, 900 items
    idx, wts = _routing(rng, T, K, E, dup=True, drop=0.1)
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    cap = ol.recv_capacity
    y_bits = W.random_bf16_rows(cap, H, 78)
    sh_bits = W.random_bf16_rows(T, H, 79)
    res_bits = W.random_bf16_rows(T, H, 80)
    y, sh, res = bf16_dev(y_bits), bf16_dev(sh_bits), bf16_dev(res_bits)
    w_dev = torch.from_numpy(wts).to(DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    for shared, residual in ((None, None), (sh, res)):
        if shared is None:
            ref = moe.moe_combine(y, lay, w_dev)
        else:
            ref, _ = moe.moe_combine_fused(y, lay, w_dev, shared, residual)
        got = torch.full_like(ref, float("nan"))
        rc = small.moe_combine_fused(y.data_ptr(), cap, T, H, K, lay.token_row.data_ptr(), w_dev.data_ptr(),
                                     None if shared is None else shared.data_ptr(),
                                     None if residual is None else residual.data_ptr(),
                                     None, ctypes.c_float(0.0), got.data_ptr(), None, st)
        assert rc == 0
        if shared is None:
            got2 = torch.full_like(ref, float("nan"))
            assert small.moe_combine(y.data_ptr(), cap, T, H, K, lay.token_row.data_ptr(), w_dev.data_ptr(),
                                     got2.data_ptr(), st) == 0
            torch.cuda.synchronize()
            assert torch.equal(got2.view(torch.int16), ref.view(torch.int16))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        if shared is None:
            exact = oracle.combine(y_bits, ol.token_row, wts)
            S = combine_bound(y_bits, ol.token_row, wts, K)
        else:
            exact, _ = oracle.combine_fused(y_bits, ol.token_row, wts, sh_bits, res_bits)
            S = combine_bound(y_bits, ol.token_row, wts, K) + np.abs(W.bf16_bits_to_f32(sh_bits)) \
                + np.abs(W.bf16_bits_to_f32(res_bits))
        check_combine(bf16_host_bits(got), exact, S, K + 2, max_rel_1e2=False)


@pytest.mark.parametrize("mode", ["bf16", "int8_token", "e4m3_token", "e5m2_token", "mxfp8_e4m3",
                                  "mxfp8_e5m2", "group_e4m3", "group_e5m2", "static", "static_channel",
                                  "static_expert", "prequantized"])
def test_dispatch_grid_stride_iterations(mode):
    """The slice dispatch kernels (unquantised, static, pre-quantised) take
    (token, slice) items beyond their grid cap in later iterations.  The
    small-grid test build (cap 64 workgroups of 4 waves) runs those
    iterations here; whole receive buffers, sentinels included, must equal
    the oracle's (the modes with one workgroup per token run through the
    same build as a check of that build).  The pre-quantised scale rows (200
    bytes over 3 slices of 64 lanes) also take a second pass."""
    import ctypes
    from combine_moe_get_dispatch_amd import build_lib
    if not os.path.exists(build_lib.SMALL_GRID_LIB_PATH):
        pytest.skip("small-grid test build not present (built by __graft_entry__.build())")
    small = moe.declare_signatures(ctypes.CDLL(build_lib.SMALL_GRID_LIB_PATH))
    rng = np.random.default_rng(79)
    T, H, K, E, R, a = 300, 1056, 5, 24, 4, 3         # 132 vectors: 3 slices, 900 items
    idx, wts = _routing(rng, T, K, E, dup=True, drop=0.1)
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    cap = ol.recv_capacity
    used = ol.recv_src >= 0
    st = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    w_dev = torch.from_numpy(wts).to(DEV)
    x_bits = W.random_bf16_rows(T, H, 81)
    x_dev = bf16_dev(x_bits)

    if mode == "prequantized":
        row_bytes, scale_bytes = 2 * H, 200
        data = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
        sc = rng.integers(0, 256, size=(T, scale_bytes), dtype=np.uint8)
        ord_, ors, orw = oracle.dispatch_prequantized(
            data, sc, ol.token_row, cap, wts, np.full((cap, row_bytes), 0xA5, np.uint8),
            np.full((cap, scale_bytes), 0x5A, np.uint8), with_weights=True)
        rd = torch.full((cap, row_bytes), 0xA5, dtype=torch.uint8, device=DEV)
        rs = torch.full((cap, scale_bytes), 0x5A, dtype=torch.uint8, device=DEV)
        rw = torch.full((cap,), -3.0, device=DEV)
        d_dev, s_dev = torch.from_numpy(data).to(DEV), torch.from_numpy(sc).to(DEV)
        assert small.moe_dispatch_prequantized(d_dev.data_ptr(), T, row_bytes, s_dev.data_ptr(), scale_bytes,
                                               K, lay.token_row.data_ptr(), w_dev.data_ptr(), cap,
                                               rd.data_ptr(), rs.data_ptr(), rw.data_ptr(), st) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rd.cpu().numpy(), ord_)
        np.testing.assert_array_equal(rs.cpu().numpy(), ors)
    elif mode == "static_expert":
        # 24 experts: 128-channel slices, 18 (block, column) items; then 1100
        # tokens x 2080 (85 items, ragged last block and column) so that the
        # grid iterates; then 300 experts at 1100 x 2080: 64-channel slices,
        # 165 items.
        shapes = [(T, H, E, R), (1100, 2080, E, R), (1100, 2080, 300, 4)]
        for T2, H2, E2, R2 in shapes:
            print(f"[grid-stride static_expert] T={T2} H={H2} E={E2}", flush=True)
            if (T2, H2, E2) == (T, H, E):
                idx2, wts2, x2, ol2, lay2 = idx, wts, x_bits, ol, lay
            else:
                idx2, wts2 = _routing(rng, T2, K, E2, dup=True, drop=0.1)
                x2 = W.random_bf16_rows(T2, H2, 83)
                ol2, lay2 = oracle.layout(idx2, E2, R2, a), gpu_layout(idx2, E2, R2, a)
            cap2 = ol2.recv_capacity
            scales = (rng.random((E2, H2), dtype=np.float32) * 40 + 1).astype(np.float32)
            orx = np.full((cap2, H2), 0x7B, np.int8)
            orx, orw = oracle.dispatch_static_expert(x2, idx2, ol2.token_row, cap2, scales, wts2, recv_x=orx,
                                                     with_weights=True)
            rx = torch.full((cap2, H2), 0x7B, dtype=torch.int8, device=DEV)
            rw = torch.full((cap2,), -3.0, device=DEV)
            sc_dev = torch.from_numpy(scales).to(DEV)
            idx_dev = torch.from_numpy(idx2).to(DEV)
            w2_dev = torch.from_numpy(wts2).to(DEV)
            assert small.moe_dispatch_static_per_expert(bf16_dev(x2).data_ptr(), T2, H2, K, idx_dev.data_ptr(), E2,
                                                        lay2.token_row.data_ptr(), w2_dev.data_ptr(), cap2,
                                                        sc_dev.data_ptr(), rx.data_ptr(), rw.data_ptr(), st) == 0
            torch.cuda.synchronize()
            np.testing.assert_array_equal(rx.cpu().numpy(), orx)
            used2 = ol2.recv_src >= 0
            np.testing.assert_array_equal(rw.cpu().numpy()[used2], orw[used2])
            assert (rw.cpu().numpy()[~used2] == -3.0).all()
        return
    elif mode.startswith("static"):
        n = H if mode == "static_channel" else 1
        scales = (rng.random(n, dtype=np.float32) * 40 + 1).astype(np.float32)
        orx = np.full((cap, H), 0x7B, np.int8)
        orx, orw = oracle.dispatch_static(x_bits, ol.token_row, cap, scales, wts, recv_x=orx,
                                          with_weights=True)
        rx = torch.full((cap, H), 0x7B, dtype=torch.int8, device=DEV)
        rw = torch.full((cap,), -3.0, device=DEV)
        sc_dev = torch.from_numpy(scales).to(DEV)
        assert small.moe_dispatch_static(x_dev.data_ptr(), T, H, K, lay.token_row.data_ptr(), w_dev.data_ptr(),
                                         cap, sc_dev.data_ptr(), n, rx.data_ptr(), rw.data_ptr(), st) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    else:
        quant = {"bf16": 0, "int8_token": 2, "e4m3_token": 0x12, "e5m2_token": 0x22, "mxfp8_e4m3": 4,
                 "mxfp8_e5m2": 0x24, "group_e4m3": 0x13, "group_e5m2": 0x23}[mode]
        orx, ors = oracle_poisoned(cap, H, quant)
        orx, ors, orw = oracle.dispatch(x_bits, ol.token_row, cap, wts, quant, recv_x=orx, recv_scales=ors,
                                        with_weights=True)
        rx, rs, rw = poisoned_recv(lay, H, quant)
        assert small.moe_dispatch(x_dev.data_ptr(), T, H, K, lay.token_row.data_ptr(), w_dev.data_ptr(), cap,
                                  quant, rx.data_ptr(), None if rs is None else rs.data_ptr(), rw.data_ptr(),
                                  st) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(recv_to_host(rx, quant), orx)
        if rs is not None and rs.dtype == torch.float32:
            np.testing.assert_array_equal(rs.cpu().numpy().view(np.uint32), ors.view(np.uint32))
        elif rs is not None:
            np.testing.assert_array_equal(rs.cpu().numpy(), ors)
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])
    assert (rw.cpu().numpy()[~used] == -3.0).all()


ALL_MODES = [0, 2, 4, 0x12, 0x22, 0x24, 0x13, 0x23]


def _random_config(i):
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([1, 2, 3, 8, 12, 64, 96, 256, 512]))
    R = int(rng.choice([r for r in (1, 2, 3, 4, 8, 16, 64) if E % r == 0]))
    dup = bool(rng.random() < 0.3)
    K = int(rng.integers(1, min(16, E) + 1)) if not dup else int(rng.integers(1, 17))
    T = int(rng.choice([0, 1, 2, 63, 64, 65, 257, int(rng.integers(3, 900))]))
    H = 32 * int(rng.choice([1, 2, 3, 5, 16, 33, 64, 100, 128]))
    a = int(rng.choice([1, 2, 7, 32, 128]))
    quant = ALL_MODES[i % len(ALL_MODES)]
    drop = float(rng.choice([0.0, 0.0, 0.3, 1.0]))
    return rng, T, H, E, R, K, a, quant, dup, drop


@pytest.mark.parametrize("i", range(200), ids=[f"cfg{i}" for i in range(200)])
def test_random_configurations(i):
    """Seeded random shapes over the whole valid range (including T = 0, one
    expert, all entries dropped, ragged hidden sizes, every quant mode): the
    full path against the oracle, plus the expert-side weighting round trip
    (rows scaled by the per-row weights dispatch returns, then an unweighted
    combine)."""
    rng, T, H, E, R, K, a, quant, dup, drop = _random_config(i)
    print(f"[cfg{i}] T={T} H={H} E={E} R={R} K={K} a={a} quant={quant:#x} dup={dup} drop={drop}", flush=True)
    idx, wts = _routing(rng, T, K, E, dup, drop)
    wts[idx < 0] = 0.0
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    run_full_case(x, idx, wts, E, R, a, quant, max_rel_1e2=False)
    if quant != 0 or T == 0:
        return
    # expert applies the row weights that dispatch returned; combine unweighted
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    rx, _, rw = poisoned_recv(lay, H, 0)
    moe.moe_dispatch(bf16_dev(x), lay, torch.from_numpy(wts).to(DEV), 0, recv_x=rx, recv_weights=rw)
    used = torch.from_numpy(ol.recv_src >= 0).to(DEV)
    y = torch.zeros_like(rx)
    y[used] = (rx[used].float() * rw[used, None]).to(torch.bfloat16)
    y_bits = bf16_host_bits(y)
    out = moe.moe_combine(y, lay, None)
    exact = oracle.combine(y_bits, ol.token_row, None)
    S = combine_bound(y_bits, ol.token_row, None, K)
    check_combine(bf16_host_bits(out), exact, S, K, max_rel_1e2=False)


STATIC_KINDS = ["one", "channel", "expert"]


@pytest.mark.parametrize("i", range(60), ids=[f"static{i}" for i in range(60)])
def test_random_static_configurations(i):
    """Static int8 on seeded random shapes (T = 0 to ~900 with ragged token
    blocks, hidden sizes that end mid column slice, 1 to 512 experts so that
    both slice widths run, duplicates and dropped entries): one
    coefficient, per-channel and per-expert scales, whole receive buffers
    (sentinels included) and row weights against the oracle."""
    rng, T, H, E, R, K, a, _, dup, drop = _random_config(500 + i)
    kind = STATIC_KINDS[i % 3]
    # every fourth case: sparse NaN and infinite elements and scales, so that
    # lanes and column slices needing the exact conversion sit beside ones
    # that do not
    nonfinite = i % 4 == 3
    print(f"[static{i}] {kind} T={T} H={H} E={E} R={R} K={K} a={a} dup={dup} drop={drop} "
          f"nonfinite={nonfinite}", flush=True)
    idx, wts = _routing(rng, T, K, E, dup, drop)
    x = W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 3).astype(np.float32))
    if nonfinite:
        m = rng.random((T, H)) < 0.002
        x[m] = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1], np.uint16)[rng.integers(0, 4, int(m.sum()))]

    def odd_scales(s):
        if nonfinite and s.size > 1:
            m = rng.random(s.shape) < 0.001
            s[m] = np.array([np.inf, np.nan, -np.inf], np.float32)[rng.integers(0, 3, int(m.sum()))]
        return s

    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    cap = ol.recv_capacity
    rx = torch.full((cap, H), 0x3C, dtype=torch.int8, device=DEV)
    rw = torch.full((cap,), -3.0, device=DEV)
    orx0 = np.full((cap, H), 0x3C, np.int8)
    if kind == "expert":
        scales = odd_scales(rng.uniform(0.5, 60.0, (E, H)).astype(np.float32))
        orx, orw = oracle.dispatch_static_expert(x, idx, ol.token_row, cap, scales, wts, recv_x=orx0,
                                                 with_weights=True)
        moe.moe_dispatch_static_per_expert(bf16_dev(x), lay, torch.from_numpy(idx).to(DEV),
                                           torch.from_numpy(scales).to(DEV), torch.from_numpy(wts).to(DEV),
                                           recv_x=rx, recv_weights=rw)
    else:
        scales = odd_scales(rng.uniform(0.5, 60.0, H if kind == "channel" else 1).astype(np.float32))
        orx, orw = oracle.dispatch_static(x, ol.token_row, cap, scales, wts, recv_x=orx0, with_weights=True)
        moe.moe_dispatch_static(bf16_dev(x), lay, torch.from_numpy(scales).to(DEV),
                                torch.from_numpy(wts).to(DEV), recv_x=rx, recv_weights=rw)
    np.testing.assert_array_equal(rx.cpu().numpy(), orx)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])
    assert (rw.cpu().numpy()[~used] == -3.0).all()


BENCH_WORKLOADS = W.WORKLOADS + W.NEXT_WORKLOADS


@pytest.mark.parametrize("w", BENCH_WORKLOADS, ids=[w.name for w in BENCH_WORKLOADS])
def test_bench_workload_full_size_sampled(w):
    """Every workload bench.py can time, at its full size and through the same
    calls and launch configuration: the whole layout against the oracle; the
    rows (codes, scales, weights) of a seeded sample of 256 tokens bit-exact;
    the combine of the sample (with the fused epilogues where the workload
    has them) within the combine bound, on seeded bf16 expert outputs."""
    T, H, K, E, R, a = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, w.expert_alignment
    print(f"[full-size] {w.name}", flush=True)
    if w.prequant:
        data, scales, idx, wts = W.generate_prequant(w)
        x_bits = None
    else:
        inp = W.generate(w)
        idx, wts, x_bits = inp.topk_idx, inp.topk_weights, inp.x_bits
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    assert_layout_equal(layout_to_host(lay), ol)
    cap = ol.recv_capacity
    w_dev = torch.from_numpy(wts).to(DEV)
    rng = np.random.default_rng(zlib.crc32(w.name.encode()))
    sample = np.sort(rng.choice(T, min(256, T), replace=False))
    rows = ol.token_row[sample]                       # [S, K], -1 where dropped
    sub_rows = np.where(rows >= 0, np.arange(rows.size, dtype=np.int32).reshape(rows.shape), -1).astype(np.int32)
    take = torch.from_numpy(np.maximum(rows, 0).reshape(-1).astype(np.int64)).to(DEV)
    valid = (rows >= 0).reshape(-1)

    if w.prequant:
        rd = torch.empty((cap, data.shape[1]), dtype=torch.uint8, device=DEV)
        rsc = torch.empty((cap, scales.shape[1]), dtype=torch.uint8, device=DEV)
        rw = torch.empty(cap, dtype=torch.float32, device=DEV)
        moe.moe_dispatch_prequantized(torch.from_numpy(data).to(DEV), torch.from_numpy(scales).to(DEV), lay,
                                      w_dev, rd, rsc, rw)
        od, osc, ow = oracle.dispatch_prequantized(data[sample], scales[sample], sub_rows, rows.size,
                                                   wts[sample], with_weights=True)
        np.testing.assert_array_equal(rd[take].cpu().numpy()[valid], od[valid])
        np.testing.assert_array_equal(rsc[take].cpu().numpy()[valid], osc[valid])
    elif w.static_per_expert:
        sc = W.expert_scales(w)
        rx = torch.empty((cap, H), dtype=torch.int8, device=DEV)
        rw = torch.empty(cap, dtype=torch.float32, device=DEV)
        moe.moe_dispatch_static_per_expert(bf16_dev(x_bits), lay, torch.from_numpy(idx).to(DEV),
                                           torch.from_numpy(sc).to(DEV), w_dev, recv_x=rx, recv_weights=rw)
        orx, ow = oracle.dispatch_static_expert(x_bits[sample], idx[sample], sub_rows, rows.size, sc,
                                                wts[sample], with_weights=True)
        np.testing.assert_array_equal(rx[take].cpu().numpy()[valid], orx[valid])
    elif w.static_scale > 0:
        sc = np.array([w.static_scale], np.float32)
        rx = torch.empty((cap, H), dtype=torch.int8, device=DEV)
        rw = torch.empty(cap, dtype=torch.float32, device=DEV)
        moe.moe_dispatch_static(bf16_dev(x_bits), lay, torch.from_numpy(sc).to(DEV), w_dev, recv_x=rx,
                                recv_weights=rw)
        orx, ow = oracle.dispatch_static(x_bits[sample], sub_rows, rows.size, sc, wts[sample], with_weights=True)
        np.testing.assert_array_equal(rx[take].cpu().numpy()[valid], orx[valid])
    else:
        rx, rs, rw = moe.allocate_recv(lay, H, w.quant_mode, with_weights=True)
        moe.moe_dispatch(bf16_dev(x_bits), lay, w_dev, w.quant_mode, recv_x=rx, recv_scales=rs, recv_weights=rw)
        orx, ors, ow = oracle.dispatch(x_bits[sample], sub_rows, rows.size, wts[sample], w.quant_mode,
                                       with_weights=True)
        np.testing.assert_array_equal(recv_to_host(rx[take], w.quant_mode)[valid], orx[valid])
        if rs is not None:
            got = rs[take].cpu().numpy()
            if got.dtype == np.float32:
                got, ors = got.view(np.uint32), ors.view(np.uint32)
            np.testing.assert_array_equal(got[valid], ors[valid])
    np.testing.assert_array_equal(rw[take].cpu().numpy()[valid], ow[valid])

    # combine on seeded expert outputs; the sample's rows gathered for the oracle
    y_sub = W.random_bf16_rows(rows.size, H, 31)
    y = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    y[take[torch.from_numpy(valid).to(DEV)]] = bf16_dev(y_sub)[torch.from_numpy(valid).to(DEV)]
    sel = torch.from_numpy(sample.astype(np.int64)).to(DEV)
    if w.epilogue:
        sh_bits, res_bits = W.random_bf16_rows(T, H, 21), W.random_bf16_rows(T, H, 22)
        gamma_bits = np.full(H, 0x3F80, np.uint16)
        out, out_norm = moe.moe_combine_fused(y, lay, w_dev, bf16_dev(sh_bits), bf16_dev(res_bits),
                                              bf16_dev(gamma_bits), 1e-6)
        exact, _ = oracle.combine_fused(y_sub, sub_rows, wts[sample], sh_bits[sample], res_bits[sample],
                                        gamma_bits, 1e-6, with_norm=True)
        S = combine_bound(y_sub, sub_rows, wts[sample], K) + np.abs(W.bf16_bits_to_f32(sh_bits[sample])) \
            + np.abs(W.bf16_bits_to_f32(res_bits[sample]))
        check_combine(bf16_host_bits(out[sel]), exact, S, K + 2, max_rel_1e2=False)
    else:
        out = moe.moe_combine(y, lay, w_dev)
        exact = oracle.combine(y_sub, sub_rows, wts[sample])
        S = combine_bound(y_sub, sub_rows, wts[sample], K)
        check_combine(bf16_host_bits(out[sel]), exact, S, K, max_rel_1e2=False)


def test_binding_rejects_mismatched_layouts():
    """A layout whose tensors do not match its sizes (truncated, wrong dtype)
    cannot be made, and calls take only layouts, so no such pointer reaches a
    kernel; the genuine layout still works."""
    import collections
    import dataclasses
    rng = np.random.default_rng(91)
    T, H, K, E, R, a = 64, 256, 4, 16, 4, 2
    idx, wts = _routing(rng, T, K, E)
    lay = gpu_layout(idx, E, R, a)
    x = bf16_dev(W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    y = torch.zeros((lay.recv_capacity, H), dtype=torch.bfloat16, device=DEV)
    for field, bad in (("token_row", lay.token_row[:-1]), ("token_row", lay.token_row.to(torch.int64)),
                       ("recv_src", lay.recv_src[:-1]), ("token_row", lay.token_row.cpu())):
        with pytest.raises((ValueError, TypeError)):
            dataclasses.replace(lay, **{field: bad})
    fake = collections.namedtuple("Fake", [f.name for f in dataclasses.fields(lay)])(
        *[getattr(lay, f.name) for f in dataclasses.fields(lay)])
    with pytest.raises(TypeError):
        moe.moe_dispatch(x, fake)
    with pytest.raises(TypeError):
        moe.moe_combine(y, fake)
    with pytest.raises(TypeError):
        moe.moe_combine_fused(y, fake)
    with pytest.raises(TypeError):
        moe.moe_get_dispatch_layout(torch.from_numpy(idx).to(DEV), E, R, a, out=fake)
    moe.moe_combine(y, lay)
    moe.moe_dispatch(x, lay)
    torch.cuda.synchronize()


def test_binding_uses_the_current_stream():
    """The stream handle passed to the library is torch's current stream:
    the default one, one set by a stream context, and for a device given
    without an index; work queued on a side stream and waited for lands."""
    dev_noindex = torch.device("cuda")
    handle = lambda d: moe._stream(d).value or 0      # the default stream's handle is 0
    assert handle(DEV) == torch.cuda.current_stream(DEV).cuda_stream
    assert handle(dev_noindex) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    rng = np.random.default_rng(93)
    T, H, K, E, R = 48, 512, 4, 16, 4
    idx, wts = _routing(rng, T, K, E)
    x = bf16_dev(W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert handle(DEV) == side.cuda_stream != 0
        lay = gpu_layout(idx, E, R, 1)
        rx, _, _ = moe.moe_dispatch(x, lay)
    torch.cuda.current_stream().wait_stream(side)
    ol = oracle.layout(idx, E, R, 1)
    assert_layout_equal(layout_to_host(lay), ol)
    orx, _, _ = oracle.dispatch(bf16_host_bits(x), ol.token_row, ol.recv_capacity)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(bf16_host_bits(rx)[used], orx[used])
