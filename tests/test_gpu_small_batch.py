"""GPU parity of the one-launch layout + dispatch for decode-sized batches
(moe_layout_and_dispatch: bf16 rows, or per-token int8 / FP8 e4m3fn / e5m2
codes and scales) against the oracle, and against the two-call form on the
same inputs.

Bar: every layout output bit-exact; every valid receive row, code and scale
bit-exact; rows no entry names keep the sentinel they were filled with; row
weights bit-exact.  Seeded random shapes cover T = 0, single tokens, the limits
(3072 entries, 16384 token x rank cells, 512 tokens, hidden 8192), one
expert, duplicated and dropped entries, out-of-range ids, alignment and a
capacity above the bound.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_get_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe
    from gpu_util import (DEV, assert_layout_equal, bf16_dev, bf16_host_bits, gpu_layout,
                          layout_to_host, oracle_poisoned, recv_to_host, scale_sentinel, sentinel)

MODES = [0, 2, 0x12, 0x22]   # bf16, int8 / e4m3fn / e5m2 per token


def _config(i):
    rng = np.random.default_rng(7000 + i)
    E = int(rng.choice([1, 2, 3, 8, 12, 64, 96, 256, 512]))
    R = int(rng.choice([r for r in (1, 2, 3, 4, 8, 16, 32, 64) if E % r == 0]))
    K = int(rng.integers(1, 17))
    T = int(rng.choice([0, 1, 2, 7, 63, 64, 65, 128, 200, 384, 512]))
    while T * K > 3072 or T * R > 16384:
        T //= 2
    H = 32 * int(rng.choice([1, 3, 32, 100, 224, 256]))
    a = int(rng.choice([1, 2, 7, 32, 128]))
    dup = bool(rng.random() < 0.3)
    drop = float(rng.choice([0.0, 0.0, 0.3, 1.0]))
    bad_ids = bool(rng.random() < 0.15)
    extra_cap = int(rng.choice([0, 0, 5]))
    weights = bool(rng.random() < 0.7)
    quant = MODES[i % len(MODES)]
    return rng, T, H, E, R, K, a, dup, drop, bad_ids, extra_cap, weights, quant


def _routing(rng, T, K, E, dup, drop, bad_ids):
    if dup or K > E:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    if drop > 0:
        idx[rng.random((T, K)) < drop] = -1
    if bad_ids and T * K > 0:
        m = rng.random((T, K)) < 0.05
        idx[m] = rng.choice([E, E + 3, -2])
    wts = rng.random((T, K)).astype(np.float32)
    return idx, wts


def _run(T, H, E, R, K, a, idx, wts, extra_cap, weights, rng, quant=0):
    x_bits = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    ol = oracle.layout(idx, E, R, a, recv_capacity=oracle.recv_capacity_bound(T, K, E, a) + extra_cap)
    cap = ol.recv_capacity
    assert moe.moe_layout_and_dispatch_fits(T, H, K, R)
    lay = moe.allocate_layout(T, K, E, R, a, cap, DEV)
    rx, rs, _ = moe.allocate_recv(lay, H, quant)
    if quant == 0:
        rx.view(torch.int16).fill_(np.int16(np.uint16(sentinel(0)).view(np.int16)))
    else:
        rx.view(torch.uint8).fill_(sentinel(quant))
        rs.fill_(scale_sentinel(quant))
    rw = torch.full((cap,), -3.0, dtype=torch.float32, device=DEV)
    w_dev = torch.from_numpy(wts).to(DEV) if weights else None
    moe.moe_layout_and_dispatch(torch.from_numpy(idx).to(DEV), bf16_dev(x_bits), E, R, a, w_dev, cap,
                                quant, out=lay, recv_x=rx, recv_scales=rs, recv_weights=rw)
    assert_layout_equal(layout_to_host(lay), ol)
    orx, ors = oracle_poisoned(cap, H, quant)
    orx, ors, orw = oracle.dispatch(x_bits, ol.token_row, cap, wts if weights else None, quant,
                                    recv_x=orx, recv_scales=ors, with_weights=True)
    np.testing.assert_array_equal(recv_to_host(rx, quant), orx)
    if quant != 0:
        np.testing.assert_array_equal(rs.cpu().numpy().view(np.uint32), ors.view(np.uint32))
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(rw.cpu().numpy()[used], orw[used])
    assert (rw.cpu().numpy()[~used] == -3.0).all()


@pytest.mark.parametrize("i", range(120), ids=[f"cfg{i}" for i in range(120)])
def test_layout_and_dispatch_random(i):
    rng, T, H, E, R, K, a, dup, drop, bad_ids, extra_cap, weights, quant = _config(i)
    print(f"[small cfg{i}] T={T} H={H} E={E} R={R} K={K} a={a} dup={dup} drop={drop} bad={bad_ids} "
          f"extra_cap={extra_cap} weights={weights} quant={quant:#x}", flush=True)
    idx, wts = _routing(rng, T, K, E, dup, drop, bad_ids)
    _run(T, H, E, R, K, a, idx, wts, extra_cap, weights, rng, quant)


@pytest.mark.parametrize("quant", MODES)
@pytest.mark.parametrize("T,H,E,R,K", [(384, 64, 256, 8, 8),      # 3072 entries
                                       (512, 32, 64, 32, 6),      # 512 tokens, 16384 cells
                                       (128, 8192, 256, 8, 8),    # largest hidden size
                                       (128, 7168, 256, 8, 8),    # the decode workload's shape
                                       (3, 7168, 1, 1, 16)])      # one expert, every entry on it
def test_layout_and_dispatch_limits(T, H, E, R, K, quant):
    print(f"[small limits] T={T} H={H} E={E} R={R} K={K} quant={quant:#x}", flush=True)
    rng = np.random.default_rng(T + H + K)
    idx, wts = _routing(rng, T, K, E, dup=E < K, drop=0.1, bad_ids=False)
    _run(T, H, E, R, K, 1, idx, wts, 0, True, rng, quant)


@pytest.mark.parametrize("quant", MODES[1:])
def test_layout_and_dispatch_quant_row_maximum_everywhere(quant):
    """Per-token codes with each row's maximum at a different position: row t
    holds it in lane t (512 lanes of a 4096-wide row), at element t % 8 of
    the lane's vector, so every lane and every element slot holds one."""
    rng = np.random.default_rng(79 + quant)
    T, H, E, R, K = 512, 4096, 64, 8, 4
    v = rng.uniform(-4.0, 4.0, (T, H)).astype(np.float32)
    pos = np.arange(T) * 8 + np.arange(T) % 8
    v[np.arange(T), pos] = np.where(np.arange(T) % 2 == 0, 5.0, -5.0)
    x_bits = W.f32_to_bf16_bits(v)
    idx, _ = _routing(rng, T, K, E, dup=False, drop=0.0, bad_ids=False)
    lay, rx, rs, _ = moe.moe_layout_and_dispatch(torch.from_numpy(idx).to(DEV), bf16_dev(x_bits), E, R, 1,
                                                 quant_mode=quant)
    ol = oracle.layout(idx, E, R, 1)
    orx, ors, _ = oracle.dispatch(x_bits, ol.token_row, ol.recv_capacity, None, quant)
    used = ol.recv_src >= 0
    np.testing.assert_array_equal(recv_to_host(rx, quant)[used], orx[used])
    np.testing.assert_array_equal(rs.cpu().numpy()[used].view(np.uint32), ors[used].view(np.uint32))


def test_layout_and_dispatch_equals_two_calls():
    """The one-launch path and the two calls write identical outputs, and the
    binding falls back to the two calls for a batch that does not fit."""
    rng = np.random.default_rng(77)
    for T, H, quant in ((128, 7168, 0), (128, 7168, 0x12), (600, 256, 0), (64, 256, 4)):
        E, R, K, a = 256, 8, 4, 7
        idx, wts = _routing(rng, T, K, E, dup=False, drop=0.1, bad_ids=False)
        x = bf16_dev(W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
        d_idx, d_w = torch.from_numpy(idx).to(DEV), torch.from_numpy(wts).to(DEV)
        lay1, rx1, rs1, rw1 = moe.moe_layout_and_dispatch(d_idx, x, E, R, a, d_w, quant_mode=quant,
                                                          with_weights=True)
        lay2 = gpu_layout(idx, E, R, a)
        rx2, rs2, rw2 = moe.moe_dispatch(x, lay2, d_w, quant, with_weights=True)
        g1, g2 = layout_to_host(lay1), layout_to_host(lay2)
        for k in g1:
            np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)
        used = torch.from_numpy(g2["recv_src"] >= 0).to(DEV)
        assert torch.equal(rx1[used].view(torch.uint8), rx2[used].view(torch.uint8))
        if quant != 0:
            assert torch.equal(rs1[used].view(torch.uint8), rs2[used].view(torch.uint8))
        assert torch.equal(rw1[used], rw2[used])
        assert moe.moe_layout_and_dispatch_fits(T, H, K, R) == (T <= 512)
    torch.cuda.synchronize()


def test_layout_and_dispatch_graph_replays_match_eager():
    """The one-launch call allocates nothing and never synchronises, so a
    step (it, then a combine) can be captured in a HIP graph.  Replay it
    several times, with eager work and synchronisations in between, against
    the eager result."""
    rng = np.random.default_rng(78)
    T, H, K, E, R, a = 128, 1024, 8, 64, 8, 4
    idx, wts = _routing(rng, T, K, E, dup=False, drop=0.05, bad_ids=False)
    idx_d = torch.from_numpy(idx).to(DEV)
    x = bf16_dev(W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    w = torch.from_numpy(wts).to(DEV)
    lay = moe.allocate_layout(T, K, E, R, a, device=DEV)
    rx = torch.empty((lay.recv_capacity, H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.moe_layout_and_dispatch(idx_d, x, E, R, a, None, out=lay, recv_x=rx)
        moe.moe_combine(rx, lay, w, out=out)

    def snapshot():
        torch.cuda.synchronize()
        used = lay.recv_src >= 0
        return (lay.token_row.clone(), lay.recv_src.clone(), lay.expert_offsets.clone(),
                lay.is_token_in_rank.clone(), rx.view(torch.int16)[used].clone(), out.view(torch.int16).clone())

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
        for t_ in (lay.token_row, lay.recv_src, lay.expert_offsets, lay.is_token_in_rank, out):
            t_.fill_(7)
        rx.view(torch.int16).fill_(3)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for r_, g_ in zip(ref, got):
            assert torch.equal(r_, g_)
