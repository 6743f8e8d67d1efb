"""Pins for the oracle's layout (counts, aligned offsets, stable rows).

The oracle's layout is a counting sort.  It is pinned here against
  * an independent, operational formulation (build the receive buffer by
    appending each expert's entries in flat order and padding the segment to
    the alignment) on every small routing pattern,
  * a hand-worked example,
  * invariants on the five measured workloads, and
  * torch's bincount and stable sort (library routines).
"""
import itertools

import numpy as np
import pytest

from combine_moe_get_dispatch_amd import workloads as W


def layout_by_appending(idx, E, R, a):
    """Receive buffer built operationally: for expert 0, 1, ... append the
    flat indices t*K+k routed to it in increasing order, then append padding
    (-1) until the segment length is a multiple of the alignment."""
    T, K = idx.shape
    L = E // R
    buf, starts = [], []
    for e in range(E):
        starts.append(len(buf))
        mine = [t * K + k for t in range(T) for k in range(K) if idx[t, k] == e]
        buf.extend(mine)
        while (len(buf) - starts[-1]) % a:
            buf.append(-1)
    starts.append(len(buf))
    row_of = {src: pos for pos, src in enumerate(buf) if src >= 0}
    token_row = np.array([[row_of.get(t * K + k, -1) for k in range(K)] for t in range(T)],
                         dtype=np.int32).reshape(T, K)
    owned = [set(range(r * L, (r + 1) * L)) for r in range(R)]
    itr = np.array([[int(any(int(idx[t, k]) in owned[r] for k in range(K))) for r in range(R)]
                    for t in range(T)], dtype=np.int32).reshape(T, R)
    per_expert = np.array([sum(1 for t in range(T) for k in range(K) if idx[t, k] == e)
                           for e in range(E)], dtype=np.int32)
    return dict(buf=buf, starts=np.array(starts, np.int32), token_row=token_row, itr=itr,
                ntpr=itr.sum(axis=0).astype(np.int32), ntpe=per_expert)


def check_against_appending(orc, idx, E, R, a):
    ref = layout_by_appending(idx, E, R, a)
    lay = orc.layout(idx, E, R, a)
    np.testing.assert_array_equal(lay.expert_offsets, ref["starts"])
    np.testing.assert_array_equal(lay.num_recv_tokens_per_expert, np.diff(ref["starts"]))
    np.testing.assert_array_equal(lay.num_tokens_per_expert, ref["ntpe"])
    np.testing.assert_array_equal(lay.token_row, ref["token_row"])
    np.testing.assert_array_equal(lay.is_token_in_rank, ref["itr"])
    np.testing.assert_array_equal(lay.num_tokens_per_rank, ref["ntpr"])
    n = len(ref["buf"])
    np.testing.assert_array_equal(lay.recv_src[:n], np.array(ref["buf"], np.int32))
    assert (lay.recv_src[n:] == -1).all()
    assert lay.error_flag == 0


def test_hand_worked_example(orc):
    # topk_idx = [[0,2],[2,-1],[1,2]], 4 experts over 2 ranks (2 local each), alignment 2.
    # entries per expert: e0 {0}, e1 {4}, e2 {1,2,5}, e3 {}  -> counts 1,1,3,0
    # aligned: 2,2,4,0 -> offsets 0,2,4,8,8; rows: (0,0)->0 (0,1)->4 (1,0)->5 (2,0)->2 (2,1)->6
    # capacity bound T*K + E*(a-1) = 6 + 4 = 10.
    idx = np.array([[0, 2], [2, -1], [1, 2]], np.int64)
    lay = orc.layout(idx, 4, 2, 2)
    assert lay.recv_capacity == 10
    assert lay.num_tokens_per_expert.tolist() == [1, 1, 3, 0]
    assert lay.num_recv_tokens_per_expert.tolist() == [2, 2, 4, 0]
    assert lay.expert_offsets.tolist() == [0, 2, 4, 8, 8]
    assert lay.token_row.tolist() == [[0, 4], [5, -1], [2, 6]]
    assert lay.recv_src.tolist() == [0, -1, 4, -1, 1, 2, 5, -1, -1, -1]
    assert lay.is_token_in_rank.tolist() == [[1, 1], [0, 1], [1, 1]]
    assert lay.num_tokens_per_rank.tolist() == [2, 3]
    assert lay.error_flag == 0


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


@pytest.mark.parametrize("E", [1, 2, 3, 4])
def test_exhaustive_small_patterns(orc, E):
    """Every routing pattern with T*K <= 4 (values -1..E-1, so duplicates and
    dropped entries included), every rank count dividing E, alignments 1..3."""
    for T, K in [(0, 1), (1, 1), (1, 2), (2, 1), (2, 2), (1, 4), (4, 1), (3, 1)]:
        for vals in itertools.product(range(-1, E), repeat=T * K):
            idx = np.array(vals, np.int64).reshape(T, K)
            for R in _divisors(E):
                for a in (1, 2, 3):
                    check_against_appending(orc, idx, E, R, a)


def test_random_small_patterns(orc):
    rng = np.random.default_rng(5)
    for _ in range(1500):
        T = int(rng.integers(1, 7))
        K = int(rng.integers(1, 5))
        E = int(rng.integers(1, 9))
        R = int(rng.choice(_divisors(E)))
        a = int(rng.integers(1, 6))
        idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
        check_against_appending(orc, idx, E, R, a)


def test_out_of_range_ids_are_flagged_and_dropped(orc):
    idx = np.array([[0, 4], [-2, 1], [3, 99]], np.int64)
    lay = orc.layout(idx, 4, 2, 1)
    assert lay.error_flag == 1
    clean = np.where((idx < -1) | (idx >= 4), -1, idx)
    ref = orc.layout(clean, 4, 2, 1)
    for a, b in zip(lay[:7], ref[:7]):
        np.testing.assert_array_equal(a, b)
    assert ref.error_flag == 0


def check_invariants(lay, idx, E, R, a):
    T, K = idx.shape
    M = T * K
    flat = idx.reshape(-1)
    valid = flat >= 0
    V = int(valid.sum())
    c = lay.num_tokens_per_expert.astype(np.int64)
    ac = lay.num_recv_tokens_per_expert.astype(np.int64)
    off = lay.expert_offsets.astype(np.int64)
    assert c.sum() == V
    assert (ac % a == 0).all() and (c <= ac).all() and (ac < c + a).all()
    assert ((c == 0) == (ac == 0)).all()
    assert off[0] == 0 and (np.diff(off) == ac).all()
    N = int(off[-1])
    assert N <= lay.recv_capacity == M + E * (a - 1)
    np.testing.assert_array_equal(lay.num_tokens_per_rank, lay.is_token_in_rank.sum(axis=0))
    L = E // R
    itr_ref = np.zeros((T, R), np.int32)
    tt = np.repeat(np.arange(T), K)
    itr_ref[tt[valid], flat[valid] // L] = 1
    np.testing.assert_array_equal(lay.is_token_in_rank, itr_ref)
    rows = lay.token_row.reshape(-1)
    assert (rows[~valid] == -1).all()
    vr = rows[valid]
    assert len(np.unique(vr)) == V
    e_of = flat[valid]
    assert (vr >= off[e_of]).all() and (vr < off[e_of] + c[e_of]).all()
    src = lay.recv_src
    np.testing.assert_array_equal(src[vr], np.nonzero(valid)[0])
    used = np.zeros(len(src), bool)
    used[vr] = True
    assert (src[~used] == -1).all()
    for e in range(E):
        seg = src[off[e]:off[e] + c[e]]
        assert (np.diff(seg) > 0).all()


@pytest.mark.parametrize("w", W.WORKLOADS, ids=[w.name for w in W.WORKLOADS])
def test_invariants_on_workloads(orc, w):
    idx, _ = W.generate_routing(w)
    lay = orc.layout(idx, w.num_experts, w.num_ranks, w.expert_alignment)
    check_invariants(lay, idx, w.num_experts, w.num_ranks, w.expert_alignment)


@pytest.mark.parametrize("w", W.WORKLOADS[:4], ids=[w.name for w in W.WORKLOADS[:4]])
def test_against_torch_bincount_and_stable_sort(orc, w):
    import torch
    idx, _ = W.generate_routing(w)
    E = w.num_experts
    lay = orc.layout(idx, E, w.num_ranks, w.expert_alignment)
    flat = torch.from_numpy(idx.reshape(-1))
    valid = flat >= 0
    counts = torch.bincount(flat[valid], minlength=E).numpy()
    np.testing.assert_array_equal(lay.num_tokens_per_expert, counts)
    # stable sort of the valid flat indices by expert id gives the row order
    vidx = torch.nonzero(valid).reshape(-1)
    _, order = torch.sort(flat[valid], stable=True)
    expect = vidx[order].numpy()
    got = np.concatenate([lay.recv_src[lay.expert_offsets[e]:lay.expert_offsets[e] + counts[e]]
                          for e in range(E)])
    np.testing.assert_array_equal(got, expect)


def test_zero_tokens(orc):
    idx = np.zeros((0, 4), np.int64)
    lay = orc.layout(idx, 8, 2, 4)
    assert lay.recv_capacity == 8 * 3
    assert (lay.num_tokens_per_expert == 0).all() and (lay.expert_offsets == 0).all()
    assert (lay.num_tokens_per_rank == 0).all() and (lay.recv_src == -1).all()


def test_all_dropped(orc):
    idx = -np.ones((5, 3), np.int64)
    lay = orc.layout(idx, 6, 3, 2)
    assert (lay.token_row == -1).all() and (lay.expert_offsets == 0).all()
    assert (lay.is_token_in_rank == 0).all() and (lay.recv_src == -1).all()


def test_deterministic(orc):
    idx, _ = W.generate_routing(W.WORKLOADS[2])
    a = orc.layout(idx, 256, 16, 128)
    b = orc.layout(idx, 256, 16, 128)
    for x, y in zip(a[:7], b[:7]):
        np.testing.assert_array_equal(x, y)
