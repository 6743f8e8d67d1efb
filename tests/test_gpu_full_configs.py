"""GPU parity on every element of the five reference configurations, at their
full sizes and through the calls bench.py times:

  128 x 1024, 16 experts / 4 ranks, top-2, bf16;
  4096 x 7168, 256 experts / 8 ranks, top-8, bf16;
  8192 x 7168, 256 experts / 16 ranks, top-8 Zipf, alignment 128, int8 per token;
  8192 x 4096, 128 experts / 8 ranks, top-8 with 10 % dropped entries,
      alignment 32, MXFP8 e4m3fn;
  32768 x 7168, 512 experts / 64 ranks, top-16, alignment 128, bf16.

The whole layout is compared at once.  Rows, codes, scales and row weights are
compared in token blocks: the oracle dispatches a block's tokens into a
compact buffer (one row per valid entry, in (token, k) order), and the GPU
rows those entries were given are gathered and compared bit for bit, so that
host memory stays bounded (the largest receive buffer is 8.45 GB).  Combine
then runs once over all tokens with identity experts (the rows themselves,
or their bf16 dequantised values), and every output element is held to the
combine bound and to a maximum relative error of 1e-2 against the oracle's
fp64 sum.
"""
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
                          recv_to_host)

ENTRIES_PER_BLOCK = 16384   # routing entries compared per block (235 MB of bf16 rows at H = 7168)


def _host_scales(rs, take):
    if rs is None:
        return None
    got = rs[take].cpu().numpy()
    return got


@pytest.mark.parametrize("w", W.WORKLOADS[:5], ids=lambda w: w.name)
def test_config_every_element(w):
    T, H, K, E, R, a, q = (w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                           w.expert_alignment, w.quant_mode)
    print(f"[every-element] {w.name}: {w.describe()}", flush=True)
    inp = W.generate(w)
    idx, wts, x_bits = inp.topk_idx, inp.topk_weights, inp.x_bits
    ol = oracle.layout(idx, E, R, a)
    lay = gpu_layout(idx, E, R, a)
    assert_layout_equal(layout_to_host(lay), ol)
    cap = ol.recv_capacity

    w_dev = torch.from_numpy(wts).to(DEV)
    rx, rs, rw = moe.allocate_recv(lay, H, q, with_weights=True)
    moe.moe_dispatch(bf16_dev(x_bits), lay, w_dev, q, recv_x=rx, recv_scales=rs, recv_weights=rw)
    y = rx if q == 0 else torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    out_h = bf16_host_bits(moe.moe_combine(rx, lay, w_dev)) if q == 0 else None

    bt = max(1, ENTRIES_PER_BLOCK // K)
    kept = []          # quantised configs: (token slice, compact rows, expert outputs) per block
    worst = 0.0
    n_rows = 0
    for t0 in range(0, T, bt):
        tb = slice(t0, min(T, t0 + bt))
        rows = ol.token_row[tb]
        valid = (rows >= 0).reshape(-1)
        sub_rows = np.where(rows >= 0, np.arange(rows.size, dtype=np.int32).reshape(rows.shape),
                            -1).astype(np.int32)
        take = torch.from_numpy(np.maximum(rows, 0).reshape(-1).astype(np.int64)).to(DEV)
        orx, ors, ow = oracle.dispatch(x_bits[tb], sub_rows, rows.size, wts[tb], q, with_weights=True)
        g = recv_to_host(rx[take], q)
        np.testing.assert_array_equal(g[valid], orx[valid], err_msg=f"rows of tokens {t0}..")
        gs = _host_scales(rs, take)
        if gs is not None:
            if gs.dtype == np.float32:
                np.testing.assert_array_equal(gs[valid].view(np.uint32), ors[valid].view(np.uint32))
            else:
                np.testing.assert_array_equal(gs[valid], ors[valid])
        np.testing.assert_array_equal(rw[take].cpu().numpy()[valid], ow[valid])
        n_rows += int(valid.sum())

        if q == 0:
            exact = oracle.combine(orx, sub_rows, wts[tb])
            S = combine_bound(orx, sub_rows, wts[tb], K)
            worst = max(worst, check_combine(out_h[tb], exact, S, K, max_rel_1e2=True))
        else:
            # identity experts: bf16 of the dequantised rows, the oracle's from
            # its own rows, the GPU's from the (equal) rows it produced
            y_or = dequant_identity_expert(orx, ors, q)
            y_g = dequant_identity_expert(g, gs, q)
            vt = torch.from_numpy(valid).to(DEV)
            y[take[vt]] = bf16_dev(y_g)[vt]
            kept.append((tb, sub_rows, y_or))
    assert n_rows == int((ol.token_row >= 0).sum())

    if q != 0:
        out_h = bf16_host_bits(moe.moe_combine(y, lay, w_dev))
        for tb, sub_rows, y_or in kept:
            exact = oracle.combine(y_or, sub_rows, wts[tb])
            S = combine_bound(y_or, sub_rows, wts[tb], K)
            worst = max(worst, check_combine(out_h[tb], exact, S, K, max_rel_1e2=True))
    torch.cuda.synchronize()
    print(f"[every-element] {w.name}: {n_rows} rows bit-exact, combine max relative error {worst:.3e}",
          flush=True)
