"""GPU parity for the dynamic quantisers with the maximum at every position.

A row's (or group's, or block's) maximum decides its scale, so a reduction
that misses one lane, one element of a lane's vector or the tail of a row
would change the codes only when the maximum sits there, which random rows
rarely arrange.  Here row p holds its unique largest magnitude at position
p, for every position of the row: with H = 7168 (one 16-byte vector per lane
of an 896-lane workgroup) and H = 16384 (two vectors per lane), every lane,
every element of its vectors and every block and group slot holds a row
maximum once.  Codes and scales must match the oracle bit for bit, through
the library's dispatch, for every dynamic quantisation mode.
"""
import functools

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe
    from gpu_util import DEV, bf16_dev, gpu_layout, recv_to_host

MODES = [(2, "int8"), (0x12, "fp8_e4m3_per_token"), (0x22, "fp8_e5m2_per_token"),
         (0x13, "fp8_e4m3_per_group"), (0x23, "fp8_e5m2_per_group"), (4, "mxfp8_e4m3"),
         (0x24, "mxfp8_e5m2")]


@functools.lru_cache(maxsize=2)
def _rows(H):
    """[H, H] bf16 bits: row p is uniform in (-4, 4) with +-5 at position p
    (bf16 by dropping the low 16 bits of each fp32 value; 5 is exact)."""
    rng = np.random.default_rng(H)
    v = rng.random((H, H), dtype=np.float32)
    v *= np.float32(8.0)
    v -= np.float32(4.0)
    r = np.arange(H)
    v[r, r] = np.where(r % 2 == 0, 5.0, -5.0)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("H", [7168, 16384])
@pytest.mark.parametrize("quant,name", MODES, ids=[n for _, n in MODES])
def test_dynamic_quant_row_maximum_at_every_position(quant, name, H):
    print(f"[max-positions] {name} H={H} rows={H}", flush=True)
    x_bits = _rows(H)
    T, K, E, R = H, 1, 8, 2
    idx = (np.arange(T, dtype=np.int64) % E).reshape(T, K)
    ol = oracle.layout(idx, E, R, 1)
    lay = gpu_layout(idx, E, R, 1)
    rx, rs, _ = moe.moe_dispatch(bf16_dev(x_bits), lay, None, quant)
    orx, ors, _ = oracle.dispatch(x_bits, ol.token_row, ol.recv_capacity, None, quant)
    np.testing.assert_array_equal(recv_to_host(rx, quant), orx)
    got = rs.cpu().numpy()
    if got.dtype == np.float32:
        got, ors = got.view(np.uint32), ors.view(np.uint32)
    np.testing.assert_array_equal(got, ors)
    torch.cuda.synchronize()
