"""Helpers shared by the GPU tests: run the HIP path through the C ABI binding
and compare it with the oracle on the same seeded inputs."""
import os

import numpy as np
import torch


import oracle
import combine_moe_get_dispatch_amd as moe
from combine_moe_get_dispatch_amd import build_lib
from combine_moe_get_dispatch_amd import workloads as W

if not os.path.exists(moe.LIB_PATH):      # build only when nothing is built
    build_lib.build(verbose=True)
elif build_lib.is_stale():
    print(f"warning: {moe.LIB_PATH} is older than a source or header it is built from; "
          "the GPU tests run the library as built", flush=True)

DEV = torch.device("cuda", 0)

PER_TOKEN = (2, 0x12, 0x22)
PER_GROUP = (0x13, 0x23)
MX = (4, 0x24)
E5M2 = (0x22, 0x24, 0x23)


def sentinel(quant):
    return 0xFFFF if quant == 0 else (0x55 if quant == 2 else 0x7F)   # bf16 NaN / int8 85 / fp8 NaN


def scale_sentinel(quant):
    return -7.0 if quant in PER_TOKEN + PER_GROUP else 0xFF


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_layout(idx: np.ndarray, E: int, R: int, a: int, cap=None):
    lay = moe.moe_get_dispatch_layout(torch.from_numpy(idx).to(DEV), E, R, a, recv_capacity=cap)
    return lay


def layout_to_host(lay):
    return dict(
        num_tokens_per_rank=lay.num_tokens_per_rank.cpu().numpy(),
        num_tokens_per_expert=lay.num_tokens_per_expert.cpu().numpy(),
        is_token_in_rank=lay.is_token_in_rank.cpu().numpy(),
        num_recv_tokens_per_expert=lay.num_recv_tokens_per_expert.cpu().numpy(),
        expert_offsets=lay.expert_offsets.cpu().numpy(),
        token_row=lay.token_row.cpu().numpy(),
        recv_src=lay.recv_src.cpu().numpy(),
        error_flag=int(lay.error_flag.cpu().numpy()[0]),
    )


def assert_layout_equal(gl, ol):
    for name in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                 "num_recv_tokens_per_expert", "expert_offsets", "token_row", "recv_src"):
        np.testing.assert_array_equal(gl[name], getattr(ol, name), err_msg=name)
    assert gl["error_flag"] == ol.error_flag


def poisoned_recv(lay, H, quant):
    """Receive buffers pre-filled with a sentinel, so that stray or missing
    writes show."""
    rx, rs, rw = moe.allocate_recv(lay, H, quant, with_weights=True)
    if quant == 0:
        rx.view(torch.int16).fill_(np.int16(np.uint16(sentinel(0)).view(np.int16)))
    else:
        rx.view(torch.uint8).fill_(sentinel(quant))
    if rs is not None:
        rs.fill_(scale_sentinel(quant))
    rw.fill_(-3.0)
    return rx, rs, rw


def oracle_poisoned(cap, H, quant):
    if quant == 0:
        return np.full((cap, H), sentinel(0), np.uint16), None
    rx = np.full((cap, H), sentinel(quant), np.int8 if quant == 2 else np.uint8)
    if quant in PER_TOKEN:
        rs = np.full(cap, scale_sentinel(quant), np.float32)
    elif quant in PER_GROUP:
        rs = np.full((cap, (H + 127) // 128), scale_sentinel(quant), np.float32)
    else:
        rs = np.full((cap, H // 32), scale_sentinel(quant), np.uint8)
    return rx, rs


def recv_to_host(rx, quant):
    if quant == 0:
        return bf16_host_bits(rx)
    if quant == 2:
        return rx.cpu().numpy()
    return rx.view(torch.uint8).cpu().numpy()


def dequant_identity_expert(rx_host: np.ndarray, rs_host, quant: int) -> np.ndarray:
    """The identity expert for quantised rows: bf16(decode(codes) * scale),
    computed on the CPU with torch (test harness, not part of the path)."""
    if quant == 0:
        return rx_host
    if quant == 2:
        codes = torch.from_numpy(rx_host.astype(np.float32))
    else:
        fp8 = torch.float8_e5m2 if quant in E5M2 else torch.float8_e4m3fn
        codes = torch.from_numpy(rx_host).view(fp8).float()
    if quant in PER_TOKEN:
        y = codes * torch.from_numpy(rs_host)[:, None]
    elif quant in PER_GROUP:
        cap, H = rx_host.shape
        per_elem = torch.from_numpy(rs_host).repeat_interleave(128, dim=1)[:, :H]
        y = codes * per_elem
    else:
        cap, H = rx_host.shape
        sc = torch.from_numpy(rs_host.astype(np.float32) - 127.0)
        y = (codes.view(cap, H // 32, 32) * torch.exp2(sc)[:, :, None]).view(cap, H)
    y = torch.nan_to_num(y, nan=0.0, posinf=0.0, neginf=0.0)   # padding rows hold sentinels
    return y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def combine_bound(y_bits, token_row, w, K):
    """|gpu - exact| <= 2^-8 |exact| + (K+1) 2^-24 sum_k |w y|: one bf16
    rounding (2^-9 relative, doubled for margin) on top of an fp32 fma chain
    of K terms."""
    y_abs = (y_bits & np.uint16(0x7FFF)).astype(np.uint16)
    w_abs = None if w is None else np.abs(w).astype(np.float32)
    S = oracle.combine(y_abs, token_row, w_abs)
    return S


def check_combine(g_bits: np.ndarray, exact: np.ndarray, S: np.ndarray, K: int, max_rel_1e2=True):
    g = W.bf16_bits_to_f32(g_bits).astype(np.float64)
    err = np.abs(g - exact)
    bound = 2.0 ** -8 * np.abs(exact) + (K + 1) * 2.0 ** -24 * S
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} elements exceed the bound; worst {err[bad].max()}"
    zero = exact == 0
    assert (g[zero] == 0).all()
    if max_rel_1e2:
        nz = ~zero
        rel = np.max(err[nz] / np.abs(exact[nz])) if nz.any() else 0.0
        assert rel <= 1e-2, rel
        return float(rel)
    return None
