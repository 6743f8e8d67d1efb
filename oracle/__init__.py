"""CPU oracle for MoE token dispatch / combine -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from the product library.

The arithmetic lives in ``moe_oracle.c`` (plain C, built with gcc); this file
only builds it, loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from collections import namedtuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_CAPACITY = -2

QUANT_NONE = 0
QUANT_INT8 = 2
QUANT_MXFP8 = 4
QUANT_FP8_E4M3_PT = 0x12
QUANT_FP8_E5M2_PT = 0x22
QUANT_MXFP8_E5M2 = 0x24
QUANT_FP8_E4M3_PG = 0x13
QUANT_FP8_E5M2_PG = 0x23
GROUP = 128
PER_GROUP_MODES = (QUANT_FP8_E4M3_PG, QUANT_FP8_E5M2_PG)
PER_TOKEN_SCALE_MODES = (QUANT_INT8, QUANT_FP8_E4M3_PT, QUANT_FP8_E5M2_PT)
MX_MODES = (QUANT_MXFP8, QUANT_MXFP8_E5M2)

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libmoe_oracle.so``."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    global _lib
    _lib = None
    return _LIB_PATH


_lib = None
_P = ctypes.c_void_p


# A prebuilt copy of this oracle to load instead of oracle/libmoe_oracle.so.
# Set only by the mutation test, which builds the oracle with one planted
# mistake and checks that the pin tests fail against it.
_OVERRIDE = os.environ.get("MOE_ORACLE_LIB_OVERRIDE")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _OVERRIDE:
            path = _OVERRIDE
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            path = _LIB_PATH
        L = ctypes.CDLL(path)
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_recv_capacity_bound.argtypes = [i32, i32, i32, i32]
        L.oracle_recv_capacity_bound.restype = i64
        L.oracle_check_layout_args.argtypes = [i32, i32, i32, i32, i32, i64]
        L.oracle_check_layout_args.restype = i32
        L.oracle_check_rows_args.argtypes = [i32, i32, i32, i64, i32]
        L.oracle_check_rows_args.restype = i32
        L.oracle_layout.argtypes = [_P, i32, i32, i32, i32, i32, i64] + [_P] * 8
        L.oracle_layout.restype = i32
        L.oracle_dispatch.argtypes = [_P, i32, i32, i32, _P, _P, i64, i32, _P, _P, _P]
        L.oracle_dispatch.restype = i32
        L.oracle_combine.argtypes = [_P, i64, i32, i32, i32, _P, _P, _P]
        L.oracle_combine.restype = i32
        L.oracle_cast_to_fp8_e4m3fn_array.argtypes = [_P, i64, _P]
        L.oracle_cast_to_fp8_e4m3fn_array.restype = None
        L.oracle_quant_int8_rows.argtypes = [_P, i32, i32, _P, _P]
        L.oracle_quant_int8_rows.restype = None
        L.oracle_quant_mxfp8_rows.argtypes = [_P, i32, i32, _P, _P]
        L.oracle_quant_mxfp8_rows.restype = None
        L.oracle_check_prequant_args.argtypes = [i32, i32, i32, i32, i64]
        L.oracle_check_prequant_args.restype = i32
        L.oracle_dispatch_prequantized.argtypes = [_P, i32, i32, _P, i32, i32, _P, _P, i64, _P, _P, _P]
        L.oracle_dispatch_prequantized.restype = i32
        L.oracle_cast_to_fp8_e5m2_array.argtypes = [_P, i64, _P]
        L.oracle_cast_to_fp8_e5m2_array.restype = None
        L.oracle_quant_mx_e5m2_rows.argtypes = [_P, i32, i32, _P, _P]
        L.oracle_quant_mx_e5m2_rows.restype = None
        L.oracle_quant_fp8_pertoken_rows.argtypes = [_P, i32, i32, i32, _P, _P]
        L.oracle_quant_fp8_pertoken_rows.restype = None
        L.oracle_check_static_args.argtypes = [i32, i32, i32, i64, i32]
        L.oracle_check_static_args.restype = i32
        L.oracle_dispatch_static.argtypes = [_P, i32, i32, i32, _P, _P, i64, _P, i32, _P, _P]
        L.oracle_dispatch_static.restype = i32
        L.oracle_quant_fp8_pergroup_rows.argtypes = [_P, i32, i32, i32, _P, _P]
        L.oracle_quant_fp8_pergroup_rows.restype = None
        L.oracle_check_static_expert_args.argtypes = [i32, i32, i32, i32, i64]
        L.oracle_check_static_expert_args.restype = i32
        L.oracle_dispatch_static_expert.argtypes = [_P, i32, i32, i32, _P, i32, _P, _P, i64, _P, _P, _P]
        L.oracle_dispatch_static_expert.restype = i32
        L.oracle_quant_static_int8_rows.argtypes = [_P, i32, i32, _P, i32, _P]
        L.oracle_quant_static_int8_rows.restype = None
        L.oracle_combine_fused.argtypes = [_P, i64, i32, i32, i32, _P, _P, _P, _P, _P,
                                           ctypes.c_double, _P, _P]
        L.oracle_combine_fused.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle returned status {code}")
        self.code = code


def recv_capacity_bound(T: int, K: int, E: int, a: int) -> int:
    return int(lib().oracle_recv_capacity_bound(T, K, E, a))


def check_layout_args(T, K, E, R, a, cap) -> int:
    return int(lib().oracle_check_layout_args(T, K, E, R, a, cap))


def check_rows_args(T, H, K, cap, quant_mode) -> int:
    return int(lib().oracle_check_rows_args(T, H, K, cap, quant_mode))


Layout = namedtuple("Layout", [
    "num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
    "num_recv_tokens_per_expert", "expert_offsets", "token_row", "recv_src",
    "error_flag", "recv_capacity"])


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int, expert_alignment: int = 1,
           recv_capacity: int | None = None) -> Layout:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    E, R, a = num_experts, num_ranks, expert_alignment
    cap = recv_capacity_bound(T, K, E, a) if recv_capacity is None else recv_capacity
    ntpr = np.zeros(R, np.int32)
    ntpe = np.zeros(E, np.int32)
    itr = np.zeros((T, R), np.int32)
    nrtpe = np.zeros(E, np.int32)
    off = np.zeros(E + 1, np.int32)
    row = np.zeros((T, K), np.int32)
    src = np.zeros(max(cap, 0), np.int32)
    flag = np.zeros(1, np.int32)
    rc = lib().oracle_layout(_ptr(idx), T, K, E, R, a, cap, _ptr(ntpr), _ptr(ntpe), _ptr(itr),
                             _ptr(nrtpe), _ptr(off), _ptr(row), _ptr(src), _ptr(flag))
    if rc != OK:
        raise OracleError(rc)
    return Layout(ntpr, ntpe, itr, nrtpe, off, row, src, int(flag[0]), cap)


def dispatch(x_bits: np.ndarray, token_row: np.ndarray, recv_capacity: int,
             topk_weights: np.ndarray | None = None, quant_mode: int = QUANT_NONE,
             recv_x: np.ndarray | None = None, recv_scales: np.ndarray | None = None,
             with_weights: bool = False):
    """Returns (recv_x, recv_scales, recv_weights).  Buffers may be passed in
    pre-filled with a sentinel; rows that hold no entry are left untouched."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    K = row.shape[1]
    cap = recv_capacity
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    if recv_x is None:
        dt = np.uint16 if quant_mode == QUANT_NONE else (np.int8 if quant_mode == QUANT_INT8 else np.uint8)
        recv_x = np.zeros((cap, H), dt)
    if recv_scales is None:
        if quant_mode in PER_TOKEN_SCALE_MODES:
            recv_scales = np.zeros(cap, np.float32)
        elif quant_mode in MX_MODES:
            recv_scales = np.zeros((cap, H // 32), np.uint8)
        elif quant_mode in PER_GROUP_MODES:
            recv_scales = np.zeros((cap, (H + GROUP - 1) // GROUP), np.float32)
    recv_w = np.zeros(cap, np.float32) if with_weights else None
    rc = lib().oracle_dispatch(_ptr(x), T, H, K, _ptr(row), _ptr(w), cap, quant_mode,
                               _ptr(recv_x), _ptr(recv_scales), _ptr(recv_w))
    if rc != OK:
        raise OracleError(rc)
    return recv_x, recv_scales, recv_w


def check_static_args(T, H, K, cap, num_scales) -> int:
    return int(lib().oracle_check_static_args(T, H, K, cap, num_scales))


def dispatch_static(x_bits, token_row, recv_capacity, scales, topk_weights=None, recv_x=None,
                    with_weights=False):
    """Static int8 quantisation (scales: 1 or H fp32 values).  Returns (recv_x, recv_weights)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    K = row.shape[1]
    sc = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    if recv_x is None:
        recv_x = np.zeros((recv_capacity, H), np.int8)
    recv_w = np.zeros(recv_capacity, np.float32) if with_weights else None
    rc = lib().oracle_dispatch_static(_ptr(x), T, H, K, _ptr(row), _ptr(w), recv_capacity,
                                      _ptr(sc), sc.size, _ptr(recv_x), _ptr(recv_w))
    if rc != OK:
        raise OracleError(rc)
    return recv_x, recv_w


def check_static_expert_args(T, H, K, E, cap) -> int:
    return int(lib().oracle_check_static_expert_args(T, H, K, E, cap))


def dispatch_static_expert(x_bits, topk_idx, token_row, recv_capacity, scales, topk_weights=None,
                           recv_x=None, with_weights=False):
    """Static int8 quantisation with one fp32 scale row per expert (scales
    [E, H]): each entry's copy is quantised with its expert's row.  Returns
    (recv_x int8 [cap, H], recv_weights or None)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    K = row.shape[1] if row.ndim == 2 else 1
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    if sc.ndim != 2 or sc.shape[1] != H:
        raise ValueError("scales must be [num_experts, hidden]")
    E = sc.shape[0]
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    if recv_x is None:
        recv_x = np.zeros((recv_capacity, H), np.int8)
    recv_w = np.zeros(recv_capacity, np.float32) if with_weights else None
    rc = lib().oracle_dispatch_static_expert(_ptr(x), T, H, K, _ptr(idx), E, _ptr(row), _ptr(w),
                                             recv_capacity, _ptr(sc), _ptr(recv_x), _ptr(recv_w))
    if rc != OK:
        raise OracleError(rc)
    return recv_x, recv_w


def quant_fp8_pergroup_rows(x_bits: np.ndarray, fmt: str = "e4m3"):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros((T, (H + GROUP - 1) // GROUP), np.float32)
    lib().oracle_quant_fp8_pergroup_rows(_ptr(x), T, H, {"e4m3": 1, "e5m2": 2}[fmt], _ptr(q), _ptr(s))
    return q, s


def quant_static_int8_rows(x_bits: np.ndarray, scales):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    sc = np.ascontiguousarray(scales, dtype=np.float32).reshape(-1)
    q = np.zeros((T, H), np.int8)
    lib().oracle_quant_static_int8_rows(_ptr(x), T, H, _ptr(sc), sc.size, _ptr(q))
    return q


def check_prequant_args(T, row_bytes, scale_bytes, K, cap) -> int:
    return int(lib().oracle_check_prequant_args(T, row_bytes, scale_bytes, K, cap))


def dispatch_prequantized(data: np.ndarray, scales, token_row: np.ndarray, recv_capacity: int,
                          topk_weights=None, recv_data=None, recv_scales=None, with_weights=False):
    """Copy pre-quantised rows (data [T, row_bytes] and scales [T, scale_bytes],
    any byte dtype) to their layout rows.  Returns (recv_data, recv_scales, recv_weights)."""
    d = np.ascontiguousarray(data).view(np.uint8)
    T, row_bytes = d.shape
    if scales is None:
        sc, scale_bytes = None, 0
    else:
        sc = np.ascontiguousarray(scales).view(np.uint8)
        scale_bytes = sc.shape[1]
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    K = row.shape[1]
    cap = recv_capacity
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    if recv_data is None:
        recv_data = np.zeros((cap, row_bytes), np.uint8)
    if recv_scales is None and scale_bytes:
        recv_scales = np.zeros((cap, scale_bytes), np.uint8)
    recv_w = np.zeros(cap, np.float32) if with_weights else None
    rc = lib().oracle_dispatch_prequantized(_ptr(d), T, row_bytes, _ptr(sc), scale_bytes, K,
                                            _ptr(row), _ptr(w), cap, _ptr(recv_data),
                                            _ptr(recv_scales), _ptr(recv_w))
    if rc != OK:
        raise OracleError(rc)
    return recv_data, recv_scales, recv_w


def combine(y_bits: np.ndarray, token_row: np.ndarray, topk_weights: np.ndarray | None = None) -> np.ndarray:
    """fp64 weighted sum [T, H]."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    cap, H = y.shape
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    T, K = row.shape
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    out = np.zeros((T, H), np.float64)
    rc = lib().oracle_combine(_ptr(y), cap, T, H, K, _ptr(row), _ptr(w), _ptr(out))
    if rc != OK:
        raise OracleError(rc)
    return out


def combine_fused(y_bits, token_row, topk_weights=None, shared=None, residual=None, gamma=None,
                  eps: float = 1e-6, with_norm: bool = False):
    """fp64 (out, norm): out = weighted sum + shared + residual; norm = RMSNorm(out) * gamma."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    cap, H = y.shape
    row = np.ascontiguousarray(token_row, dtype=np.int32)
    T, K = row.shape
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    sh = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint16)
    rs = None if residual is None else np.ascontiguousarray(residual, dtype=np.uint16)
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.uint16)
    out = np.zeros((T, H), np.float64)
    norm = np.zeros((T, H), np.float64) if with_norm else None
    rc = lib().oracle_combine_fused(_ptr(y), cap, T, H, K, _ptr(row), _ptr(w), _ptr(sh), _ptr(rs),
                                    _ptr(g), float(eps), _ptr(out), _ptr(norm))
    if rc != OK:
        raise OracleError(rc)
    return out, norm


def cast_to_fp8_e4m3fn(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().oracle_cast_to_fp8_e4m3fn_array(_ptr(v), v.size, _ptr(out))
    return out


def cast_to_fp8_e5m2(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().oracle_cast_to_fp8_e5m2_array(_ptr(v), v.size, _ptr(out))
    return out


def quant_mx_e5m2_rows(x_bits: np.ndarray):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros((T, H // 32), np.uint8)
    lib().oracle_quant_mx_e5m2_rows(_ptr(x), T, H, _ptr(q), _ptr(s))
    return q, s


def quant_fp8_pertoken_rows(x_bits: np.ndarray, fmt: str = "e4m3"):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros(T, np.float32)
    lib().oracle_quant_fp8_pertoken_rows(_ptr(x), T, H, {"e4m3": 1, "e5m2": 2}[fmt], _ptr(q), _ptr(s))
    return q, s


def quant_int8_rows(x_bits: np.ndarray):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.int8)
    s = np.zeros(T, np.float32)
    lib().oracle_quant_int8_rows(_ptr(x), T, H, _ptr(q), _ptr(s))
    return q, s


def quant_mxfp8_rows(x_bits: np.ndarray):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    s = np.zeros((T, H // 32), np.uint8)
    lib().oracle_quant_mxfp8_rows(_ptr(x), T, H, _ptr(q), _ptr(s))
    return q, s


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the OpenMP loops of dispatch and combine use from now on."""
    lib().oracle_set_num_threads(int(n))
