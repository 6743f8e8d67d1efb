"""MoE token dispatch / combine on one AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libmoe_dispatch_combine.so``
(declared in ``include/moe_dispatch_combine.h``).  The three calls keep the
C names:

    layout = moe_get_dispatch_layout(topk_idx, num_experts, num_ranks, expert_alignment)
    recv_x, recv_scales, recv_weights = moe_dispatch(x, layout, topk_weights, quant_mode)
    out = moe_combine(expert_out, layout, topk_weights)

This module only checks tensor metadata and passes device pointers and
torch's current HIP stream to the library; every step of the path runs in
the library's HIP kernels.  There is no CPU fallback: if the library is not
built, the first call raises.  torch is used for device memory and streams.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_dispatch_combine.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_CAPACITY = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 8 << 20

QUANT_NONE = 0
QUANT_INT8_PER_TOKEN = 2
QUANT_MXFP8_E4M3 = 4
QUANT_FP8_E4M3_PER_TOKEN = 0x12
QUANT_FP8_E5M2_PER_TOKEN = 0x22
QUANT_MXFP8_E5M2 = 0x24
QUANT_FP8_E4M3_PER_GROUP = 0x13
QUANT_FP8_E5M2_PER_GROUP = 0x23
QUANT_GROUP = 128
PER_GROUP_MODES = (QUANT_FP8_E4M3_PER_GROUP, QUANT_FP8_E5M2_PER_GROUP)
PER_TOKEN_SCALE_MODES = (QUANT_INT8_PER_TOKEN, QUANT_FP8_E4M3_PER_TOKEN, QUANT_FP8_E5M2_PER_TOKEN)
MX_MODES = (QUANT_MXFP8_E4M3, QUANT_MXFP8_E5M2)

FLAG_BAD_EXPERT_ID = 1

__all__ = [
    "moe_get_dispatch_layout", "moe_get_dispatch_layout_noalloc", "moe_dispatch", "moe_dispatch_static", "moe_dispatch_static_per_expert",
    "moe_dispatch_prequantized",
    "moe_combine", "moe_combine_fused",
    "moe_recv_capacity_bound",
    "moe_layout_workspace_bytes", "DispatchLayout", "allocate_layout", "allocate_recv",
    "num_recv_tokens_per_expert_list", "MoeError", "lib",
    "QUANT_NONE", "QUANT_INT8_PER_TOKEN", "QUANT_MXFP8_E4M3", "QUANT_FP8_E4M3_PER_TOKEN",
    "QUANT_FP8_E5M2_PER_TOKEN", "QUANT_MXFP8_E5M2", "QUANT_FP8_E4M3_PER_GROUP",
    "QUANT_FP8_E5M2_PER_GROUP",
]


class MoeError(RuntimeError):
    def __init__(self, func: str, code: int):
        msg = lib().moe_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def declare_signatures(L: ctypes.CDLL) -> ctypes.CDLL:
    """Give the C ABI's functions their argument and result types on a loaded
    copy of the library."""
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.moe_recv_capacity_bound.argtypes = [i32, i32, i32, i32]
    L.moe_recv_capacity_bound.restype = i64
    L.moe_layout_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.moe_layout_workspace_bytes.restype = sz
    L.moe_get_dispatch_layout.argtypes = [P, i32, i32, i32, i32, i32, i64] + [P] * 8 + [P, sz, P]
    L.moe_get_dispatch_layout.restype = i32
    L.moe_dispatch.argtypes = [P, i32, i32, i32, P, P, i64, i32, P, P, P, P]
    L.moe_dispatch.restype = i32
    L.moe_dispatch_static.argtypes = [P, i32, i32, i32, P, P, i64, P, i32, P, P, P]
    L.moe_dispatch_static.restype = i32
    L.moe_get_dispatch_layout_noalloc.argtypes = [P, i32, i32, i32, i32, i32, i64] + [P] * 8 + [P]
    L.moe_get_dispatch_layout_noalloc.restype = i32
    L.moe_dispatch_static_per_expert.argtypes = [P, i32, i32, i32, P, i32, P, P, i64, P, P, P, P]
    L.moe_dispatch_static_per_expert.restype = i32
    L.moe_dispatch_prequantized.argtypes = [P, i32, i32, P, i32, i32, P, P, i64, P, P, P, P]
    L.moe_dispatch_prequantized.restype = i32
    L.moe_combine.argtypes = [P, i64, i32, i32, i32, P, P, P, P]
    L.moe_combine.restype = i32
    L.moe_combine_fused.argtypes = [P, i64, i32, i32, i32, P, P, P, P, P, ctypes.c_float, P, P, P]
    L.moe_combine_fused.restype = i32
    L.moe_layout_and_dispatch_fits.argtypes = [i32, i32, i32, i32]
    L.moe_layout_and_dispatch_fits.restype = i32
    L.moe_layout_and_dispatch.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i64, P, i32] + [P] * 8 + [P, P, P, P]
    L.moe_layout_and_dispatch.restype = i32
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    return L


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with combine_moe_get_dispatch_amd.build_lib.build() "
                "(hipcc, gfx950). There is no CPU fallback.")
        _lib = declare_signatures(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# torch's raw accessor for the current stream's handle returns the same value
# as torch.cuda.current_stream(device).cuda_stream (it honours stream
# contexts and graph capture alike) without building a Stream object: 0.08
# against 1.9 us per call, which matters for decode-sized batches, whose
# eager steps are bound by host-side launch cost.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device) -> ctypes.c_void_p:
    if _raw_stream is not None:
        index = device.index if device.index is not None else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(index))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_fields(t: torch.Tensor, name: str, dtype, shape, device):
    """Shape, dtype, contiguity and device of one layout tensor (any device
    type: a layout may be allocated on the host, calls refuse it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _validate_layout(layout):
    """Every tensor of a layout matches its sizes and sits on one device."""
    T, K, E, R, cap = (layout.num_tokens, layout.num_topk, layout.num_experts, layout.num_ranks,
                       layout.recv_capacity)
    if min(T, K, E, R, layout.expert_alignment) < 0 or cap < 0:
        raise ValueError("layout sizes must be non-negative")
    dev = layout.token_row.device
    _check_fields(layout.token_row, "layout.token_row", torch.int32, (T, K), dev)
    _check_fields(layout.num_tokens_per_rank, "layout.num_tokens_per_rank", torch.int32, (R,), dev)
    _check_fields(layout.num_tokens_per_expert, "layout.num_tokens_per_expert", torch.int32, (E,), dev)
    _check_fields(layout.is_token_in_rank, "layout.is_token_in_rank", torch.int32, (T, R), dev)
    _check_fields(layout.num_recv_tokens_per_expert, "layout.num_recv_tokens_per_expert", torch.int32,
                  (E,), dev)
    _check_fields(layout.expert_offsets, "layout.expert_offsets", torch.int32, (E + 1,), dev)
    _check_fields(layout.recv_src, "layout.recv_src", torch.int32, (cap,), dev)
    _check_fields(layout.error_flag, "layout.error_flag", torch.int32, (1,), dev)
    _check_fields(layout.workspace, "layout.workspace", torch.uint8, None, dev)


def _check_layout(layout, device):
    """A call's layout: a DispatchLayout (validated when it was made) on the
    call's device."""
    if not isinstance(layout, DispatchLayout):
        raise TypeError("layout must be a DispatchLayout")
    if layout.token_row.device != device:
        raise ValueError(f"layout is on {layout.token_row.device}, expected {device}")


def moe_recv_capacity_bound(num_tokens: int, num_topk: int, num_experts: int,
                            expert_alignment: int) -> int:
    return int(lib().moe_recv_capacity_bound(num_tokens, num_topk, num_experts, expert_alignment))


def moe_layout_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int, num_ranks: int) -> int:
    return int(lib().moe_layout_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks))


@dataclasses.dataclass(frozen=True)
class DispatchLayout:
    """Outputs of moe_get_dispatch_layout; (expert_offsets, token_row,
    recv_src) plus the sizes form the handle combine needs.

    Every tensor is checked against the sizes when the layout is made (here
    or through dataclasses.replace), and the fields cannot be reassigned, so
    calls only check the layout's device.  Its tensors must not be resized
    or re-pointed in place afterwards."""
    num_tokens_per_rank: torch.Tensor          # int32 [R]
    num_tokens_per_expert: torch.Tensor        # int32 [E]
    is_token_in_rank: torch.Tensor             # int32 [T, R]
    num_recv_tokens_per_expert: torch.Tensor   # int32 [E], aligned
    expert_offsets: torch.Tensor               # int32 [E + 1]
    token_row: torch.Tensor                    # int32 [T, K]
    recv_src: torch.Tensor                     # int32 [cap]
    error_flag: torch.Tensor                   # int32 [1]
    workspace: torch.Tensor                    # uint8 [workspace bytes]
    num_tokens: int
    num_topk: int
    num_experts: int
    num_ranks: int
    expert_alignment: int
    recv_capacity: int

    def __post_init__(self):
        _validate_layout(self)
        # pointer arguments of the layout call, fixed with the tensors
        object.__setattr__(self, "_layout_ptrs", tuple(_ptr(t) for t in (
            self.num_tokens_per_rank, self.num_tokens_per_expert, self.is_token_in_rank,
            self.num_recv_tokens_per_expert, self.expert_offsets, self.token_row, self.recv_src,
            self.error_flag, self.workspace)))
        object.__setattr__(self, "_token_row_ptr", _ptr(self.token_row))


def allocate_layout(num_tokens: int, num_topk: int, num_experts: int, num_ranks: int,
                    expert_alignment: int = 1, recv_capacity: Optional[int] = None,
                    device=None) -> DispatchLayout:
    device = torch.device("cuda") if device is None else torch.device(device)
    T, K, E, R, a = num_tokens, num_topk, num_experts, num_ranks, expert_alignment
    bound = moe_recv_capacity_bound(T, K, E, a)
    if bound < 0:
        raise ValueError("invalid layout sizes")
    cap = bound if recv_capacity is None else int(recv_capacity)
    ws = moe_layout_workspace_bytes(T, K, E, R)
    i32 = dict(dtype=torch.int32, device=device)
    return DispatchLayout(
        torch.empty(R, **i32), torch.empty(E, **i32), torch.empty((T, R), **i32),
        torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty((T, K), **i32),
        torch.empty(max(cap, 0), **i32), torch.empty(1, **i32),
        torch.empty(max(ws, 1), dtype=torch.uint8, device=device),
        T, K, E, R, a, cap)


def moe_get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                            expert_alignment: int = 1, recv_capacity: Optional[int] = None,
                            out: Optional[DispatchLayout] = None) -> DispatchLayout:
    """Counts, aligned expert offsets and stable expert-grouped rows for
    ``topk_idx`` (int64 [T, K], -1 = no expert)."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    T, K = topk_idx.shape
    _check(topk_idx, "topk_idx", torch.int64)
    if out is None:
        out = allocate_layout(T, K, num_experts, num_ranks, expert_alignment, recv_capacity,
                              topk_idx.device)
    elif (out.num_tokens, out.num_topk, out.num_experts, out.num_ranks, out.expert_alignment) != (
            T, K, num_experts, num_ranks, expert_alignment):
        raise ValueError("preallocated layout was made for other sizes")
    _check_layout(out, topk_idx.device)
    rc = lib().moe_get_dispatch_layout(
        _ptr(topk_idx), T, K, num_experts, num_ranks, expert_alignment, out.recv_capacity,
        *out._layout_ptrs, out.workspace.numel(), _stream(topk_idx.device))
    if rc != MOE_OK:
        raise MoeError("moe_get_dispatch_layout", rc)
    return out


def moe_get_dispatch_layout_noalloc(topk_idx: torch.Tensor, out: DispatchLayout) -> DispatchLayout:
    """moe_get_dispatch_layout into the preallocated ``out`` with the
    library's built-in scratch instead of ``out.workspace``: the call
    allocates nothing (for graph capture and allocation-free loops).  Calls
    that overlap on one GPU share that scratch and must not run at the same
    time.  Sizes needing more than NOALLOC_SCRATCH_BYTES of workspace raise."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    T, K = topk_idx.shape
    _check(topk_idx, "topk_idx", torch.int64)
    if (out.num_tokens, out.num_topk) != (T, K):
        raise ValueError("preallocated layout was made for other sizes")
    _check_layout(out, topk_idx.device)
    rc = lib().moe_get_dispatch_layout_noalloc(
        _ptr(topk_idx), T, K, out.num_experts, out.num_ranks, out.expert_alignment, out.recv_capacity,
        *out._layout_ptrs[:8], _stream(topk_idx.device))
    if rc != MOE_OK:
        raise MoeError("moe_get_dispatch_layout_noalloc", rc)
    return out


def num_recv_tokens_per_expert_list(layout: DispatchLayout) -> list:
    """Aligned rows per expert as a host list (waits for the GPU)."""
    return layout.num_recv_tokens_per_expert.cpu().tolist()


_RECV_DTYPE = {QUANT_NONE: torch.bfloat16, QUANT_INT8_PER_TOKEN: torch.int8,
               QUANT_MXFP8_E4M3: torch.float8_e4m3fn, QUANT_FP8_E4M3_PER_TOKEN: torch.float8_e4m3fn,
               QUANT_FP8_E5M2_PER_TOKEN: torch.float8_e5m2, QUANT_MXFP8_E5M2: torch.float8_e5m2,
               QUANT_FP8_E4M3_PER_GROUP: torch.float8_e4m3fn, QUANT_FP8_E5M2_PER_GROUP: torch.float8_e5m2}


def allocate_recv(layout: DispatchLayout, hidden: int, quant_mode: int = QUANT_NONE,
                  with_weights: bool = False):
    """Receive buffers for ``quant_mode``: rows [cap, H] of the mode's element
    type, scales fp32 [cap] (per-token modes), fp32 [cap, ceil(H/128)]
    (per-group modes), uint8 e8m0 [cap, H/32] (MX modes) or None (bf16),
    optional fp32 row weights [cap]."""
    dev = layout.token_row.device
    cap = layout.recv_capacity
    if quant_mode not in _RECV_DTYPE:
        raise ValueError(f"unsupported quant_mode {quant_mode}")
    rx = torch.empty((cap, hidden), dtype=_RECV_DTYPE[quant_mode], device=dev)
    if quant_mode in PER_TOKEN_SCALE_MODES:
        rs = torch.empty(cap, dtype=torch.float32, device=dev)
    elif quant_mode in MX_MODES:
        rs = torch.empty((cap, hidden // 32), dtype=torch.uint8, device=dev)
    elif quant_mode in PER_GROUP_MODES:
        rs = torch.empty((cap, (hidden + QUANT_GROUP - 1) // QUANT_GROUP), dtype=torch.float32,
                         device=dev)
    else:
        rs = None
    rw = torch.empty(cap, dtype=torch.float32, device=dev) if with_weights else None
    return rx, rs, rw


def moe_dispatch(x: torch.Tensor, layout: DispatchLayout, topk_weights: Optional[torch.Tensor] = None,
                 quant_mode: int = QUANT_NONE, recv_x: Optional[torch.Tensor] = None,
                 recv_scales: Optional[torch.Tensor] = None,
                 recv_weights: Optional[torch.Tensor] = None, with_weights: bool = False):
    """Copy (and optionally quantise) every token of ``x`` (bf16 [T, H]) into
    its experts' rows.  Returns (recv_x, recv_scales, recv_weights)."""
    T, K, cap = layout.num_tokens, layout.num_topk, layout.recv_capacity
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError(f"x must be [{T}, hidden]")
    H = x.shape[1]
    dev = x.device
    _check_layout(layout, dev)
    _check(x, "x", torch.bfloat16, device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if quant_mode not in _RECV_DTYPE:
        raise ValueError(f"unsupported quant_mode {quant_mode}")
    if recv_x is None:
        recv_x, rs, rw = allocate_recv(layout, H, quant_mode, with_weights and recv_weights is None)
        recv_scales = rs if recv_scales is None else recv_scales
        recv_weights = rw if recv_weights is None else recv_weights
    _check(recv_x, "recv_x", _RECV_DTYPE[quant_mode], (cap, H), dev)
    if quant_mode in PER_TOKEN_SCALE_MODES:
        _check(recv_scales, "recv_scales", torch.float32, (cap,), dev)
    elif quant_mode in MX_MODES:
        _check(recv_scales, "recv_scales", torch.uint8, (cap, H // 32), dev)
    elif quant_mode in PER_GROUP_MODES:
        _check(recv_scales, "recv_scales", torch.float32,
               (cap, (H + QUANT_GROUP - 1) // QUANT_GROUP), dev)
    if recv_weights is not None:
        _check(recv_weights, "recv_weights", torch.float32, (cap,), dev)
    rc = lib().moe_dispatch(_ptr(x), T, H, K, layout._token_row_ptr, _ptr(topk_weights), cap,
                            quant_mode, _ptr(recv_x), _ptr(recv_scales), _ptr(recv_weights),
                            _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_dispatch", rc)
    return recv_x, recv_scales, recv_weights


def moe_layout_and_dispatch_fits(num_tokens: int, hidden: int, num_topk: int, num_ranks: int) -> bool:
    return bool(lib().moe_layout_and_dispatch_fits(num_tokens, hidden, num_topk, num_ranks))


ONE_LAUNCH_MODES = (QUANT_NONE, QUANT_INT8_PER_TOKEN, QUANT_FP8_E4M3_PER_TOKEN, QUANT_FP8_E5M2_PER_TOKEN)


def moe_layout_and_dispatch(topk_idx: torch.Tensor, x: torch.Tensor, num_experts: int, num_ranks: int,
                            expert_alignment: int = 1, topk_weights: Optional[torch.Tensor] = None,
                            recv_capacity: Optional[int] = None, quant_mode: int = QUANT_NONE,
                            out: Optional[DispatchLayout] = None, recv_x: Optional[torch.Tensor] = None,
                            recv_scales: Optional[torch.Tensor] = None,
                            recv_weights: Optional[torch.Tensor] = None, with_weights: bool = False):
    """moe_get_dispatch_layout and moe_dispatch: in one launch when the batch
    is decode-sized (moe_layout_and_dispatch_fits) and ``quant_mode`` is
    bf16 or a per-token mode, else as the two calls; the results are the
    same either way.  Returns (layout, recv_x, recv_scales, recv_weights)."""
    if topk_idx.dim() != 2 or x.dim() != 2 or x.shape[0] != topk_idx.shape[0]:
        raise ValueError("topk_idx must be [num_tokens, num_topk] and x [num_tokens, hidden]")
    T, K = topk_idx.shape
    H = x.shape[1]
    if quant_mode not in ONE_LAUNCH_MODES or not moe_layout_and_dispatch_fits(T, H, K, num_ranks):
        lay = moe_get_dispatch_layout(topk_idx, num_experts, num_ranks, expert_alignment, recv_capacity,
                                      out)
        rx, rs, rw = moe_dispatch(x, lay, topk_weights, quant_mode, recv_x=recv_x, recv_scales=recv_scales,
                                  recv_weights=recv_weights, with_weights=with_weights)
        return lay, rx, rs, rw
    dev = topk_idx.device
    _check(topk_idx, "topk_idx", torch.int64)
    _check(x, "x", torch.bfloat16, device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if out is None:
        out = allocate_layout(T, K, num_experts, num_ranks, expert_alignment, recv_capacity, dev)
    elif (out.num_tokens, out.num_topk, out.num_experts, out.num_ranks, out.expert_alignment) != (
            T, K, num_experts, num_ranks, expert_alignment):
        raise ValueError("preallocated layout was made for other sizes")
    _check_layout(out, dev)
    cap = out.recv_capacity
    if recv_x is None:
        recv_x = torch.empty((cap, H), dtype=_RECV_DTYPE[quant_mode], device=dev)
    _check(recv_x, "recv_x", _RECV_DTYPE[quant_mode], (cap, H), dev)
    if quant_mode != QUANT_NONE:
        if recv_scales is None:
            recv_scales = torch.empty(cap, dtype=torch.float32, device=dev)
        _check(recv_scales, "recv_scales", torch.float32, (cap,), dev)
    if recv_weights is None and with_weights:
        recv_weights = torch.empty(cap, dtype=torch.float32, device=dev)
    if recv_weights is not None:
        _check(recv_weights, "recv_weights", torch.float32, (cap,), dev)
    rc = lib().moe_layout_and_dispatch(
        _ptr(topk_idx), _ptr(x), T, H, K, num_experts, num_ranks, expert_alignment, cap,
        _ptr(topk_weights), quant_mode, *out._layout_ptrs[:8], _ptr(recv_x),
        _ptr(recv_scales if quant_mode != QUANT_NONE else None), _ptr(recv_weights), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_layout_and_dispatch", rc)
    return out, recv_x, recv_scales if quant_mode != QUANT_NONE else None, recv_weights


def moe_dispatch_static(x: torch.Tensor, layout: DispatchLayout, scales: torch.Tensor,
                        topk_weights: Optional[torch.Tensor] = None,
                        recv_x: Optional[torch.Tensor] = None,
                        recv_weights: Optional[torch.Tensor] = None, with_weights: bool = False):
    """Static int8 quantisation with the caller's fp32 scales (1 value, or H
    per-channel values) and dispatch.  Returns (recv_x int8 [cap, H], recv_weights)."""
    T, K, cap = layout.num_tokens, layout.num_topk, layout.recv_capacity
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError(f"x must be [{T}, hidden]")
    H = x.shape[1]
    dev = x.device
    _check_layout(layout, dev)
    _check(x, "x", torch.bfloat16, device=dev)
    _check(scales, "scales", torch.float32, device=dev)
    if scales.numel() not in (1, H):
        raise ValueError("scales must hold 1 or hidden values")
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if recv_x is None:
        recv_x = torch.empty((cap, H), dtype=torch.int8, device=dev)
    if recv_weights is None and with_weights:
        recv_weights = torch.empty(cap, dtype=torch.float32, device=dev)
    _check(recv_x, "recv_x", torch.int8, (cap, H), dev)
    if recv_weights is not None:
        _check(recv_weights, "recv_weights", torch.float32, (cap,), dev)
    rc = lib().moe_dispatch_static(_ptr(x), T, H, K, layout._token_row_ptr, _ptr(topk_weights),
                                   cap, _ptr(scales), scales.numel(), _ptr(recv_x),
                                   _ptr(recv_weights), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_dispatch_static", rc)
    return recv_x, recv_weights


def moe_dispatch_static_per_expert(x: torch.Tensor, layout: DispatchLayout, topk_idx: torch.Tensor,
                                   scales: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                                   recv_x: Optional[torch.Tensor] = None,
                                   recv_weights: Optional[torch.Tensor] = None,
                                   with_weights: bool = False):
    """Static int8 quantisation with one fp32 scale row per expert (scales
    [num_experts, H]) and dispatch: each copy of a token is quantised with
    the row of the expert it goes to.  ``topk_idx`` is the int64 [T, K] the
    layout was made from.  Returns (recv_x int8 [cap, H], recv_weights)."""
    T, K, E, cap = layout.num_tokens, layout.num_topk, layout.num_experts, layout.recv_capacity
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError(f"x must be [{T}, hidden]")
    H = x.shape[1]
    dev = x.device
    _check_layout(layout, dev)
    _check(x, "x", torch.bfloat16, device=dev)
    _check(topk_idx, "topk_idx", torch.int64, (T, K), dev)
    _check(scales, "scales", torch.float32, (E, H), dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if recv_x is None:
        recv_x = torch.empty((cap, H), dtype=torch.int8, device=dev)
    if recv_weights is None and with_weights:
        recv_weights = torch.empty(cap, dtype=torch.float32, device=dev)
    _check(recv_x, "recv_x", torch.int8, (cap, H), dev)
    if recv_weights is not None:
        _check(recv_weights, "recv_weights", torch.float32, (cap,), dev)
    rc = lib().moe_dispatch_static_per_expert(_ptr(x), T, H, K, _ptr(topk_idx), E, layout._token_row_ptr,
                                              _ptr(topk_weights), cap, _ptr(scales), _ptr(recv_x),
                                              _ptr(recv_weights), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_dispatch_static_per_expert", rc)
    return recv_x, recv_weights


def _bytes2d(t: torch.Tensor, name: str, rows: int, dev) -> torch.Tensor:
    if t.device != dev or t.dim() != 2 or t.shape[0] != rows or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [{rows}, n] tensor on {dev}")
    return t.view(torch.uint8)


def moe_dispatch_prequantized(data: torch.Tensor, scales: Optional[torch.Tensor],
                              layout: DispatchLayout, topk_weights: Optional[torch.Tensor] = None,
                              recv_data: Optional[torch.Tensor] = None,
                              recv_scales: Optional[torch.Tensor] = None,
                              recv_weights: Optional[torch.Tensor] = None,
                              with_weights: bool = False):
    """Copy pre-quantised tokens -- the (data, scale) tuple input of MXFP8 /
    MXFP4 dispatch: data [T, H] float8 or [T, H/2] packed float4, scales
    [T, H/32] e8m0 bytes -- unchanged into their experts' rows.  Any element
    dtype is accepted; rows are moved as bytes.  Returns (recv_data,
    recv_scales, recv_weights) with the input dtypes."""
    T, K, cap = layout.num_tokens, layout.num_topk, layout.recv_capacity
    dev = data.device
    _check_layout(layout, dev)
    if dev.type != "cuda":
        raise ValueError("data must be on a HIP device")
    d8 = _bytes2d(data, "data", T, dev)
    row_bytes = d8.shape[1]
    s8 = None if scales is None else _bytes2d(scales, "scales", T, dev)
    scale_bytes = 0 if s8 is None else s8.shape[1]
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if recv_data is None:
        recv_data = torch.empty((cap,) + tuple(data.shape[1:]), dtype=data.dtype, device=dev)
    if recv_scales is None and scales is not None:
        recv_scales = torch.empty((cap,) + tuple(scales.shape[1:]), dtype=scales.dtype, device=dev)
    if recv_weights is None and with_weights:
        recv_weights = torch.empty(cap, dtype=torch.float32, device=dev)
    rd8 = _bytes2d(recv_data, "recv_data", cap, dev)
    rs8 = None if recv_scales is None else _bytes2d(recv_scales, "recv_scales", cap, dev)
    if rd8.shape[1] != row_bytes or (rs8 is not None and rs8.shape[1] != scale_bytes):
        raise ValueError("receive buffers do not match the row sizes of the input")
    if recv_weights is not None:
        _check(recv_weights, "recv_weights", torch.float32, (cap,), dev)
    rc = lib().moe_dispatch_prequantized(_ptr(d8), T, row_bytes, _ptr(s8), scale_bytes, K,
                                         layout._token_row_ptr, _ptr(topk_weights), cap,
                                         _ptr(rd8), _ptr(rs8), _ptr(recv_weights), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_dispatch_prequantized", rc)
    return recv_data, recv_scales, recv_weights


def moe_combine(expert_out: torch.Tensor, layout: DispatchLayout,
                topk_weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = bf16(sum_k w[t,k] * expert_out[row(t,k)]), fp32 accumulation."""
    T, K, cap = layout.num_tokens, layout.num_topk, layout.recv_capacity
    if expert_out.dim() != 2 or expert_out.shape[0] != cap:
        raise ValueError(f"expert_out must be [{cap}, hidden]")
    H = expert_out.shape[1]
    dev = expert_out.device
    _check_layout(layout, dev)
    _check(expert_out, "expert_out", torch.bfloat16, device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, H), dev)
    rc = lib().moe_combine(_ptr(expert_out), cap, T, H, K, layout._token_row_ptr,
                           _ptr(topk_weights), _ptr(out), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_combine", rc)
    return out


def moe_combine_fused(expert_out: torch.Tensor, layout: DispatchLayout,
                      topk_weights: Optional[torch.Tensor] = None,
                      shared_out: Optional[torch.Tensor] = None,
                      residual: Optional[torch.Tensor] = None,
                      rms_weight: Optional[torch.Tensor] = None, rms_eps: float = 1e-6,
                      out: Optional[torch.Tensor] = None, out_norm: Optional[torch.Tensor] = None,
                      with_norm: bool = False):
    """Combine plus epilogues: out = sum_k w y (+ shared_out) (+ residual);
    out_norm = RMSNorm(out) * rms_weight when rms_weight is given.
    Returns (out, out_norm)."""
    T, K, cap = layout.num_tokens, layout.num_topk, layout.recv_capacity
    if expert_out.dim() != 2 or expert_out.shape[0] != cap:
        raise ValueError(f"expert_out must be [{cap}, hidden]")
    H = expert_out.shape[1]
    dev = expert_out.device
    _check_layout(layout, dev)
    _check(expert_out, "expert_out", torch.bfloat16, device=dev)
    if topk_weights is not None:
        _check(topk_weights, "topk_weights", torch.float32, (T, K), dev)
    for name, t_ in (("shared_out", shared_out), ("residual", residual)):
        if t_ is not None:
            _check(t_, name, torch.bfloat16, (T, H), dev)
    want_norm = with_norm or out_norm is not None
    if want_norm:
        if rms_weight is None:
            raise ValueError("rms_weight is required for the normalised output")
        _check(rms_weight, "rms_weight", torch.bfloat16, (H,), dev)
        if out_norm is None:
            out_norm = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _check(out_norm, "out_norm", torch.bfloat16, (T, H), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (T, H), dev)
    rc = lib().moe_combine_fused(_ptr(expert_out), cap, T, H, K, layout._token_row_ptr,
                                 _ptr(topk_weights), _ptr(shared_out), _ptr(residual),
                                 _ptr(rms_weight if want_norm else None), float(rms_eps), _ptr(out),
                                 _ptr(out_norm if want_norm else None), _stream(dev))
    if rc != MOE_OK:
        raise MoeError("moe_combine_fused", rc)
    return out, out_norm
