"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-side argument checks agree with the oracle's rules.
No kernel is launched here: every call below fails validation (or is a pure
host query) before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dispatch_combine.h")


@pytest.fixture(scope="module")
def L():
    from combine_moe_get_dispatch_amd import build_lib
    if build_lib.is_stale():
        build_lib.build(verbose=False)
    import combine_moe_get_dispatch_amd as m
    return m.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("moe_get_dispatch_layout", "moe_dispatch", "moe_combine",
              "moe_layout_workspace_bytes", "moe_recv_capacity_bound", "moe_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from combine_moe_get_dispatch_amd import LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(L, n)


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c11", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-x", "c", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_capacity_and_workspace_queries(L, orc):
    for args in [(4096, 8, 256, 1), (8192, 8, 256, 128), (32768, 16, 512, 128), (0, 4, 8, 4),
                 (-1, 4, 8, 4), (8, 0, 8, 1), (8, 2, 8, 0)]:
        assert L.moe_recv_capacity_bound(*args) == orc.recv_capacity_bound(*args)
    assert L.moe_layout_workspace_bytes(0, 8, 256, 8) == 0
    assert L.moe_layout_workspace_bytes(4096, 8, 256, 7) == 0
    ws = L.moe_layout_workspace_bytes(4096, 8, 256, 8)
    assert 0 < ws < 1 << 20 and ws % 4 == 0


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(L.moe_status_string(code), bytes)
    assert b"scratch" in L.moe_status_string(-5)


def test_noalloc_layout_host_rules(L, orc):
    """moe_get_dispatch_layout_noalloc: the layout's argument rules, and sizes
    whose workspace exceeds the built-in scratch rejected on the host."""
    import combine_moe_get_dispatch_amd as m
    f = L.moe_get_dispatch_layout_noalloc

    def call(T, K, E, R, a=1, cap=None, outs=None):
        cap = orc.recv_capacity_bound(T, K, E, a) if cap is None else cap
        outs = [BAD] * 8 if outs is None else outs
        return f(BAD, T, K, E, R, a, cap, *outs, None)

    assert L.moe_layout_workspace_bytes(65536, 16, 512, 512) > m.NOALLOC_SCRATCH_BYTES
    assert call(65536, 16, 512, 512) == m.MOE_ERR_SCRATCH
    assert L.moe_layout_workspace_bytes(32768, 16, 512, 512) <= m.NOALLOC_SCRATCH_BYTES
    assert call(100, 17, 16, 4) == -1                      # K
    assert call(100, 4, 16, 3) == -1                       # ranks do not divide experts
    assert call(100, 4, 16, 4, cap=10) == -2               # capacity below the bound
    assert call(100, 4, 16, 4, outs=[None] + [BAD] * 7) == -1
    assert call(100, 4, 16, 4, outs=[BAD] * 6 + [None, BAD]) == -1


def test_noalloc_layout_source_allocates_nothing():
    """The no-allocation entry point and its scratch lookup call no allocating
    HIP routine (the whole C-ABI file holds none)."""
    src = open(os.path.join(ROOT, "combine_moe_get_dispatch_amd", "csrc", "moe_api.hip")).read()
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", src, flags=re.S)
    for name in ("hipMalloc", "hipFree", "hipHostMalloc", "hipMallocAsync", "hipMallocManaged",
                 "hipExtMallocWithFlags", "malloc(", "new "):
        assert name not in code, name
    assert "hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))" in code


BAD = ctypes.c_void_p(0x1000)   # never dereferenced: every call below is rejected on the host


def _layout_call(L, T, K, E, R, a, cap, ptrs=True, ws=BAD, ws_bytes=1 << 30):
    p = BAD if ptrs else None
    return L.moe_get_dispatch_layout(p, T, K, E, R, a, cap, p, p, p, p, p, p, p, p, ws, ws_bytes, None)


LAYOUT_CASES = [
    (8, 0, 4, 2, 1), (8, 17, 4, 2, 1), (8, 2, 513, 1, 1), (8, 2, 0, 1, 1), (8, 2, 6, 4, 1),
    (8, 2, 6, 7, 1), (8, 2, 6, 0, 1), (8, 2, 6, 3, 0), (-1, 2, 6, 3, 1),
]


@pytest.mark.parametrize("T,K,E,R,a", LAYOUT_CASES)
def test_layout_rejects_like_the_oracle(L, orc, T, K, E, R, a):
    cap = max(orc.recv_capacity_bound(T, K, max(E, 1), max(a, 1)), 0)
    expect = orc.check_layout_args(T, K, E, R, a, cap)
    assert expect != 0
    assert _layout_call(L, T, K, E, R, a, cap) == expect


def test_layout_capacity_errors(L, orc):
    bound = orc.recv_capacity_bound(100, 4, 16, 8)
    assert _layout_call(L, 100, 4, 16, 4, 8, bound - 1) == -2 == orc.check_layout_args(100, 4, 16, 4, 8, bound - 1)
    assert _layout_call(L, 100, 4, 16, 4, 8, 1 << 31) == orc.check_layout_args(100, 4, 16, 4, 8, 1 << 31)
    assert _layout_call(L, 1 << 28, 16, 16, 4, 8, 1 << 31) == -1


def test_layout_rejects_null_outputs_and_small_workspace(L):
    cap = 100 * 4 + 16 * 7
    assert _layout_call(L, 100, 4, 16, 4, 8, cap, ptrs=False) == -1
    # a batch too large for the one-workgroup layout needs the count table
    T = 3000
    cap = T * 4 + 16 * 7
    need = L.moe_layout_workspace_bytes(T, 4, 16, 4)
    assert need > 0
    assert _layout_call(L, T, 4, 16, 4, 8, cap, ws=None) == -3
    assert _layout_call(L, T, 4, 16, 4, 8, cap, ws_bytes=need - 1) == -3
    assert _layout_call(L, T, 4, 16, 4, 8, cap, ws=ctypes.c_void_p(0x1008)) == -3   # misaligned


def test_scan_layout_workspace(L):
    # many ranks force small chunks; from 131072 count-table cells on the layout
    # adds a column scan, whose prefix table and totals live in the workspace
    K, E, R, Ep = 2, 512, 512, 512
    assert L.moe_layout_workspace_bytes(8192, K, E, R) == 4 * (256 * (Ep + R + 1) + 256 * Ep + Ep)
    assert L.moe_layout_workspace_bytes(8160, K, E, R) == 4 * 255 * (Ep + R + 1)


def test_small_batches_need_no_workspace(L):
    # one workgroup takes the whole batch when T*K <= 3072 and T*R <= 16384
    assert L.moe_layout_workspace_bytes(384, 8, 256, 8) == 0
    assert L.moe_layout_workspace_bytes(3072, 1, 64, 4) == 0
    assert L.moe_layout_workspace_bytes(385, 8, 256, 8) > 0
    assert L.moe_layout_workspace_bytes(512, 8, 256, 8) > 0
    assert L.moe_layout_workspace_bytes(1024, 2, 512, 32) > 0     # T*R > 16384


ROWS_CASES = [(16, 48, 4, 0), (16, 16, 4, 0), (16, 16416, 4, 0), (16, 1024, 4, 1), (16, 1024, 4, 3),
              (16, 1024, 0, 0), (16, 1024, 17, 0), (-1, 1024, 4, 0), (16, 1024, 4, 5)]


@pytest.mark.parametrize("T,H,K,q", ROWS_CASES)
def test_dispatch_and_combine_reject_like_the_oracle(L, orc, T, H, K, q):
    expect = orc.check_rows_args(T, H, K, 1000, q)
    assert expect != 0
    assert L.moe_dispatch(BAD, T, H, K, BAD, BAD, 1000, q, BAD, BAD, BAD, None) == expect
    if q == 0:
        assert L.moe_combine(BAD, 1000, T, H, K, BAD, BAD, BAD, None) == expect


def test_dispatch_pointer_rules(L):
    assert L.moe_dispatch(None, 4, 64, 2, BAD, None, 100, 0, BAD, None, None, None) == -1
    assert L.moe_dispatch(ctypes.c_void_p(0x1008), 4, 64, 2, BAD, None, 100, 0, BAD, None, None, None) == -1
    assert L.moe_dispatch(BAD, 4, 64, 2, BAD, None, 100, 2, BAD, None, None, None) == -1
    assert L.moe_dispatch(None, 0, 64, 2, None, None, 100, 0, None, None, None, None) == 0
    assert L.moe_combine(BAD, 100, 4, 64, 2, BAD, None, ctypes.c_void_p(0x1004), None) == -1
    assert L.moe_combine(None, 100, 0, 64, 2, None, None, None, None) == 0


@pytest.mark.parametrize("q", [0x14, 0x32, 0x42, 0x33, 6])
def test_unknown_quant_modes_rejected(L, orc, q):
    assert orc.check_rows_args(16, 1024, 4, 1000, q) == -1
    assert L.moe_dispatch(BAD, 16, 1024, 4, BAD, BAD, 1000, q, BAD, BAD, BAD, None) == -1


PREQUANT_CASES = [(4, 8, 1, 2, 10), (4, 24, 1, 2, 10), (4, 32784, 0, 2, 10), (4, 32, 4097, 2, 10),
                  (4, 32, -1, 2, 10), (4, 32, 1, 0, 10), (4, 32, 1, 17, 10), (-1, 32, 1, 2, 10),
                  (4, 32, 1, 2, -1)]


@pytest.mark.parametrize("T,rb,sb,K,cap", PREQUANT_CASES)
def test_prequantized_rejects_like_the_oracle(L, orc, T, rb, sb, K, cap):
    expect = orc.check_prequant_args(T, rb, sb, K, cap)
    assert expect != 0
    assert L.moe_dispatch_prequantized(BAD, T, rb, BAD, sb, K, BAD, None, cap, BAD, BAD, None, None) == expect


def test_prequantized_pointer_rules(L):
    f = L.moe_dispatch_prequantized
    assert f(None, 4, 64, BAD, 2, 2, BAD, None, 100, BAD, BAD, None, None) == -1
    assert f(ctypes.c_void_p(0x1008), 4, 64, BAD, 2, 2, BAD, None, 100, BAD, BAD, None, None) == -1
    assert f(BAD, 4, 64, None, 2, 2, BAD, None, 100, BAD, BAD, None, None) == -1
    assert f(BAD, 4, 64, BAD, 2, 2, BAD, None, 100, BAD, None, None, None) == -1
    assert f(None, 0, 64, None, 2, 2, None, None, 100, None, None, None, None) == 0


@pytest.mark.parametrize("n", [0, 2, 1023, 1025])
def test_static_rejects_like_the_oracle(L, orc, n):
    expect = orc.check_static_args(16, 1024, 4, 1000, n)
    assert expect == -1
    assert L.moe_dispatch_static(BAD, 16, 1024, 4, BAD, None, 1000, BAD, n, BAD, None, None) == -1


def test_static_pointer_rules(L):
    f = L.moe_dispatch_static
    assert f(BAD, 16, 1024, 4, BAD, None, 1000, None, 1, BAD, None, None) == -1
    assert f(BAD, 16, 1024, 4, BAD, None, 1000, ctypes.c_void_p(0x1004), 1024, BAD, None, None) == -1
    assert f(BAD, 16, 48, 4, BAD, None, 1000, BAD, 1, BAD, None, None) == -1
    assert f(None, 0, 1024, 4, None, None, 1000, None, 1, None, None, None) == 0


@pytest.mark.parametrize("E", [0, 513])
def test_static_per_expert_rejects_like_the_oracle(L, orc, E):
    assert orc.check_static_expert_args(16, 1024, 4, E, 1000) == -1
    assert L.moe_dispatch_static_per_expert(BAD, 16, 1024, 4, BAD, E, BAD, None, 1000, BAD, BAD, None,
                                            None) == -1


def test_static_per_expert_pointer_rules(L):
    f = L.moe_dispatch_static_per_expert
    assert f(BAD, 16, 1024, 4, None, 8, BAD, None, 1000, BAD, BAD, None, None) == -1    # ids missing
    assert f(BAD, 16, 1024, 4, BAD, 8, BAD, None, 1000, None, BAD, None, None) == -1    # scales missing
    assert f(BAD, 16, 1024, 4, BAD, 8, None, None, 1000, BAD, BAD, None, None) == -1    # token_row missing
    assert f(BAD, 16, 1024, 4, BAD, 8, BAD, None, 1000, ctypes.c_void_p(0x1004), BAD, None, None) == -1
    assert f(BAD, 16, 1024, 4, ctypes.c_void_p(0x1004), 8, BAD, None, 1000, BAD, BAD, None, None) == -1
    assert f(BAD, 16, 1024, 4, BAD, 8, BAD, None, 1000, BAD, BAD, ctypes.c_void_p(0x1002), None) == -1
    assert f(BAD, 16, 48, 4, BAD, 8, BAD, None, 1000, BAD, BAD, None, None) == -1        # H % 32
    assert f(BAD, 16, 1024, 17, BAD, 8, BAD, None, 1000, BAD, BAD, None, None) == -1     # K
    assert f(None, 0, 1024, 4, None, 8, None, None, 1000, None, None, None, None) == 0


def test_combine_fused_rules(L):
    f = L.moe_combine_fused
    assert f(BAD, 1000, 16, 48, 4, BAD, None, None, None, None, 1e-6, BAD, None, None) == -1
    assert f(BAD, 1000, 16, 64, 4, BAD, None, None, None, None, 1e-6, BAD, BAD, None) == -1      # norm without gamma
    assert f(BAD, 1000, 16, 64, 4, BAD, None, None, None, BAD, -1.0, BAD, BAD, None) == -1       # eps < 0
    assert f(BAD, 1000, 16, 64, 4, BAD, None, None, None, BAD, float("nan"), BAD, BAD, None) == -1
    assert f(BAD, 1000, 16, 64, 4, BAD, None, ctypes.c_void_p(0x1002), None, None, 0.0, BAD, None, None) == -1
    assert f(BAD, 1000, 16, 64, 4, None, None, None, None, None, 0.0, BAD, None, None) == -1
    assert f(None, 1000, 0, 64, 4, None, None, None, None, None, 0.0, None, None, None) == 0


def test_layout_and_dispatch_limits_and_rules(L, orc):
    """The one-launch layout + dispatch: its size limits, and host-side
    rejections (nothing reaches HIP in any of these calls)."""
    assert L.moe_layout_and_dispatch_fits(512, 8192, 6, 32) == 1
    assert L.moe_layout_and_dispatch_fits(0, 32, 1, 1) == 1
    assert L.moe_layout_and_dispatch_fits(513, 1024, 1, 1) == 0      # tokens
    assert L.moe_layout_and_dispatch_fits(384, 1024, 9, 8) == 0      # 3456 entries
    assert L.moe_layout_and_dispatch_fits(512, 1024, 2, 64) == 0     # 32768 token x rank cells
    assert L.moe_layout_and_dispatch_fits(128, 8224, 8, 8) == 0      # hidden

    def call(T=128, H=7168, K=8, E=256, R=8, a=1, cap=None, idx=BAD, x=BAD, rx=BAD, outs=None, q=0, rs=BAD,
             rw=None):
        cap = orc.recv_capacity_bound(T, K, E, a) if cap is None else cap
        outs = [BAD] * 8 if outs is None else outs
        return L.moe_layout_and_dispatch(idx, x, T, H, K, E, R, a, cap, None, q, *outs, rx, rs, rw, None)

    assert call(T=600, K=1) == -1                       # beyond the one-launch limits
    assert call(H=8224) == -1
    assert call(H=100) == -1                            # not a multiple of 32
    assert call(E=255) == -1                            # ranks do not divide experts
    assert call(K=17) == -1
    assert call(cap=100) == -2                          # below the capacity bound
    assert call(x=None) == -1
    assert call(idx=None) == -1
    assert call(x=ctypes.c_void_p(0x1008)) == -1        # not 16-byte aligned
    assert call(rx=ctypes.c_void_p(0x1004)) == -1
    assert call(outs=[BAD] * 6 + [None, BAD]) == -1     # recv_src missing
    assert call(outs=[None] + [BAD] * 7) == -1          # num_tokens_per_rank missing
    for q in (4, 0x13, 0x24, 0x14, 1):                  # only bf16 and the per-token modes
        assert call(q=q) == -1
    assert call(q=2, rs=None) == -1                     # per-token scales missing
    assert call(q=2, rs=ctypes.c_void_p(0x1002)) == -1  # fp32 scales not 4-byte aligned
    assert call(rw=ctypes.c_void_p(0x1006)) == -1       # fp32 row weights not 4-byte aligned


def test_missing_library_raises_and_nothing_falls_back(tmp_path):
    """With the HIP library absent the binding raises on first use: there is
    no CPU path to fall back on.  Run in a fresh interpreter whose binding
    looks for the library at a path that does not exist."""
    code = f"""
import torch
import combine_moe_get_dispatch_amd as m
m.LIB_PATH = {str(tmp_path / 'absent.so')!r}
m._lib = None
for f in (m.lib,
          lambda: m.moe_get_dispatch_layout(torch.zeros((4, 2), dtype=torch.int64), 4, 2),
          lambda: m.moe_recv_capacity_bound(4, 2, 4, 1)):
    try:
        f()
    except (RuntimeError, ValueError) as e:
        print(type(e).__name__, str(e)[:60])
    else:
        raise SystemExit("call succeeded without the library")
"""
    out = subprocess.run(["python", "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.strip().splitlines()
    assert len(lines) == 3 and lines[0].startswith("RuntimeError") and "missing" in lines[0]
