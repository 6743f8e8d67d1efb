"""moe_get_dispatch_layout_noalloc -- the layout with its workspace in the
library's built-in scratch, for callers that cannot allocate -- against
moe_get_dispatch_layout with a caller workspace, through the C ABI.  Every
output must be bit-identical, on two calls in a row whose second is smaller,
for each layout path (chunked, chunked with the column scan, one workgroup),
on the default stream and on a side stream."""
import ctypes

import numpy as np
import pytest
import torch

from combine_moe_get_dispatch_amd import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import combine_moe_get_dispatch_amd as moe

DEV = torch.device("cuda", 0)

# (T, K, E, R, a, routing): first call, then a smaller second call
PAIRS = [
    ("chunked", (8192, 8, 256, 16, 128, "zipf"), (3000, 4, 32, 4, 1, "uniform")),
    ("column_scan", (16384, 16, 512, 512, 1, "uniform"), (5000, 8, 64, 8, 7, "uniform")),
    ("chunked_then_one_workgroup", (4096, 8, 256, 8, 1, "uniform"), (128, 8, 256, 8, 1, "uniform")),
]

FIELDS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "num_recv_tokens_per_expert",
          "expert_offsets", "token_row", "recv_src", "error_flag")


def _inputs(T, K, E, R, a, routing, seed):
    w = W.Workload("noalloc", T, 32, E, R, K, a, 0, routing=routing, zipf_s=1.1 if routing == "zipf" else 0.0,
                   drop_prob=0.05, seed_index=seed)
    idx, _ = W.generate_routing(w)
    return torch.from_numpy(idx).to(DEV)


def _poisoned_layout(T, K, E, R, a):
    lay = moe.allocate_layout(T, K, E, R, a, device=DEV)
    for f in FIELDS:
        getattr(lay, f).fill_(-77)
    return lay


def _noalloc(idx, lay, stream):
    L = moe.lib()
    T, K = idx.shape
    ptrs = [ctypes.c_void_p(getattr(lay, f).data_ptr()) for f in FIELDS]
    return L.moe_get_dispatch_layout_noalloc(ctypes.c_void_p(idx.data_ptr()), T, K, lay.num_experts,
                                             lay.num_ranks, lay.expert_alignment, lay.recv_capacity, *ptrs,
                                             ctypes.c_void_p(stream.cuda_stream))


@pytest.mark.parametrize("name,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_layout_matches_the_workspace_layout(name, first, second):
    side = torch.cuda.Stream()
    for n, (T, K, E, R, a, routing) in enumerate((first, second)):
        print(f"[noalloc] {name} call {n + 1}: T={T} K={K} E={E} R={R} a={a} {routing}", flush=True)
        assert moe.moe_layout_workspace_bytes(T, K, E, R) <= moe.NOALLOC_SCRATCH_BYTES
        idx = _inputs(T, K, E, R, a, routing, 40 + n)
        ref = moe.moe_get_dispatch_layout(idx, E, R, a)
        got = _poisoned_layout(T, K, E, R, a)
        stream = torch.cuda.current_stream(DEV) if n == 0 else side
        if n == 1:
            side.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(stream):
            assert _noalloc(idx, got, stream) == moe.MOE_OK
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(got, f), getattr(ref, f)), f"{name} call {n + 1}: {f}"
        assert int(got.error_flag.item()) == 0


def test_noalloc_layout_binding_and_repeated_calls():
    """The binding's wrapper, called repeatedly on one layout: each result
    equals the workspace layout of the same ids (the scratch keeps the last
    call's contents and needs no clearing)."""
    T, K, E, R, a = 4096, 8, 256, 8, 1
    out = _poisoned_layout(T, K, E, R, a)
    for seed in (50, 51, 52):
        idx = _inputs(T, K, E, R, a, "uniform", seed)
        ref = moe.moe_get_dispatch_layout(idx, E, R, a)
        moe.moe_get_dispatch_layout_noalloc(idx, out)
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(out, f), getattr(ref, f)), f"seed {seed}: {f}"
