"""The allocation-free routing entry point, moe_route_noalloc, called
through the C ABI: bit-exact against moe_route (the workspace entry point)
on two calls in a row, the second smaller than the first (the fixed scratch
keeps the first call's contents), and a size beyond its scratch rejected
before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from parity import banner, to_np

pytestmark = pytest.mark.gpu

try:
    import gemm_bit_weight_amd as gbw
except ImportError as e:
    gbw = None
    _IMPORT_ERROR = e

DEV = "cuda"
KEYS = ("topk_ids", "topk_w", "expert_offsets", "pair_token", "pair_pos")


def setup_module():
    assert gbw is not None, f"HIP library missing: {_IMPORT_ERROR}"
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _noalloc_c(logits, topk):
    """One call straight through the C ABI (ctypes), outputs preset to -1."""
    T, E = logits.shape
    out = dict(topk_ids=torch.full((T, topk), -1, dtype=torch.int32, device=DEV),
               topk_w=torch.full((T, topk), -1.0, dtype=torch.float32, device=DEV),
               expert_offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=DEV),
               pair_token=torch.full((T * topk,), -1, dtype=torch.int32, device=DEV),
               pair_pos=torch.full((T, topk), -1, dtype=torch.int32, device=DEV))
    lib = ctypes.CDLL(gbw.library_path())
    lib.moe_route_noalloc.restype = ctypes.c_int
    lib.moe_route_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + \
        [ctypes.c_void_p] * 6
    st = lib.moe_route_noalloc(logits.data_ptr(), T, E, topk, *(out[k].data_ptr() for k in KEYS),
                               torch.cuda.current_stream().cuda_stream)
    return st, out


def test_noalloc_route_matches_workspace_route():
    for T, E, k in ((8192, 128, 8), (1000, 64, 4)):       # the second call smaller than the first
        banner(f"moe_route_noalloc T={T} E={E} k={k}")
        logits = synth.normal((T, E), 1.0, T + E, "noalloc.l", DEV)
        st, got = _noalloc_c(logits, k)
        assert st == 0, gbw.status_string(st)
        ref = gbw.moe_route(logits, k)
        torch.cuda.synchronize()
        for key in KEYS:
            assert np.array_equal(to_np(got[key]), to_np(ref[key])), key


def test_noalloc_route_rejects_sizes_beyond_its_scratch():
    banner("moe_route_noalloc too large")
    T, E = 64 * 1025, 128                                   # ceil(T/64) * E = 131200 > 131072
    logits = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    st, out = _noalloc_c(logits, 8)
    assert st == 2                                          # GBW_E_SHAPE
    assert b"scratch" in gbw._lib.gbw_last_error()
    torch.cuda.synchronize()
    assert (out["expert_offsets"] == -1).all()               # nothing was launched
