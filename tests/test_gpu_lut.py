"""GPU parity: the codebook (LUT) GEMM against the oracle.

Outputs must satisfy max_n |y - y_ref| <= 1e-3 * ||y_ref row||_2; the
integer-valued case (centroids j - 8, integer x) must be bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_rows_close, banner, to_np, u16

pytestmark = pytest.mark.gpu

try:
    import gemm_bit_weight_amd as gbw
except ImportError as e:
    gbw = None
    _IMPORT_ERROR = e

DEV = "cuda"


def setup_module():
    assert gbw is not None, f"HIP library missing: {_IMPORT_ERROR}"
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _ref(d, group):
    return oracle.lut_gemm(u16(d["x"]), to_np(d["idx"]), to_np(d["centroids"]), group)


@pytest.mark.parametrize("M,N,K,group", [(1, 64, 256, 128), (3, 100, 512, 64), (8, 256, 1024, 128),
                                         (17, 130, 384, 32), (64, 512, 2048, 128), (70, 96, 640, 128),
                                         (128, 64, 256, 64)])
def test_lut_gemm_small(M, N, K, group):
    banner(f"lut_gemm {M}x{N}x{K} group {group}")
    w = synth.clustered_weight(N, K, group=group, seed=M + N, device="cpu", iters=4)
    x = synth.normal((M, K), 1.0, M, "lut.tx", "cpu").to(torch.bfloat16)
    d = dict(x=x, idx=w["idx"], centroids=w["centroids"])
    ref = _ref(d, group)
    y = gbw.lut_gemm(x.to(DEV), w["idx"].to(DEV), w["centroids"].to(DEV), group)
    assert_rows_close(to_np(y), ref, what="lut_gemm")
    assert torch.equal(y, gbw.lut_gemm(x.to(DEV), w["idx"].to(DEV), w["centroids"].to(DEV), group))


def test_lut_gemm_integer_case_bitexact():
    banner("lut_gemm integer case")
    rng = np.random.default_rng(40)
    M, N, K, group = 24, 200, 1024, 128
    idx = rng.integers(0, 16, (N, K))
    cents = np.tile((np.arange(16) - 8).astype(np.float16), (N, K // group, 1))
    xi = rng.integers(-8, 9, (M, K))
    xb = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16)
    y = gbw.lut_gemm(xb.to(DEV), torch.from_numpy(oracle.pack_nibbles(idx)).to(DEV),
                     torch.from_numpy(cents).to(DEV), group)
    assert np.array_equal(to_np(y).astype(np.float64), (xi @ (idx - 8).T).astype(np.float64))


@pytest.mark.parametrize("M", [1, 8, 64])
def test_lut_gemm_full_size(M):
    """The measured shape: K = N = 4096, 128-wide groups, all outputs compared."""
    banner(f"lut_gemm full 4096x4096 M={M}")
    d = synth.lut_problem(M, N=4096, K=4096, group=128, seed=0, device=DEV, iters=10)
    y = gbw.lut_gemm(d["x"], d["idx"], d["centroids"], 128)
    ref = _ref(d, 128)
    assert_rows_close(to_np(y), ref, what=f"lut_gemm full M={M}")


def test_lut_gemm_rejects_bad_shapes():
    x = torch.zeros((4, 200), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gbw.GbwError):
        gbw.lut_gemm(x, torch.zeros((8, 100), dtype=torch.uint8, device=DEV),
                     torch.zeros((8, 2, 16), dtype=torch.float16, device=DEV), 128)
