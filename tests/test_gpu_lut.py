"""GPU parity: the codebook (LUT) GEMM against the oracle.

Outputs must satisfy max_n |y - y_ref| <= 1e-3 * ||y_ref row||_2; the
integer-valued case (centroids j - 8, integer x) must be bit-exact.  x covers
the whole bf16 range (values up to 1e30 and below 2^-24) and every
workspace path of the split-K kernel (a reused zeroed workspace, one that is
too short, none).
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.native as on
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
    return on.lut_gemm(u16(d["x"]), to_np(d["idx"]), to_np(d["centroids"]), group)


@pytest.mark.parametrize("M,N,K,group", [(1, 64, 256, 128), (3, 100, 512, 64), (8, 256, 1024, 128),
                                         (17, 130, 384, 32), (64, 512, 2048, 128), (70, 96, 640, 128),
                                         (128, 64, 256, 64), (3, 100, 4608, 64), (16, 50, 2176, 32),
                                         (11, 70, 8320, 128)])
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


@pytest.mark.parametrize("M", [1, 8, 16, 40, 64, 100])
def test_lut_gemm_whole_bf16_range(M):
    """x rows and 128-chunks at very different magnitudes: whole rows near
    1e30, rows below 2^-24, chunks that mix 1e30 with 2^-30 and ordinary
    N(0,1) values; the oracle is finite everywhere, and so must the GPU be."""
    banner(f"lut_gemm bf16 range M={M} N=192 K=1024")
    N, K, group = 192, 1024, 128
    w = synth.clustered_weight(N, K, group=group, seed=60 + M, device="cpu", iters=4)
    x = synth.normal((M, K), 1.0, 61 + M, "lut.range", "cpu")
    row_gain = torch.tensor([1e30, 2.0 ** -30, 1.0, 3e-38, 2.0 ** -100, 6e4, 7e4, 1e-8][:M] +
                            [1.0] * max(0, M - 8)).reshape(-1, 1)
    x = x * row_gain
    if M > 2:                                  # a row whose chunks mix huge and tiny values
        x[2, :128] *= 1e30
        x[2, 128:256] *= 2.0 ** -30
        x[2, 300] = 1e30
    if M > 9:
        x[9:, 512:640] *= 2.0 ** -40           # one tiny chunk in every other row
    xb = x.to(torch.bfloat16)
    assert torch.isfinite(xb.float()).all()
    d = dict(x=xb, idx=w["idx"], centroids=w["centroids"])
    ref = _ref(d, group)
    y = gbw.lut_gemm(xb.to(DEV), w["idx"].to(DEV), w["centroids"].to(DEV), group)
    assert torch.isfinite(y).all()
    assert_rows_close(to_np(y), ref, what="lut_gemm bf16 range")


@pytest.mark.parametrize("M", [24, 64])
def test_lut_gemm_workspace_paths(M):
    """The split-K kernel with one zeroed workspace reused over several calls
    (its arrival counters must be left at zero: every call gives the same
    bits), with a workspace one byte too short and with none (both the
    one-workgroup-per-tile path)."""
    banner(f"lut_gemm workspace paths M={M} N=512 K=4096")
    N, K, group = 512, 4096, 128
    w = synth.clustered_weight(N, K, group=group, seed=70, device="cpu", iters=4)
    x = synth.normal((M, K), 1.0, 71, "lut.ws", "cpu").to(torch.bfloat16)
    ref = _ref(dict(x=x, idx=w["idx"], centroids=w["centroids"]), group)
    xd, idx, cent = x.to(DEV), w["idx"].to(DEV), w["centroids"].to(DEV)
    need = gbw.workspace_size(gbw.OP_LUT_GEMM, M, N, K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ys = [gbw.lut_gemm(xd, idx, cent, group, ws=ws) for _ in range(4)]
    assert_rows_close(to_np(ys[0]), ref, what="split-K")
    assert all(torch.equal(ys[0], yy) for yy in ys[1:])
    short = torch.zeros(need - 1, dtype=torch.uint8, device=DEV)
    y_short = gbw.lut_gemm(xd, idx, cent, group, ws=short)
    y_none = gbw.lut_gemm(xd, idx, cent, group, ws=False)
    assert_rows_close(to_np(y_short), ref, what="short workspace")
    assert torch.equal(y_short, y_none)


def test_lut_gemm_empty_extents():
    """M = 0 or N = 0 returns without touching the output."""
    banner("lut_gemm empty extents")
    K, group = 256, 128
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((8, K // 2), dtype=torch.uint8, device=DEV)
    cent = torch.zeros((8, K // group, 16), dtype=torch.float16, device=DEV)
    assert gbw.lut_gemm(x0, idx, cent, group).shape == (0, 8)
    x = torch.ones((3, K), dtype=torch.bfloat16, device=DEV)
    y = gbw.lut_gemm(x, idx[:0], cent[:0], group)
    assert y.shape == (3, 0)
    torch.cuda.synchronize()


def test_lut_gemm_rejects_bad_shapes():
    x = torch.zeros((4, 200), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gbw.GbwError):
        gbw.lut_gemm(x, torch.zeros((8, 100), dtype=torch.uint8, device=DEV),
                     torch.zeros((8, 2, 16), dtype=torch.float16, device=DEV), 128)
