"""GPU parity: online quantization, decode, MXFP4 GEMM and the PRQuant
tail-residual GEMM against the oracle.

Encodings, decoded weights and residuals must match bit for bit; GEMM outputs
must satisfy max_n |y - y_ref| <= 1e-3 * ||y_ref row||_2 (the oracle's value
is the exact value of the quantized GEMM), and integer-valued cases must be
bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.native as on
import synth
from parity import assert_rows_close, banner, to_np, vq_ref_block_scales

pytestmark = pytest.mark.gpu

try:
    import gemm_bit_weight_amd as gbw
except ImportError as e:  # collected on CPU-only hosts too; the GPU run must have the library
    gbw = None
    _IMPORT_ERROR = e

DEV = "cuda"


def _q8(x_t):
    """oracle E8M0 quantization of a torch tensor (bf16 or fp32)."""
    return oracle.quantize_e8m0_b32(x_t.float().cpu().numpy())


def _gpu_act(codes, scales, fmt=0, ts=None):
    return gbw.Act(fmt, torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                   None if ts is None else torch.tensor([ts], dtype=torch.float32, device=DEV))


def _gpu_w(codes, scales):
    N = codes.shape[0]
    return gbw.Weight(gbw.FMT_E8M0_B32, N, codes.shape[1] * 2, torch.from_numpy(codes).to(DEV),
                      torch.from_numpy(scales).to(DEV))


def setup_module():
    assert gbw is not None, f"HIP library missing: {_IMPORT_ERROR}"
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def _special_rows(K):
    x = np.zeros((6, K), np.float32)
    x[1, :] = -0.0
    x[2, ::3] = 1e-40                    # subnormal block amax
    x[3, :] = np.tile([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5], K // 8)  # midpoints at scale 2^-1
    x[3, 7::8] = 4.0
    x[4, :] = np.tile([3e38, -1.0, 1e-30, 7.9], K // 4)
    x[5, :] = np.linspace(-1000, 1000, K)
    return x


@pytest.mark.parametrize("rows,K,dtype", [(16, 512, "bf16"), (512, 512, "f32"), (13, 96, "bf16"),
                                          (128, 9728, "bf16"), (2560, 9728, "f32"), (6, 256, "special")])
def test_quantize_e8m0_bitexact(rows, K, dtype):
    banner(f"quantize e8m0 {rows}x{K} {dtype}")
    if dtype == "special":
        x = torch.from_numpy(_special_rows(K)).to(DEV)
    else:
        d = synth.dense_linear(rows, 8, K, seed=1, device=DEV)
        x = d["x"] if dtype == "bf16" else synth.normal((rows, K), 0.02, 1, "q.w", DEV)
    a = gbw.mx_quantize(x.contiguous(), gbw.FMT_E8M0_B32)
    c, s = _q8(x)
    assert np.array_equal(to_np(a.scales), s)
    assert np.array_equal(to_np(a.codes), c)


def test_quantize_tail_copy_bitexact():
    banner("quantize e8m0 tail copy 128x9728 tail 256")
    p = synth.tail_residual_problem(128, 64, 9728, seed=0, device=DEV)
    a = gbw.mx_quantize(p["x"], gbw.FMT_E8M0_B32, tail_copy=256)
    c, s = _q8(p["x"])
    cc, ss = oracle.tail_copy(c, s, 256)
    assert np.array_equal(to_np(a.codes), cc)
    assert np.array_equal(to_np(a.scales), ss)


@pytest.mark.parametrize("rows,K,kind", [(13, 96, "bf16"), (128, 9728, "outliers"), (2560, 9728, "f32"),
                                        (40, 512, "wide")])
def test_quantize_e8m0_block_hadamard_bitexact(rows, K, kind):
    """mx_quantize(rotate=True): the oracle rotates each 32-block in fp32 in
    the same butterfly order, then quantizes; codes and scales bit for bit."""
    banner(f"quantize e8m0 block-hadamard {rows}x{K} {kind}")
    if kind == "bf16":
        x = synth.normal((rows, K), 1.0, 6, "h.x", DEV).to(torch.bfloat16)
    elif kind == "outliers":
        x = synth.tail_residual_problem(rows, 64, K, seed=0, device=DEV)["x"]
    elif kind == "f32":
        x = synth.normal((rows, K), 0.02, 6, "h.w", DEV)
    else:
        g = synth.normal((rows, K), 1.0, 7, "h.wide", DEV)
        e = torch.arange(rows * K // 32, device=DEV).reshape(rows, K // 32) % 41 - 20
        x = (g * torch.exp2(e.float()).repeat_interleave(32, dim=1)).contiguous()
    a = gbw.mx_quantize(x.contiguous(), gbw.FMT_E8M0_B32, rotate=True)
    c, s = oracle.quantize_e8m0_b32(oracle.fwht32_fp32(x.float().cpu().numpy()))
    assert np.array_equal(to_np(a.scales), s)
    assert np.array_equal(to_np(a.codes), c)
    if kind == "outliers":
        at = gbw.mx_quantize(x, gbw.FMT_E8M0_B32, rotate=True, tail_copy=256)
        cc, ss = oracle.tail_copy(c, s, 256)
        assert np.array_equal(to_np(at.codes), cc) and np.array_equal(to_np(at.scales), ss)


def test_block_hadamard_gemm_parity_and_error():
    """Q(XH) Q(WH)^T through mx_gemm against the oracle's GEMM of the oracle's
    rotated quantization; with outlier channels it is closer to X W^T than
    the plain MXFP4 GEMM (the reason for the rotation)."""
    banner("mx_gemm block-hadamard 128x2560x9728")
    p = synth.tail_residual_problem(128, 2560, 9728, seed=0, device=DEV)
    x, w = p["x"], p["w"]
    a = gbw.mx_quantize(x, gbw.FMT_E8M0_B32, rotate=True)
    wq = gbw.mx_quantize(w, gbw.FMT_E8M0_B32, rotate=True)
    y = to_np(gbw.mx_gemm(a, gbw.weight_from_act(wq))).astype(np.float64)
    ac, as_ = on.quantize_e8m0_b32(oracle.fwht32_fp32(x.float().cpu().numpy()))
    wc, ws = on.quantize_e8m0_b32(oracle.fwht32_fp32(w.cpu().numpy()))
    assert np.array_equal(to_np(a.codes), ac) and np.array_equal(to_np(wq.codes), wc)
    assert np.array_equal(to_np(a.scales), as_) and np.array_equal(to_np(wq.scales), ws)
    ref = on.mx_gemm(ac, as_, wc, ws)
    assert_rows_close(y, ref, what="rotated mx_gemm")
    y_plain = to_np(gbw.mx_gemm(gbw.mx_quantize(x, gbw.FMT_E8M0_B32),
                                gbw.weight_from_act(gbw.mx_quantize(w, gbw.FMT_E8M0_B32)))).astype(np.float64)
    exact = x.double().cpu().numpy() @ w.double().cpu().numpy().T
    e_rot = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    e_plain = np.linalg.norm(y_plain - exact) / np.linalg.norm(exact)
    print(f"[stats] y-NRMSE rotated {e_rot:.4f} plain {e_plain:.4f}", flush=True)
    assert e_rot < e_plain


def test_block_hadamard_rejects_16_element_blocks():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gbw.GbwError):
        gbw.mx_quantize(x, gbw.FMT_E4M3_B16, rotate=True)


_TS_FORMATS = {"e4m3": (gbw.FMT_E4M3_B16, oracle.quantize_e4m3_b16, oracle.formats.tensor_scale_e4m3),
               "e5m3": (gbw.FMT_E5M3_B16, oracle.quantize_e5m3_b16, oracle.formats.tensor_scale_e5m3)}


@pytest.mark.parametrize("fmt", ["e4m3", "e5m3"])
@pytest.mark.parametrize("rows,K,dtype,static", [(64, 2048, "bf16", False), (37, 48, "f32", False),
                                                 (300, 768, "bf16", True), (6, 256, "special", False),
                                                 (40, 512, "wide", False)])
def test_quantize_e4m3_bitexact(rows, K, dtype, static, fmt):
    banner(f"quantize {fmt} {rows}x{K} {dtype} static={static}")
    gfmt, oq, ots = _TS_FORMATS[fmt]
    if dtype == "special":
        x = torch.from_numpy(_special_rows(K)[:, :K]).to(DEV)
        x[4] = x[5]                                   # keep the tensor amax finite and moderate
    elif dtype == "bf16":
        x = synth.normal((rows, K), 1.0, 2, "q4.x", DEV).to(torch.bfloat16)
    elif dtype == "wide":
        # 16-element blocks spread over 2^-40 .. 2^20: subnormal, normal and top block scales
        g = synth.normal((rows, K), 1.0, 5, "q4.wide", DEV)
        e = torch.arange(rows * K // 16, device=DEV).reshape(rows, K // 16) % 61 - 40
        x = (g * torch.exp2(e.float()).repeat_interleave(16, dim=1)).contiguous()
    else:
        x = synth.normal((rows, K), 0.02, 2, "q4.w", DEV)
    xn = x.float().cpu().numpy()
    if static:
        amax = np.float32(7.5)
        ts = torch.tensor([ots(amax)], dtype=torch.float32, device=DEV)
        a = gbw.mx_quantize(x, gfmt, tensor_scale=ts, dynamic=False)
        c, s, st = oq(xn, tensor_amax=amax)
    else:
        a = gbw.mx_quantize(x, gfmt)
        c, s, st = oq(xn)
    assert to_np(a.tensor_scale)[0] == st
    assert np.array_equal(to_np(a.scales), s)
    assert np.array_equal(to_np(a.codes), c)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m3"])
def test_quantize_e4m3_empty_tensor_scale(fmt):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    a = gbw.mx_quantize(x, _TS_FORMATS[fmt][0])
    assert to_np(a.tensor_scale)[0] == 1.0


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def test_dequantize_e8m0_and_e4m3_bitexact():
    banner("dequantize e8m0/e4m3")
    w = synth.normal((192, 512), 0.02, 3, "dq.w", "cpu").numpy()
    c, s = oracle.quantize_e8m0_b32(w)
    out = gbw.mx_dequantize(_gpu_w(c, s))
    assert np.array_equal(to_np(out).astype(np.float64), oracle.dequantize(c, s, "e8m0_b32"))
    # E4M3 with two tensor-scale segments (gate rows, up rows)
    cg, sg, tg = oracle.quantize_e4m3_b16(w[:96])
    cu, su, tu = oracle.quantize_e4m3_b16(w[96:] * 3)
    W = gbw.Weight(gbw.FMT_E4M3_B16, 192, 512, torch.from_numpy(np.concatenate([cg, cu])).to(DEV),
                   torch.from_numpy(np.concatenate([sg, su])).to(DEV), None,
                   torch.tensor([tg, tu], dtype=torch.float32, device=DEV), 2, 1)
    out = to_np(gbw.mx_dequantize(W))
    ref = np.concatenate([oracle.dequantize(cg, sg, "e4m3_b16", tg), oracle.dequantize(cu, su, "e4m3_b16", tu)])
    assert np.array_equal(out.astype(np.float64), ref.astype(np.float32).astype(np.float64))
    # E5M3 likewise, with a spread of block magnitudes that reaches subnormal and top UE5M3 scales
    w5 = w * np.exp2(np.arange(192 * 32).reshape(192, 32) % 50 - 30).repeat(16, axis=1)
    cg, sg, tg = oracle.quantize_e5m3_b16(w5[:96].astype(np.float32))
    cu, su, tu = oracle.quantize_e5m3_b16(w5[96:].astype(np.float32))
    W = gbw.Weight(gbw.FMT_E5M3_B16, 192, 512, torch.from_numpy(np.concatenate([cg, cu])).to(DEV),
                   torch.from_numpy(np.concatenate([sg, su])).to(DEV), None,
                   torch.tensor([tg, tu], dtype=torch.float32, device=DEV), 2, 1)
    out = to_np(gbw.mx_dequantize(W))
    ref = np.concatenate([oracle.dequantize(cg, sg, "e5m3_b16", tg), oracle.dequantize(cu, su, "e5m3_b16", tu)])
    assert np.array_equal(out.astype(np.float64), ref.astype(np.float32).astype(np.float64))
    assert (np.concatenate([sg, su]) < 8).any() and (np.concatenate([sg, su]) == 0xFE).any()


def test_dequantize_vq_bitexact():
    banner("dequantize vq")
    v = synth.vq_weight(3, 128, 192, seed=4, device="cpu")
    W = gbw.Weight(gbw.FMT_VQ4_E8M0, 128, 192, v["idx"].to(DEV), v["scales"].to(DEV), v["codebook"].to(DEV),
                   None, 1, 3)
    cb = v["codebook"].numpy().view(np.uint16)
    for e in range(3):
        out = to_np(gbw.mx_dequantize(W, expert=e))
        ref = oracle.vq_dequantize(v["idx"][e].numpy(), cb[e], v["scales"][e].numpy())
        assert np.array_equal(out.astype(np.float64), ref)


_VQ_FMT = {"prescale": gbw.FMT_VQ4_E8M0, "postscale": gbw.FMT_VQ4_POST, "prescale_plus": gbw.FMT_VQ4_PLUS}


@pytest.mark.parametrize("scales,qblock,N,K", [("postscale", 64, 128, 192), ("postscale", 128, 256, 384),
                                               ("postscale", 256, 256, 512), ("prescale_plus", 64, 128, 512),
                                               ("prescale_plus", 256, 256, 768), ("prescale", 128, 384, 256)])
def test_dequantize_vq_scale_layouts_bitexact(scales, qblock, N, K):
    """MXCode PostScale / PreScale+ block scales and QBlocks of 64-256: the
    device decode equals the oracle's, expert by expert."""
    banner(f"dequantize vq {scales} qblock={qblock} N={N} K={K}")
    E = 3
    v = synth.vq_weight(E, N, K, qblock=qblock, seed=5, device="cpu", scales=scales)
    W = gbw.Weight(_VQ_FMT[scales], N, K, v["idx"].to(DEV), v["scales"].to(DEV), v["codebook"].to(DEV),
                   None, 1, E, qblock=qblock,
                   scale_codebook=v["scale_codebook"].to(DEV) if "scale_codebook" in v else None)
    cb = v["codebook"].numpy().view(np.uint16)
    for e in range(E):
        out = to_np(gbw.mx_dequantize(W, expert=e))
        ref = oracle.vq_dequantize(v["idx"][e].numpy(), cb[e], vq_ref_block_scales(v, e, scales, K, qblock), qblock)
        assert np.array_equal(out.astype(np.float64), ref)


_VQ16_FMT = {("e4m3", "prescale"): gbw.FMT_VQ4_E4M3, ("e4m3", "postscale"): gbw.FMT_VQ4_E4M3_POST,
             ("e4m3", "prescale_plus"): gbw.FMT_VQ4_E4M3_PLUS, ("e5m3", "prescale"): gbw.FMT_VQ4_E5M3,
             ("e5m3", "postscale"): gbw.FMT_VQ4_E5M3_POST, ("e5m3", "prescale_plus"): gbw.FMT_VQ4_E5M3_PLUS}


@pytest.mark.parametrize("scale_fmt", ["e4m3", "e5m3"])
@pytest.mark.parametrize("scales,qblock,N,K", [("prescale", 64, 128, 192), ("postscale", 128, 256, 384),
                                               ("prescale_plus", 64, 128, 384), ("prescale_plus", 256, 256, 512)])
def test_dequantize_vq_b16_bitexact(scale_fmt, scales, qblock, N, K):
    """VQ codes with E4M3 / UE5M3 block scales per 16 (PreScale, PostScale,
    PreScale+) and two tensor-scale row segments: the device decode equals
    the oracle's, expert by expert."""
    banner(f"dequantize vq {scale_fmt} {scales} qblock={qblock} N={N} K={K}")
    E = 2
    v = synth.vq_weight(E, N, K, qblock=qblock, seed=6, device="cpu", scales=scales, scale_fmt=scale_fmt,
                        ts_segments=2)
    W = gbw.Weight(_VQ16_FMT[(scale_fmt, scales)], N, K, v["idx"].to(DEV), v["scales"].to(DEV),
                   v["codebook"].to(DEV), v["tensor_scale"].to(DEV), 2, E, qblock=qblock,
                   scale_codebook=v["scale_codebook"].to(DEV) if "scale_codebook" in v else None)
    cb = v["codebook"].numpy().view(np.uint16)
    ofmt = "e4m3_b16" if scale_fmt == "e4m3" else "e5m3_b16"
    for e in range(E):
        out = to_np(gbw.mx_dequantize(W, expert=e))
        codes = oracle.vq_decode_codes(v["idx"][e].numpy(), cb[e], qblock)
        sc = vq_ref_block_scales(v, e, scales, K, qblock, 16)
        ts = v["tensor_scale"][e].numpy()
        ref = np.concatenate([oracle.dequantize(codes[:N // 2], sc[:N // 2], ofmt, ts[0]),
                              oracle.dequantize(codes[N // 2:], sc[N // 2:], ofmt, ts[1])])
        assert np.array_equal(out.astype(np.float64), ref.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# MXFP4 GEMM
# ---------------------------------------------------------------------------

def _dense_case(M, N, K, seed):
    """GPU operands quantized by the library, the reference from the oracle's
    own quantization of the same synthetic inputs (the codes agree bit for
    bit)."""
    d = synth.dense_linear(M, N, K, seed=seed, device=DEV)
    a = gbw.mx_quantize(d["x"], gbw.FMT_E8M0_B32)
    wq = gbw.mx_quantize(d["w"], gbw.FMT_E8M0_B32)
    w = gbw.weight_from_act(wq)
    ac, as_ = on.quantize_e8m0_b32(d["x"].float().cpu().numpy())
    wc, ws = on.quantize_e8m0_b32(d["w"].cpu().numpy())
    assert np.array_equal(to_np(a.codes), ac) and np.array_equal(to_np(a.scales), as_)
    assert np.array_equal(to_np(wq.codes), wc) and np.array_equal(to_np(wq.scales), ws)
    ref = on.mx_gemm(ac, as_, wc, ws)
    assert on.last_inexact == 0
    return a, w, ref


def test_mx_gemm_single_linear_16x512x512():
    banner("mx_gemm 16x512x512 seed 0")
    a, w, ref = _dense_case(16, 512, 512, 0)
    y = gbw.mx_gemm(a, w)
    assert_rows_close(to_np(y), ref, what="mx_gemm 16x512x512")
    # every path sums in a fixed order: two runs agree bit for bit
    assert torch.equal(y, gbw.mx_gemm(a, w))
    y1 = gbw.mx_gemm(a, w, ws=False)                   # serial-K path (no workspace)
    assert torch.equal(y1, gbw.mx_gemm(a, w, ws=False))
    assert_rows_close(to_np(y1), ref, what="serial")


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 20, 96), (17, 300, 160), (33, 64, 544), (100, 129, 1056),
                                   (128, 2560, 9728), (200, 70, 256), (17, 64, 128), (40, 130, 640),
                                   (96, 64, 4096), (129, 100, 1280), (70, 4100, 1024), (65, 4098, 256),
                                   (17, 8192, 384)])
def test_mx_gemm_ragged(M, N, K):
    banner(f"mx_gemm {M}x{N}x{K}")
    a, w, ref = _dense_case(M, N, K, 7)
    assert_rows_close(to_np(gbw.mx_gemm(a, w)), ref, what=f"mx_gemm {M}x{N}x{K}")
    y = gbw.mx_gemm(a, w)
    assert torch.equal(y, gbw.mx_gemm(a, w))
    assert_rows_close(to_np(gbw.mx_gemm(a, w, ws=False)), ref, what="serial")


@pytest.mark.parametrize("M,N,K", [(16, 256, 1024), (9, 70, 96), (64, 512, 2048), (128, 2560, 9728),
                                   (40, 100, 640), (70, 4100, 1024)])
def test_mx_gemm_wide_scale_codes(M, N, K):
    """Random E2M1 codes with E8M0 scale codes over 1 .. 253: a low
    activation scale against a high weight scale in every block (each product
    of two scales within 2^+-7, so every sum is exact and finite).  Covers
    the 16-row and 32-row kernels and the serial path."""
    banner(f"mx_gemm wide scale codes {M}x{N}x{K}")
    ac = synth.random_codes(M, K, 8, "wide.a")
    wc = synth.random_codes(N, K, 8, "wide.w")
    asc, wsc = synth.paired_scale_codes(M, N, K, 8, "wide.s")
    ref = on.mx_gemm(ac.numpy(), asc.numpy(), wc.numpy(), wsc.numpy())
    assert on.last_inexact == 0
    A = _gpu_act(ac.numpy(), asc.numpy())
    W = _gpu_w(wc.numpy(), wsc.numpy())
    assert_rows_close(to_np(gbw.mx_gemm(A, W)), ref, what="wide-scale mx_gemm")
    assert_rows_close(to_np(gbw.mx_gemm(A, W, ws=False)), ref, what="wide-scale mx_gemm serial")
    print(f"[stats] scale codes a {int(asc.min())}..{int(asc.max())} w {int(wsc.min())}..{int(wsc.max())}",
          flush=True)


def test_dense_empty_extents():
    """M = 0 or N = 0: every GEMM entry point returns without touching its
    output; a zero-row quantization returns an empty result."""
    banner("dense empty extents")
    K = 256
    codes = np.zeros((4, K // 2), np.uint8)
    scales = np.full((4, K // 32), 127, np.uint8)
    A0 = gbw.Act(gbw.FMT_E8M0_B32, torch.empty((0, K // 2), dtype=torch.uint8, device=DEV),
                 torch.empty((0, K // 32), dtype=torch.uint8, device=DEV))
    W = _gpu_w(codes, scales)
    y = torch.full((0, 4), 7.0, device=DEV)
    assert gbw.mx_gemm(A0, W, out=y).shape == (0, 4)
    R = _gpu_w(np.ascontiguousarray(codes[:, :64]), np.ascontiguousarray(scales[:, :4]))
    assert gbw.residual_tail_gemm(A0, W, R, 128, out=y).shape == (0, 4)
    A = _gpu_act(codes, scales)
    W0 = gbw.Weight(gbw.FMT_E8M0_B32, 0, K, torch.empty((0, K // 2), dtype=torch.uint8, device=DEV),
                    torch.empty((0, K // 32), dtype=torch.uint8, device=DEV))
    y4 = torch.full((4, 0), 7.0, device=DEV)
    assert gbw.mx_gemm(A, W0, out=y4).shape == (4, 0)
    q = gbw.mx_quantize(torch.empty((0, K), dtype=torch.bfloat16, device=DEV), gbw.FMT_E8M0_B32)
    assert q.codes.shape == (0, K // 2) and q.scales.shape == (0, K // 32)
    torch.cuda.synchronize()


def test_mx_gemm_long_k():
    """K = 32768 (256 steps of 128; the 16-row kernel's longest K ranges) at
    M = 16, N = 1024."""
    banner("mx_gemm 16x1024x32768")
    a, w, ref = _dense_case(16, 1024, 32768, 11)
    assert_rows_close(to_np(gbw.mx_gemm(a, w)), ref, what="mx_gemm long K")
    assert_rows_close(to_np(gbw.mx_gemm(a, w, ws=False)), ref, what="mx_gemm long K serial")


def test_split_k_workspace_shared_across_shapes():
    """One zeroed workspace, sized for the largest call, serves a sequence of
    split-K GEMMs of different shapes (both split-K kernels, with and without
    the tail segment): every call leaves the arrival counters at zero, so each
    result is bitwise the one a fresh workspace gives."""
    banner("split-K workspace shared across shapes")
    shapes = [(128, 2560, 2048, 256), (40, 1024, 4096, 0), (16, 512, 4096, 0), (70, 640, 1024, 128),
              (128, 2560, 2048, 256)]
    cases = []
    for i, (M, N, K, tail) in enumerate(shapes):
        p, a, wq, r, rq = _tail_case(M, N, K, max(tail, 96), seed=20 + i)
        cases.append((a, gbw.weight_from_act(wq), gbw.weight_from_act(rq) if tail else None, tail, K))
    need = max(gbw.workspace_size(gbw.OP_MX_GEMM, a.rows, w.N, K + t) for a, w, rw, t, K in cases)
    shared = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for a, w, rw, t, K in cases:
        y_shared = gbw.residual_tail_gemm(a, w, rw, t, ws=shared)
        y_fresh = gbw.residual_tail_gemm(a, w, rw, t)
        assert torch.equal(y_shared, y_fresh)
    torch.cuda.synchronize()
    assert int(shared[:65536].count_nonzero()) == 0  # the counters are back at zero


def test_mx_gemm_integer_special_case_bitexact():
    """All scales 127: Y = int64 GEMM / 4 exactly (|Y| < 2^22)."""
    banner("mx_gemm integer case")
    rng = np.random.default_rng(30)
    M, N, K = 48, 96, 1024
    a = rng.integers(0, 16, (M, K))
    w = rng.integers(0, 16, (N, K))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12])
    ai = np.where(a & 8, -twice[a & 7], twice[a & 7]).astype(np.int64)
    wi = np.where(w & 8, -twice[w & 7], twice[w & 7]).astype(np.int64)
    A = _gpu_act(oracle.pack_nibbles(a), np.full((M, K // 32), 127, np.uint8))
    W = _gpu_w(oracle.pack_nibbles(w), np.full((N, K // 32), 127, np.uint8))
    want = (ai @ wi.T).astype(np.float64) / 4
    assert np.abs(want).max() < 2 ** 22
    for ws in (None, False):
        y = to_np(gbw.mx_gemm(A, W, ws=ws)).astype(np.float64)
        assert np.array_equal(y, want)


# ---------------------------------------------------------------------------
# PRQuant residual
# ---------------------------------------------------------------------------

def _tail_case(M, N, K, tail, seed=0):
    p = synth.tail_residual_problem(M, N, K, tail=tail, seed=seed, device=DEV)
    a = gbw.mx_quantize(p["x"], gbw.FMT_E8M0_B32)
    wq = gbw.mx_quantize(p["w"], gbw.FMT_E8M0_B32)
    r = gbw.mx_residual(p["w"], wq.codes, wq.scales, tail)
    rq = gbw.mx_quantize(r, gbw.FMT_E8M0_B32)
    return p, a, wq, r, rq


def test_mx_residual_bitexact():
    banner("mx_residual 256x2048 tail 256")
    p, a, wq, r, rq = _tail_case(8, 256, 2048, 256)
    wn = to_np(p["w"])
    wc, ws = on.quantize_e8m0_b32(wn)
    assert np.array_equal(to_np(wq.codes), wc) and np.array_equal(to_np(wq.scales), ws)
    ref = oracle.residual_weight(wn, wc, ws, 256)
    assert np.array_equal(to_np(r), ref)


def test_residual_tail_gemm_wide_scale_codes():
    """The tail-residual GEMM on random codes whose E8M0 scales span 1 .. 253
    (low activation scales against high weight and residual scales)."""
    banner("residual_tail_gemm wide scale codes 128x512x2048 tail 256")
    M, N, K, t = 128, 512, 2048, 256
    ac = synth.random_codes(M, K, 9, "wt.a")
    wc = synth.random_codes(N, K, 9, "wt.w")
    rc = synth.random_codes(N, t, 9, "wt.r")
    asc, wsc = synth.paired_scale_codes(M, N, K, 9, "wt.s")
    rsc = wsc[:, -t // 32:].contiguous()        # the residual blocks carry the weight's tail scales
    ref = on.residual_tail_gemm(ac.numpy(), asc.numpy(), wc.numpy(), wsc.numpy(), rc.numpy(), rsc.numpy(), t)
    assert on.last_inexact == 0
    A = _gpu_act(ac.numpy(), asc.numpy())
    y = gbw.residual_tail_gemm(A, _gpu_w(wc.numpy(), wsc.numpy()), _gpu_w(rc.numpy(), rsc.numpy()), t)
    assert_rows_close(to_np(y), ref, what="wide-scale residual_tail_gemm")


@pytest.mark.parametrize("M,N,K,tail", [(8, 256, 2048, 256), (13, 100, 1024, 96), (128, 2560, 9728, 256),
                                        (64, 64, 512, 0), (33, 200, 1024, 128), (70, 96, 2048, 256),
                                        (100, 2600, 2048, 256)])
def test_residual_tail_gemm(M, N, K, tail):
    banner(f"residual_tail_gemm {M}x{N}x{K} tail {tail}")
    p, a, wq, r, rq = _tail_case(M, N, K, max(tail, 96))
    t = tail
    w = gbw.weight_from_act(wq)
    rw = gbw.weight_from_act(rq) if t else None
    # the oracle's own chain from the synthetic inputs: Q(X), Q(W), R = W_tail - deq(Q(W))_tail, Q(R)
    ac, as_ = on.quantize_e8m0_b32(p["x"].float().cpu().numpy())
    wn = p["w"].cpu().numpy()
    wc, ws = on.quantize_e8m0_b32(wn)
    rc, rs = on.quantize_e8m0_b32(oracle.residual_weight(wn, wc, ws, max(tail, 96)))
    for g, o in ((a.codes, ac), (a.scales, as_), (wq.codes, wc), (wq.scales, ws), (rq.codes, rc), (rq.scales, rs)):
        assert np.array_equal(to_np(g), o)
    ref = on.residual_tail_gemm(ac, as_, wc, ws, rc[:, :t // 2], rs[:, :t // 32], t)
    assert on.last_inexact == 0
    y = to_np(gbw.residual_tail_gemm(a, w, rw, t))
    assert_rows_close(y, ref, what="residual_tail_gemm")
    yd = to_np(gbw.residual_tail_gemm(a, w, rw, t, ws=False))
    assert_rows_close(yd, ref, what="residual_tail_gemm serial")
    if t:
        # the augmented GEMM is the plain GEMM over [A, A_tail] x [W, R]
        at = gbw.mx_quantize(p["x"], gbw.FMT_E8M0_B32, tail_copy=t)
        wcat = torch.cat([p["w"], r], dim=1).contiguous()
        waug = gbw.weight_from_act(gbw.mx_quantize(wcat, gbw.FMT_E8M0_B32))
        yaug = to_np(gbw.mx_gemm(at, waug))
        assert_rows_close(yaug, ref, what="augmented")


def test_split_k_gemms_in_a_replayed_graph():
    """The split-K GEMMs captured in one HIP graph (their arrival counters are
    never cleared by a memset node: every call leaves them zero) and
    replayed several times, with eager work and synchronizations between the
    replays: every replay gives the eager result bit for bit."""
    banner("split-K GEMMs in a replayed graph")
    p, a, wq, r, rq = _tail_case(128, 2560, 2048, 256, seed=31)
    w, rw = gbw.weight_from_act(wq), gbw.weight_from_act(rq)
    lut = synth.lut_problem(64, N=1024, K=4096, group=128, seed=32, device=DEV, iters=4)
    ws_mx = torch.zeros(gbw.workspace_size(gbw.OP_MX_GEMM, 128, 2560, 2048 + 256), dtype=torch.uint8, device=DEV)
    ws_lut = torch.zeros(gbw.workspace_size(gbw.OP_LUT_GEMM, 64, 1024, 4096), dtype=torch.uint8, device=DEV)
    y_mx = torch.empty((128, 2560), dtype=torch.float32, device=DEV)
    y_lut = torch.empty((64, 1024), dtype=torch.float32, device=DEV)

    def calls():
        gbw.residual_tail_gemm(a, w, rw, 256, out=y_mx, ws=ws_mx)
        gbw.lut_gemm(lut["x"], lut["idx"], lut["centroids"], 128, out=y_lut, ws=ws_lut)

    calls()
    torch.cuda.synchronize()
    eager_mx, eager_lut = y_mx.clone(), y_lut.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    for rep in range(4):
        y_mx.fill_(float("nan"))
        y_lut.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_mx, eager_mx), f"replay {rep}: residual_tail_gemm"
        assert torch.equal(y_lut, eager_lut), f"replay {rep}: lut_gemm"
        calls()  # eager work between replays, on the same workspaces
        torch.cuda.synchronize()
        assert torch.equal(y_mx, eager_mx) and torch.equal(y_lut, eager_lut)
    assert int(ws_mx[:65536].count_nonzero()) == 0 and int(ws_lut[:65536].count_nonzero()) == 0
