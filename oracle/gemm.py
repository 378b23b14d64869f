"""GEMM references: MX GEMM, tail-residual GEMM, LUT GEMM, VQ decode (MXCode
PreScale, PostScale and PreScale+ block scales).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Each GEMM decodes its operands to float64 and contracts with a float64
matmul.  For the block-scaled formats every product e2m1*e2m1*2^(sa+sb-254)
(or (e2m1*sd)_a*(e2m1*sd)_w) has at most 12 significant bits and, for the
value ranges used here, a dot product spans far fewer than 53 bits, so the
float64 result is the exact value of the quantized GEMM whatever order the
matmul sums in.  Tiny brute-force cases with exact rationals pin this.

Layout conventions: activations A are [M][K]; weights W are [N][K] with K
contiguous (a "K x N" weight stored per output column); Y = deq(A) deq(W)^T.
"""

import numpy as np

from .formats import (
    FMT_E4M3_B16,
    TENSOR_SCALED,
    FMT_E8M0_B32,
    bf16_bits_to_f32,
    dequantize,
    pack_nibbles,
    unpack_nibbles,
)


def mx_gemm(a_codes, a_scales, w_codes, w_scales, fmt=FMT_E8M0_B32, a_ts=None, w_ts=None):
    """Y[m][n] = sum_k deq(A)[m][k] * deq(W)[n][k] in float64.

    For E4M3-B16 and E5M3-B16 the tensor scales are applied once to the exact sum:
    Y = S_Ta * S_Tw * sum_k (e2m1*sd)_a (e2m1*sd)_w.
    """
    a = dequantize(a_codes, a_scales, fmt)
    w = dequantize(w_codes, w_scales, fmt)
    y = a @ w.T
    if fmt in TENSOR_SCALED:
        sa = 1.0 if a_ts is None else float(np.float32(a_ts))
        sw = 1.0 if w_ts is None else float(np.float32(w_ts))
        y = y * sa * sw
    return y


def residual_weight(w_f32, w_codes, w_scales, tail):
    """Offline weight residual of PRQuant §4 Eq. (2): R = W_tail - Q(W_tail).

    W is [N][K] fp32; (w_codes, w_scales) its E8M0-B32 quantization over all
    K.  Because the tail starts on a 32-element block boundary, the tail of
    Q(W) is Q(W_tail).  R is formed as one fp32 subtraction per element.
    """
    w = np.asarray(w_f32, dtype=np.float32)
    N, K = w.shape
    if tail % 32 or tail > K or tail < 0:
        raise ValueError("tail must be a multiple of 32 and at most K")
    deq = dequantize(w_codes, w_scales, FMT_E8M0_B32).astype(np.float32)  # exact in fp32
    return (w[:, K - tail:] - deq[:, K - tail:]).astype(np.float32)


def tail_copy(codes, scales, tail):
    """PRQuant online copy (§4 "Kernel design"): append the quantized tail
    blocks of each row, with their scales -> rows of width K + tail."""
    if tail == 0:
        return codes.copy(), scales.copy()
    K = codes.shape[1] * 2
    c = np.concatenate([codes, codes[:, (K - tail) // 2:]], axis=1)
    s = np.concatenate([scales, scales[:, (K - tail) // 32:]], axis=1)
    return c, s


def residual_tail_gemm(a_codes, a_scales, w_codes, w_scales, r_codes, r_scales, tail):
    """Augmented MXFP4 GEMM (PRQuant §4, W_aug^q = Q([W, R_W])):

    Y = deq(A) deq(W)^T + deq(A[:, K-tail:]) deq(R)^T

    i.e. one GEMM over K + tail whose activation is [A, A_tail] and whose
    weight is [W, R].  R is [N][tail] E8M0-B32.
    """
    y = mx_gemm(a_codes, a_scales, w_codes, w_scales, FMT_E8M0_B32)
    if tail:
        K = a_codes.shape[1] * 2
        at_c = a_codes[:, (K - tail) // 2:]
        at_s = a_scales[:, (K - tail) // 32:]
        y = y + mx_gemm(at_c, at_s, r_codes, r_scales, FMT_E8M0_B32)
    return y


# ----------------------------------------------------------------------------
# Codebook / LUT weights (CodeQuant)
# ----------------------------------------------------------------------------

def lut_decode(idx_packed, centroids_f16, group):
    """Decoded weight W[n][k] = C[n][k // group][idx[n][k]] as float64.

    idx_packed [N][K/2] (4-bit indices, element 2i in bits 3:0);
    centroids_f16 [N][K/group][16] float16.
    """
    idx = unpack_nibbles(idx_packed).astype(np.int64)
    N, K = idx.shape
    c = np.asarray(centroids_f16).astype(np.float64)
    g = np.arange(K) // group
    return c[np.arange(N)[:, None], g[None, :], idx]


def lut_gemm(x_bf16_bits, idx_packed, centroids_f16, group):
    """Y[m][n] = sum_k bf16(X)[m][k] * fp16(C[n][k/group][idx[n][k]]) in float64."""
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    w = lut_decode(idx_packed, centroids_f16, group)
    return x @ w.T


# ----------------------------------------------------------------------------
# VQ -> MX weights (MXCode PreScale)
# ----------------------------------------------------------------------------

def vq_decode_codes(idx, codebook, qblock=64):
    """MXCode PreScale decode to the MXFP4 code stream.

    idx [N][K/4] uint8: vector j of row n covers elements 4j..4j+3;
    codebook [N/qblock][K/qblock][256] uint16: 4 E2M1 codes, element i of the
    vector in bits 4i+3:4i; QBlock (n // qblock, k // qblock) owns the table.
    Returns packed E2M1 codes [N][K/2].
    """
    idx = np.asarray(idx).astype(np.int64)
    N, KV = idx.shape
    K = KV * 4
    cb = np.asarray(codebook).astype(np.int64)
    rb = (np.arange(N) // qblock)[:, None]
    kb = (np.arange(KV) * 4 // qblock)[None, :]
    keys = cb[rb, kb, idx]                                   # [N][K/4]
    nib = np.stack([(keys >> (4 * i)) & 0xF for i in range(4)], axis=-1)
    return pack_nibbles(nib.reshape(N, K))


def vq_dequantize(idx, codebook, scales, qblock=64):
    """Decoded VQ weight as float64: E2M1 code from the QBlock LUT times the
    E8M0-B32 prescale."""
    codes = vq_decode_codes(idx, codebook, qblock)
    return dequantize(codes, scales, FMT_E8M0_B32)


# ----------------------------------------------------------------------------
# MXCode PostScale and PreScale+: where the block scales come from
# ----------------------------------------------------------------------------
# The E2M1 code stream is the PreScale one in both (vq_decode_codes); only the
# E8M0 block scale of each 32-element block along K is stored differently.

def postscale_block_scales(qscales, K, qblock=64, block=32):
    """MXCode PostScale (abstract: the learned codebook itself is quantized
    to MXFP4).  Reading: the QBlock's codebook is one block-scaled FP4
    tensor with one scale, so every block of weights in QBlock
    (n // qblock, k // qblock) has that scale.

    qscales [N/qblock][K/qblock] uint8 -> block scale codes [N][K/block]
    (block 32 for E8M0-B32, 16 for E4M3-B16 and E5M3-B16).
    """
    qs = np.asarray(qscales, dtype=np.uint8)
    N = qs.shape[0] * qblock
    assert qs.shape[1] * qblock == K and K % block == 0
    rows = np.arange(N) // qblock
    cols = (np.arange(K // block) * block) // qblock
    return qs[rows[:, None], cols[None, :]]


def prescale_plus_block_scales(sidx, scale_codebook, ds=8):
    """MXCode PreScale+ (abstract: the PreScale scales are compressed by VQ;
    Table 4 caption: Ks = 256 entries, ds = 8).  Reading: the block scales of
    one row are cut along K into vectors of ds consecutive scales; vector j of
    row n is entry sidx[n][j] of the matrix's scale codebook.

    sidx [N][K/(block ds)] uint8, scale_codebook [Ks][ds] scale codes
    -> block scale codes [N][K/block] (block 32 for E8M0-B32, 16 for
    E4M3-B16 and E5M3-B16).
    """
    si = np.asarray(sidx).astype(np.int64)
    scb = np.asarray(scale_codebook, dtype=np.uint8)
    assert scb.shape[1] == ds
    return scb[si].reshape(si.shape[0], si.shape[1] * ds)


def mxcode_bpe(method, block, qblock, N, K, d=4, n_entries=256, ks=256, ds=8, scale_bits=8):
    """Stored bits per weight element as MXCode Table 2 counts them: VQ
    indices, FP4 codebooks and scales (Table 1: the FP32 tensor scale of the
    16-element formats is not counted).

    method: "native" (plain block-scaled FP4), "prescale" (per-block scales
    kept), "postscale" (one scale per QBlock codebook), "prescale_plus"
    (block scales vector-quantized, one Ks x ds scale codebook per matrix).
    block: elements per scale block (32 for E8M0-B32, 16 for E4M3-B16).
    """
    if method == "native":
        return 4.0 + scale_bits / block
    idx = np.log2(n_entries) / d                      # one index per d weights
    fp4_codebook = n_entries * d * 4 / qblock ** 2     # one table per QBlock
    if method == "prescale":
        return idx + fp4_codebook + scale_bits / block
    if method == "postscale":
        return idx + fp4_codebook + scale_bits / qblock ** 2
    if method == "prescale_plus":
        scale_idx = np.log2(ks) / (ds * block)         # one index per ds scales
        scale_codebook = ks * ds * scale_bits / (N * K)
        return idx + fp4_codebook + scale_idx + scale_codebook
    raise ValueError(method)
