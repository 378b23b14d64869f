"""Pins for the oracle's GEMMs: MX GEMM, tail-residual GEMM, LUT GEMM, VQ decode.

The checks are exact rational brute force on tiny inputs, integer special
cases against int64 matmuls, closed forms, and identities the pages state
(PRQuant §4: the block-aligned tail copy equals quantizing the concatenation;
the augmented GEMM equals the main plus residual product; Eq. (1)'s channel
permutation leaves the product unchanged).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _e2m1_frac(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def _brute_mx(a_codes, a_sc, w_codes, w_sc):
    """Exact rational GEMM straight from the bit fields, one term at a time."""
    M, N = a_codes.shape[0], w_codes.shape[0]
    K = a_codes.shape[1] * 2
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                ca = (int(a_codes[m, k // 2]) >> (4 * (k % 2))) & 0xF
                cw = (int(w_codes[n, k // 2]) >> (4 * (k % 2))) & 0xF
                sa = Fraction(2) ** (int(a_sc[m, k // 32]) - 127)
                sw = Fraction(2) ** (int(w_sc[n, k // 32]) - 127)
                acc += _e2m1_frac(ca) * sa * _e2m1_frac(cw) * sw
            y[m][n] = acc
    return y


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 2, 96), (4, 4, 128)])
def test_mx_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    # scale spread kept so a dot product spans < 53 bits (then fp64 is exact)
    a_sc = rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
    w_sc = rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
    y = oracle.mx_gemm(a_codes, a_sc, w_codes, w_sc)
    ref = _brute_mx(a_codes, a_sc, w_codes, w_sc)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(y[m, n])) == ref[m][n]


def test_mx_gemm_all_codes_enumerated():
    """Every (a, w) element code pair appears once along K=256."""
    a = np.repeat(np.arange(16), 16)
    w = np.tile(np.arange(16), 16)
    ac = oracle.pack_nibbles(a[None, :])
    wc = oracle.pack_nibbles(w[None, :])
    sc = np.full((1, 8), 127, np.uint8)
    y = oracle.mx_gemm(ac, sc, wc, sc)
    vals = [_e2m1_frac(c) for c in range(16)]
    assert Fraction(float(y[0, 0])) == sum(vals) * sum(vals)


def test_mx_gemm_integer_special_case():
    """All scales 127: element values are multiples of 0.5 and Y is a quarter
    of an int64 GEMM of twice the values."""
    rng = np.random.default_rng(7)
    M, N, K = 16, 24, 512
    a = rng.integers(0, 16, (M, K))
    w = rng.integers(0, 16, (N, K))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12])
    ai = np.where(a & 8, -twice[a & 7], twice[a & 7]).astype(np.int64)
    wi = np.where(w & 8, -twice[w & 7], twice[w & 7]).astype(np.int64)
    sc = np.full((M, K // 32), 127, np.uint8)
    scw = np.full((N, K // 32), 127, np.uint8)
    y = oracle.mx_gemm(oracle.pack_nibbles(a), sc, oracle.pack_nibbles(w), scw)
    assert np.array_equal(y * 4, (ai @ wi.T).astype(np.float64))


def test_mx_gemm_k_permutation_and_transpose():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    w = (rng.standard_normal((12, 256)) * 0.02).astype(np.float32)
    ac, as_ = oracle.quantize_e8m0_b32(x)
    wc, ws = oracle.quantize_e8m0_b32(w)
    y = oracle.mx_gemm(ac, as_, wc, ws)
    # permuting whole 32-blocks of K on both sides leaves Y unchanged (Eq. (1))
    bp = rng.permutation(8)
    colp = (bp[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    xp, wp = x[:, colp], w[:, colp]
    acp, asp = oracle.quantize_e8m0_b32(xp)
    wcp, wsp = oracle.quantize_e8m0_b32(wp)
    assert np.array_equal(oracle.mx_gemm(acp, asp, wcp, wsp), y)
    # swapping the roles of A and W gives Y^T
    assert np.array_equal(oracle.mx_gemm(wc, ws, ac, as_), y.T)


@pytest.mark.parametrize("fmt", ["e4m3_b16", "e5m3_b16"])
def test_mx_gemm_tensor_scaled_formats(fmt):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    w = (rng.standard_normal((7, 64)) * 0.02).astype(np.float32)
    q = oracle.quantize_e4m3_b16 if fmt == "e4m3_b16" else oracle.quantize_e5m3_b16
    ac, as_, ats = q(x)
    wc, ws, wts = q(w)
    y = oracle.mx_gemm(ac, as_, wc, ws, fmt, ats, wts)
    a = oracle.dequantize(ac, as_, fmt, ats)
    b = oracle.dequantize(wc, ws, fmt, wts)
    # brute force over exact rationals
    for m in range(5):
        for n in range(7):
            ref = sum(Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(64))
            assert abs(Fraction(float(y[m, n])) - ref) <= abs(ref) * Fraction(1, 2 ** 50)
    # sanity: W4A4 output error is of the size FP4 quantization gives (y-NRMSE ~0.1-0.2)
    ref = x.astype(np.float64) @ w.T.astype(np.float64)
    assert np.linalg.norm(y - ref) < 0.3 * np.linalg.norm(ref)


# ---------------------------------------------------------------------------
# PRQuant tail residual
# ---------------------------------------------------------------------------

def _tail_problem(M=8, N=16, K=512, tail=128, seed=10):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, K - 20:] *= 50
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return x, w, tail


def test_residual_tail_gemm_equals_augmented_concat():
    x, w, tail = _tail_problem()
    K = x.shape[1]
    ac, as_ = oracle.quantize_e8m0_b32(x)
    wc, ws = oracle.quantize_e8m0_b32(w)
    r = oracle.residual_weight(w, wc, ws, tail)
    rc, rs = oracle.quantize_e8m0_b32(r)
    y = oracle.residual_tail_gemm(ac, as_, wc, ws, rc, rs, tail)
    # the augmented form: [A, A_tail] against Q([W, R]) in one GEMM over K+tail
    acat, ascat = oracle.tail_copy(ac, as_, tail)
    wcat, wscat = oracle.quantize_e8m0_b32(np.concatenate([w, r], axis=1))
    assert np.array_equal(wcat[:, :K // 2], wc)          # W_aug^q = [Q(W), Q(R)]
    assert np.array_equal(oracle.mx_gemm(acat, ascat, wcat, wscat), y)
    # the tail copy equals quantizing the concatenation [X, X_tail] (block aligned)
    qc, qs = oracle.quantize_e8m0_b32(np.concatenate([x, x[:, K - tail:]], axis=1))
    assert np.array_equal(qc, acat) and np.array_equal(qs, ascat)


def test_residual_reduces_error_and_special_cases():
    x, w, tail = _tail_problem()
    ac, as_ = oracle.quantize_e8m0_b32(x)
    wc, ws = oracle.quantize_e8m0_b32(w)
    r = oracle.residual_weight(w, wc, ws, tail)
    rc, rs = oracle.quantize_e8m0_b32(r)
    y0 = oracle.mx_gemm(ac, as_, wc, ws)
    # tail = 0 reduces to the plain GEMM
    assert np.array_equal(oracle.residual_tail_gemm(ac, as_, wc, ws, rc[:, :0], rs[:, :0], 0), y0)
    # R is exactly W_tail - deq(Q(W))_tail, so W_tail = deq + R in fp64
    K = x.shape[1]
    deq = oracle.dequantize(wc, ws, "e8m0_b32")
    assert np.array_equal(deq[:, K - tail:] + r.astype(np.float64), w[:, K - tail:].astype(np.float64))
    # the residual term moves the weight closer: |W - (deq + deq(Rq))| < |W - deq| on the tail
    rdeq = oracle.dequantize(rc, rs, "e8m0_b32")
    e0 = np.linalg.norm(w[:, K - tail:] - deq[:, K - tail:])
    e1 = np.linalg.norm(w[:, K - tail:] - deq[:, K - tail:] - rdeq)
    assert e1 < 0.25 * e0
    # weights already on the MXFP4 grid: R = 0, Rq all zero, same Y bit for bit
    wg = deq.astype(np.float32)
    wgc, wgs = oracle.quantize_e8m0_b32(wg)
    rg = oracle.residual_weight(wg, wgc, wgs, tail)
    assert np.all(rg == 0)
    rgc, rgs = oracle.quantize_e8m0_b32(rg)
    assert np.all(rgc == 0) and np.all(rgs == 0)
    assert np.array_equal(oracle.residual_tail_gemm(ac, as_, wgc, wgs, rgc, rgs, tail),
                          oracle.mx_gemm(ac, as_, wgc, wgs))


# ---------------------------------------------------------------------------
# LUT (codebook) GEMM
# ---------------------------------------------------------------------------

def _bf16_bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_lut_decode_brute_force():
    rng = np.random.default_rng(11)
    N, K, group = 3, 256, 128
    idx = rng.integers(0, 16, (N, K))
    cents = rng.standard_normal((N, K // group, 16)).astype(np.float16)
    w = oracle.lut_decode(oracle.pack_nibbles(idx), cents, group)
    for n in range(N):
        for k in range(K):
            assert w[n, k] == float(cents[n, k // group, idx[n, k]])


def test_lut_gemm_integer_special_case():
    """Centroids j - 8 and integer X in [-8, 8]: Y is an exact integer GEMM
    of (idx - 8) with X."""
    rng = np.random.default_rng(12)
    M, N, K, group = 8, 40, 512, 128
    idx = rng.integers(0, 16, (N, K))
    cents = np.tile((np.arange(16) - 8).astype(np.float16), (N, K // group, 1))
    xi = rng.integers(-8, 9, (M, K))
    y = oracle.lut_gemm(_bf16_bits(xi), oracle.pack_nibbles(idx), cents, group)
    assert np.array_equal(y, (xi @ (idx - 8).T).astype(np.float64))


def test_lut_gemm_all_zero_indices_closed_form():
    rng = np.random.default_rng(13)
    M, N, K, group = 4, 6, 384, 128
    cents = rng.standard_normal((N, K // group, 16)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xb = _bf16_bits(x)
    y = oracle.lut_gemm(xb, np.zeros((N, K // 2), np.uint8), cents, group)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    gsum = xf.reshape(M, K // group, group).sum(-1)            # per-group sums of X
    ref = gsum @ cents[:, :, 0].astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# VQ -> MX decode (MXCode PreScale)
# ---------------------------------------------------------------------------

def test_vq_lossless_case_reproduces_mx_codes():
    """A QBlock with at most 256 distinct 4-element keys is represented
    exactly: decoding the VQ gives back the MXFP4 codes."""
    rng = np.random.default_rng(14)
    N, K, qb = 128, 128, 64
    # few distinct values so each QBlock has <= 256 distinct keys
    w = rng.choice([-0.04, 0.0, 0.03], size=(N, K)).astype(np.float32)
    codes, scales = oracle.quantize_e8m0_b32(w)
    el = oracle.unpack_nibbles(codes).astype(np.int64)                   # [N][K]
    keys = el[:, 0::4] | (el[:, 1::4] << 4) | (el[:, 2::4] << 8) | (el[:, 3::4] << 12)
    cb = np.zeros((N // qb, K // qb, 256), np.uint16)
    idx = np.zeros((N, K // 4), np.uint8)
    for bn in range(N // qb):
        for bk in range(K // qb):
            blk = keys[bn * qb:(bn + 1) * qb, bk * qb // 4:(bk + 1) * qb // 4]
            uniq = np.unique(blk)
            assert len(uniq) <= 256
            cb[bn, bk, :len(uniq)] = uniq
            idx[bn * qb:(bn + 1) * qb, bk * qb // 4:(bk + 1) * qb // 4] = np.searchsorted(uniq, blk)
    assert np.array_equal(oracle.vq_decode_codes(idx, cb, qb), codes)
    assert np.array_equal(oracle.vq_dequantize(idx, cb, scales, qb), oracle.dequantize(codes, scales, "e8m0_b32"))


def test_vq_lut_size_and_bpe():
    """A 256-entry table of 16-bit keys is 512 B (within the 1 KB LUT limit);
    per 64x64 QBlock: 1024 B of indices + 512 B LUT + 128 B of E8M0 = 3.25 bits/weight."""
    cb = np.zeros((1, 1, 256), np.uint16)
    assert cb.nbytes == 512 <= 1024
    idx = np.zeros((64, 16), np.uint8)
    sc = np.zeros((64, 2), np.uint8)
    assert (idx.nbytes + cb.nbytes + sc.nbytes) * 8 / (64 * 64) == 3.25
