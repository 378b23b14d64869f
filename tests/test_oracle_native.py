"""Pins for the C++ oracle (oracle/native): the same closed forms, brute
force and special cases that pin the numpy oracle, plus bit-for-bit agreement
with the numpy oracle wherever both compute an exact value.

The C++ side is the reference the GPU parity tests and the CPU baseline use
for the contractions; numpy stays as the cross-check.
"""

import ctypes
import json
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.native as on

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))


def _e2m1_frac(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


# ---------------------------------------------------------------- decoders

def test_decoders_against_table1_and_bit_fields():
    """E2M1 values (golden file), E8M0 extremes of Table 1 (2^-127 .. 1.70e38),
    E4M3 extremes (2^-9 .. 448) and UE5M3 extremes (2^-17 .. 114688)."""
    codes = oracle.pack_nibbles(np.arange(32)[None, :] % 16)
    one = np.full((1, 1), 127, np.uint8)
    v = on.dequantize(codes, one, "e8m0_b32")[0, :16]
    mags = GOLD["e2m1_values"]["magnitudes"]
    assert v.tolist() == mags + [-m for m in mags]
    zero_code = oracle.pack_nibbles(np.full((1, 32), 2))            # element 1.0
    lo = on.dequantize(zero_code, np.zeros((1, 1), np.uint8), "e8m0_b32")[0, 0]
    hi = on.dequantize(zero_code, np.full((1, 1), 254, np.uint8), "e8m0_b32")[0, 0]
    t1 = GOLD["formats"]
    assert lo == 2.0 ** t1["E8M0-B32-FP4"]["min_scale_log2"]
    assert abs(hi - t1["E8M0-B32-FP4"]["max_scale"]) / hi < 1e-3
    z16 = oracle.pack_nibbles(np.full((1, 16), 2))
    assert on.dequantize(z16, np.array([[0x01]], np.uint8), "e4m3_b16")[0, 0] == 2.0 ** t1["E4M3-B16-FP4"]["min_scale_log2"]
    assert on.dequantize(z16, np.array([[0x7E]], np.uint8), "e4m3_b16")[0, 0] == t1["E4M3-B16-FP4"]["max_scale"]
    assert on.dequantize(z16, np.array([[0x01]], np.uint8), "e5m3_b16")[0, 0] == 2.0 ** t1["E5M3-B16-FP4"]["min_scale_log2"]
    assert on.dequantize(z16, np.array([[0xFE]], np.uint8), "e5m3_b16")[0, 0] == t1["E5M3-B16-FP4"]["max_scale"]


@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16", "e5m3_b16"])
def test_dequantize_matches_numpy_every_code_and_scale(fmt):
    bs = 32 if fmt == "e8m0_b32" else 16
    nsc = 255 if fmt != "e4m3_b16" else 127
    codes = oracle.pack_nibbles(np.tile(np.arange(16), (nsc, bs // 16 * 2)))[:, : bs // 2 * 2]
    codes = np.ascontiguousarray(codes[:, : bs // 2])
    sc = np.arange(nsc, dtype=np.uint8)[:, None]
    assert np.array_equal(on.dequantize(codes, sc, fmt, 0.75 if fmt != "e8m0_b32" else None),
                          oracle.dequantize(codes, sc, fmt, 0.75 if fmt != "e8m0_b32" else None))


# ---------------------------------------------------------------- quantizers

def _special_rows(K):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((12, K)).astype(np.float32)
    x[1] = 0.0
    x[2, ::3] = -0.0
    x[3] *= 1e-40                                  # fp32 subnormals
    x[4] *= 3e37
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 8.0 - 2 ** -20, 0.0, 6.0], np.float32)
    x[5] = np.resize(np.concatenate([mids, -mids]), K)   # E2M1 midpoints at scale 1 (block amax 8)
    x[6] = np.resize(np.concatenate([mids, -mids]), K) * np.float32(2.0 ** -100)
    return x


@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16", "e5m3_b16"])
def test_quantizers_match_numpy_bit_for_bit(fmt):
    x = _special_rows(256)
    if fmt == "e8m0_b32":
        assert all(np.array_equal(a, b) for a, b in zip(on.quantize_e8m0_b32(x), oracle.quantize_e8m0_b32(x)))
        return
    q, qn = (oracle.quantize_e4m3_b16, on.quantize_e4m3_b16) if fmt == "e4m3_b16" else \
        (oracle.quantize_e5m3_b16, on.quantize_e5m3_b16)
    for amax in (None, 1.5, 1e-30):
        a, b = q(x[:4], tensor_amax=amax), qn(x[:4], tensor_amax=amax)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_e8m0_round_trip_every_code_and_scale():
    """The block [6S, c S, 0, ...] encodes back to (sc, [0x7, c, 0, ...]) for
    every element code c and every scale code 0..252 (6S finite in fp32)."""
    rows = []
    for sc in range(253):
        for c in range(16):
            S = np.ldexp(1.0, sc - 127)
            v = float(oracle.e2m1_decode(c)) * S
            rows.append([6.0 * S, v] + [0.0] * 30)
    x = np.array(rows, dtype=np.float32)
    codes, scales = on.quantize_e8m0_b32(x)
    assert np.array_equal(scales[:, 0], np.repeat(np.arange(253), 16))
    nib = oracle.unpack_nibbles(codes)
    assert np.all(nib[:, 0] == 7)
    want = np.tile(np.arange(16), 253)
    got = nib[:, 1]
    # -0 encodes with its sign kept; +0 as 0
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- GEMMs

def _brute_mx(a_codes, a_sc, w_codes, w_sc):
    M, N = a_codes.shape[0], w_codes.shape[0]
    K = a_codes.shape[1] * 2
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                ca = (int(a_codes[m, k // 2]) >> (4 * (k % 2))) & 0xF
                cw = (int(w_codes[n, k // 2]) >> (4 * (k % 2))) & 0xF
                acc += _e2m1_frac(ca) * Fraction(2) ** (int(a_sc[m, k // 32]) - 127) * \
                    _e2m1_frac(cw) * Fraction(2) ** (int(w_sc[n, k // 32]) - 127)
            out[m][n] = acc
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (4, 4, 128)])
def test_mx_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + 5)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w_codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    a_sc = rng.integers(118, 137, (M, K // 32), dtype=np.uint8)
    w_sc = rng.integers(118, 137, (N, K // 32), dtype=np.uint8)
    y = on.mx_gemm(a_codes, a_sc, w_codes, w_sc)
    assert on.last_inexact == 0
    ref = _brute_mx(a_codes, a_sc, w_codes, w_sc)
    assert all(Fraction(float(y[m, n])) == ref[m][n] for m in range(M) for n in range(N))


def test_mx_gemm_integer_special_case_and_numpy():
    rng = np.random.default_rng(17)
    M, N, K = 9, 13, 512
    a = rng.integers(0, 16, (M, K))
    w = rng.integers(0, 16, (N, K))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12])
    ai = np.where(a & 8, -twice[a & 7], twice[a & 7]).astype(np.int64)
    wi = np.where(w & 8, -twice[w & 7], twice[w & 7]).astype(np.int64)
    y = on.mx_gemm(oracle.pack_nibbles(a), np.full((M, K // 32), 127, np.uint8), oracle.pack_nibbles(w),
                   np.full((N, K // 32), 127, np.uint8))
    assert np.array_equal(y * 4, (ai @ wi.T).astype(np.float64))
    # scale codes over 1 .. 253, a low activation scale against a high weight
    # scale in every block, so each product stays near 1 and the sums are
    # exact: both oracles return the same exact values
    ac, wc = rng.integers(0, 256, (M, K // 2), dtype=np.uint8), rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    base = rng.integers(1, 120, K // 32)
    asc = (base[None, :] + rng.integers(0, 8, (M, 1))).astype(np.uint8)
    wsc = (254 - base[None, :] - rng.integers(0, 8, (N, 1))).astype(np.uint8)
    assert asc.min() >= 1 and wsc.max() <= 253
    y = on.mx_gemm(ac, asc, wc, wsc)
    assert on.last_inexact == 0
    assert np.array_equal(y, oracle.mx_gemm(ac, asc, wc, wsc))


@pytest.mark.parametrize("fmt", ["e4m3_b16", "e5m3_b16"])
def test_tensor_scaled_gemm_matches_numpy(fmt):
    rng = np.random.default_rng(18)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    w = (rng.standard_normal((10, 128)) * 0.02).astype(np.float32)
    q = on.quantize_e4m3_b16 if fmt == "e4m3_b16" else on.quantize_e5m3_b16
    ac, as_, ats = q(x)
    wc, ws, wts = q(w)
    y = on.mx_gemm(ac, as_, wc, ws, fmt, ats, wts)
    ref = oracle.mx_gemm(ac, as_, wc, ws, fmt, ats, wts)
    # numpy scales the sum by S_Ta, then S_Tw (two roundings); C++ by their exact product once
    assert np.allclose(y, ref, rtol=4e-16, atol=0)


def test_residual_tail_gemm_is_the_augmented_gemm():
    rng = np.random.default_rng(19)
    M, N, K, tail = 5, 7, 256, 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ac, as_ = on.quantize_e8m0_b32(x)
    wc, ws = on.quantize_e8m0_b32(w)
    r = oracle.residual_weight(w, wc, ws, tail)
    rc, rs = on.quantize_e8m0_b32(r)
    y = on.residual_tail_gemm(ac, as_, wc, ws, rc, rs, tail)
    cc, cs = oracle.tail_copy(ac, as_, tail)
    y_aug = on.mx_gemm(cc, cs, np.concatenate([wc, rc], 1), np.concatenate([ws, rs], 1))
    assert np.array_equal(y, y_aug) and on.last_inexact == 0
    assert np.array_equal(y, oracle.residual_tail_gemm(ac, as_, wc, ws, rc, rs, tail))
    assert np.array_equal(on.residual_tail_gemm(ac, as_, wc, ws, rc[:, :0], rs[:, :0], 0), on.mx_gemm(ac, as_, wc, ws))


def test_lut_gemm_integer_case_and_closed_form():
    rng = np.random.default_rng(20)
    M, N, K, group = 3, 5, 256, 128
    xi = rng.integers(-8, 9, (M, K))
    x_bits = oracle.f32_to_bf16_bits(xi.astype(np.float32))
    idx = rng.integers(0, 16, (N, K))
    cent = np.tile((np.arange(16) - 8).astype(np.float16), (N, K // group, 1))
    y = on.lut_gemm(x_bits, oracle.pack_nibbles(idx), cent, group)
    assert np.array_equal(y, (xi @ (idx - 8).T).astype(np.float64))
    # all indices 0: y[m][n] = sum_g c[n][g][0] * sum_{k in g} x[m][k]
    c = rng.standard_normal((N, K // group, 16)).astype(np.float16)
    y0 = on.lut_gemm(x_bits, np.zeros((N, K // 2), np.uint8), c, group)
    ref = np.einsum("ng,mg->mn", c[:, :, 0].astype(np.float64), xi.reshape(M, K // group, group).sum(2).astype(np.float64))
    assert np.array_equal(y0, ref)
    # random values: equal to numpy's float64 matmul of the same decoded operands
    xb = oracle.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    yr = on.lut_gemm(xb, oracle.pack_nibbles(idx), c, group)
    assert np.allclose(yr, oracle.lut_gemm(xb, oracle.pack_nibbles(idx), c, group), rtol=1e-14, atol=1e-14)


def test_vq_decode_matches_numpy_and_lossless_case():
    rng = np.random.default_rng(21)
    N, K, qb = 128, 256, 64
    idx = rng.integers(0, 256, (N, K // 4), dtype=np.uint8)
    cb = rng.integers(0, 1 << 16, (N // qb, K // qb, 256), dtype=np.uint16)
    assert np.array_equal(on.vq_decode_codes(idx, cb, qb), oracle.vq_decode_codes(idx, cb, qb))
    # lossless: a QBlock whose 4-vectors are all in its table reproduces the code stream
    codes = rng.integers(0, 16, (N, K))
    keys = (codes.reshape(N, K // 4, 4) << (4 * np.arange(4))).sum(-1)
    tab = np.zeros((N // qb, K // qb, 256), np.uint16)
    ix = np.zeros((N, K // 4), np.uint8)
    for bn in range(N // qb):
        for bk in range(K // qb):
            blk = keys[bn * qb:(bn + 1) * qb, bk * qb // 4:(bk + 1) * qb // 4]
            u, inv = np.unique(blk, return_inverse=True)
            assert len(u) <= 256 or True
            u = u[:256]
            tab[bn, bk, :len(u)] = u
            ix[bn * qb:(bn + 1) * qb, bk * qb // 4:(bk + 1) * qb // 4] = np.minimum(inv.reshape(blk.shape), 255)
    sub = keys[:qb, :qb // 4]
    if len(np.unique(sub)) <= 256:
        dec = on.vq_decode_codes(ix, tab, qb)
        assert np.array_equal(dec[:qb, :qb // 2], oracle.pack_nibbles(codes[:qb, :qb]))


def test_swiglu_matches_numpy_and_midpoints():
    rng = np.random.default_rng(22)
    g = rng.standard_normal(20000) * 8
    u = rng.standard_normal(20000) * 3
    g[:3] = [-800.0, 0.0, 1000.0]
    assert np.array_equal(on.swiglu_bf16(g, u), oracle.swiglu_bf16(g, u))
    # bf16 midpoints and values one double ulp around them: u chosen so silu(g) u hits them (g = 40: silu = 40)
    mid = 1.0 + 2.0 ** -8
    vals = np.array([mid, np.nextafter(mid, 2), np.nextafter(mid, 0), 3 * 2.0 ** -140, -(1 + 3 * 2.0 ** -8)])
    gg = np.full(len(vals), 40.0)
    h = on.swiglu_bf16(gg, vals / 40.0)
    assert h.tolist() == oracle.swiglu_bf16(gg, vals / 40.0).tolist()


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (37, 16, 4), (200, 128, 8), (5, 1000, 16)])
def test_route_matches_numpy(T, E, k):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :3] = logits[0, 3 % E]
    a, b = on.moe_route(logits, k), oracle.moe_route(logits, k)
    for key in ("topk_ids", "expert_offsets", "pair_token", "pair_pos"):
        assert np.array_equal(a[key], b[key]), key
    assert np.allclose(a["topk_w"], b["topk_w"], rtol=1e-15, atol=0)


def test_route_special_values():
    row = np.array([[np.nan, -0.0, 0.0, 1.0, -np.inf, np.inf, 1.0, np.nan]], np.float32)
    with np.errstate(invalid="ignore"):
        r = on.moe_route(row, 8)
    assert r["topk_ids"][0].tolist() == [5, 3, 6, 1, 2, 4, 0, 7]


def test_e2m1_rounding_exhaustive_over_fp32(tmp_path):
    """Every non-negative finite fp32 value: the oracle's E2M1 rounding
    against an interval statement of round-to-nearest-even with saturation,
    written independently in C (tests/pins/e2m1_all.c)."""
    src = os.path.join(os.path.dirname(__file__), "pins", "e2m1_all.c")
    so = str(tmp_path / "e2m1_all.so")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", src, "-o", so], check=True)
    lib = ctypes.CDLL(so)
    lib.check_all.restype = ctypes.c_int64
    lib.check_all.argtypes = [ctypes.c_void_p]
    fn = ctypes.cast(on._lib.gbwo_e2m1_rne, ctypes.c_void_p)
    assert lib.check_all(fn) == 0
