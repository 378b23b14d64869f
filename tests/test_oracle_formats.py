"""Pins for the oracle's block-scaled FP4 codecs and quantizers.

Each test checks the oracle against something other than itself: values the
MXCode page prints in its Table 1 (tests/golden/mx_formats.json), the E2M1
bit-field definition, torch's float8_e4m3fn decode/cast, an independent
interval table for round-to-nearest-even, round trips and invariants.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))


# ---------------------------------------------------------------------------
# decoders
# ---------------------------------------------------------------------------

def _e2m1_from_bits(c):
    """E2M1 from its bit fields: sign | exp(2, bias 1) | mantissa(1)."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def test_e2m1_value_set_matches_spec():
    want = GOLD["e2m1_values"]["magnitudes"]
    got = oracle.e2m1_decode(np.arange(16))
    assert list(got[:8]) == want
    assert list(-got[8:]) == want
    for c in range(16):
        assert Fraction(float(got[c])) == _e2m1_from_bits(c)
    assert np.signbit(got[8])  # 0x8 is negative zero


def test_e8m0_extremes_table1():
    f = GOLD["formats"]["E8M0-B32-FP4"]
    assert oracle.e8m0_decode(0) == 2.0 ** f["min_scale_log2"]
    top = oracle.e8m0_decode(254)
    assert top == 2.0 ** 127
    assert f"{top:.2e}" == f"{f['max_scale']:.2e}"
    assert np.isnan(oracle.e8m0_decode(255))
    codes = np.arange(255)
    assert np.array_equal(np.log2(oracle.e8m0_decode(codes)), codes - 127)


def test_e4m3_extremes_table1_and_torch_decode():
    f = GOLD["formats"]["E4M3-B16-FP4"]
    dec = oracle.e4m3_decode(np.arange(256))
    pos = dec[1:127]
    assert pos.min() == 2.0 ** f["min_scale_log2"]
    assert pos.max() == f["max_scale"]
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(dec)
    assert np.array_equal(np.isnan(ref), np.isnan(dec))
    assert np.array_equal(ref[~both_nan], dec[~both_nan])


def test_ue5m3_extremes_table1_and_fp16_bit_layout():
    """UE5M3 has fp16's exponent field (5 bits, bias 15) and the top 3 of its
    mantissa bits: for exponent fields 0..30 a code c is numpy's float16 with
    bits c << 7; exponent field 31 (infinite/NaN in fp16) continues the
    binade scale by one more factor of two.  Table 1: smallest scale 2^-17,
    largest 114688."""
    f = GOLD["formats"]["E5M3-B16-FP4"]
    dec = oracle.ue5m3_decode(np.arange(256))
    low = np.arange(0, 248)
    ref = (low.astype(np.uint16) << 7).view(np.float16).astype(np.float64)
    assert np.array_equal(dec[low], ref)
    top = np.arange(248, 255)
    assert np.array_equal(dec[top], 2.0 * dec[top - 8])
    pos = dec[1:255]
    assert pos.min() == 2.0 ** f["min_scale_log2"]
    assert pos.max() == f["max_scale"]
    assert np.all(np.diff(dec[:255]) > 0)
    assert np.isnan(dec[255])


# ---------------------------------------------------------------------------
# E2M1 round-to-nearest-even
# ---------------------------------------------------------------------------

def _interval_table(v):
    """Independent statement of RNE onto E2M1 with saturation, written as
    closed/open intervals (ties go to the even code 0, 1, 2, 4)."""
    out = []
    for x in v:
        if x <= 0.25:
            out.append(0)
        elif x < 0.75:
            out.append(1)
        elif x <= 1.25:
            out.append(2)
        elif x < 1.75:
            out.append(3)
        elif x <= 2.5:
            out.append(4)
        elif x < 3.5:
            out.append(5)
        elif x <= 5.0:
            out.append(6)
        else:
            out.append(7)
    return np.array(out)


def test_e2m1_rne_midpoints_and_sweep():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(oracle.e2m1_round_magnitude(mids)) == [0, 2, 2, 4, 4, 6, 6]
    for m in mids:
        lo, hi = np.nextafter(m, 0), np.nextafter(m, 10)
        assert oracle.e2m1_round_magnitude([lo])[0] == _interval_table([lo])[0]
        assert oracle.e2m1_round_magnitude([hi])[0] == _interval_table([hi])[0]
    v = np.concatenate([np.arange(0, 9000) / 1024.0, [1e30, 7.99, 6.0, 0.0]])
    assert np.array_equal(oracle.e2m1_round_magnitude(v), _interval_table(v))


def test_e2m1_rne_over_fp32_bit_patterns():
    """Stride through the non-negative fp32 bit patterns (every exponent, a
    spread of mantissas, all neighbours of the midpoints) and compare with the
    interval table."""
    bits = np.arange(0, 0x7F800000, 4093, dtype=np.uint64).astype(np.uint32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-3, 4)[None, :]).reshape(-1).astype(np.uint32)
    v = np.concatenate([bits, near]).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e2m1_round_magnitude(v), _interval_table(v))


# ---------------------------------------------------------------------------
# E8M0-B32 quantizer
# ---------------------------------------------------------------------------

def test_pack_order():
    assert oracle.pack_nibbles(np.array([[0x1, 0x2, 0xF, 0x0]]))[0].tolist() == [0x21, 0x0F]
    assert oracle.unpack_nibbles(np.array([[0x21]], np.uint8))[0].tolist() == [1, 2]


def test_e8m0_roundtrip_every_code_and_scale():
    """A block [6S, c*S, 0, ...] with S = 2^(sc-127) encodes back to scale sc
    and codes [7, c, 0, ...] for every element code c and every sc whose 6S is
    a finite fp32 (the OCP floor rule: floor(log2(6S)) - 2 = sc - 127)."""
    rows = []
    want_sc = []
    want_c = []
    for sc in range(0, 253):
        S = 2.0 ** (sc - 127)
        for c in range(16):
            blk = np.zeros(32)
            blk[0] = 6 * S
            blk[1] = float(oracle.e2m1_decode(c)) * S
            rows.append(blk)
            want_sc.append(sc)
            want_c.append(c)
    x = np.array(rows, dtype=np.float32)
    assert np.array_equal(x.astype(np.float64), np.array(rows))  # all exact in fp32
    codes, scales = oracle.quantize_e8m0_b32(x)
    el = oracle.unpack_nibbles(codes)
    # sc <= 1 is clamped: 6S is below 2^-125 and the scale code floors to 0
    ok = np.array(want_sc) >= 2
    assert np.array_equal(scales[ok, 0], np.array(want_sc)[ok])
    assert np.all(el[ok, 0] == 7)
    assert np.array_equal(el[ok, 1], np.array(want_c)[ok])
    assert np.all(el[ok, 2:] == 0)


def test_e8m0_scale_rule_and_zero_blocks():
    x = np.zeros((3, 64), np.float32)
    x[0, :32] = 1.0            # amax 1 -> floor(log2 1) - 2 = -2 -> code 125
    x[0, 32:] = 7.9            # amax 7.9 -> 2 - 2 = 0 -> code 127, 7.9 clips to 6
    x[1, :32] = -0.0           # all (negative) zero -> code 0, sign kept
    x[2, 5] = 1e-40            # subnormal amax -> code 0
    codes, scales = oracle.quantize_e8m0_b32(x)
    el = oracle.unpack_nibbles(codes)
    assert scales.tolist() == [[125, 127], [0, 0], [0, 0]]
    assert np.all(el[0, :32] == 6)         # 1.0 / 2^-2 = 4 -> code 6 (value 4)
    assert np.all(el[0, 32:] == 7)         # 7.9 saturates at 6
    assert np.all(el[1, :32] == 8)         # -0 keeps its sign
    assert np.all(el[2] == 0)


def test_e8m0_idempotent_and_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    codes, scales = oracle.quantize_e8m0_b32(x)
    d = oracle.dequantize(codes, scales, "e8m0_b32")
    c2, s2 = oracle.quantize_e8m0_b32(d.astype(np.float32))
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # each element is within half a grid step unless it saturated at 6S
    S = oracle.e8m0_decode(scales).repeat(32, axis=1)
    err = np.abs(d - x)
    sat = np.abs(x) > 6 * S
    assert np.all(err[~sat] <= 1.0 * S[~sat] + 1e-300)
    assert np.all(err[~sat & (np.abs(x) < 4 * S)] <= 0.5 * S[~sat & (np.abs(x) < 4 * S)])


def test_bpe_table1():
    K = 4096
    x = np.random.default_rng(0).standard_normal((8, K)).astype(np.float32)
    c, s = oracle.quantize_e8m0_b32(x)
    assert (c.nbytes + s.nbytes) * 8 / x.size == GOLD["formats"]["E8M0-B32-FP4"]["bpe"]
    c, s, _ = oracle.quantize_e4m3_b16(x)
    assert (c.nbytes + s.nbytes) * 8 / x.size == GOLD["formats"]["E4M3-B16-FP4"]["bpe"]
    c, s, _ = oracle.quantize_e5m3_b16(x)
    assert (c.nbytes + s.nbytes) * 8 / x.size == GOLD["formats"]["E5M3-B16-FP4"]["bpe"]


# ---------------------------------------------------------------------------
# E4M3 rounding and the E4M3-B16 quantizer
# ---------------------------------------------------------------------------

def test_e4m3_rne_matches_torch_cast():
    rng = np.random.default_rng(2)
    s = np.concatenate([
        np.exp2(rng.uniform(-14, 8.8, 200000)),
        oracle.e4m3_decode(np.arange(1, 127)),                       # grid points
        (oracle.e4m3_decode(np.arange(0, 126)) + oracle.e4m3_decode(np.arange(1, 127))) / 2,  # midpoints
        [0.0, 448.0, 2.0 ** -10, 3 * 2.0 ** -11],
    ]).astype(np.float32)
    s = np.minimum(s, np.float32(448.0))
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_round(s), ref.astype(np.int64))
    assert oracle.e4m3_round(np.float32([1e6, 449.0, 480.0]))[0] == 0x7E


def test_e4m3_b16_tensor_amax_element_maps_to_top_codes():
    """S_T = amax/(6*448): the tensor's largest element sits in a block whose
    scale is 448 (code 0x7E) and encodes to magnitude code 7 (6)."""
    rng = np.random.default_rng(3)
    for trial in range(50):
        x = (rng.standard_normal((4, 64)) * np.exp(rng.uniform(-20, 20))).astype(np.float32)
        codes, scales, st = oracle.quantize_e4m3_b16(x)
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, c // 16] == 0x7E
        assert (oracle.unpack_nibbles(codes)[r, c] & 7) == 7
        assert st == np.float32(np.float32(np.abs(x).max()) / np.float32(2688.0))


def test_e4m3_b16_elements_are_nearest_grid_points():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((16, 128)) * rng.uniform(0.01, 5, (16, 1))).astype(np.float32)
    codes, scales, st = oracle.quantize_e4m3_b16(x)
    sd = oracle.e4m3_decode(scales).astype(np.float32)
    den = (sd * st).astype(np.float32).astype(np.float64).repeat(16, axis=1)
    el = oracle.e2m1_decode(oracle.unpack_nibbles(codes))
    q = (np.abs(x) / den.astype(np.float32)).astype(np.float64)
    # brute force: distance to every E2M1 magnitude, pick the nearest
    grid = np.array(GOLD["e2m1_values"]["magnitudes"])
    dist = np.abs(q[..., None] - grid)
    best = dist.min(axis=-1)
    chosen = np.abs(q - np.abs(el))
    assert np.all(chosen == best)
    assert np.array_equal(np.signbit(el), np.signbit(x))


def test_e4m3_b16_block_scale_uses_torch_rounding():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-3, 3, (32, 16)).repeat(16, 1))).astype(np.float32)
    codes, scales, st = oracle.quantize_e4m3_b16(x)
    amax = np.abs(x.reshape(32, 16, 16)).max(-1).astype(np.float32)
    s = (amax / np.float32(np.float32(6.0) * st)).astype(np.float32)
    ref = torch.from_numpy(np.minimum(s, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)


def test_e4m3_b16_decoded_values_fit_bf16_exactly():
    """e2m1 * sd has at most 6 significant bits: exact in bf16 (8 bits)."""
    el = oracle.e2m1_decode(np.arange(16))
    sd = oracle.e4m3_decode(np.arange(0, 127))
    prod = (el[:, None] * sd[None, :]).astype(np.float32)
    bf = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf, prod)


def test_e4m3_b16_zero_tensor():
    codes, scales, st = oracle.quantize_e4m3_b16(np.zeros((2, 32), np.float32))
    assert st == 1.0 and np.all(scales == 0) and np.all(codes == 0)


# ---------------------------------------------------------------------------
# UE5M3 rounding and the E5M3-B16 quantizer
# ---------------------------------------------------------------------------

def _nearest_code_brute(s, grid):
    """Brute force: the grid index nearest to s, ties to the even index,
    values above the grid saturating to its last point."""
    out = []
    for v in s:
        if v >= grid[-1]:
            out.append(len(grid) - 1)
            continue
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        out.append(int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0]))
    return np.array(out)


def test_ue5m3_rne_brute_force():
    rng = np.random.default_rng(12)
    grid = oracle.ue5m3_decode(np.arange(255))
    s = np.concatenate([
        np.exp2(rng.uniform(-20, 17.2, 4000)),
        grid,                                                   # every grid point
        (grid[:-1] + grid[1:]) / 2,                             # every midpoint (ties)
        [0.0, 2.0 ** -18, 3 * 2.0 ** -19, 114688.0, 118784.0, 1e30],
    ]).astype(np.float32)
    assert np.array_equal(oracle.ue5m3_round(s), _nearest_code_brute(s.astype(np.float64), grid))
    assert list(oracle.ue5m3_round(np.float32([114688.0, 118784.0, 3e38]))) == [0xFE, 0xFE, 0xFE]


def test_e5m3_b16_tensor_amax_element_maps_to_top_codes():
    """S_T = amax/(6*114688): the largest element's block gets scale code 0xFE
    (114688) and the element encodes to magnitude code 7 (6)."""
    rng = np.random.default_rng(13)
    for trial in range(50):
        x = (rng.standard_normal((4, 64)) * np.exp(rng.uniform(-30, 30))).astype(np.float32)
        codes, scales, st = oracle.quantize_e5m3_b16(x)
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, c // 16] == 0xFE
        assert (oracle.unpack_nibbles(codes)[r, c] & 7) == 7
        assert st == np.float32(np.float32(np.abs(x).max()) / np.float32(688128.0))


def test_e5m3_b16_elements_and_scales_are_nearest_grid_points():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((16, 128)) * np.exp(rng.uniform(-8, 8, (16, 8)).repeat(16, 1))).astype(np.float32)
    codes, scales, st = oracle.quantize_e5m3_b16(x)
    # block scales: brute-force nearest UE5M3 grid point of amax / (6 S_T)
    amax = np.abs(x.reshape(16, 8, 16)).max(-1).astype(np.float32)
    sv = (amax / np.float32(np.float32(6.0) * st)).astype(np.float32)
    grid = oracle.ue5m3_decode(np.arange(255))
    assert np.array_equal(scales.reshape(-1), _nearest_code_brute(sv.reshape(-1).astype(np.float64), grid))
    # elements: nearest E2M1 magnitude of |x| / (sd S_T)
    sd = oracle.ue5m3_decode(scales).astype(np.float32)
    den = (sd * st).astype(np.float32).repeat(16, axis=1)
    q = (np.abs(x) / den).astype(np.float32).astype(np.float64)
    el = oracle.e2m1_decode(oracle.unpack_nibbles(codes))
    e2 = np.array(GOLD["e2m1_values"]["magnitudes"])
    assert np.all(np.abs(q - np.abs(el)) == np.abs(q[..., None] - e2).min(axis=-1))
    assert np.array_equal(np.signbit(el), np.signbit(x))


def test_e5m3_b16_decoded_values_exact_in_bf16_not_fp16():
    """e2m1 * sd (UE5M3) has at most 6 significant bits and spans
    [2^-18, 6*114688]: exact in bf16; beyond fp16's largest finite value."""
    el = oracle.e2m1_decode(np.arange(16))
    sd = oracle.ue5m3_decode(np.arange(0, 255))
    prod = (el[:, None] * sd[None, :]).astype(np.float32)
    bf = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf, prod)
    assert np.abs(prod).max() == 6 * 114688.0 > 65504.0


def test_e5m3_b16_zero_tensor():
    codes, scales, st = oracle.quantize_e5m3_b16(np.zeros((2, 32), np.float32))
    assert st == 1.0 and np.all(scales == 0) and np.all(codes == 0)


def test_bf16_helpers():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38], np.float32)
    b = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    assert np.array_equal(oracle.bf16_bits_to_f32(b), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("fmt", ["e8m0_b32", "e4m3_b16", "e5m3_b16"])
def test_dequantize_shapes(fmt):
    x = np.random.default_rng(6).standard_normal((3, 64)).astype(np.float32)
    if fmt == "e8m0_b32":
        c, s = oracle.quantize_e8m0_b32(x)
        d = oracle.dequantize(c, s, fmt)
    else:
        q = oracle.quantize_e4m3_b16 if fmt == "e4m3_b16" else oracle.quantize_e5m3_b16
        c, s, st = q(x)
        d = oracle.dequantize(c, s, fmt, st)
    assert d.shape == x.shape
    assert np.max(np.abs(d - x)) < 0.5 * np.max(np.abs(x))
