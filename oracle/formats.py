"""Block-scaled FP4 formats: decoders (closed forms) and quantizers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Formats, as "MXCode: MX-Native Codebook Quantization", Table 1 lists them:
  * E8M0-B32-FP4: E2M1 elements, one E8M0 scale per 32 elements along K,
    smallest scale 2^-127, largest 1.70e38, 4.25 bits per element.
  * E4M3-B16-FP4: E2M1 elements, one E4M3 scale per 16 elements, smallest
    scale 2^-9, largest 448, an optional FP32 tensor scale, 4.50 bits per
    element.
  * E5M3-B16-FP4: E2M1 elements, one UE5M3 scale per 16 elements, smallest
    scale 2^-17, largest 114688, an optional FP32 tensor scale, 4.50 bits per
    element.
The E2M1 value set {0, 0.5, 1, 1.5, 2, 3, 4, 6} is the OCP MX element type
that the PRQuant page cites for MXFP4 (§1, "block-wise duality").

Packing (the pages are silent; this is the reading used everywhere here):
byte i of a row holds element 2i in bits 3:0 and element 2i+1 in bits 7:4;
bit 3 of a nibble is the sign.

Readings taken where the pages leave a step open:
  * E8M0 scale rule: the OCP floor rule, scale exponent = floor(log2 amax)
    - 2 (2 = emax of E2M1), written as the biased code max(0, E(amax) - 2)
    where E(.) is the fp32 biased exponent field; a zero or subnormal block
    gets code 0.
  * Element rounding: round to nearest E2M1 value, ties to the even code
    (mantissa bit 0), saturating at 6; the sign of x is kept even when the
    magnitude rounds to 0.
  * E4M3-B16: tensor scale S_T = amax / (6*448) (1.0 for an all-zero
    tensor), block scale code = E4M3 round-to-nearest-even of
    amax_blk / (6*S_T) saturating at 448, element = RNE(|x| / (sd*S_T)),
    every step an fp32 operation in that order.
  * UE5M3: unsigned, 5 exponent bits with bias 15 (the bias that makes the
    smallest subnormal (1/8)*2^-14 the 2^-17 of Table 1) and 3 mantissa bits;
    the all-ones code 0xFF is reserved (not finite), so the largest finite
    code 0xFE = 1.75*2^16 = 114688, the Table 1 maximum.
  * E5M3-B16: the E4M3-B16 steps with UE5M3 block scales and
    S_T = amax / (6*114688).
"""

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ----------------------------------------------------------------------------
# Decoders (closed forms)
# ----------------------------------------------------------------------------

def e2m1_decode(codes):
    """E2M1 nibble -> float64: magnitude table indexed by bits 2:0, sign bit 3."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e8m0_decode(codes):
    """E8M0 byte e -> 2^(e-127); e = 255 is NaN (never produced here)."""
    e = np.asarray(codes).astype(np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def e4m3_decode(codes):
    """E4M3 ("fn" variant) byte -> float64.

    Exponent field 0: (m/8) * 2^-6 (subnormal); otherwise (1 + m/8) * 2^(e-7).
    0x7F / 0xFF are NaN, there is no infinity.  Bit 7 is the sign.
    """
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def ue5m3_decode(codes):
    """UE5M3 byte -> float64 (unsigned; 5 exponent bits, bias 15; 3 mantissa bits).

    Exponent field 0: (m/8) * 2^-14 (subnormal); otherwise (1 + m/8) * 2^(e-15).
    0xFF is reserved and decodes to NaN.
    """
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0x1F
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -14, (1.0 + m / 8.0) * np.ldexp(1.0, e - 15))
    return np.where(c == 0xFF, np.nan, mag)


# ----------------------------------------------------------------------------
# Round-to-nearest-even onto a finite grid
# ----------------------------------------------------------------------------

def _round_to_grid(v, grid):
    """Index of the grid value nearest to v (v >= 0, float64, exact).

    ``grid`` is strictly increasing and index parity is the code's mantissa
    parity, so a tie goes to the even index.  Values above the last grid point
    saturate to it.
    """
    v = np.asarray(v, dtype=np.float64)
    n = len(grid)
    hi = np.searchsorted(grid, v, side="left")          # first grid >= v
    hi_c = np.clip(hi, 0, n - 1)
    lo_c = np.clip(hi - 1, 0, n - 1)
    d_lo = v - grid[lo_c]
    d_hi = grid[hi_c] - v
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    idx = np.where(pick_hi, hi_c, lo_c)
    idx = np.where(hi == 0, 0, idx)                      # v <= grid[0]
    idx = np.where(hi >= n, n - 1, idx)                  # saturate
    return idx.astype(np.int64)


def e2m1_round_magnitude(v):
    """|v| (float64) -> E2M1 magnitude code 0..7, RNE, saturating at 6."""
    return _round_to_grid(np.abs(np.asarray(v, dtype=np.float64)), E2M1_MAGNITUDES)


_E4M3_POS_GRID = e4m3_decode(np.arange(0, 127))          # codes 0x00..0x7E, increasing


def e4m3_round(s):
    """Non-negative fp32 s -> unsigned E4M3 code, RNE, saturating at 448 (0x7E)."""
    return _round_to_grid(np.asarray(s, dtype=np.float64), _E4M3_POS_GRID)


_UE5M3_GRID = ue5m3_decode(np.arange(0, 255))           # codes 0x00..0xFE, increasing


def ue5m3_round(s):
    """Non-negative fp32 s -> UE5M3 code, RNE, saturating at 114688 (0xFE)."""
    return _round_to_grid(np.asarray(s, dtype=np.float64), _UE5M3_GRID)


# ----------------------------------------------------------------------------
# Packing helpers and bf16 bit conversions
# ----------------------------------------------------------------------------

def pack_nibbles(codes):
    """[..., 2n] nibble codes -> [..., n] bytes, element 2i in bits 3:0."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    """[..., n] bytes -> [..., 2n] nibble codes."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.asarray(bits).astype(np.uint32)
    return (b << 16).view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bits by round-to-nearest-even (NaN not expected)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# E8M0-B32-FP4 quantizer
# ----------------------------------------------------------------------------

def quantize_e8m0_b32(x):
    """x [rows][K] (fp32 values; bf16 inputs are widened exactly first)
    -> (codes uint8 [rows][K/2], scales uint8 [rows][K/32]).

    Steps per block of 32 consecutive K elements:
      1. amax = max |x| (exact);
      2. scale code sc = max(0, E(amax) - 2), E = fp32 biased exponent field;
      3. v = x * 2^(127 - sc) (power-of-two scaling, exact in float64);
      4. element code = sign(x) | RNE_sat(|v|) onto the E2M1 magnitudes.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    E = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    sc = np.maximum(E - 2, 0)
    v = blk.astype(np.float64) * np.ldexp(1.0, 127 - sc)[..., None]
    mag = e2m1_round_magnitude(v)
    sign = np.signbit(blk).astype(np.int64)
    codes = (mag | (sign << 3)).reshape(rows, K)
    return pack_nibbles(codes), sc.astype(np.uint8)


# ----------------------------------------------------------------------------
# E4M3-B16-FP4 quantizer with FP32 tensor scale
# ----------------------------------------------------------------------------

E4M3_MAX = np.float32(448.0)
E2M1_MAX = np.float32(6.0)


def tensor_scale_e4m3(amax):
    """S_T = amax / (6 * 448) in fp32; 1.0 for an all-zero tensor."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(2688.0))


def quantize_e4m3_b16(x, tensor_amax=None):
    """x [rows][K] fp32 -> (codes [rows][K/2], scales uint8 [rows][K/16], S_T fp32).

    ``tensor_amax`` (fp32) overrides the tensor's own amax; by default the
    tensor scale is dynamic (amax of x).  Every step below is an fp32
    operation, in this order:
      S_T = A / 2688; d = 6 * S_T; s = amax_blk / d; sc = E4M3_RNE_sat(s);
      sd = decode(sc); den = sd * S_T; code = sign(x) | RNE_sat(|x| / den)
    and a block with sd == 0 (or den == 0) encodes as signed zeros.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    A = np.float32(np.max(np.abs(x))) if tensor_amax is None else np.float32(tensor_amax)
    if x.size == 0:
        A = np.float32(0.0)
    S_T = tensor_scale_e4m3(A)
    blk = x.reshape(rows, K // 16, 16)
    amax = np.max(np.abs(blk), axis=2).astype(np.float32) if x.size else np.zeros((rows, K // 16), np.float32)
    d = np.float32(E2M1_MAX * S_T)
    s = (amax / d).astype(np.float32)
    sc = e4m3_round(s)
    sd = e4m3_decode(sc).astype(np.float32)
    den = (sd * S_T).astype(np.float32)
    ok = den > 0
    safe = np.where(ok, den, np.float32(1.0)).astype(np.float32)
    q = (np.abs(blk) / safe[..., None]).astype(np.float32)
    mag = e2m1_round_magnitude(q)
    mag = np.where(ok[..., None], mag, 0)
    sign = np.signbit(blk).astype(np.int64)
    codes = (mag | (sign << 3)).reshape(rows, K)
    return pack_nibbles(codes), sc.astype(np.uint8), np.float32(S_T)


# ----------------------------------------------------------------------------
# E5M3-B16-FP4 quantizer with FP32 tensor scale
# ----------------------------------------------------------------------------

UE5M3_MAX = np.float32(114688.0)


def tensor_scale_e5m3(amax):
    """S_T = amax / (6 * 114688) in fp32; 1.0 for an all-zero tensor."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    return np.float32(a / np.float32(688128.0))


def quantize_e5m3_b16(x, tensor_amax=None):
    """x [rows][K] fp32 -> (codes [rows][K/2], scales uint8 [rows][K/16], S_T fp32).

    The E4M3-B16 steps with UE5M3 block scales (MXCode Table 1, E5M3-B16-FP4
    row), every step an fp32 operation, in this order:
      S_T = A / 688128; d = 6 * S_T; s = amax_blk / d; sc = UE5M3_RNE_sat(s);
      sd = decode(sc); den = sd * S_T; code = sign(x) | RNE_sat(|x| / den)
    and a block with sd == 0 (or den == 0) encodes as signed zeros.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    A = np.float32(np.max(np.abs(x))) if tensor_amax is None else np.float32(tensor_amax)
    if x.size == 0:
        A = np.float32(0.0)
    S_T = tensor_scale_e5m3(A)
    blk = x.reshape(rows, K // 16, 16)
    amax = np.max(np.abs(blk), axis=2).astype(np.float32) if x.size else np.zeros((rows, K // 16), np.float32)
    d = np.float32(E2M1_MAX * S_T)
    s = (amax / d).astype(np.float32)
    sc = ue5m3_round(s)
    sd = ue5m3_decode(sc).astype(np.float32)
    den = (sd * S_T).astype(np.float32)
    ok = den > 0
    safe = np.where(ok, den, np.float32(1.0)).astype(np.float32)
    q = (np.abs(blk) / safe[..., None]).astype(np.float32)
    mag = e2m1_round_magnitude(q)
    mag = np.where(ok[..., None], mag, 0)
    sign = np.signbit(blk).astype(np.int64)
    codes = (mag | (sign << 3)).reshape(rows, K)
    return pack_nibbles(codes), sc.astype(np.uint8), np.float32(S_T)


# ----------------------------------------------------------------------------
# Dequantization
# ----------------------------------------------------------------------------

FMT_E8M0_B32 = "e8m0_b32"
FMT_E4M3_B16 = "e4m3_b16"
FMT_E5M3_B16 = "e5m3_b16"
TENSOR_SCALED = (FMT_E4M3_B16, FMT_E5M3_B16)   # formats with an FP32 tensor scale


def dequantize(codes, scales, fmt, tensor_scale=None):
    """Packed codes [rows][K/2] + block scales -> float64 [rows][K].

    E8M0-B32: e2m1 * 2^(sc-127).  E4M3-B16 / E5M3-B16: e2m1 * decode(sc) * S_T
    (S_T defaults to 1, so the product of the two left factors is returned).
    """
    el = e2m1_decode(unpack_nibbles(codes))
    rows, K = el.shape
    if fmt == FMT_E8M0_B32:
        s = e8m0_decode(scales)
        return (el.reshape(rows, K // 32, 32) * s[..., None]).reshape(rows, K)
    if fmt in TENSOR_SCALED:
        s = e4m3_decode(scales) if fmt == FMT_E4M3_B16 else ue5m3_decode(scales)
        out = (el.reshape(rows, K // 16, 16) * s[..., None]).reshape(rows, K)
        if tensor_scale is not None:
            out = out * np.float64(np.float32(tensor_scale))
        return out
    raise ValueError(fmt)
