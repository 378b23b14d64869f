// Online activation quantization (E8M0-B32 and E4M3-B16 FP4), the tensor
// amax pass, decode-to-fp32 and the offline PRQuant weight residual.
//
// Formats: "MXCode: MX-Native Codebook Quantization", Table 1.  Tail copy:
// "PRQuant: Permutation Residual Quantization for Low-Overhead Inference",
// §4 "Kernel design for efficient inference" (online copy).  Residual: same
// page, §4 Eq. (2).
//
// Layout: one lane owns 8 consecutive K elements (one 16-byte bf16 load, two
// for fp32); 4 neighbouring lanes form an E8M0 block of 32 and 2 form an E4M3
// block of 16, so every wave-wide load is one contiguous 1 KiB (bf16) and the
// block amax needs one or two lane swaps.  Each lane stores its 8 nibbles as
// one 32-bit word.
#include "common.hpp"

namespace gbw {

constexpr int kQuantThreads = 256;
constexpr int kAmaxBlocks = 256;  // amax partials; every E4M3 quantizer block reduces all of them

template <typename T>
struct In8;

template <>
struct In8<uint16_t> {  // bf16 bits
  __device__ static void load(const uint16_t* p, float (&v)[8]) {
    const v4i q = load16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)q[i];
      v[2 * i] = __uint_as_float(w << 16);
      v[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  }
};

template <>
struct In8<float> {
  __device__ static void load(const float* p, float (&v)[8]) {
    const v4i a = load16(p), b = load16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __int_as_float(a[i]);
      v[4 + i] = __int_as_float(b[i]);
    }
  }
};

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// Row and first column of 8-element unit u of a [rows][K] tensor.  The unit
// count fits 32 bits in every tensor below 2^35 elements, where a 32-bit
// division (a dozen VALU operations) replaces the 64-bit one.
template <bool WIDE>
__device__ __forceinline__ void unit_pos(int64_t u, int64_t K, int64_t& row, int64_t& col) {
  if (WIDE) {
    row = u / (K / 8);
    col = (u % (K / 8)) * 8;
  } else {
    const uint32_t kg = (uint32_t)(K / 8), uu = (uint32_t)u;
    const uint32_t r = uu / kg;
    row = r;
    col = (int64_t)(uu - r * kg) * 8;
  }
}

// max over lanes (lane ^ 1) and, if span == 4, (lane ^ 2): non-negative fp32
// bit patterns order like unsigned integers.
template <int SPAN>
__device__ __forceinline__ uint32_t group_max(uint32_t a) {
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  if (SPAN == 4) a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  return a;
}

// ---------------------------------------------------------------------------
// E8M0-B32
// ---------------------------------------------------------------------------
// Normalized order-32 Walsh-Hadamard transform of the 32-block a quad of
// lanes holds (lane 4k+q: elements 8q..8q+7 of the block): stages of span 1,
// 2, 4 inside the lane, 8 and 16 across lanes q^1 and q^2, each pair (a, b)
// -> (a + b, a - b) in fp32, then one multiply by fp32(1/sqrt(32)).
__device__ __forceinline__ void fwht32_quad(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  const int q = threadIdx.x & 3;
#pragma unroll
  for (int m = 1; m <= 2; m <<= 1) {
    const bool upper = (q & m) != 0;  // this lane holds the (i + h) side of each pair
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float o = __shfl_xor(v[i], m);
      v[i] = upper ? o - v[i] : v[i] + o;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= 0x1.6a09e6p-3f;  // fp32(1/sqrt(32))
}

// Four 8-element units per thread (all four loads in flight before any
// arithmetic); the units of one load instruction are 64 consecutive units of
// the row-major tensor (1 KiB contiguous), and a lane quad always holds one
// whole 32-element block.
constexpr int kQ8Units = 4;    // E4M3-B16 / E5M3-B16: units per thread (the per-workgroup tensor-amax
                               // reduction is paid once per 1024 units)
constexpr int kQ8UnitsE8 = 2;  // E8M0-B32: units per thread (more, smaller workgroups than 4 units:
                               // 8192 x 4096 bf16 in 17.7 against 18.5 us)

template <typename T, bool WIDE, bool ROT>
__global__ __launch_bounds__(kQuantThreads) void k_quant_e8m0(const T* __restrict__ x, int64_t rows,
                                                             int64_t K, int64_t tail,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t total = rows * (K / 8);
  const int64_t g0 = (int64_t)blockIdx.x * (kQuantThreads * kQ8UnitsE8) + threadIdx.x;
  float v[kQ8UnitsE8][8];
  int64_t row[kQ8UnitsE8], col[kQ8UnitsE8];
#pragma unroll
  for (int u = 0; u < kQ8UnitsE8; ++u) {
    const int64_t g = g0 + (int64_t)u * kQuantThreads;
    const int64_t gg = g < total ? g : total - 1;  // keep the whole wave in the shuffles
    unit_pos<WIDE>(gg, K, row[u], col[u]);
    In8<T>::load(x + row[u] * K + col[u], v[u]);
  }
  const int64_t W = K + tail;
  const bool lead = (threadIdx.x & 3) == 0;
#pragma unroll
  for (int u = 0; u < kQ8UnitsE8; ++u) {
    if (ROT) fwht32_quad(v[u]);
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, abs_bits(v[u][i]));
    am = group_max<4>(am);
    const uint32_t sc = e8m0_scale_code(__uint_as_float(am));
    // v_cvt_scalef32_pk_fp4_f32: x / 2^(sc-127) (exact: a power of two, also
    // for the subnormal 2^-127), RNE onto E2M1, saturating at 6, sign kept --
    // the rounding rule above, one instruction per two elements
    const float scale = e8m0_value(sc);
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[u][0], v[u][1], scale, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[u][2], v[u][3], scale, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[u][4], v[u][5], scale, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[u][6], v[u][7], scale, 3);
    if (g0 + (int64_t)u * kQuantThreads >= total) continue;
    *reinterpret_cast<uint32_t*>(codes + row[u] * (W / 2) + col[u] / 2) = word;
    if (lead) scales[row[u] * (W / 32) + col[u] / 32] = (uint8_t)sc;
    if (tail > 0 && col[u] >= K - tail) {
      const int64_t c2 = K + (col[u] - (K - tail));
      *reinterpret_cast<uint32_t*>(codes + row[u] * (W / 2) + c2 / 2) = word;
      if (lead) scales[row[u] * (W / 32) + c2 / 32] = (uint8_t)sc;
    }
  }
}

// ---------------------------------------------------------------------------
// tensor amax (deterministic two-pass: per-block partial maxima, reduced by
// every consumer block)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void k_amax_partial(const T* __restrict__ x, int64_t n8,
                                                               uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kQuantThreads / 64];
  // four 8-element units per thread in flight at a time
  uint32_t am = 0;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t i0 = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i0 < n8; i0 += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      In8<T>::load(x + (i < n8 ? i : i0) * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) am = max(am, abs_bits(v[u][j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) m = max(m, red[i]);
    partial[blockIdx.x] = m;
  }
}

// S_T = amax / (6 * 448) (E4M3 scales) or amax / (6 * 114688) (UE5M3 scales)
// in fp32, 1 for an all-zero tensor.
template <bool E5>
__device__ __forceinline__ float tensor_scale_from_amax(float a) {
  return a == 0.0f ? 1.0f : a / (E5 ? 688128.0f : 2688.0f);
}

__device__ float block_reduce_partials(const uint32_t* __restrict__ partial, int n) {
  __shared__ uint32_t red[kQuantThreads / 64];
  uint32_t am = 0;
  for (int i = threadIdx.x; i < n; i += kQuantThreads) am = max(am, partial[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kQuantThreads / 64; ++i) m = max(m, red[i]);
  return __uint_as_float(m);
}

// ---------------------------------------------------------------------------
// E4M3-B16 and E5M3-B16 (E5 = true: UE5M3 block scales) with FP32 tensor scale
// ---------------------------------------------------------------------------
template <typename T, bool WIDE, bool E5>
__global__ __launch_bounds__(kQuantThreads) void k_quant_e4m3(const T* __restrict__ x, int64_t rows,
                                                             int64_t K, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             float* __restrict__ tensor_scale,
                                                             const uint32_t* __restrict__ partial,
                                                             int n_partial) {
  float S_T;
  if (partial != nullptr) {
    S_T = tensor_scale_from_amax<E5>(block_reduce_partials(partial, n_partial));
    if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = S_T;
  } else {
    S_T = tensor_scale[0];
  }
  // kQ8Units 8-element units per thread, as in the E8M0 quantizer (the
  // tensor-amax reduction above is paid once per 1024 units)
  const int64_t total = rows * (K / 8);
  const int64_t g0 = (int64_t)blockIdx.x * (kQuantThreads * kQ8Units) + threadIdx.x;
  float v[kQ8Units][8];
  int64_t row[kQ8Units], col[kQ8Units];
#pragma unroll
  for (int u = 0; u < kQ8Units; ++u) {
    const int64_t g = g0 + (int64_t)u * kQuantThreads;
    const int64_t gg = g < total ? g : total - 1;  // keep the whole wave in the shuffles
    unit_pos<WIDE>(gg, K, row[u], col[u]);
    In8<T>::load(x + row[u] * K + col[u], v[u]);
  }
  const float d = 6.0f * S_T;
#pragma unroll
  for (int u = 0; u < kQ8Units; ++u) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, abs_bits(v[u][i]));
    am = group_max<2>(am);
    const float s = __uint_as_float(am) / d;
    const uint32_t sc = E5 ? ue5m3_rne_sat(s) : e4m3_rne_sat(s);
    const float den = (E5 ? ue5m3_value(sc) : e4m3_value(sc)) * S_T;
    // element = RNE onto E2M1 of the fp32 quotient x / den (sign kept; a block
    // whose scale decodes to 0 encodes signed zeros): the division in fp32,
    // then v_cvt_scalef32_pk_fp4_f32 at scale 1 for the rounding
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = den > 0.0f ? v[u][i] / den : v[u][i] * 0.0f;
    uint32_t word = 0;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[0], q[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[2], q[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[4], q[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q[6], q[7], 1.0f, 3);
    if (g0 + (int64_t)u * kQuantThreads >= total) continue;
    *reinterpret_cast<uint32_t*>(codes + row[u] * (K / 2) + col[u] / 2) = word;
    if ((threadIdx.x & 1) == 0) scales[row[u] * (K / 16) + col[u] / 16] = (uint8_t)sc;
  }
}

// ---------------------------------------------------------------------------
// decode to fp32 (same decoders as the GEMM kernels) and the residual
// ---------------------------------------------------------------------------
// One decoded weight element.  VQ formats (qsh = log2 of the QBlock edge):
// the E2M1 code is nibble k%4 of the QBlock table entry the index selects;
// the E8M0 scale is stored per 32 along K (PreScale), per QBlock (PostScale)
// or is element (k/32)%8 of the scale-table entry of the row's index for
// elements 256*(k/256) .. (PreScale+).
__device__ __forceinline__ float decode_elem(int32_t fmt, const uint8_t* codes, const uint8_t* scales,
                                             const uint16_t* codebook, const uint8_t* scb, int32_t qsh,
                                             const float* ts, int32_t ts_seg, int64_t N, int64_t K, int64_t n,
                                             int64_t k) {
  if (fmt >= GBW_FMT_VQ4_E4M3 && fmt <= GBW_FMT_VQ4_E5M3_PLUS) {
    // 16-element blocks: E4M3 (formats 6-8) or UE5M3 (9-11) scales, FP32 tensor scale
    const int lay = (fmt - GBW_FMT_VQ4_E4M3) % 3;  // 0 PreScale, 1 PostScale, 2 PreScale+
    const bool e5 = fmt >= GBW_FMT_VQ4_E5M3;
    const uint32_t idx = codes[n * (K / 4) + k / 4];
    const int64_t qblk = (n >> qsh) * (K >> qsh) + (k >> qsh);
    const uint32_t c = (codebook[qblk * 256 + idx] >> (4 * (k & 3))) & 0xFu;
    uint32_t sc;
    if (lay == 1)
      sc = scales[qblk];
    else if (lay == 2)
      sc = scb[(uint32_t)scales[n * (K / 128) + k / 128] * 8 + (k / 16) % 8];
    else
      sc = scales[n * (K / 16) + k / 16];
    const float v = e2m1_value(c) * (e5 ? ue5m3_value(sc) : e4m3_value(sc));
    return v * ts[n / (N / ts_seg)];
  }
  if (fmt == GBW_FMT_VQ4_E8M0 || fmt == GBW_FMT_VQ4_POST || fmt == GBW_FMT_VQ4_PLUS) {
    const uint32_t idx = codes[n * (K / 4) + k / 4];
    const int64_t qblk = (n >> qsh) * (K >> qsh) + (k >> qsh);
    const uint32_t key = codebook[qblk * 256 + idx];
    const uint32_t c = (key >> (4 * (k & 3))) & 0xFu;
    uint32_t sc;
    if (fmt == GBW_FMT_VQ4_POST)
      sc = scales[qblk];
    else if (fmt == GBW_FMT_VQ4_PLUS)
      sc = scb[(uint32_t)scales[n * (K / 256) + k / 256] * 8 + (k / 32) % 8];
    else
      sc = scales[n * (K / 32) + k / 32];
    return e2m1_value(c) * e8m0_value(sc);
  }
  const uint32_t c = (codes[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 0xFu;
  if (fmt == GBW_FMT_E8M0_B32) return e2m1_value(c) * e8m0_value(scales[n * (K / 32) + k / 32]);
  const uint32_t sc = scales[n * (K / 16) + k / 16];
  const float v = e2m1_value(c) * (fmt == GBW_FMT_E5M3_B16 ? ue5m3_value(sc) : e4m3_value(sc));
  const int64_t seg = n / (N / ts_seg);
  return v * ts[seg];
}

__global__ void k_dequant(int32_t fmt, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                          const uint16_t* __restrict__ codebook, const uint8_t* __restrict__ scb, int32_t qsh,
                          const float* __restrict__ ts, int32_t ts_seg, int64_t N, int64_t K,
                          float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i % K;
  out[i] = decode_elem(fmt, codes, scales, codebook, scb, qsh, ts, ts_seg, N, K, n, k);
}

__global__ void k_residual(const float* __restrict__ w, int64_t N, int64_t K, int64_t tail,
                           const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                           float* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * tail) return;
  const int64_t n = i / tail, k = K - tail + i % tail;
  const float d = decode_elem(GBW_FMT_E8M0_B32, codes, scales, nullptr, nullptr, 6, nullptr, 1, N, K, n, k);
  r[i] = w[n * K + k] - d;
}

__global__ void k_set_scalar(float* p, float v) {
  if (threadIdx.x == 0) p[0] = v;
}

size_t ws_quantize(int64_t rows, int64_t K, int32_t fmt) {
  (void)rows;
  (void)K;
  return fmt == GBW_FMT_E4M3_B16 || fmt == GBW_FMT_E5M3_B16 ? (size_t)kAmaxBlocks * sizeof(uint32_t) : 0;
}

}  // namespace gbw

using namespace gbw;

extern "C" int mx_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t K, int32_t fmt,
                           int64_t tail_copy, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || K < 0 || tail_copy < 0) return fail(GBW_E_ARG, "mx_quantize: negative extent");
  if (x_dtype != GBW_DTYPE_BF16 && x_dtype != GBW_DTYPE_F32) return fail(GBW_E_ARG, "mx_quantize: bad dtype");
  if (fmt != GBW_FMT_E8M0_B32 && fmt != GBW_FMT_E4M3_B16 && fmt != GBW_FMT_E5M3_B16)
    return fail(GBW_E_ARG, "mx_quantize: bad format");
  const bool tscaled = fmt != GBW_FMT_E8M0_B32;  // E4M3-B16 or E5M3-B16: FP32 tensor scale
  if ((flags & GBW_ROTATE_H32) && fmt != GBW_FMT_E8M0_B32)
    return fail(GBW_E_UNSUPPORTED, "mx_quantize: the block rotation is for E8M0-B32 (32-element blocks)");
  const int bs = fmt == GBW_FMT_E8M0_B32 ? 32 : 16;
  if (K % bs) return fail(GBW_E_SHAPE, "mx_quantize: K=%lld not a multiple of %d", (long long)K, bs);
  if (tail_copy && (fmt != GBW_FMT_E8M0_B32 || tail_copy % 32 || tail_copy > K))
    return fail(GBW_E_SHAPE, "mx_quantize: tail_copy must be a multiple of 32, <= K, E8M0 only");
  const bool dynamic = tscaled && (flags & GBW_TS_DYNAMIC);
  if (tscaled && !tensor_scale) return fail(GBW_E_ARG, "mx_quantize: E4M3/E5M3 needs tensor_scale");
  if (rows == 0 || K == 0) {
    if (!dynamic) return GBW_OK;
    int st0 = check_device();
    if (st0) return st0;
    // an empty tensor has amax 0, so its tensor scale is 1
    hipLaunchKernelGGL(k_set_scalar, dim3(1), dim3(64), 0, as_stream(stream), tensor_scale, 1.0f);
    return check_launch("mx_quantize(empty)");
  }
  if (!x || !codes || !scales) return fail(GBW_E_ARG, "mx_quantize: null pointer");
  if (!aligned16(x) || !aligned16(codes)) return fail(GBW_E_ALIGN, "mx_quantize: x/codes not 16-byte aligned");
  if (dynamic && (!ws || ws_bytes < ws_quantize(rows, K, fmt)))
    return fail(GBW_E_WORKSPACE, "mx_quantize: dynamic tensor scale needs %zu bytes of workspace",
                ws_quantize(rows, K, fmt));
  int st = check_device();
  if (st) return st;
  hipStream_t s = as_stream(stream);
  const int64_t total = rows * (K / 8);
  const unsigned blocks8 = (unsigned)cdiv(total > 0 ? total : 1, kQuantThreads * kQ8Units);      // E4M3 / E5M3
  const unsigned blocks8e = (unsigned)cdiv(total > 0 ? total : 1, kQuantThreads * kQ8UnitsE8);  // E8M0
  const bool bf = x_dtype == GBW_DTYPE_BF16;
  const bool wide = total > (int64_t)UINT32_MAX;
  if (fmt == GBW_FMT_E8M0_B32) {
#define GBW_Q8(T, W, R)                                                                                       \
  hipLaunchKernelGGL((k_quant_e8m0<T, W, R>), dim3(blocks8e), dim3(kQuantThreads), 0, s, (const T*)x, rows, K, \
                     tail_copy, codes, scales)
#define GBW_Q8F(R)                                                              \
  if (bf) {                                                                     \
    if (wide) GBW_Q8(uint16_t, true, R); else GBW_Q8(uint16_t, false, R);       \
  } else {                                                                      \
    if (wide) GBW_Q8(float, true, R); else GBW_Q8(float, false, R);             \
  }
    if (flags & GBW_ROTATE_H32) {
      GBW_Q8F(true)
    } else {
      GBW_Q8F(false)
    }
#undef GBW_Q8F
#undef GBW_Q8
    return check_launch("mx_quantize(e8m0)");
  }
  uint32_t* partial = nullptr;
  if (dynamic) {
    partial = reinterpret_cast<uint32_t*>(ws);
    if (bf)
      hipLaunchKernelGGL(k_amax_partial<uint16_t>, dim3(kAmaxBlocks), dim3(kQuantThreads), 0, s,
                         (const uint16_t*)x, total, partial);
    else
      hipLaunchKernelGGL(k_amax_partial<float>, dim3(kAmaxBlocks), dim3(kQuantThreads), 0, s,
                         (const float*)x, total, partial);
    if ((st = check_launch("mx_quantize(amax)"))) return st;
  }
#define GBW_Q4(T, W, E5)                                                                                          \
  hipLaunchKernelGGL((k_quant_e4m3<T, W, E5>), dim3(blocks8), dim3(kQuantThreads), 0, s, (const T*)x, rows, K, codes, \
                     scales, tensor_scale, partial, kAmaxBlocks)
#define GBW_Q4F(E5)                                                   \
  if (bf) {                                                           \
    if (wide) GBW_Q4(uint16_t, true, E5); else GBW_Q4(uint16_t, false, E5); \
  } else {                                                            \
    if (wide) GBW_Q4(float, true, E5); else GBW_Q4(float, false, E5);       \
  }
  if (fmt == GBW_FMT_E5M3_B16) {
    GBW_Q4F(true)
  } else {
    GBW_Q4F(false)
  }
#undef GBW_Q4F
#undef GBW_Q4
  return check_launch("mx_quantize(e4m3/e5m3)");
}

extern "C" int mx_dequantize(const gbw_weight* w, int32_t expert, float* out, void* stream) {
  if (!w || !out) return fail(GBW_E_ARG, "mx_dequantize: null pointer");
  if (w->N < 0 || w->K < 0 || expert < 0 || expert >= w->n_experts)
    return fail(GBW_E_ARG, "mx_dequantize: bad extent or expert");
  if (!w->codes || !w->scales) return fail(GBW_E_ARG, "mx_dequantize: null codes/scales");
  const int64_t N = w->N, K = w->K;
  const int qb = w->qblock ? w->qblock : 64;
  const int qsh = qb == 256 ? 8 : qb == 128 ? 7 : 6;
  int64_t cbytes, sbytes;
  switch (w->fmt) {
    case GBW_FMT_E8M0_B32:
      if (K % 32) return fail(GBW_E_SHAPE, "mx_dequantize: K %% 32");
      cbytes = N * K / 2;
      sbytes = N * K / 32;
      break;
    case GBW_FMT_E4M3_B16:
    case GBW_FMT_E5M3_B16:
      if (K % 16) return fail(GBW_E_SHAPE, "mx_dequantize: K %% 16");
      if (!w->tensor_scale || w->ts_per_expert < 1 || N % w->ts_per_expert)
        return fail(GBW_E_ARG, "mx_dequantize: bad tensor scale");
      cbytes = N * K / 2;
      sbytes = N * K / 16;
      break;
    case GBW_FMT_VQ4_E8M0:
    case GBW_FMT_VQ4_POST:
    case GBW_FMT_VQ4_PLUS:
    case GBW_FMT_VQ4_E4M3:
    case GBW_FMT_VQ4_E4M3_POST:
    case GBW_FMT_VQ4_E4M3_PLUS:
    case GBW_FMT_VQ4_E5M3:
    case GBW_FMT_VQ4_E5M3_POST:
    case GBW_FMT_VQ4_E5M3_PLUS: {
      if (qb != 64 && qb != 128 && qb != 256) return fail(GBW_E_ARG, "mx_dequantize: QBlock edge must be 64, 128 or 256");
      if (K % qb || N % qb) return fail(GBW_E_SHAPE, "mx_dequantize: VQ needs N, K multiples of the QBlock edge");
      if (!w->codebook) return fail(GBW_E_ARG, "mx_dequantize: VQ needs a codebook");
      const bool b16 = w->fmt >= GBW_FMT_VQ4_E4M3;
      const int lay = b16 ? (w->fmt - GBW_FMT_VQ4_E4M3) % 3 : w->fmt == GBW_FMT_VQ4_POST ? 1 : w->fmt == GBW_FMT_VQ4_PLUS ? 2 : 0;
      const int bs = b16 ? 16 : 32;
      cbytes = N * K / 4;
      sbytes = lay == 0 ? N * K / bs : lay == 1 ? (N / qb) * (K / qb) : N * K / (8 * bs);
      if (lay == 2 && (K % (8 * bs) || !w->scale_codebook))
        return fail(w->scale_codebook ? GBW_E_SHAPE : GBW_E_ARG,
                    "mx_dequantize: PreScale+ needs K a multiple of 8 scale blocks and a scale codebook");
      if (b16 && (!w->tensor_scale || w->ts_per_expert < 1 || N % w->ts_per_expert))
        return fail(GBW_E_ARG, "mx_dequantize: bad tensor scale");
      break;
    }
    default:
      return fail(GBW_E_ARG, "mx_dequantize: bad format");
  }
  if (N == 0 || K == 0) return GBW_OK;
  int st = check_device();
  if (st) return st;
  const bool vq = w->fmt == GBW_FMT_VQ4_E8M0 || w->fmt == GBW_FMT_VQ4_POST || w->fmt == GBW_FMT_VQ4_PLUS ||
                  (w->fmt >= GBW_FMT_VQ4_E4M3 && w->fmt <= GBW_FMT_VQ4_E5M3_PLUS);
  const bool plus = w->fmt == GBW_FMT_VQ4_PLUS || w->fmt == GBW_FMT_VQ4_E4M3_PLUS || w->fmt == GBW_FMT_VQ4_E5M3_PLUS;
  const uint16_t* cb = vq ? w->codebook + (int64_t)expert * (N / qb) * (K / qb) * 256 : nullptr;
  const uint8_t* scb = plus ? w->scale_codebook + (int64_t)expert * 2048 : nullptr;
  const float* ts = w->tensor_scale ? w->tensor_scale + (int64_t)expert * w->ts_per_expert : nullptr;
  const int64_t n = N * K;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, as_stream(stream), w->fmt,
                     w->codes + expert * cbytes, w->scales + expert * sbytes, cb, scb, qsh, ts,
                     w->ts_per_expert > 0 ? w->ts_per_expert : 1, N, K, out);
  return check_launch("mx_dequantize");
}

extern "C" int mx_residual(const float* w, int64_t N, int64_t K, int64_t tail, const uint8_t* codes,
                           const uint8_t* scales, float* r, void* stream) {
  if (N < 0 || K < 0 || tail < 0) return fail(GBW_E_ARG, "mx_residual: negative extent");
  if (K % 32 || tail % 32 || tail > K) return fail(GBW_E_SHAPE, "mx_residual: bad K/tail");
  if (N == 0 || tail == 0) return GBW_OK;
  if (!w || !codes || !scales || !r) return fail(GBW_E_ARG, "mx_residual: null pointer");
  int st = check_device();
  if (st) return st;
  const int64_t n = N * tail;
  hipLaunchKernelGGL(k_residual, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, as_stream(stream), w, N, K,
                     tail, codes, scales, r);
  return check_launch("mx_residual");
}
