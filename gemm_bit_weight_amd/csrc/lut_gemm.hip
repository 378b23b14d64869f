// Codebook (clustered) weight GEMM: 4-bit indices into a 16-entry fp16
// centroid table per (output row, K group).
//
// y[m][n] = sum_k bf16(x[m][k]) * fp16(C[n][k / group][idx[n][k]])
//
// "CodeQuant: Unified Clustering and Quantization for Enhanced Outlier
// Smoothing in Low-Precision Mixture-of-Experts", Fig. 1 (stage 3 clusters
// the weights, stage 4 deploys them through a LUT kernel) and Fig. 4 (one
// tile of the matmul; a lookup table built once per tile, then looked up).
// The pages' kernel keeps its table in shared memory; here each lane keeps
// the 16-entry table of its own (row, group) in eight VGPRs, split into a
// low-byte plane and a high-byte plane, and looks up four indices at once
// with byte permutes (v_perm_b32) -- no LDS traffic and no bank conflicts for
// the lookups.  The decoded fp16 weights feed fp16 MFMA (16x16x32) directly;
// fp32 accumulation.
//
// Data path per wave: 16 output rows n; per K group of 128 a lane (n, q)
// holds elements [32q, 32q + 32) of that group: one 16-byte index load, its
// table (two 16-byte loads), four MFMA steps of 8 elements.  Inside each
// 8-element step the decode yields the elements in the order 0,2,4,6,1,3,5,7
// (even nibbles, then odd); x is staged in LDS as fp16 in the same order, so
// both MFMA operands pair the same K indices.
//
// x (bf16) is converted to fp16 once per workgroup while it is staged; values
// with |x| < 2^-17 lose low bits in fp16's subnormal range (a relative error
// far below the output tolerance), every other bf16 value is exact in fp16.
#include "common.hpp"

namespace gbw {

// byte-wise table lookup: each byte of s (0..15) selects one byte of the
// 16-byte table t[0..3]
__device__ __forceinline__ uint32_t lut16(uint32_t s7, uint32_t mask, const uint32_t (&t)[4]) {
  const uint32_t lo = __builtin_amdgcn_perm(t[1], t[0], s7);  // entries 0..7
  const uint32_t hi = __builtin_amdgcn_perm(t[3], t[2], s7);  // entries 8..15
  return (hi & mask) | (lo & ~mask);
}

// Eight 4-bit indices (one dword) -> eight fp16 centroids as four fp16x2
// words, element order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ void decode8(uint32_t w, const uint32_t (&L)[4], const uint32_t (&H)[4], uint32_t (&o)[4]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t s = half == 0 ? (w & 0x0F0F0F0Fu) : ((w >> 4) & 0x0F0F0F0Fu);
    const uint32_t s7 = s & 0x07070707u;
    const uint32_t b3 = (s >> 3) & 0x01010101u;
    const uint32_t mask = (b3 << 8) - b3;  // 0xFF in every byte whose index is >= 8
    const uint32_t lo = lut16(s7, mask, L);
    const uint32_t hi = lut16(s7, mask, H);
    o[2 * half + 0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[2 * half + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
}

// 16 fp16 centroids (8 dwords, entry 2i in the low half of dword i) -> low-
// and high-byte planes of four dwords each.
__device__ __forceinline__ void split_table(const v4i a, const v4i b, uint32_t (&L)[4], uint32_t (&H)[4]) {
  const uint32_t d[8] = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3],
                         (uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    L[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x06040200u);
    H[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07050301u);
  }
}

struct LutArgs {
  int64_t M, N, K;
  int32_t group;
  const uint16_t* x;     // [M][K] bf16
  const uint8_t* idx;    // [N][K/2]
  const uint16_t* cent;  // [N][K/group][16] fp16
  float* y;              // [M][N]
  float* part;           // [splits][M][N]
  int32_t chunks_per_split;  // 128-element chunks of K per workgroup
  int32_t split;
};

// Workgroup: NW waves x 16 rows of W each; 16*TM rows of x; KR chunks of 128
// along K (one split).
template <int TM, int NW, int KR>
__global__ __launch_bounds__(64 * NW) void k_lut_gemm(const LutArgs p) {
  constexpr int XR = 16 * TM;
  constexpr int LDX = KR * 128 * 2 + 16;  // LDS bytes per x row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint8_t xs[XR * LDX];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * NW + wave) * 16;
  const int64_t m0 = (int64_t)blockIdx.z * XR;
  const int c0 = blockIdx.y * p.chunks_per_split;
  const int nc = min((int)(p.K / 128) - c0, p.chunks_per_split);
  const int64_t G = p.K / p.group;

  // --- weight slice: all loads issued up front --------------------------
  int64_t n = n0 + r16;
  n = n < p.N ? n : p.N - 1;
  v4i iq[KR], ca[KR], cb[KR];
#pragma unroll
  for (int c = 0; c < KR; ++c) {
    const int cc = c0 + (c < nc ? c : nc - 1);
    const int64_t k = (int64_t)cc * 128 + 32 * q;  // this lane's first element
    iq[c] = load16(p.idx + n * (p.K / 2) + k / 2);
    const uint16_t* t = p.cent + (n * G + k / p.group) * 16;
    ca[c] = load16(t);
    cb[c] = load16(t + 8);
  }

  // --- x range -> LDS as fp16, 8-element chunks in order 0,2,4,6,1,3,5,7 --
  // all global loads first (one round trip), then convert and store
  constexpr int XCH = XR * KR * 16;  // 8-element chunks
  constexpr int PER = XCH / (64 * NW);
  static_assert(XCH % (64 * NW) == 0, "x range must split evenly over the workgroup");
  v4i xv[PER];
  bool xok[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int u = threadIdx.x + t * 64 * NW;
    const int row = u / (KR * 16), j = u % (KR * 16);
    int64_t m = m0 + row;
    xok[t] = m < p.M && j / 16 < nc;
    m = m < p.M ? m : p.M - 1;
    const int jj = j / 16 < nc ? j : j % 16;  // stay inside this split's range
    xv[t] = load16(p.x + m * p.K + (int64_t)c0 * 128 + jj * 8);
  }
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int u = threadIdx.x + t * 64 * NW;
    const int row = u / (KR * 16), j = u % (KR * 16);
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (xok[t]) {
      const v4i v = xv[t];
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_to_f32((uint32_t)v[e] & 0xFFFFu);
        f[2 * e + 1] = bf16_to_f32((uint32_t)v[e] >> 16);
      }
      const int ord[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 h0 = (_Float16)f[ord[2 * e]], h1 = (_Float16)f[ord[2 * e + 1]];
        o[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      }
    }
    *reinterpret_cast<v4i*>(xs + row * LDX + j * 16) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  }
  __syncthreads();

  v4f acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < KR; ++c) {
    if (c < nc) {
      uint32_t L[4], H[4];
      split_table(ca[c], cb[c], L, H);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        decode8((uint32_t)iq[c][s], L, H, o);
        const v8h bfrag = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4i xa = *reinterpret_cast<const v4i*>(xs + (16 * i + r16) * LDX + (c * 128 + 32 * q + 8 * s) * 2);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xa), bfrag, acc[i], 0, 0, 0);
        }
      }
    }
  }

  const int64_t nn = n0 + r16;
  if (nn >= p.N) return;
  float* out = p.split ? p.part + (int64_t)blockIdx.y * p.M * p.N : p.y;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 16 * i + 4 * q + r;
      if (m < p.M) out[m * p.N + nn] = acc[i][r];
    }
}

// Decode shape (M <= 16): one workgroup per 16 output rows n over the whole
// of K, so a call is one kernel with no partial sums in HBM.  Wave w takes
// the 128-element chunks w, w + NW, ...; a lane (r16 = n, q) holds elements
// [32q, 32q + 32) of a chunk as above.  Every weight load of a batch of CB
// chunks is issued before the first is used, so a CU has all its weight
// bytes in flight at once.  The x rows of the wave's chunks (M x 128 each)
// are converted once, by the wave that uses them, into its own LDS slice
// (fp16, decode order); rows >= M of that slice are never written and feed
// only output rows that are never stored.  The NW per-wave 16 x 16 partial
// products are summed in LDS in wave order (a fixed order: repeatable).
template <int NW, int CB>
__global__ __launch_bounds__(64 * NW) void k_lut_gemv(const LutArgs p) {
  constexpr int XROW = 128 * 2 + 16;  // LDS bytes per x row in a chunk slot (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint8_t xs[NW][CB][16 * XROW];
  __shared__ float red[NW][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t n = n0 + r16 < p.N ? n0 + r16 : p.N - 1;
  const int chunks = (int)(p.K / 128);
  const int64_t G = p.K / p.group;
  const int M = (int)p.M;
  const uint8_t* wr = p.idx + n * (p.K / 2);
  const uint16_t* cr = p.cent + n * G * 16;

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int cb0 = wave; cb0 < chunks; cb0 += NW * CB) {
    v4i iq[CB], ca[CB], cc[CB];
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int c0 = cb0 + NW * b;
      const int c = c0 < chunks ? c0 : chunks - 1;  // clamped: redundant loads hit L2
      const int64_t k = (int64_t)c * 128 + 32 * q;  // this lane's first element
      iq[b] = load16(wr + k / 2);
      const uint16_t* t = cr + (k / p.group) * 16;
      ca[b] = load16(t);
      cc[b] = load16(t + 8);
    }
    // x: M rows x 128 of each chunk, 16 pieces of 8 per row -> fp16 in the
    // order 0,2,4,6,1,3,5,7 into this wave's slot
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int c0 = cb0 + NW * b;
      const int c = c0 < chunks ? c0 : chunks - 1;
      for (int u = lane; u < M * 16; u += 64) {
        const int m = u >> 4, j = u & 15;
        const v4i v = load16(p.x + (int64_t)m * p.K + (int64_t)c * 128 + 8 * j);
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16_to_f32((uint32_t)v[e] & 0xFFFFu);
          f[2 * e + 1] = bf16_to_f32((uint32_t)v[e] >> 16);
        }
        const v8h h = v8h{(_Float16)f[0], (_Float16)f[2], (_Float16)f[4], (_Float16)f[6],
                          (_Float16)f[1], (_Float16)f[3], (_Float16)f[5], (_Float16)f[7]};
        *reinterpret_cast<v8h*>(&xs[wave][b][m * XROW + 16 * j]) = h;
      }
    }
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      if (cb0 + NW * b >= chunks) break;
      uint32_t L[4], H[4];
      split_table(ca[b], cc[b], L, H);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        decode8((uint32_t)iq[b][s], L, H, o);
        const v8h bfrag = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
        const v8h afrag = *reinterpret_cast<const v8h*>(&xs[wave][b][r16 * XROW + (32 * q + 8 * s) * 2]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag, bfrag, acc, 0, 0, 0);
      }
    }
  }
  // acc[r]: x row 4q + r, output row n0 + r16
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][(4 * q + r) * 16 + r16] = acc[r];
  __syncthreads();
  for (int i = threadIdx.x; i < 256; i += 64 * NW) {
    const int m = i >> 4, c = i & 15;
    if (m < M && n0 + c < p.N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][i];
      p.y[(int64_t)m * p.N + n0 + c] = v;
    }
  }
}

constexpr int kGemvNW = 16, kGemvCB = 2;

// splits of K: enough workgroups for every CU, at most one resident round
static int lut_splits(int64_t M, int64_t N, int64_t K, int nw, int kr_max) {
  const int64_t tiles = cdiv(N, 16 * nw) * cdiv(M, 64);
  const int chunks = (int)(K / 128);
  int splits = (int)cdiv(chunks, kr_max);
  const int64_t slots = 2 * (int64_t)device_cu_count();
  while ((int64_t)(splits + 1) * tiles <= slots && splits < chunks) ++splits;
  const int per = (int)cdiv(chunks, splits);
  return (int)cdiv(chunks, per);
}

constexpr int kLutNW = 8;
constexpr int kLutKR = 4;

size_t ws_lut_gemm(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || N <= 0 || K <= 0 || K % 128) return 0;  // M <= 16: one kernel, no partials
  const int splits = lut_splits(M, N, K, kLutNW, kLutKR);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

template <int TM>
static int launch_lut(LutArgs& p, int splits, hipStream_t st) {
  p.chunks_per_split = (int)cdiv(p.K / 128, splits);
  p.split = splits > 1;
  hipLaunchKernelGGL((k_lut_gemm<TM, kLutNW, kLutKR>),
                     dim3((unsigned)cdiv(p.N, 16 * kLutNW), (unsigned)splits, (unsigned)cdiv(p.M, 16 * TM)),
                     dim3(64 * kLutNW), 0, st, p);
  int s = check_launch("lut_gemm");
  if (s || splits == 1) return s;
  return launch_splitk_reduce(p.part, splits, p.M * p.N, p.y, st);
}

}  // namespace gbw

using namespace gbw;

extern "C" int lut_gemm(int64_t M, int64_t N, int64_t K, int32_t group, const uint16_t* x_bf16, const uint8_t* idx,
                        const uint16_t* centroids_f16, float* y, int32_t flags, void* ws, size_t ws_bytes,
                        void* stream) {
  (void)flags;
  if (M < 0 || N < 0 || K < 0) return fail(GBW_E_ARG, "lut_gemm: negative extent");
  if (group != 32 && group != 64 && group != 128)
    return fail(GBW_E_SHAPE, "lut_gemm: group must be 32, 64 or 128");
  if (K % 128) return fail(GBW_E_SHAPE, "lut_gemm: K must be a multiple of 128");
  if (M == 0 || N == 0) return GBW_OK;
  if (K == 0) return fail(GBW_E_SHAPE, "lut_gemm: K must be positive");
  if (!x_bf16 || !idx || !centroids_f16 || !y) return fail(GBW_E_ARG, "lut_gemm: null pointer");
  if (!aligned16(x_bf16) || !aligned16(idx) || !aligned16(centroids_f16))
    return fail(GBW_E_ALIGN, "lut_gemm: x/idx/centroids not 16-byte aligned");
  int st = check_device();
  if (st) return st;
  LutArgs p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.group = group;
  p.x = x_bf16;
  p.idx = idx;
  p.cent = centroids_f16;
  p.y = y;
  p.part = reinterpret_cast<float*>(ws);
  hipStream_t s = as_stream(stream);
  if (M <= 16) {
    hipLaunchKernelGGL((k_lut_gemv<kGemvNW, kGemvCB>), dim3((unsigned)cdiv(N, 16)), dim3(64 * kGemvNW), 0, s, p);
    return check_launch("lut_gemm");
  }
  int splits = lut_splits(M, N, K, kLutNW, kLutKR);
  const int need = (int)cdiv(K / 128, kLutKR);
  if (splits > 1 && (!ws || ws_bytes < (size_t)splits * M * N * sizeof(float))) {
    const int fit = ws ? (int)(ws_bytes / ((size_t)M * N * sizeof(float))) : 0;
    if (fit >= need && fit >= 2)
      splits = fit;
    else if (need == 1)
      splits = 1;
    else
      return fail(GBW_E_WORKSPACE, "lut_gemm: needs %zu bytes of workspace", ws_lut_gemm(M, N, K));
  }
  if (M <= 32) return launch_lut<2>(p, splits, s);
  return launch_lut<4>(p, splits, s);
}
