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
// the lookups.  The decoded fp16 weights feed fp16 MFMA directly; fp32
// accumulation.
//
// Activations: bf16 has fp32's exponent range, fp16 a much narrower one, so
// x is not converted to fp16 as it is.  Each 128-element chunk of an x row is
// multiplied by a power of two 2^s chosen from the chunk's largest magnitude
// (that magnitude lands in [2^14, 2^15), far from fp16's 65504), converted to
// fp16, contracted, and the chunk's fp32 partial sum is multiplied by 2^-s
// before it joins the row's sum.  Both multiplies are exact; every bf16 value
// within 2^31 of its chunk's largest is exact in fp16 after the scaling (a
// smaller one contributes less than 2^-31 of that chunk's largest product,
// and is rounded).  So any finite bf16 input works, 1e30 and 2^-30 alike.
//
// Decode order: inside each 8-element piece the decode yields the elements
// in the order 0,2,4,6,1,3,5,7 (even nibbles, then odd); x is staged in LDS as
// fp16 in the same order, so both MFMA operands pair the same K indices.
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

// max over the 16 lanes of a DPP row (lanes 16r .. 16r + 15)
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm: lane ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm: lane ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true));  // row_ror:8
  return v;
}

// Power-of-two prescale exponent of an x chunk from the bf16 magnitude bits
// of its largest element: 2^s puts that element in [2^14, 2^15); zero and
// bf16-subnormal chunks take the largest exponent used, 126 (every value
// stays below 2); clamped to [-126, 126] so 2^s and 2^-s are normal fp32.
__device__ __forceinline__ int chunk_prescale(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 7);  // biased exponent field (255: inf / NaN)
  int s = e == 0 ? 126 : 141 - e;       // 14 - (e - 127)
  return s < -126 ? -126 : (s > 126 ? 126 : s);
}
__device__ __forceinline__ float pow2f(int s) { return __uint_as_float((uint32_t)(s + 127) << 23); }

// Eight bf16 (four dwords, element 2i in the low half of dword i), times
// 2^s, to fp16 in the decode order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ v4i x8_to_f16(v4i v, float scale) {
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_to_f32((uint32_t)v[e] & 0xFFFFu) * scale;
    f[2 * e + 1] = bf16_to_f32((uint32_t)v[e] >> 16) * scale;
  }
  const v8h h = v8h{(_Float16)f[0], (_Float16)f[2], (_Float16)f[4], (_Float16)f[6],
                    (_Float16)f[1], (_Float16)f[3], (_Float16)f[5], (_Float16)f[7]};
  return __builtin_bit_cast(v4i, h);
}

struct LutArgs {
  int64_t M, N, K;
  int32_t group;
  const uint16_t* x;     // [M][K] bf16
  const uint8_t* idx;    // [N][K/2]
  const uint16_t* cent;  // [N][K/group][16] fp16
  float* y;              // [M][N]
  float* part;           // [tiles][splits][32 MT x 64] fp32 partial tiles (splits > 1)
  uint32_t* counters;    // one arrival counter per output tile (splits > 1), zero between calls
  int32_t chunks_per_split;  // 128-element chunks of K per workgroup
  int32_t splits;
};

// ---------------------------------------------------------------------------
// M <= 16: one workgroup per 16 output rows n over the whole of K
// ---------------------------------------------------------------------------
// The 16 rows' indices and tables are contiguous in HBM ([N][K/2] and
// [N][K/group][16]); a segment of up to KSEG elements of all 16 rows is
// copied into LDS by direct loads, each instruction one contiguous kilobyte
// of one row (LDS rows padded by 16 bytes, so the 16 rows a fragment read
// touches fall in different banks).  Each wave has at most two 128-element
// chunks of a segment, w and w + NW; their x rows are loaded into registers
// before the copy is waited for.  Then wave w converts each chunk's x rows
// (16 lanes per row, the chunk's prescale from a 16-lane maximum) into its
// own LDS slot -- rows >= M are never written and feed only outputs that are
// never stored -- and a lane (r16 = n, q) decodes elements [32q, 32q + 32)
// of row n and feeds them to four v_mfma_f32_16x16x32_f16 steps.  The NW
// per-wave 16 x 16 partial products are summed in LDS in wave order (a fixed
// order: repeatable).
template <int NW, int XRND>
__global__ __launch_bounds__(64 * NW) void k_lut_gemv(const LutArgs p) {
  constexpr int XROW = 128 * 2 + 16;         // LDS bytes per x row of a chunk slot (16-byte pad)
  constexpr int WLDS = 64 * 1024;            // weight segment: 16 rows of indices + tables
  __shared__ __attribute__((aligned(16))) uint8_t sw[WLDS + 2 * 16 * 16];
  __shared__ __attribute__((aligned(16))) uint8_t xs[NW][16 * XROW];
  __shared__ __attribute__((aligned(16))) float invs[NW][16];
  __shared__ float red[NW][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int M = (int)p.M;  // XRND = ceil(M / 4): rounds of 64 x pieces (16 lanes per row)
  const int64_t G = p.K / p.group;
  const int kseg = p.group == 32 ? 2048 : 4096;   // elements per segment: 16 rows fit WLDS
  static_assert(NW == 16, "a segment of 4096 elements is two chunks per wave");
  const int tpc = 128 / p.group;                  // tables per 128-element chunk
  const int64_t tb_row = (int64_t)G * 32;         // table bytes per row in HBM

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < p.K; k0 += kseg) {
    const int seg = (int)(p.K - k0 < kseg ? p.K - k0 : kseg);
    const int ib = seg / 2, tbb = seg / p.group * 32;  // index and table bytes per row of the segment
    const int irow = ib + 16, trow = tbb + 16;          // LDS row strides
    uint8_t* const si = sw;
    uint8_t* const st = sw + 16 * irow;
    const int nch = seg / 128;  // <= 2 NW: a wave has at most two chunks of a segment
    // x of the wave's chunks wave and wave + NW, loaded before the weights
    // are waited for (rows >= M load row M - 1 and are never stored)
    v4i xv[2][XRND];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = wave + NW * i < nch ? wave + NW * i : nch - 1;
#pragma unroll
      for (int t = 0; t < XRND; ++t) {
        const int m = min((lane + 64 * t) >> 4, M - 1);
        xv[i][t] = load16(p.x + (int64_t)m * p.K + k0 + (int64_t)c * 128 + 8 * (lane & 15));
      }
    }
    // copy: 16 rows x ib index bytes, then 16 rows x tbb table bytes, 1 KiB per instruction
    const int ipc = (ib + 1023) / 1024, tpcs = (tbb + 1023) / 1024;  // pieces per row
    for (int pc = wave; pc < 16 * (ipc + tpcs); pc += NW) {
      const bool isidx = pc < 16 * ipc;
      const int rel = isidx ? pc : pc - 16 * ipc;
      const int r = rel / (isidx ? ipc : tpcs), part = rel % (isidx ? ipc : tpcs);
      const int len = isidx ? ib : tbb;
      const int o = part * 1024 + lane * 16;
      int64_t n = n0 + r;
      n = n < p.N ? n : p.N - 1;
      if (o < len) {
        const uint8_t* src = isidx ? p.idx + n * (p.K / 2) + k0 / 2 + o
                                   : reinterpret_cast<const uint8_t*>(p.cent) + n * tb_row + (k0 / p.group) * 32 + o;
        // streaming: each weight byte is read once per call (measured: 7.8 -> 7.5 us
        // at M = 1 and 8.6 -> 8.2 us at M = 8 with the weights in HBM)
        load_lds16<true>(src, (isidx ? si + r * irow : st + r * trow) + part * 1024);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = wave + NW * i;
      if (c >= nch) break;  // uniform over the wave
      // x rows of the chunk -> prescaled fp16 in decode order, this wave's slot
#pragma unroll
      for (int t = 0; t < XRND; ++t) {
        const int u = lane + 64 * t;
        const int m = u >> 4, j = u & 15;
        const int sx = chunk_prescale(row16_max_u32(bf16x8_absmax_bits(xv[i][t])));
        if (m < M) {  // the same for all 16 lanes of a DPP row
          *reinterpret_cast<v4i*>(&xs[wave][m * XROW + 16 * j]) = x8_to_f16(xv[i][t], pow2f(sx));
          if (j == 0) invs[wave][m] = pow2f(-sx);
        }
      }
      const v4i iq = *reinterpret_cast<const v4i*>(si + r16 * irow + c * 64 + 16 * q);
      const uint8_t* tr = st + r16 * trow + (c * tpc + (32 * q) / p.group) * 32;
      uint32_t L[4], H[4];
      split_table(*reinterpret_cast<const v4i*>(tr), *reinterpret_cast<const v4i*>(tr + 16), L, H);
      v4f part = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t o[4];
        decode8((uint32_t)iq[s], L, H, o);
        const v8h bfrag = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
        const v8h afrag = *reinterpret_cast<const v8h*>(&xs[wave][r16 * XROW + (32 * q + 8 * s) * 2]);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(afrag, bfrag, part, 0, 0, 0);
      }
      // part[r]: x row 4q + r; undo that row's prescale for this chunk
      const v4f inv = *reinterpret_cast<const v4f*>(&invs[wave][4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += part[r] * inv[r];
    }
    __syncthreads();  // the segment's LDS copy is free again
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

// ---------------------------------------------------------------------------
// M > 16: 64 output columns x 32*MT rows of x per workgroup, K split S ways
// ---------------------------------------------------------------------------
// Eight waves: two blocks of 32 output columns (n) x four K groups.  The
// workgroup owns one range of the K chunks (split blockIdx.y of S); K group
// g takes its chunks g, g + 4, ... .  Per round of four chunks (one per K
// group) the two waves of a K group convert that chunk's x rows into the
// group's LDS slot (prescaled fp16, 16 lanes per row), barrier; then each
// wave contracts its 32 columns: v_mfma_f32_32x32x16_f16, lane l holding
// column (or x row) l % 32 and, in step s, elements 64(l/32) + 8s .. + 7 of
// the chunk for A and B alike, eight steps per chunk into a zeroed
// accumulator that joins the running sum through the rows' inverse
// prescales; barrier.  The four K groups' sums meet in LDS in group order.
// With S > 1 every workgroup writes its tile to a partial slab; the last of
// the tile's S workgroups to arrive (an atomic counter per tile) adds the
// slabs in split order -- a fixed order whatever the arrival order, so the
// result is bitwise repeatable -- writes y and resets the counter.  The
// partial tiles of one call are written and read back within it, mostly
// from L2.
template <int MT>
__global__ __launch_bounds__(512) void k_lut_gemm(const LutArgs p) {
  constexpr int XR = 32 * MT;          // x rows per tile
  constexpr int XROW = 128 * 2 + 16;   // LDS bytes per x row of a chunk slot
  constexpr int XSB = 4 * XR * XROW;   // the four slots
  constexpr int REDB = 8 * MT * 16 * 64 * 4 + XR * 64 * 4;  // per-wave partial sums, then the tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[XSB > REDB ? XSB : REDB];
  __shared__ __attribute__((aligned(16))) float invs[4][XR];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = wave & 1, kg = wave >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t ntile0 = (int64_t)blockIdx.x * 64;
  const int64_t n0 = ntile0 + 32 * nb;
  const int64_t m0 = (int64_t)blockIdx.z * XR;
  const int chunks = (int)(p.K / 128);
  const int cs0 = blockIdx.y * p.chunks_per_split;
  const int nc = min(chunks - cs0, p.chunks_per_split);  // >= 1: the host makes no empty split
  const int rounds = (nc + 3) / 4;
  const int64_t G = p.K / p.group;
  const int64_t n = n0 + l32 < p.N ? n0 + l32 : p.N - 1;
  uint8_t* const xs = smem + kg * XR * XROW;

  v16f acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = v16f{};

  constexpr int XP = XR * 16 / 128;  // x pieces (8 elements) per lane per chunk
  // Rounds go two at a time: every load of both (the lane's indices and
  // tables, its share of the chunk's x rows) is issued before the first is
  // used, so a workgroup has its whole K range in flight at once.
  for (int rb = 0; rb < rounds; rb += 2) {
    v4i iq[2][2], ta[2][2], tb[2][2], xv[2][XP];
    bool has[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int cl = 4 * (rb + r) + kg;  // chunk of the range for this K group
      has[r] = cl < nc;                  // the same for both waves of the group
      const int c = cs0 + (has[r] ? cl : nc - 1);
      const uint8_t* ir = p.idx + n * (p.K / 2) + (int64_t)c * 64 + 32 * h;
      iq[r][0] = load16(ir);
      iq[r][1] = load16(ir + 16);
      const int64_t g0 = ((int64_t)c * 128 + 64 * h) / p.group;  // table of elements 64h .. 64h + 31
      const int64_t g1 = ((int64_t)c * 128 + 64 * h + 32) / p.group;
      const uint16_t* t0 = p.cent + (n * G + g0) * 16;
      const uint16_t* t1 = p.cent + (n * G + g1) * 16;
      ta[r][0] = load16(t0);
      tb[r][0] = load16(t0 + 8);
      ta[r][1] = load16(t1);  // the same table unless group == 32
      tb[r][1] = load16(t1 + 8);
#pragma unroll
      for (int t = 0; t < XP; ++t) {
        const int u = nb * 64 + lane + 128 * t;
        const int64_t m = m0 + (u >> 4);
        xv[r][t] = m < p.M ? load16(p.x + m * p.K + (int64_t)c * 128 + 8 * (u & 15)) : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (rb + r >= rounds) break;  // uniform over the workgroup
      // x: XR rows x 16 pieces of this K group's chunk over its 128 lanes
#pragma unroll
      for (int t = 0; t < XP; ++t) {
        const int u = nb * 64 + lane + 128 * t;
        const int row = u >> 4, j = u & 15;
        const int s = chunk_prescale(row16_max_u32(bf16x8_absmax_bits(xv[r][t])));
        *reinterpret_cast<v4i*>(xs + row * XROW + 16 * j) = x8_to_f16(xv[r][t], pow2f(s));
        if (j == 0) invs[kg][row] = pow2f(-s);
      }
      __syncthreads();
      if (has[r]) {
        uint32_t L0[4], H0[4], L1[4], H1[4];
        split_table(ta[r][0], tb[r][0], L0, H0);
        split_table(ta[r][1], tb[r][1], L1, H1);
        const uint32_t wd[8] = {(uint32_t)iq[r][0][0], (uint32_t)iq[r][0][1], (uint32_t)iq[r][0][2],
                                (uint32_t)iq[r][0][3], (uint32_t)iq[r][1][0], (uint32_t)iq[r][1][1],
                                (uint32_t)iq[r][1][2], (uint32_t)iq[r][1][3]};
        v8h bf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          uint32_t o[4];
          if (s < 4)
            decode8(wd[s], L0, H0, o);
          else
            decode8(wd[s], L1, H1, o);
          bf[s] = __builtin_bit_cast(v8h, v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          v16f part = v16f{};
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const v8h af = *reinterpret_cast<const v8h*>(xs + (32 * i + l32) * XROW + (64 * h + 8 * s) * 2);
            part = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[s], part, 0, 0, 0);
          }
          // part[r]: x row 32i + 8(r/4) + 4h + r%4
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4f inv = *reinterpret_cast<const v4f*>(&invs[kg][32 * i + 8 * q + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][4 * q + e] += part[4 * q + e] * inv[e];
          }
        }
      }
      __syncthreads();
    }
  }

  // the four K groups' sums, in group order, into a row-major tile in LDS
  float* red = reinterpret_cast<float*>(smem);                // [wave][MT][16][64]
  float* tile = red + 8 * MT * 16 * 64;                       // [XR][64]: row m, column n
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave * MT + i) * 16 + r) * 64 + lane] = acc[i][r];
  __syncthreads();
  constexpr int OUTS = 2 * MT * 16 * 64;  // outputs of the tile (2 column blocks)
#pragma unroll
  for (int t = 0; t < OUTS / 512; ++t) {
    const int o = (int)threadIdx.x + 512 * t;
    const int ob = o / (MT * 1024), rem = o % (MT * 1024);  // column block, then (i, r, lane)
    const int i = rem / 1024, r = (rem / 64) % 16, l = rem % 64;
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) sum += red[(((2 * g + ob) * MT + i) * 16 + r) * 64 + l];
    tile[(32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)) * 64 + 32 * ob + (l & 31)] = sum;
  }
  __syncthreads();

  // 16-byte pieces: XR rows x 16
  constexpr int PC = XR * 16 / 512;  // pieces per thread
  const bool vec = (p.N & 3) == 0 && !(reinterpret_cast<uintptr_t>(p.y) & 15u);
  auto store_y = [&](int pc, v4f v) __attribute__((always_inline)) {
    const int64_t m = m0 + (pc >> 4), nn = ntile0 + 4 * (pc & 15);
    if (m >= p.M || nn >= p.N) return;
    float* dst = p.y + m * p.N + nn;
    if (vec && nn + 4 <= p.N) {
      *reinterpret_cast<v4f*>(dst) = v;
    } else {
      for (int e = 0; e < 4 && nn + e < p.N; ++e) dst[e] = v[e];
    }
  };
  if (p.splits == 1) {
#pragma unroll
    for (int u = 0; u < PC; ++u) {
      const int pc = (int)threadIdx.x + 512 * u;
      store_y(pc, *reinterpret_cast<const v4f*>(tile + 4 * pc));
    }
    return;
  }
  // this tile's S slots of XR x 64 fp32, one per split, contiguous; the last
  // workgroup to arrive sums them in split order
  const int64_t tile_id = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
  constexpr uint32_t SLOT = XR * 64 * 4;  // bytes
  const __amdgpu_buffer_rsrc_t rs = shared_tile_rsrc(p.part + tile_id * p.splits * (XR * 64), SLOT * p.splits);
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int pc = (int)threadIdx.x + 512 * u;
    store_shared_v4(rs, SLOT * blockIdx.y + 16 * pc, *reinterpret_cast<const v4f*>(tile + 4 * pc));
  }
  if (!arrive_last(p.counters + tile_id, p.splits, &s_last)) return;
  constexpr int SMX = 8;  // splits whose loads are in flight together
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int pc = (int)threadIdx.x + 512 * u;
    const v4f own = *reinterpret_cast<const v4f*>(tile + 4 * pc);
    v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < p.splits; sp0 += SMX) {
      v4f ld[SMX];
#pragma unroll
      for (int q = 0; q < SMX; ++q) {
        const int sp = sp0 + q;
        ld[q] = sp < p.splits && sp != (int)blockIdx.y ? load_shared_v4(rs, SLOT * sp + 16 * pc) : own;
      }
#pragma unroll
      for (int q = 0; q < SMX; ++q)
        if (sp0 + q < p.splits) sum += ld[q];
    }
    store_y(pc, sum);
  }
}

constexpr int kGemvNW = 16;

// K splits for the M > 16 kernel: about one workgroup per CU over all tiles,
// each K group with at least one chunk when K allows it
static int lut_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = cdiv(N, 64) * cdiv(M, 64);
  const int chunks = (int)(K / 128);
  const int most = chunks / 4 > 1 ? chunks / 4 : 1;
  int64_t s = cdiv(device_cu_count(), tiles);
  s = s < 1 ? 1 : (s > most ? most : s);
  const int per = (int)cdiv(chunks, s);
  return (int)cdiv(chunks, per);  // no empty split
}

size_t ws_lut_gemm(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || N <= 0 || K <= 0 || K % 128) return 0;  // M <= 16: one kernel, no partials
  if (cdiv(N, 64) * cdiv(M, 64) > kWsMaxTiles) return 0;  // too many tiles for the counters: no split
  const int splits = lut_splits(M, N, K);
  const int64_t xr = M <= 32 ? 32 : 64;  // x rows per tile
  return splits > 1 ? kWsCounterBytes + (size_t)(cdiv(N, 64) * cdiv(M, xr)) * splits * xr * 64 * sizeof(float) : 0;
}

}  // namespace gbw

using namespace gbw;

extern "C" int lut_gemm(int64_t M, int64_t N, int64_t K, int32_t group, const uint16_t* x_bf16, const uint8_t* idx,
                        const uint16_t* centroids_f16, float* y, int32_t flags, void* ws, size_t ws_bytes,
                        void* stream) {
  (void)flags;  // every path sums in a fixed order: results are bitwise repeatable
  if (M < 0 || N < 0 || K < 0) return fail(GBW_E_ARG, "lut_gemm: negative extent");
  if (group != 32 && group != 64 && group != 128)
    return fail(GBW_E_SHAPE, "lut_gemm: group must be 32, 64 or 128");
  if (K % 128) return fail(GBW_E_SHAPE, "lut_gemm: K must be a multiple of 128");
  if (M == 0 || N == 0) return GBW_OK;
  if (K == 0) return fail(GBW_E_SHAPE, "lut_gemm: K must be positive");
  if (!x_bf16 || !idx || !centroids_f16 || !y) return fail(GBW_E_ARG, "lut_gemm: null pointer");
  if (!aligned16(x_bf16) || !aligned16(idx) || !aligned16(centroids_f16))
    return fail(GBW_E_ALIGN, "lut_gemm: x/idx/centroids not 16-byte aligned");
  if (M > 16 && (int64_t)cdiv(N, 64) * cdiv(M, 64) > 0x7FFFFFFF)
    return fail(GBW_E_SHAPE, "lut_gemm: too many output tiles");
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
  hipStream_t s = as_stream(stream);
  if (M <= 16) {
    const dim3 grid((unsigned)cdiv(N, 16)), block(64 * kGemvNW);
    switch ((M + 3) / 4) {
      case 1: hipLaunchKernelGGL((k_lut_gemv<kGemvNW, 1>), grid, block, 0, s, p); break;
      case 2: hipLaunchKernelGGL((k_lut_gemv<kGemvNW, 2>), grid, block, 0, s, p); break;
      case 3: hipLaunchKernelGGL((k_lut_gemv<kGemvNW, 3>), grid, block, 0, s, p); break;
      default: hipLaunchKernelGGL((k_lut_gemv<kGemvNW, 4>), grid, block, 0, s, p); break;
    }
    return check_launch("lut_gemm");
  }
  const int chunks = (int)(K / 128);
  int splits = lut_splits(M, N, K);
  // too little workspace for the partial tiles: one workgroup per tile over
  // all of K (no workspace; slower, same results up to the summation order)
  if (splits > 1 && (!ws || ws_lut_gemm(M, N, K) == 0 || ws_bytes < ws_lut_gemm(M, N, K) || ((uintptr_t)ws & 15u)))
    splits = 1;
  p.chunks_per_split = (int)cdiv(chunks, splits);
  p.splits = splits;
  if (splits > 1) {
    p.counters = reinterpret_cast<uint32_t*>(ws);
    p.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + kWsCounterBytes);
  }
  const dim3 grid((unsigned)cdiv(N, 64), (unsigned)splits, (unsigned)cdiv(M, M <= 32 ? 32 : 64));
  if (M <= 32)
    hipLaunchKernelGGL((k_lut_gemm<1>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((k_lut_gemm<2>), grid, dim3(512), 0, s, p);
  return check_launch("lut_gemm");
}
