// Dense MXFP4 (E8M0-B32) GEMM on CDNA4 scaled MFMA, with the PRQuant tail
// residual as a second K segment.
//
// y[M][N] = deq(A) deq(W)^T  (+ deq(A[:, K-tail:]) deq(R)^T)
//
// "PRQuant: Permutation Residual Quantization for Low-Overhead Inference",
// §4 "Offline residual augmentation" (W_aug^q = Q([W, R_W])) and "Kernel design
// for efficient inference": one MXFP4 GEMM over the reduction C + k.  Here the
// extra k columns of the activation are the last k columns of A read a second
// time in place (identical to the appended copy when the tail starts on a
// 32-element block boundary), so no copy is made.
//
// Two kernels, both on the scaled FP4 MFMA with one E8M0 scale per lane (a
// lane holds 32 consecutive K elements -- exactly one E8M0 block -- as 16
// bytes, and that block's scale; activation and weight use the same lane -> K
// mapping, so each lane's products pair the same K indices):
//  * k_mx_gemm (up to 16 rows, or K not a multiple of 128):
//    v_mfma_scale_f32_16x16x128_f8f6f4; lane (row r = lane % 16, group
//    g = lane / 16); the 16x16 fp32 result is lane l, register i = row
//    4*(l/16)+i, column l%16.  Each wave streams its own 16*TN weight rows.
//  * k_mx_gemm32 (17+ rows with 128-aligned K segments): the 32x32x64 shape,
//    which runs at twice the 16x16x128 rate; the weight slice is read once
//    for all rows of the M tile (up to 128).
// Decode-shaped problems (M <= 128, N in the thousands) stream the weights
// from HBM once; the K range is split across workgroups when the (N, M) tiles
// alone cannot fill 256 CUs.  k_mx_gemm32 reduces the splits inside the
// kernel (the last workgroup of a tile to arrive adds the split tiles in
// split order); k_mx_gemm writes one fp32 partial slab per split and
// k_splitk_reduce sums them in split order.  Either way the result is
// bitwise repeatable.
#include "common.hpp"

namespace gbw {

struct MxSeg {
  const uint8_t* w_codes;   // [N][K/2]
  const uint8_t* w_scales;  // [N][K/32]
  int64_t ldw, ldws;        // bytes per weight row: codes, scales
  int64_t a_k0;             // first A column this segment reads
  int64_t K;                // segment length, multiple of 32
  int32_t steps;            // ceil(K / 128)
};

struct MxGemmArgs {
  int64_t M, N;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  int64_t lda, ldas;  // bytes per A row: codes, scales
  MxSeg seg[2];
  int32_t total_steps, steps_per_split;
  float* y;
  int64_t ldy;
  int32_t atomic;  // 1: K is split over workgroups, partials go to `part`
  float* part;     // 16-row kernel: [splits][M][N] fp32; 32-row kernel: [tiles][splits][rows x 64] fp32
  uint32_t* counters;  // 32-row kernel with splits: one arrival counter per output tile, zero between calls
  int32_t splits;
};

// Fields of the segment that K step s belongs to.  Selected with uniform
// conditionals (never a dynamic index into the argument struct, which would
// force the arguments through memory and serialize the loads).
struct StepSeg {
  const uint8_t* wc;
  const uint8_t* ws;
  int64_t ldw, ldws, a_k0, K, k;  // k: first K element of step s within the segment
};

__device__ __forceinline__ StepSeg step_seg(const MxGemmArgs& p, int s) {
  const bool b = s >= p.seg[0].steps;
  StepSeg r;
  r.wc = b ? p.seg[1].w_codes : p.seg[0].w_codes;
  r.ws = b ? p.seg[1].w_scales : p.seg[0].w_scales;
  r.ldw = b ? p.seg[1].ldw : p.seg[0].ldw;
  r.ldws = b ? p.seg[1].ldws : p.seg[0].ldws;
  r.a_k0 = b ? p.seg[1].a_k0 : p.seg[0].a_k0;
  r.K = b ? p.seg[1].K : p.seg[0].K;
  r.k = (int64_t)(b ? s - p.seg[0].steps : s) * 128;
  return r;
}

__device__ __forceinline__ v8i widen(v4i x) {
  v8i r;
  r[0] = x[0];
  r[1] = x[1];
  r[2] = x[2];
  r[3] = x[3];
  r[4] = 0;
  r[5] = 0;
  r[6] = 0;
  r[7] = 0;
  return r;
}

// One workgroup: NW waves, each owning 16*TN output columns; all waves share
// the 16*TM rows of A and one contiguous range of at most SMAX K steps (128
// elements each).  The A range is staged once in LDS (rows padded by 16 bytes
// so the 16 lanes of a fragment read spread over the banks); every weight load
// of the range is issued before the first MFMA so the whole weight slice is in
// flight at once.
template <int TM, int TN, int NW, int SMAX>
__global__ __launch_bounds__(64 * NW) void k_mx_gemm(const MxGemmArgs p) {
  constexpr int ROWS = 16 * TM;
  constexpr int LDA = SMAX * 64 + 16;             // LDS bytes per A row
  constexpr int CHUNKS = ROWS * SMAX * 4;         // 16-byte A chunks (one E8M0 block each)
  constexpr int PER = CHUNKS / (64 * NW);         // chunks per thread
  static_assert(CHUNKS % (64 * NW) == 0, "A range must split evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t sa[ROWS * LDA];
  __shared__ uint8_t ss[ROWS * SMAX * 4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.z * ROWS;
  const int64_t n0 = ((int64_t)blockIdx.x * NW + wave) * (16 * TN);
  const int s0 = blockIdx.y * p.steps_per_split;
  const int ns = min(p.total_steps - s0, p.steps_per_split);

  // --- weight slice: straight-line loads, all in flight at once -----------
  // Steps past this split's range re-read its last step (their A is zero);
  // blocks past the segment end re-read its last block (A is zero there too).
  // The row pointers of both K segments are formed once; a step only picks
  // one of them (a uniform choice) and adds its K offset.
  const bool two = p.seg[1].steps > 0;
  v4i bq[SMAX][TN];
  int bsc[SMAX][TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int64_t n = n0 + 16 * j + r16;
    n = n < p.N ? n : p.N - 1;
    const uint8_t* wc0 = p.seg[0].w_codes + n * p.seg[0].ldw;
    const uint8_t* ws0 = p.seg[0].w_scales + n * p.seg[0].ldws;
    const uint8_t* wc1 = two ? p.seg[1].w_codes + n * p.seg[1].ldw : wc0;
    const uint8_t* ws1 = two ? p.seg[1].w_scales + n * p.seg[1].ldws : ws0;
#pragma unroll
    for (int t = 0; t < SMAX; ++t) {
      const int s = s0 + (t < ns ? t : ns - 1);
      const bool b = s >= p.seg[0].steps;
      const int64_t K = b ? p.seg[1].K : p.seg[0].K;
      int64_t kk = (int64_t)(b ? s - p.seg[0].steps : s) * 128 + 32 * g;
      kk = kk < K ? kk : K - 32;
      bq[t][j] = load16((b ? wc1 : wc0) + kk / 2);
      bsc[t][j] = (b ? ws1 : ws0)[kk / 32];
    }
  }

  // --- activation range: batched loads, then LDS -------------------------
  // 16-byte chunk c of the range is row c / (4 SMAX), step (c / 4) % SMAX,
  // block c % 4; a thread's chunks c = tid + 64 NW u all share one (step,
  // block), so its K offset is computed once.
  constexpr int RPU = 64 * NW / (SMAX * 4);  // rows between a thread's consecutive chunks
  static_assert((64 * NW) % (SMAX * 4) == 0, "a thread's chunks must share their step");
  const int row0 = (int)threadIdx.x / (SMAX * 4), tq = (int)threadIdx.x % (SMAX * 4);
  const int ta = tq >> 2, blk = tq & 3;
  const int sta = s0 + (ta < ns ? ta : ns - 1);
  const bool ba = sta >= p.seg[0].steps;
  const int64_t Ka = ba ? p.seg[1].K : p.seg[0].K;
  int64_t kka = (int64_t)(ba ? sta - p.seg[0].steps : sta) * 128 + 32 * blk;
  const bool okk = ta < ns && kka < Ka;
  kka = kka < Ka ? kka : Ka - 32;
  const int64_t ka = (ba ? p.seg[1].a_k0 : p.seg[0].a_k0) + kka;
  const uint8_t* acol = p.a_codes + ka / 2;
  const uint8_t* ascol = p.a_scales + ka / 32;
  v4i av[PER];
  uint32_t asv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    int64_t m = m0 + row0 + RPU * u;
    m = m < p.M ? m : p.M - 1;
    av[u] = load16(acol + m * p.lda);
    asv[u] = ascol[m * p.ldas];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int row = row0 + RPU * u;
    *reinterpret_cast<v4i*>(sa + row * LDA + tq * 16) = okk ? av[u] : v4i{0, 0, 0, 0};
    ss[row * SMAX * 4 + tq] = (uint8_t)(okk ? asv[u] : 127u);
  }
  __syncthreads();

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < SMAX; ++t) {
    if (t < ns) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = 16 * i + r16;
        const v4i af = *reinterpret_cast<const v4i*>(sa + row * LDA + t * 64 + g * 16);
        const int as = ss[row * SMAX * 4 + t * 4 + g];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(af), widen(bq[t][j]), acc[i][j], 4, 4,
                                                                        0, as, 0, bsc[t][j]);
      }
    }
  }
  if (n0 >= p.N) return;

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + 16 * j + r16;
      if (n >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + 16 * i + 4 * g + q;
        if (m >= p.M) continue;
        // one split: the output itself; several: this split's slab of the workspace
        float* dst = p.atomic ? p.part + (int64_t)blockIdx.y * p.M * p.N + m * p.N + n : p.y + m * p.ldy + n;
        *dst = acc[i][j][q];
      }
    }
}

// ---------------------------------------------------------------------------
// 32x32x64 path for 17..128 rows per tile with 128-aligned K segments
// ---------------------------------------------------------------------------
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (the full FP4 rate on gfx950; 16x16x128
// runs at the FP8 rate).  Operand lane l holds row l % 32 and one 32-element
// E8M0 block (16 bytes) of K; the fp32 result holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 in register r.  Within a 128-element K step, MFMA h
// (0, 1) gives lane half j block 2h + j, for the activation and the weight
// alike, with that block's own scale.
//
// A workgroup (4 waves) owns 64 output columns, all 32*TM rows of its M tile
// and a range of at most 2*HALF K steps: waves 0/1 take columns 0-31/32-63
// over the first half of the steps, waves 2/3 the same columns over the
// second half.  Each wave issues, step by step, its share of the step's
// activation blocks and scales and its own weight codes and scales, all to
// registers, so every byte of the range is in flight at once and arrives in
// step order.  Step t waits only for its own registers, writes its share of
// the step's activation to LDS (the two waves of a half share it), meets the
// other waves at a barrier and runs its MFMAs while later steps are still
// arriving.  (Direct-to-LDS loads would save the registers, but the compiler
// then waits for every one of them before the first LDS read.)  The two
// halves' sums meet in LDS in a fixed order.
//
// With the K range split over S workgroups, each writes its 64-column tile
// to its own slot of the workspace; the last of the tile's S workgroups to
// arrive (an atomic counter per tile) adds the S slots in split order -- a
// fixed order whatever the arrival order, so results are bitwise repeatable
// -- writes y and resets the counter.  No second kernel runs.
// 16-byte slot of logical block `blk` in LDS row `rr` (0..15) of a 1 KB
// activation block: rows are 64 bytes, so 8 (or 16) consecutive rows read by
// one ds_read_b128 pass land in distinct banks
__device__ __forceinline__ int a_slot(int rr, int blk) { return blk ^ (((rr >> 2) & 3) ^ (rr & 2)); }

template <int TM>
struct Mx32Cfg {
  static constexpr int ROWS = 32 * TM;
  static constexpr int RB = ROWS / 16;               // 1 KB activation blocks per step
  static constexpr int RBW = RB / 2;                 // of them loaded by each wave of a half
  static constexpr int SR = ROWS > 64 ? ROWS : 64;   // scale dwords per step slot (a 4-byte direct load fills 64)
  static constexpr int LPS = RBW + 1 + 3;            // loads per wave per step: activation, its scales, weight x 3
  static constexpr int HALF = 56 / LPS;              // K steps per wave at most (registers: (RBW + 2) x 4 + 2 a step)
  static constexpr int LDS = 2 * HALF * RB * 1024 + 2 * HALF * SR * 4;
};

template <int TM>
__global__ __launch_bounds__(256) void k_mx_gemm32(const MxGemmArgs p) {
  using C = Mx32Cfg<TM>;
  constexpr int ROWS = C::ROWS, RB = C::RB, RBW = C::RBW, SR = C::SR, LPS = C::LPS, HALF = C::HALF;
  static_assert(TM == 1 || TM == 2 || TM == 4, "tile");
  static_assert(2 * TM * 16 * 64 * 4 + ROWS * 64 * 4 <= 2 * HALF * RB * 1024, "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) uint8_t sa[2 * HALF * RB * 1024];  // [half][step][RB KB]
  __shared__ __attribute__((aligned(16))) uint32_t ssc[2 * HALF * SR];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave & 1, kh = wave >> 1;
  const int c = lane & 31, j = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.z * ROWS;
  const int64_t ntile0 = (int64_t)blockIdx.x * 64;
  const int64_t n0 = ntile0 + cg * 32;
  const int s0 = blockIdx.y * p.steps_per_split;
  const int ns = min(p.total_steps - s0, p.steps_per_split);  // 1 .. 2 HALF
  const int h0 = (ns + 1) >> 1;
  const int tb = kh ? h0 : 0;         // this wave's first step within the range
  const int cnt = kh ? ns - h0 : h0;  // and its step count (0 when ns = 1, kh = 1)
  const int last = tb + cnt - 1 > 0 ? tb + cnt - 1 : 0;
  const int steps0 = p.seg[0].steps;
  // first A column of range step t (segment 1 starts at its own A column)
  auto a_col = [&](int t) __attribute__((always_inline)) {
    const int s = s0 + t;
    return s >= steps0 ? p.seg[1].a_k0 + (int64_t)(s - steps0) * 128 : (int64_t)s * 128;
  };

  int64_t n = n0 + c;
  n = n < p.N ? n : p.N - 1;
  const bool two = p.seg[1].steps > 0;
  const uint8_t* wc0 = p.seg[0].w_codes + n * p.seg[0].ldw;
  const uint8_t* ws0 = p.seg[0].w_scales + n * p.seg[0].ldws;
  const uint8_t* wc1 = two ? p.seg[1].w_codes + n * p.seg[1].ldw : wc0;
  const uint8_t* ws1 = two ? p.seg[1].w_scales + n * p.seg[1].ldws : ws0;
  const int rr = lane >> 2;                                        // row of a 1 KB block this lane fills
  const int ablk = (lane & 3) ^ (((rr >> 2) & 3) ^ (rr & 2));      // inverse of a_slot for this lane's slot
  const int srow = ROWS > 64 ? cg * 64 : 0;                        // scale rows of this wave's direct load

  // --- issue: per step, this wave's activation blocks, scales and weights ---
  // (steps past the wave's count re-read its last step; nothing uses them).
  // Every load of the range is in flight before any is waited for, in step
  // order; each goes to registers, so step t waits only for its own loads.
  v4i av[HALF][RBW];
  uint32_t asv[HALF];
  v4i bq[HALF][2];
  uint32_t bs[HALF];
#pragma unroll
  for (int t = 0; t < HALF; ++t) {
    const int st = min(tb + t, last);
    const int64_t ac = a_col(st);
#pragma unroll
    for (int u = 0; u < RBW; ++u) {
      int64_t m = m0 + (cg + 2 * u) * 16 + rr;
      m = m < p.M ? m : p.M - 1;
      av[t][u] = load16(p.a_codes + m * p.lda + (ac + 32 * ablk) / 2);
    }
    {
      int64_t m = m0 + srow + lane;
      m = m < p.M ? m : p.M - 1;
      asv[t] = *reinterpret_cast<const uint32_t*>(p.a_scales + m * p.ldas + ac / 32);
    }
    const int s = s0 + st;
    const bool sb = s >= steps0;
    const int64_t kb = (int64_t)(sb ? s - steps0 : s) * 64;  // byte offset of the step in the code row
    const uint8_t* wc = (sb ? wc1 : wc0) + kb + 16 * j;
    bq[t][0] = load16(wc);       // block j
    bq[t][1] = load16(wc + 32);  // block 2 + j
    bs[t] = *reinterpret_cast<const uint32_t*>((sb ? ws1 : ws0) + kb / 16);  // the step's 4 scales
  }

  v16f acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v16f{};
#pragma unroll
  for (int t = 0; t < HALF; ++t) {
    // the step's activation blocks and scales -> this half's LDS slot (each
    // wave writes its share; the wait is for those registers only), then a
    // bare barrier: __syncthreads() would also wait for every later step's
    // loads still in flight
    const int slot = kh * HALF + t;
#pragma unroll
    for (int u = 0; u < RBW; ++u)
      *reinterpret_cast<v4i*>(sa + (slot * RB + cg + 2 * u) * 1024 + lane * 16) = av[t][u];
    ssc[slot * SR + srow + lane] = asv[t];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (t < cnt) {
      const int bsc0 = (int)((bs[t] >> (8 * j)) & 0xFFu), bsc1 = (int)((bs[t] >> (8 * (2 + j))) & 0xFFu);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int R = 32 * i + c, r16 = R & 15;
        const uint8_t* row = sa + (slot * RB + (R >> 4)) * 1024 + r16 * 64;
        const v4i a0 = *reinterpret_cast<const v4i*>(row + 16 * a_slot(r16, j));
        const v4i a1 = *reinterpret_cast<const v4i*>(row + 16 * a_slot(r16, 2 + j));
        const uint32_t asw = ssc[slot * SR + R];
        const int asc0 = (int)((asw >> (8 * j)) & 0xFFu), asc1 = (int)((asw >> (8 * (2 + j))) & 0xFFu);
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a0), widen(bq[t][0]), acc[i], 4, 4, 0, asc0,
                                                                  0, bsc0);
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a1), widen(bq[t][1]), acc[i], 4, 4, 0, asc1,
                                                                  0, bsc1);
      }
    }
  }

  // --- the halves' sums meet in LDS; the tile is staged row-major --------
  __syncthreads();  // every wave is done reading the activation range
  float* red = reinterpret_cast<float*>(sa);                 // [2 column groups][TM * 16][64 lanes]
  float* tile = red + 2 * TM * 16 * 64;                      // [ROWS][64] fp32
  if (kh) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((cg * TM + i) * 16 + v) * 64 + lane] = acc[i][v];
  }
  __syncthreads();
  if (!kh) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * i + 8 * (v >> 2) + 4 * j + (v & 3);
        tile[r * 64 + cg * 32 + c] = acc[i][v] + red[((cg * TM + i) * 16 + v) * 64 + lane];
      }
  }
  __syncthreads();

  // --- stores: 16-byte pieces, 16 per tile row ----------------------------
  constexpr int PIECES = ROWS * 16 / 256;  // per thread
  const bool vec = (p.N & 3) == 0 && (p.ldy & 3) == 0 && !(reinterpret_cast<uintptr_t>(p.y) & 15u);
  auto store_y = [&](int r, int q, v4f v) __attribute__((always_inline)) {
    const int64_t m = m0 + r, nn = ntile0 + 4 * q;
    if (m >= p.M || nn >= p.N) return;
    float* dst = p.y + m * p.ldy + nn;
    if (vec && nn + 4 <= p.N) {
      *reinterpret_cast<v4f*>(dst) = v;
    } else {
      for (int e = 0; e < 4 && nn + e < p.N; ++e) dst[e] = v[e];
    }
  };
  if (!p.atomic) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pc = (int)threadIdx.x + 256 * u, r = pc >> 4, q = pc & 15;
      store_y(r, q, *reinterpret_cast<const v4f*>(tile + r * 64 + 4 * q));
    }
    return;
  }
  const int64_t tile_id = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
  // this tile's S slots of ROWS x 64 fp32, one per split, contiguous
  constexpr uint32_t SLOT = ROWS * 64 * 4;  // bytes
  const __amdgpu_buffer_rsrc_t rs = shared_tile_rsrc(p.part + tile_id * p.splits * (ROWS * 64), SLOT * p.splits);
#pragma unroll
  for (int u = 0; u < PIECES; ++u) {
    const int pc = (int)threadIdx.x + 256 * u;
    store_shared_v4(rs, SLOT * blockIdx.y + 16 * pc, *reinterpret_cast<const v4f*>(tile + 4 * pc));
  }
  if (!arrive_last(p.counters + tile_id, p.splits, &s_last)) return;
  // the last arrival: every piece of up to SMX other splits' slots in flight
  // at once (one memory round trip; 48 registers of 16 bytes), then the sums
  // in split order
  constexpr int PB = PIECES;
  constexpr int SMX = 48 / PB;  // splits per pass of the load batch (more passes beyond)
#pragma unroll
  for (int u0 = 0; u0 < PIECES; u0 += PB) {
    v4f sum[PB];
#pragma unroll
    for (int b = 0; b < PB; ++b) sum[b] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < p.splits; sp0 += SMX) {
      v4f ld[SMX][PB];
#pragma unroll
      for (int q = 0; q < SMX; ++q)
#pragma unroll
        for (int b = 0; b < PB; ++b) {
          const int sp = sp0 + q, pc = (int)threadIdx.x + 256 * (u0 + b);
          ld[q][b] = sp < p.splits && sp != (int)blockIdx.y ? load_shared_v4(rs, SLOT * sp + 16 * pc)
                                                              : *reinterpret_cast<const v4f*>(tile + 4 * pc);
        }
#pragma unroll
      for (int q = 0; q < SMX; ++q)
#pragma unroll
        for (int b = 0; b < PB; ++b)
          if (sp0 + q < p.splits) sum[b] += ld[q][b];
    }
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      const int pc = (int)threadIdx.x + 256 * (u0 + b);
      store_y(pc >> 4, pc & 15, sum[b]);
    }
  }
}

// Split count: enough K splits that the grid fills the CUs, but never more
// workgroups than can be resident at once (a second partial round of
// workgroups would double the latency of this one-pass kernel).  A K range
// that one workgroup loads in a single batch (at most SMAX steps) is not
// split: there the partial slabs and the second kernel that sums them cost
// more than the extra workgroups gain.
template <int TM, int TN, int NW, int SMAX>
static int pick_splits(int64_t M, int64_t N, int total_steps) {
  if (total_steps <= SMAX) return 1;
  const int64_t tiles = cdiv(N, 16 * TN * NW) * cdiv(M, 16 * TM);
  constexpr int lds = 16 * TM * (SMAX * 64 + 16) + 16 * TM * SMAX * 4;
  const int per_cu = lds > 80 * 1024 ? 1 : 2;
  const int64_t slots = (int64_t)per_cu * device_cu_count();
  int splits = (int)cdiv(total_steps, SMAX);
  while ((int64_t)(splits + 1) * tiles <= slots && splits < total_steps) ++splits;
  const int steps = (int)cdiv(total_steps, splits);
  return (int)cdiv(total_steps, steps);
}

template <int TM, int TN, int NW, int SMAX>
static int launch_mx(MxGemmArgs& p, int splits, hipStream_t st) {
  const int64_t n_tiles = cdiv(p.N, 16 * TN * NW);
  const int64_t m_tiles = cdiv(p.M, 16 * TM);
  p.steps_per_split = (int)cdiv(p.total_steps, splits);
  splits = (int)cdiv(p.total_steps, p.steps_per_split);  // no empty split
  p.atomic = splits > 1;
  hipLaunchKernelGGL((k_mx_gemm<TM, TN, NW, SMAX>), dim3((unsigned)n_tiles, (unsigned)splits, (unsigned)m_tiles),
                     dim3(64 * NW), 0, st, p);
  int s = check_launch("mx_gemm");
  if (s || splits == 1) return s;
  return launch_splitk_reduce(p.part, splits, p.M * p.N, p.y, st);
}

// Serial-K variant for GBW_DETERMINISTIC: the K loop runs inside one wave, so
// every output is summed in one fixed order.
template <int TM, int NW>
__global__ __launch_bounds__(64 * NW) void k_mx_gemm_serial(const MxGemmArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.z * (16 * TM);
  const int64_t n0 = ((int64_t)blockIdx.x * NW + wave) * 16;
  if (n0 >= p.N) return;
  const uint8_t* arow[TM];
  const uint8_t* asrow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t r = m0 + 16 * i + r16;
    r = r < p.M ? r : p.M - 1;
    arow[i] = p.a_codes + r * p.lda;
    asrow[i] = p.a_scales + r * p.ldas;
  }
  int64_t n = n0 + r16;
  n = n < p.N ? n : p.N - 1;
  v4f acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.total_steps; ++s) {
    const StepSeg sg = step_seg(p, s);
    const int64_t kk = sg.k + 32 * g;
    const bool valid = kk < sg.K;
    const v4i bf = valid ? load16(sg.wc + n * sg.ldw + kk / 2) : v4i{0, 0, 0, 0};
    const int bs = valid ? (int)sg.ws[n * sg.ldws + kk / 32] : 127;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t ka = sg.a_k0 + kk;
      const v4i af = valid ? load16(arow[i] + ka / 2) : v4i{0, 0, 0, 0};
      const int as = valid ? (int)asrow[i][ka / 32] : 127;
      acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(af), widen(bf), acc[i], 4, 4, 0, as, 0, bs);
    }
  }
  const int64_t nn = n0 + r16;
  if (nn >= p.N) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + 16 * i + 4 * g + q;
      if (m < p.M) p.y[m * p.ldy + nn] = acc[i][q];
    }
}

template <int TM>
static int launch_serial(MxGemmArgs& p, hipStream_t st) {
  if (TM == 2) return launch_serial<4>(p, st);
  p.atomic = 0;
  hipLaunchKernelGGL((k_mx_gemm_serial<TM, 4>), dim3((unsigned)cdiv(p.N, 64), 1, (unsigned)cdiv(p.M, 16 * TM)),
                     dim3(256), 0, st, p);
  return check_launch("mx_gemm(serial)");
}

static int check_act(const gbw_act* a, int64_t M, const char* who) {
  if (!a) return fail(GBW_E_ARG, "%s: null activation", who);
  if (a->fmt != GBW_FMT_E8M0_B32) return fail(GBW_E_UNSUPPORTED, "%s: activation must be E8M0-B32", who);
  if (a->rows < M) return fail(GBW_E_SHAPE, "%s: activation has %lld rows < M", who, (long long)a->rows);
  if (a->K <= 0 || a->K % 32) return fail(GBW_E_SHAPE, "%s: activation K must be a positive multiple of 32", who);
  if (M > 0 && (!a->codes || !a->scales)) return fail(GBW_E_ARG, "%s: null activation pointer", who);
  if (M > 0 && !aligned16(a->codes)) return fail(GBW_E_ALIGN, "%s: activation codes not 16-byte aligned", who);
  return GBW_OK;
}

static int check_w(const gbw_weight* w, int64_t K, const char* who) {
  if (!w) return fail(GBW_E_ARG, "%s: null weight", who);
  if (w->fmt != GBW_FMT_E8M0_B32) return fail(GBW_E_UNSUPPORTED, "%s: weight must be E8M0-B32", who);
  if (w->n_experts != 1) return fail(GBW_E_ARG, "%s: dense GEMM takes one expert", who);
  if (w->N < 0 || w->K != K) return fail(GBW_E_SHAPE, "%s: weight K %lld != %lld", who, (long long)w->K, (long long)K);
  if (w->N > 0 && (!w->codes || !w->scales)) return fail(GBW_E_ARG, "%s: null weight pointer", who);
  if (w->N > 0 && !aligned16(w->codes)) return fail(GBW_E_ALIGN, "%s: weight codes not 16-byte aligned", who);
  return GBW_OK;
}

// K steps (of 128) per workgroup at most: 16 for long K (fewer split-K
// partials), 8 otherwise (a workgroup loads all SMAX steps' registers)
constexpr int mx_smax(int64_t steps) { return steps >= 48 ? 16 : 8; }

template <int TM, int SMAX>
static int dispatch_tm(MxGemmArgs& p, size_t ws_bytes, hipStream_t st) {
  int splits = pick_splits<TM, 1, 4, SMAX>(p.M, p.N, p.total_steps);
  const size_t slab = (size_t)p.M * p.N * sizeof(float);
  // the partial slabs follow the workspace's counter region (never touched here)
  if (p.part) {
    p.part = ws_bytes > kWsCounterBytes ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(p.part) + kWsCounterBytes)
                                        : nullptr;
    ws_bytes = ws_bytes > kWsCounterBytes ? ws_bytes - kWsCounterBytes : 0;
  }
  if (splits > 1 && (!p.part || ws_bytes < (size_t)splits * slab)) {
    // not enough workspace for the partials: the serial-K kernel needs none
    const int fit = p.part ? (int)(ws_bytes / slab) : 0;
    const int need = (int)cdiv(p.total_steps, SMAX);
    if (fit >= need && fit >= 2)
      splits = fit;
    else if (need == 1)
      splits = 1;
    else
      return launch_serial<TM>(p, st);
  }
  return launch_mx<TM, 1, 4, SMAX>(p, splits, st);
}

template <int SMAX>
static int ws_splits(int64_t M, int64_t N, int steps) {
  if (M <= 16) return pick_splits<1, 1, 4, SMAX>(M, N, steps);
  if (M <= 32) return pick_splits<2, 1, 4, SMAX>(M, N, steps);
  return pick_splits<4, 1, 4, SMAX>(M, N, steps);
}

// 32x32x64 path: splits of the K steps so that the (column, row) tiles fill
// the CUs once (one resident round), each range within 2 HALF steps
template <int TM>
static int pick_splits32(int64_t M, int64_t N, int total_steps) {
  using C = Mx32Cfg<TM>;
  const int64_t tiles = cdiv(N, 64) * cdiv(M, 32 * TM);
  const int per_cu = 1;  // one resident workgroup per CU (LDS and, for two row tiles, registers)
  const int64_t slots = (int64_t)per_cu * device_cu_count();
  int splits = (int)cdiv(total_steps, 2 * C::HALF);
  while ((int64_t)(splits + 1) * tiles <= slots && splits < total_steps) ++splits;
  const int steps = (int)cdiv(total_steps, splits);
  return (int)cdiv(total_steps, steps);
}

template <int TM>
static size_t ws_bytes32(int64_t M, int64_t N, int splits) {
  const int64_t tiles = cdiv(N, 64) * cdiv(M, 32 * TM);
  if (tiles > kWsMaxTiles) return 0;  // too many tiles for the counters: no split
  return splits > 1 ? kWsCounterBytes + (size_t)tiles * splits * (32 * TM) * 64 * sizeof(float) : 0;
}

static size_t ws32(int64_t M, int64_t N, int steps) {
  if (M <= 32) return ws_bytes32<1>(M, N, pick_splits32<1>(M, N, steps));
  if (M <= 64) return ws_bytes32<2>(M, N, pick_splits32<2>(M, N, steps));
  return ws_bytes32<4>(M, N, pick_splits32<4>(M, N, steps));
}

size_t ws_mx_gemm(int64_t M, int64_t N, int64_t Ktot) {
  if (M <= 0 || N <= 0 || Ktot <= 0) return 0;
  const int steps = (int)cdiv(Ktot, 128) + 1;  // + 1: the tail segment may start a step of its own
  // the largest workspace any kernel choice can ask for at these extents
  int splits = ws_splits<8>(M, N, steps);
  const int s16 = ws_splits<16>(M, N, steps);
  splits = splits > s16 ? splits : s16;
  size_t b = splits > 1 ? kWsCounterBytes + (size_t)splits * M * N * sizeof(float) : 0;
  if (M > 16) {
    for (int st = steps - 1; st <= steps; ++st) {
      const size_t b32 = ws32(M, N, st);
      b = b > b32 ? b : b32;
    }
  }
  return b;
}

template <int TM>
static int dispatch32(MxGemmArgs& p, size_t ws_bytes, hipStream_t st) {
  using C = Mx32Cfg<TM>;
  int splits = pick_splits32<TM>(p.M, p.N, p.total_steps);
  const size_t need = ws_bytes32<TM>(p.M, p.N, splits);
  if (splits > 1 && (!p.part || need == 0 || ws_bytes < need || (reinterpret_cast<uintptr_t>(p.part) & 15u))) {
    // not enough workspace for the split tiles: the serial-K kernel needs none
    if (cdiv(p.total_steps, 2 * C::HALF) == 1)
      splits = 1;
    else
      return launch_serial<4>(p, st);
  }
  const int64_t n_tiles = cdiv(p.N, 64), m_tiles = cdiv(p.M, 32 * TM);
  p.steps_per_split = (int)cdiv(p.total_steps, splits);
  splits = (int)cdiv(p.total_steps, p.steps_per_split);
  p.splits = splits;
  p.atomic = splits > 1;
  if (splits > 1) {
    uint8_t* ws = reinterpret_cast<uint8_t*>(p.part);
    p.counters = reinterpret_cast<uint32_t*>(ws);
    p.part = reinterpret_cast<float*>(ws + kWsCounterBytes);
  }
  hipLaunchKernelGGL((k_mx_gemm32<TM>), dim3((unsigned)n_tiles, (unsigned)splits, (unsigned)m_tiles), dim3(256), 0,
                     st, p);
  return check_launch("mx_gemm");
}

static bool aligned4(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; }

static int run_mx(int64_t M, const gbw_act* a, const gbw_weight* w, const gbw_weight* r, int64_t tail, float* y,
                  int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  (void)flags;  // every path sums in a fixed order: results are bitwise repeatable
  MxGemmArgs p{};
  p.M = M;
  p.N = w->N;
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.lda = a->K / 2;
  p.ldas = a->K / 32;
  p.seg[0] = MxSeg{w->codes, w->scales, w->K / 2, w->K / 32, 0, w->K, (int32_t)cdiv(w->K, 128)};
  if (r && tail > 0)
    p.seg[1] = MxSeg{r->codes, r->scales, tail / 2, tail / 32, a->K - tail, tail, (int32_t)cdiv(tail, 128)};
  else
    p.seg[1] = MxSeg{w->codes, w->scales, 0, 0, 0, 0, 0};
  p.total_steps = p.seg[0].steps + p.seg[1].steps;
  p.y = y;
  p.ldy = w->N;
  p.part = reinterpret_cast<float*>(ws);
  hipStream_t st = as_stream(stream);
  // 17+ rows with every K segment a whole number of 128-element steps (and
  // dword-aligned scale rows): the 32x32x64 kernel
  const bool k128 = a->K % 128 == 0 && w->K % 128 == 0 && (!r || tail % 128 == 0) && aligned4(a->scales) &&
                    aligned4(w->scales) && (!r || aligned4(r->scales));
  if (M > 16 && k128) {
    if (M <= 32) return dispatch32<1>(p, ws_bytes, st);
    if (M <= 64) return dispatch32<2>(p, ws_bytes, st);
    return dispatch32<4>(p, ws_bytes, st);
  }
  // rows per workgroup: up to 64 (more rows are more workgroups along M: a
  // 128-row tile leaves too few workgroups once K is split into 16-step ranges)
  if (mx_smax(p.total_steps) == 16) {
    if (M <= 16) return dispatch_tm<1, 16>(p, ws_bytes, st);
    if (M <= 32) return dispatch_tm<2, 16>(p, ws_bytes, st);
    return dispatch_tm<4, 16>(p, ws_bytes, st);
  }
  if (M <= 16) return dispatch_tm<1, 8>(p, ws_bytes, st);
  if (M <= 32) return dispatch_tm<2, 8>(p, ws_bytes, st);
  return dispatch_tm<4, 8>(p, ws_bytes, st);
}

}  // namespace gbw

using namespace gbw;

extern "C" int mx_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, float* y, int32_t flags, void* ws,
                       size_t ws_bytes, void* stream) {
  if (M < 0) return fail(GBW_E_ARG, "mx_gemm: negative M");
  int st;
  if ((st = check_act(a, M, "mx_gemm"))) return st;
  if ((st = check_w(w, a->K, "mx_gemm"))) return st;
  if (M == 0 || w->N == 0) return GBW_OK;
  if (!y) return fail(GBW_E_ARG, "mx_gemm: null output");
  if ((st = check_device())) return st;
  return run_mx(M, a, w, nullptr, 0, y, flags, ws, ws_bytes, stream);
}

extern "C" int residual_tail_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, const gbw_weight* r,
                                  int64_t tail, float* y, int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || tail < 0) return fail(GBW_E_ARG, "residual_tail_gemm: negative extent");
  int st;
  if ((st = check_act(a, M, "residual_tail_gemm"))) return st;
  if ((st = check_w(w, a->K, "residual_tail_gemm"))) return st;
  if (tail % 32 || tail > a->K) return fail(GBW_E_SHAPE, "residual_tail_gemm: tail must be a multiple of 32, <= K");
  if (tail > 0) {
    if ((st = check_w(r, tail, "residual_tail_gemm(residual)"))) return st;
    if (r->N != w->N) return fail(GBW_E_SHAPE, "residual_tail_gemm: residual has %lld rows, weight %lld",
                                  (long long)r->N, (long long)w->N);
  }
  if (M == 0 || w->N == 0) return GBW_OK;
  if (!y) return fail(GBW_E_ARG, "residual_tail_gemm: null output");
  if ((st = check_device())) return st;
  return run_mx(M, a, w, tail > 0 ? r : nullptr, tail, y, flags, ws, ws_bytes, stream);
}
