// Grouped expert GEMMs of the routed FFN on CDNA4 matrix cores.
//
//  GATEUP: for every pair p = (token t, expert e), g and u = deq(Xq[t]) W_e^T
//          over the fused [2I][H] gate/up weight (gate rows first), then
//          h = bf16(silu(g) * u) and (FP4 path) its MXFP4 (E8M0-B32)
//          requantization -- all in the epilogue, so h never exists in a
//          wider format in HBM.
//  DOWN:   o_p = deq(Hq[p]) W_e^T for every pair, written once to row p of a
//          pair-major slot buffer; a combine kernel forms
//          y[t] = sum_j topk_w[t][j] * o_{pair_pos[t][j]} in slot order.
//
// FFN form: "PRQuant: Permutation Residual Quantization for Low-Overhead
// Inference", §4 Eq. (1) (the gated MLP, applied to each routed expert;
// CodeQuant Fig. 1-2 show the experts of an MoE FFN).  Weight formats:
//  * MXFP4 (E8M0-B32): codes and scales stream straight into LDS;
//  * VQ -> MX ("MXCode: MX-Native Codebook Quantization", abstract, PreScale;
//    Fig. 2/3 and Table 4: d = 4, 256 entries, QBlocks of 64, 128 or 256):
//    each 8-bit index is expanded through its QBlock's 256-entry table of four
//    E2M1 codes (the table lives in LDS, 512 bytes) into an MXFP4 operand tile
//    in LDS; the E8M0 prescales are the operand's block scales.  PostScale
//    keeps one scale per QBlock table, PreScale+ an 8-bit index per 8 scales
//    along K into a 256 x 8 table per expert (held in LDS, 2 KiB): both are
//    turned into the same per-stage scale dwords when a stage is stored.  No
//    wider copy of the weights exists anywhere, in HBM or on chip;
//  * E4M3-B16 + FP32 tensor scale: exact decode to fp16 tiles, fp16 MFMA.
//
// Work decomposition: one workgroup per output tile of one expert (256 pairs
// x 256 weight rows).  The tile list is
// expert-major (m tiles, then n tiles) and is recovered by every workgroup
// from expert_offsets with a block scan; consecutive logical tiles are placed
// on the same XCD so the experts an XCD works on stay in its L2.  K advances
// one stage at a time, double-buffered in LDS; the next stage's global loads
// are in flight while the current stage's MFMAs run.  LDS operand rows carry
// 16 bytes of padding so the 16 lanes reading one MFMA fragment hit distinct
// banks.
//
// For GATEUP the weight rows of a tile are gate rows and the up rows of the
// same intermediate columns, arranged so that each wave holds g and u of the
// same (row, column) in its own accumulators.
#include <type_traits>

#include "common.hpp"

namespace gbw {

// Measurement aid, compiled in only with -DGBW_TILE_TRACE (a separate
// library; the normal build has none of it): thread 0 of each FP4 MoE
// workgroup stamps the wall clock (100 MHz) at tile entry, after the tile
// lookup, after the prologue, after the K loop and after the epilogue, and
// records its CU id and tile (rows, expert, m tile, n tile).  Slots per
// workgroup: 0 entry, 1 lookup done, 2 K loop start, 3 K loop end, 4 tile
// end, 5 CU id, 6 rows | e << 16 | mt << 32 | nt << 40.
#ifdef GBW_TILE_TRACE
constexpr int kTraceBlocks = 16384;
__device__ unsigned long long g_tile_trace[kTraceBlocks * 8];
#define GBW_TRACE(slot, val)                                                    \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks) g_tile_trace[blockIdx.x * 8 + (slot)] = (val); \
  } while (0)
#else
#define GBW_TRACE(slot, val) \
  do {                       \
  } while (0)
#endif

constexpr int kMoeBM = 256;       // pairs (A rows) per tile
constexpr int kMoeThreads = 256;  // threads that run the tile-list scan (every kernel has at least this many)
constexpr int kRowB = 80;         // LDS bytes per FP4 operand row per stage (64 of data + 16 of padding)
constexpr int kMaxMoeExperts = 256;
constexpr int kXsMaxK = 8192;     // PostScale / PreScale+: longest K whose tile scale bytes are staged in LDS

// weight formats of the FP4 kernel: MXFP4, and VQ -> MX with the block
// scales stored per 32 along K (PreScale), per QBlock table (PostScale) or
// as table-coded 8-vectors (PreScale+)
enum WFmt { W_MX = 0, W_VQ = 1, W_VQ_POST = 2, W_VQ_PLUS = 3 };

struct MoeArgs {
  int32_t stage;
  int32_t topk, E;
  int64_t T, P;
  const int32_t* off;
  const int32_t* pair_token;
  const int32_t* pair_pos;
  const float* topk_w;
  const uint8_t* a_codes;  // [rows][K/2]
  const uint8_t* a_scales; // [rows][K/32]
  int64_t K;               // reduction length (H for GATEUP, I for DOWN)
  const uint8_t* w_codes;  // MX: [E][N][K/2]; VQ: idx [E][N][K/4]
  const uint8_t* w_scales; // [E][N][K/32]; PostScale [E][N/qb][K/qb]; PreScale+ [E][N][K/256]
  const uint16_t* w_cb;    // VQ: [E][N/qb][K/qb][256]
  const uint8_t* w_scb;    // PreScale+: [E][256][8] E8M0 codes
  int32_t qsh;             // VQ: log2 of the QBlock edge (6, 7 or 8)
  const float* a_ts;       // E4M3: activation tensor scale [1]
  const float* w_ts;       // E4M3: weight tensor scales [E][ts_per]
  int32_t ts_per;
  int64_t N;               // weight rows per expert (2I or H)
  int32_t n_tiles;         // output tiles along N
  int32_t total_tiles;
  uint16_t* h_bf16;        // GATEUP: [P][I] or null
  uint8_t* h_codes;        // GATEUP: [P][(I+h_tail)/2] or null
  uint8_t* h_scales;       // GATEUP: [P][(I+h_tail)/32] or null
  int32_t h_tail;          // GATEUP: columns I-h_tail..I-1 also stored at I..I+h_tail-1
  float* y;                // DOWN: [T][H]
  void* slots;             // DOWN: [P][H] bf16 or fp32 per-pair outputs (pair-major), or null (atomics into y)
  int32_t slots_f32;       // 1: fp32 slots, 0: bf16 slots
  int32_t scales16;        // 1: K % 512 == 0 and both scale arrays 16-byte aligned
};

struct TileInfo {
  int e, mt, nt;
  int row0, rows;  // first pair of the tile, valid rows
};

template <int N>
struct IntC {
  static constexpr int value = N;
};

// 32-row bands (0, 1 or 2) of wave row wm (rows 64*wm .. 64*wm+63) that hold
// pairs; the value is the same in every lane, and is made a scalar so that a
// branch on it is a scalar branch
__device__ __forceinline__ int band_count(int rows, int wm) {
  const int r = rows - 64 * wm;
  return __builtin_amdgcn_readfirstlane(r >= 64 ? 2 : (r > 32 ? 2 : (r > 0 ? 1 : 0)));
}

// Logical tile of this workgroup: XCD-aware remap, then (expert, n tile, m tile).
// Workgroup b runs on XCD b % 8; the tiles that exist (known only here, from
// expert_offsets) are split into 8 equal runs of consecutive logical tiles, one
// per XCD, so every XCD gets the same share and its experts stay in its L2.
__device__ __forceinline__ bool find_tile(const MoeArgs& p, TileInfo& ti, int* scan) {
  const int tid = threadIdx.x;
  const bool mine = tid < kMoeThreads;  // the first 256 threads own the scan
  int cnt = 0;
  if (tid < p.E) cnt = (p.off[tid + 1] - p.off[tid] + kMoeBM - 1) / kMoeBM;
  if (mine) scan[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < kMoeThreads; o <<= 1) {
    const int add = (mine && tid >= o) ? scan[tid - o] : 0;
    __syncthreads();
    if (mine) scan[tid] += add;
    __syncthreads();
  }
  // scan[e] = m tiles of experts 0..e (inclusive)
  const int mt_total = scan[kMoeThreads - 1];
  const int valid = mt_total * p.n_tiles;
  const int per = (valid + 7) / 8;
  const int k = blockIdx.x / 8;
  const int L = (blockIdx.x % 8) * per + k;
  if (k >= per || L >= valid) return false;
  const int lm = L / p.n_tiles;  // logical m tile
  __shared__ int s_e;
  if (tid < p.E) {
    const int lo = tid ? scan[tid - 1] : 0;
    if (lm >= lo && lm < scan[tid]) s_e = tid;
  }
  __syncthreads();
  ti.e = s_e;
  // within the expert, m tiles vary fastest: the workgroups that run at the
  // same time on an XCD share each weight tile, which then comes from L2
  const int first = ti.e ? scan[ti.e - 1] : 0;
  const int mts = scan[ti.e] - first;
  const int local = L - first * p.n_tiles;
  ti.mt = local % mts;
  ti.nt = local / mts;
  ti.row0 = p.off[ti.e] + ti.mt * kMoeBM;
  ti.rows = min(kMoeBM, p.off[ti.e + 1] - ti.row0);
  return true;
}

// One pair's output element on the atomic path (no slot buffer): weighted
// straight into y[token] with an fp32 atomic.
__device__ __forceinline__ void atomic_pair_out(const MoeArgs& p, int tok, float w, int64_t n, float v) {
  unsafeAtomicAdd(p.y + (int64_t)tok * p.N + n, w * v);
}

__device__ __forceinline__ v8i widen8(v4i x) {
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

// Weight row within the expert of row j (0 .. BN-1) of B tile nt.  GATEUP
// tiles hold BN/2 gate rows and the BN/2 up rows of the same intermediate
// columns (gate rows first in the fused [2I][H] weight).
template <int BN>
__device__ __forceinline__ int64_t b_row(const MoeArgs& p, int nt, int j) {
  if (p.stage == GBW_MOE_GATEUP_SWIGLU) {
    const int64_t I = p.N / 2;
    const int64_t i0 = (int64_t)nt * (BN / 2);
    return j < BN / 2 ? i0 + j : I + i0 + (j - BN / 2);
  }
  return (int64_t)nt * BN + j;
}

// DOWN epilogue shared by the expert kernels (waves of 64 x 128, 32x32
// accumulators): acc[i][j][r] is row 64*wm + 32*i + 8*(r/4) + 4*(lane/32) +
// r%4 of the tile and column 128*wn + 32*j + lane%32 of the BN-column tile;
// `scale` multiplies every output (the tensor scales of E4M3-B16, 1
// otherwise).  With a slot buffer (pair-major [P][H]: the output row of pair
// p is row p) each wave stages its block in LDS, 16 rows at a time (8 KiB at
// most, at stg + 8 KiB * its wave index; the operand buffers are free after
// the K loop's last barrier), then writes whole 16-byte pieces of rows.
template <int BN>
__device__ __forceinline__ void down_epilogue(const MoeArgs& p, const TileInfo& ti, const v16f (&acc)[2][4], int wm,
                                              int wn, int lane, float scale, uint8_t* stg, const int* s_tok,
                                              const float* s_w) {
  const int l32 = lane & 31, g2 = lane >> 5;
  const int64_t col0 = (int64_t)ti.nt * BN + 128 * wn;
  if (!p.slots) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g2 + (r & 3);
        if (m >= ti.rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) atomic_pair_out(p, s_tok[m], s_w[m], col0 + 32 * j + l32, scale * acc[i][j][r]);
      }
    return;
  }
  const int esz = p.slots_f32 ? 4 : 2;
  uint8_t* const st = stg + (wm * (BN / 128) + wn) * (16 * 128 * 4);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int r = 8 * h + rr;
        const int mr = 8 * ((r >> 2) & 1) + 4 * g2 + (r & 3);  // row within the 16-row half
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const int c = 32 * j + l32;
          const float v0 = scale * acc[i][j][r], v1 = scale * acc[i][j + 1][r];
          if (esz == 4) {
            reinterpret_cast<float*>(st)[mr * 128 + c] = v0;
            reinterpret_cast<float*>(st)[mr * 128 + c + 32] = v1;
          } else {
            const uint32_t hp = cvt_pk_bf16(v0, v1);
            reinterpret_cast<uint16_t*>(st)[mr * 128 + c] = (uint16_t)hp;
            reinterpret_cast<uint16_t*>(st)[mr * 128 + c + 32] = (uint16_t)(hp >> 16);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      const int pieces = 128 * esz / 16;  // 16-byte pieces per row
      for (int q = lane; q < 16 * pieces; q += 64) {
        const int mr = q / pieces, pc = q % pieces;
        const int m = 64 * wm + 32 * i + 16 * h + mr;
        if (m < ti.rows) {
          uint8_t* dst = reinterpret_cast<uint8_t*>(p.slots) + ((int64_t)(ti.row0 + m) * p.N + col0) * esz + pc * 16;
          // streaming store: a slot row is read once, by the combine, after
          // this launch; it should not displace weight tiles from L2
          __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(st + mr * 128 * esz + pc * 16),
                                      reinterpret_cast<v4i*>(dst));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// FP4 experts.  A workgroup of 2*BN threads = BN/32 waves computes a tile of
// 256 pairs x BN weight rows (BN = 256, launched for both stages: 8 waves as
// 4 x 2, one workgroup per CU; BN = 128, kept in the template but not
// instantiated: 4 waves as 4 x 1, two workgroups per CU, so one workgroup's
// prologue, barriers and epilogue overlap the other's MFMAs).  A wave owns a
// 64 x 128 block as 2 x 4 accumulators of v_mfma_scale_f32_32x32x64_f8f6f4 (on
// gfx950 the 32x32x64 shape runs at the full FP4 rate; 16x16x128 at the FP8
// rate).  Lane l of a 32x32x64 operand holds row l % 32 and the 32 K elements
// of block l / 32 (one E8M0 block, 16 bytes); the fp32 result holds column
// l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 in register r.
constexpr int fp4_threads(int BN) { return 2 * BN; }

// GATEUP h tile (256 rows x BN/2 intermediate columns of bf16, staged in LDS
// with rows of BN/2 + 8 elements, so rows 4 apart fall in different banks) ->
// h codes and E8M0 scales (and h in bf16 when asked for).  Thread t handles
// groups t, t + 2BN, ... of 8 consecutive elements: group g is row g / (BN/16),
// columns 8 * (g % (BN/16)) ..; the four groups of a 32-element block sit in
// one quad of lanes.  E8M0 rule as in the MX quantizer: scale code = biased
// exponent of the block amax - 2, floored at 0.
template <int BN>
__device__ __forceinline__ void h_tile_store(const MoeArgs& p, const TileInfo& ti, const uint16_t* sHb, int tid) {
  constexpr int HR = BN / 2 + 8, GPR = BN / 16, NT = fp4_threads(BN);
  const int64_t I = p.N / 2, W = I + p.h_tail;  // W: code columns per h row
#pragma unroll 2
  for (int k = 0; k < kMoeBM * GPR / NT; ++k) {
    const int g = tid + NT * k;
    const int m = g / GPR, q = g % GPR;
    const v4i w = *reinterpret_cast<const v4i*>(&sHb[m * HR + 8 * q]);
    const uint32_t am = quad_max_u32(bf16x8_absmax_bits(w));
    const uint32_t E = am >> 7;  // biased exponent field of the bf16 amax
    const uint32_t sc = E > 2 ? E - 2 : 0;
    const uint32_t codes = e2m1x8_from_bf16(w, e8m0_value(sc));
    if (m < ti.rows) {
      const int64_t row = ti.row0 + m;
      if (p.h_codes) {
        const int64_t c = (int64_t)ti.nt * (BN / 2) + 8 * q;  // first h column of these 8
        *reinterpret_cast<uint32_t*>(p.h_codes + row * (W / 2) + c / 2) = codes;
        if ((q & 3) == 0) p.h_scales[row * (W / 32) + c / 32] = (uint8_t)sc;
        if (c >= I - p.h_tail) {  // PRQuant online tail copy
          const int64_t c2 = c + p.h_tail;
          *reinterpret_cast<uint32_t*>(p.h_codes + row * (W / 2) + c2 / 2) = codes;
          if ((q & 3) == 0) p.h_scales[row * (W / 32) + c2 / 32] = (uint8_t)sc;
        }
      }
      if (p.h_bf16) *reinterpret_cast<v4i*>(p.h_bf16 + row * I + (int64_t)ti.nt * (BN / 2) + 8 * q) = w;
    }
  }
}

template <int WF, int BN>
__global__ __launch_bounds__(fp4_threads(BN), 2) void k_moe_fp4(const MoeArgs p) {
  constexpr int NT = fp4_threads(BN), WN = BN / 128;    // threads, wave columns
  constexpr int kABuf = kMoeBM * kRowB, kBBuf = BN * kRowB;  // bytes per stage buffer
  constexpr int NA = kMoeBM * 4 / NT;                   // 16-byte A chunks per thread per stage
  constexpr int NLUT = BN / 32;                         // QBlock tables per stage (2 per 64 weight rows)
  constexpr int SB = BN > 256 ? BN : 256;               // B scale slots (>= BN; the extra ones are never read)
  constexpr bool VQ = WF != W_MX;
  constexpr bool XS = WF == W_VQ_POST || WF == W_VQ_PLUS;  // B scales not stored per 32 along K
  __shared__ __attribute__((aligned(16))) uint8_t sOp[2 * kABuf + 2 * kBBuf];
  __shared__ uint32_t sAs[2][kMoeBM];
  __shared__ uint32_t sBs[2][SB];
  __shared__ __attribute__((aligned(16))) uint16_t sLut[2][VQ ? NLUT * 256 : 4];
  __shared__ uint32_t sScb[WF == W_VQ_PLUS ? 512 : 1];  // PreScale+: the expert's 256 x 8 scale table
  // PostScale / PreScale+: the tile's stored B-scale bytes, staged once per
  // tile -- PostScale: the K/qb codes of the QBlock row of each 64-row band
  // at band * nq; PreScale+: the K/256 indices of tile row j at j * nq
  constexpr int XSB = WF == W_VQ_PLUS ? BN * (kXsMaxK / 256) : WF == W_VQ_POST ? (BN / 64) * (kXsMaxK / 64) : 4;
  __shared__ __attribute__((aligned(4))) uint8_t sXs[XSB];
  __shared__ int scan[kMoeThreads];
  __shared__ int s_tok[kMoeBM];
  __shared__ float s_w[kMoeBM];
  uint8_t* const sA0 = sOp;              // A buffer b at sA0 + b * kABuf
  uint8_t* const sB0 = sOp + 2 * kABuf;  // B buffer b at sB0 + b * kBBuf

#ifdef GBW_TILE_TRACE
  const unsigned long long t_entry = wall_clock64();
#endif
  TileInfo ti;
  if (!find_tile(p, ti, scan)) return;
  GBW_TRACE(0, t_entry);
  GBW_TRACE(1, wall_clock64());
  GBW_TRACE(5, __smid());
  GBW_TRACE(6, (unsigned long long)ti.rows | ((unsigned long long)ti.e << 16) | ((unsigned long long)ti.mt << 32) |
                   ((unsigned long long)ti.nt << 40));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int64_t K = p.K;
  const int steps = (int)(K / 128);
  const bool gate = p.stage == GBW_MOE_GATEUP_SWIGLU;

  // per-row metadata: the token of each pair (the A row of the gate/up
  // gather) and, for the atomic down path only, its routing weight (the
  // down stage with a slot buffer needs neither)
  for (int r = tid; r < kMoeBM; r += NT) {
    int tok = 0;
    float wt = 0.f;
    if (r < ti.rows && (gate || !p.slots)) {
      const int pr = ti.row0 + r;
      tok = p.pair_token[pr];
      if (!gate && !p.slots)
        for (int j = 0; j < p.topk; ++j)
          if (p.pair_pos[(int64_t)tok * p.topk + j] == pr) wt = p.topk_w[(int64_t)tok * p.topk + j];
    }
    s_tok[r] = tok;
    s_w[r] = wt;
  }
  // bytes per staged PostScale band / PreScale+ row
  const int nq = WF == W_VQ_PLUS ? (int)(p.K / 256) : WF == W_VQ_POST ? (int)(p.K >> p.qsh) : 0;
  if (WF == W_VQ_PLUS) {
    const uint32_t* scb = reinterpret_cast<const uint32_t*>(p.w_scb) + (int64_t)ti.e * 512;
    for (int i = tid; i < 512; i += NT) sScb[i] = scb[i];
    // the tile's rows are two runs of BN/2 consecutive weight rows (gate and
    // up halves, or the two halves of a down tile): (BN/2) * nq contiguous,
    // 4-byte aligned bytes each; nq <= 32 makes at most 4 dwords per thread
    const int run_dw = (BN / 2) * nq / 4;
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + u * NT;
      if (i < 2 * run_dw) {
        const int run = i >= run_dw ? 1 : 0;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            p.w_scales + ((int64_t)ti.e * p.N + b_row<BN>(p, ti.nt, run * (BN / 2))) * nq);
        v[u] = src[i - run * run_dw];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + u * NT;
      if (i < 2 * run_dw) reinterpret_cast<uint32_t*>(sXs)[i] = v[u];
    }
  } else if (WF == W_VQ_POST) {
    // (BN/64) * nq <= NT bytes: one per thread
    if (tid < (BN / 64) * nq) {
      const int band = tid / nq;
      const int64_t qrow = b_row<BN>(p, ti.nt, band * 64) >> p.qsh;
      sXs[tid] = p.w_scales[((int64_t)ti.e * (p.N >> p.qsh) + qrow) * nq + (tid - band * nq)];
    }
  }
  __syncthreads();

  // --- fixed per-thread load assignments --------------------------------
  // A codes: rows ar + (NT/4)u, 16-byte chunk ac of the 64-byte stage row.
  // Scales: with 512 threads, thread t loads the dword of A row t (t < 256) or
  // of B row t - 256; with 256 threads, of A row t and of B row t % BN.
  const int ar = tid >> 2, ac = tid & 3;
  const int64_t wN = p.N;
  auto a_src = [&](int r) __attribute__((always_inline)) {
    const int rr = r < ti.rows ? r : ti.rows - 1;
    return gate ? (int64_t)s_tok[rr] : (int64_t)(ti.row0 + rr);
  };
  const uint8_t* arow[NA];
#pragma unroll
  for (int u = 0; u < NA; ++u) arow[u] = p.a_codes + a_src(ar + (NT / 4) * u) * (K / 2);
  // PostScale / PreScale+ (XS) B scales come from LDS (sXs), not from a
  // per-32 stream: the B-scale waves of the 512-thread kernel then load the
  // scale row of A row t - 256 instead (unused, keeps one load sequence)
  const uint8_t* scl0;  // A scales (or, with 512 threads, B scales for t >= 256)
  const uint8_t* scl1;  // B scales (256 threads only)
  if (NT == 512) {
    scl0 = tid < 256 || XS ? p.a_scales + a_src(tid & 255) * (K / 32)
                           : p.w_scales + ((int64_t)ti.e * wN + b_row<BN>(p, ti.nt, tid - 256)) * (K / 32);
    scl1 = scl0;
  } else {
    scl0 = p.a_scales + a_src(tid) * (K / 32);
    scl1 = p.w_scales + ((int64_t)ti.e * wN + b_row<BN>(p, ti.nt, tid % BN)) * (K / 32);
  }
  // XS: whether this thread makes B scales (all threads with 256, t >= 256
  // with 512 -- whole waves either way), and for which tile row
  const bool xs_thr = XS && (NT != 512 || wave >= 4);
  const int xs_row = NT == 512 ? (tid & 255) : tid % BN;
  // the four E8M0 block scales of stage s of that row, as one dword
  auto xs_scales = [&](int s) __attribute__((always_inline)) {
    if (WF == W_VQ_PLUS) {
      const uint32_t si = sXs[xs_row * nq + (s >> 1)];  // 8 scales = 2 stages per index
      return sScb[(si << 1) | (uint32_t)(s & 1)];
    }
    // PostScale: the codes of the QBlocks holding the stage's two 64-wide
    // halves (the same one for QBlocks of 128 or 256)
    const uint8_t* const q = sXs + (xs_row >> 6) * nq;
    const uint32_t c0 = q[(s * 128) >> p.qsh], c1 = q[(s * 128 + 64) >> p.qsh];
    return c0 * 0x0101u | c1 * 0x01010000u;
  };
  uint32_t* const sdst0 = (NT == 512 && tid >= 256) ? &sBs[0][tid - 256] : &sAs[0][tid];  // buffer 1: + SB or 256
  const uint8_t* wrow[2];
  const uint8_t* vrow = nullptr;
  const uint16_t* cbase = nullptr;
  int lut_kb = 0;
  if (WF == W_MX) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      wrow[u] = p.w_codes + ((int64_t)ti.e * wN + b_row<BN>(p, ti.nt, ar + (NT / 4) * u)) * (K / 2);
  } else {
    // idx: wave w expands the 64 rows of band w >> 1 in stage half w & 1
    // (16-byte chunk w & 1 of each 32-byte stage row), so all of a wave's
    // lookups go to the one table of its slot (a 512-byte table spreads
    // over the 64 LDS banks with at most two of its dwords in a bank; two
    // tables per wave made lookups conflict twice as often: 2 % faster)
    vrow = p.w_codes + ((int64_t)ti.e * wN + b_row<BN>(p, ti.nt, 64 * (wave >> 1) + lane)) * (K / 4);
    // LUT: 8 bytes of table slot tid >> 6 (BN/64 row bands of 64 x 2 halves
    // of the stage); a slot holds the table of the QBlock its 64 x 64 weight
    // block lies in (with QBlocks of 128 or 256 several slots hold one table)
    const int tb = wave;  // (a scalar: the table offsets below are scalar arithmetic)
    lut_kb = tb & 1;
    const int64_t qrow = b_row<BN>(p, ti.nt, (tb >> 1) * 64) >> p.qsh;
    cbase = p.w_cb + ((int64_t)ti.e * (wN >> p.qsh) + qrow) * (K >> p.qsh) * 256 + (tid & 63) * 4;
  }
  // element offset of the table of slot half `kb` of stage s within the
  // slot's QBlock row (K <= 2^30, so 32 bits hold it)
  auto lut_off = [&](int s, int kb) __attribute__((always_inline)) {
    return (uint32_t)(((s * 128 + kb * 64) >> p.qsh) << 8);
  };

  // Software pipeline, one barrier per 128-element stage.  Iteration s:
  //   1. store stage s+1 (loaded into registers during iteration s-1) into
  //      LDS buffer (s+1)&1 and, for VQ, expand its indices there through the
  //      QBlock tables of stage s+1 (stored one iteration earlier);
  //   2. issue the global loads of stage s+2 (and the tables of stage s+3);
  //   3. the MFMAs of stage s from buffer s&1;
  //   4. barrier.
  // The last two iterations are peeled (no loads of stage s+2 in the second
  // to last, only the MFMAs in the last); the tables, which run one stage
  // further ahead, clamp their stage index to the last stage instead.
  v4i pa[NA], pb[2];
  uint32_t ps0 = 0, ps1 = 0;
  // with p.scales16 (256-wide tiles only: the 128-wide kernel has no
  // registers to spare): the scale dwords of a group of four stages.  The
  // next group's load goes to fixed registers (s4n*) and is copied to the
  // current ones (s4c*) when its first stage is stored, one iteration later:
  // choosing the destination at load time would need the loaded value at
  // once and stall on every load still in flight.
  constexpr bool S16 = BN == 256;
  v4i s4ca = v4i{0, 0, 0, 0}, s4cb = s4ca, s4na = s4ca, s4nb = s4ca;
  uint2 pl;
  uint32_t pq = 0;  // XS: the B-scale dword of the stage gload last prepared
  const int last = steps - 1;
  auto gload = [&](int s) __attribute__((always_inline)) {
    s = s < last ? s : last;
    const int64_t kb = (int64_t)s * 64;
#pragma unroll
    for (int u = 0; u < NA; ++u) pa[u] = load16(arow[u] + kb + 16 * ac);
    if (S16 && p.scales16) {
      // one 16-byte load per row covers the scale dwords of stages s .. s+3
      if ((s & 3) == 0) {
        s4na = load16(scl0 + (int64_t)s * 4);
        if (NT != 512) s4nb = load16(scl1 + (int64_t)s * 4);
      }
    } else {
      ps0 = *reinterpret_cast<const uint32_t*>(scl0 + (int64_t)s * 4);
      if (NT != 512 && !XS) ps1 = *reinterpret_cast<const uint32_t*>(scl1 + (int64_t)s * 4);
    }
    if (XS && xs_thr) pq = xs_scales(s);
    if (WF == W_MX) {
#pragma unroll
      for (int u = 0; u < 2; ++u) pb[u] = load16(wrow[u] + kb + 16 * ac);
    } else {
      pb[0] = load16(vrow + (int64_t)s * 32 + 16 * (wave & 1));
      const int sl = s + 1 < last ? s + 1 : last;  // tables run one stage ahead
      pl = *reinterpret_cast<const uint2*>(cbase + lut_off(sl, lut_kb));
    }
  };
  // stage k's registers -> LDS buffer k&1 (tables of stage k+1 -> table buffer (k+1)&1)
  auto lstore = [&](int k) __attribute__((always_inline)) {
    const int buf = k & 1;
    uint8_t* const a = sA0 + buf * kABuf;
    if (S16 && p.scales16) {
      const int kk = k < last ? k : last;
      if ((kk & 3) == 0) {
        s4ca = s4na;
        s4cb = NT != 512 ? s4nb : s4na;
      }
      const v4i a4 = s4ca, b4 = s4cb;
      const int e = kk & 3;
      ps0 = (uint32_t)(e == 0 ? a4[0] : e == 1 ? a4[1] : e == 2 ? a4[2] : a4[3]);
      ps1 = (uint32_t)(e == 0 ? b4[0] : e == 1 ? b4[1] : e == 2 ? b4[2] : b4[3]);
    }
    if (XS) {
      if (NT == 512)
        ps0 = xs_thr ? pq : ps0;
      else
        ps1 = pq;
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) *reinterpret_cast<v4i*>(a + (ar + (NT / 4) * u) * kRowB + 16 * ac) = pa[u];
    if (NT == 512) {
      sdst0[buf * (tid >= 256 ? SB : kMoeBM)] = ps0;
    } else {
      sAs[buf][tid] = ps0;
      sBs[buf][tid] = ps1;
    }
    if (WF == W_MX) {
      uint8_t* const b = sB0 + buf * kBBuf;
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<v4i*>(b + (ar + (NT / 4) * u) * kRowB + 16 * ac) = pb[u];
    } else {
      *reinterpret_cast<uint2*>(&sLut[buf ^ 1][(tid >> 6) * 256 + (tid & 63) * 4]) = pl;
    }
  };
  // VQ: expand this thread's 16 indices of stage k into 32 bytes of E2M1 codes
  auto vq_expand = [&](int k) __attribute__((always_inline)) {
    const int buf = k & 1;
    const int row = 64 * (wave >> 1) + lane, half = wave & 1;  // half = 64-element half of the stage
    const uint16_t* lut = &sLut[buf][wave * 256];
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w = (uint32_t)pb[0][d];
      o[2 * d] = (uint32_t)lut[w & 0xFF] | ((uint32_t)lut[(w >> 8) & 0xFF] << 16);
      o[2 * d + 1] = (uint32_t)lut[(w >> 16) & 0xFF] | ((uint32_t)lut[w >> 24] << 16);
    }
    uint8_t* dst = sB0 + buf * kBBuf + row * kRowB + 32 * half;
    *reinterpret_cast<v4i*>(dst) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    *reinterpret_cast<v4i*>(dst + 16) = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  // B-tile rows of this wave's four 32-row subtiles (GATEUP: j = 0, 1 gate,
  // j = 2, 3 the up rows of the same intermediate columns 64*wn + 32*(j%2) ..)
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = gate ? (j < 2 ? 64 * wn + 32 * j : BN / 2 + 64 * wn + 32 * (j - 2)) : 128 * wn + 32 * j;

  // number of this wave's 32-row bands that hold pairs (the last tile of an
  // expert is usually partly empty); the K loop is instantiated per count, so
  // the MFMA sequence carries no branch and the empty bands cost nothing
  const int nband = band_count(ti.rows, wm);

  // prologue: stage 0 (and the tables of stages 0 and 1) in LDS, stage 1 in registers
  if (VQ) {
    const uint2 t0 = *reinterpret_cast<const uint2*>(cbase + lut_off(0, lut_kb));
    *reinterpret_cast<uint2*>(&sLut[0][(tid >> 6) * 256 + (tid & 63) * 4]) = t0;
  }
  gload(0);
  lstore(0);
  __syncthreads();
  if (VQ) vq_expand(0);
  gload(1);
  __syncthreads();

  // MFMAs of one stage from LDS buffer buf: all fragments of a 64-element
  // step are read first, then the NB x 4 MFMAs
  auto mma = [&](int buf, auto nb) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
    const uint8_t* const a = sA0 + buf * kABuf;
    const uint8_t* const b = sB0 + buf * kBBuf;
#pragma unroll
    for (int t = 0; t < 2; ++t) {  // two 64-element MFMA steps per 128-element stage
      v4i bf[4], af[2];
      int bsc[4], asc[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = brow[j] + l32;
        bf[j] = *reinterpret_cast<const v4i*>(b + row * kRowB + 32 * t + 16 * g2);
        bsc[j] = (int)((sBs[buf][row] >> (8 * (2 * t + g2))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int row = 64 * wm + 32 * i + l32;
        af[i] = *reinterpret_cast<const v4i*>(a + row * kRowB + 32 * t + 16 * g2);
        asc[i] = (int)((sAs[buf][row] >> (8 * (2 * t + g2))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen8(af[i]), widen8(bf[j]), acc[i][j], 4, 4,
                                                                       0, asc[i], 0, bsc[j]);
    }
  };
  // the last two stages are peeled: no loads past the last stage, no store
  // or expansion of a stage that does not exist
  auto kloop = [&](auto nb) __attribute__((always_inline)) {
    int s = 0;
    for (; s < steps - 2; ++s) {
      lstore(s + 1);
      if (VQ) vq_expand(s + 1);
      gload(s + 2);
      mma(s & 1, nb);
      __syncthreads();
    }
    if (s == steps - 2) {
      lstore(s + 1);
      if (VQ) vq_expand(s + 1);
      mma(s & 1, nb);
      __syncthreads();
      ++s;
    }
    mma(s & 1, nb);
    __syncthreads();
  };
  GBW_TRACE(2, wall_clock64());
  if (nband == 2)
    kloop(IntC<2>{});
  else if (nband == 1)
    kloop(IntC<1>{});
  else
    kloop(IntC<0>{});
  GBW_TRACE(3, wall_clock64());

  // ---------------------------------------------------------------------
  // epilogues; acc[i][j][r] is row 64*wm + 32*i + 8*(r/4) + 4*g2 + r%4 of
  // the tile and row brow[j] + l32 of the B tile.  The last barrier of the
  // K loop has freed the operand buffers.
  // ---------------------------------------------------------------------
  if (!gate) {
    static_assert(fp4_threads(BN) / 64 * 8192 <= 2 * kABuf + 2 * kBBuf, "down staging fits the operand buffers");
    down_epilogue<BN>(p, ti, acc, wm, wn, lane, 1.0f, sA0, s_tok, s_w);
#ifdef GBW_TILE_TRACE
    __syncthreads();
    GBW_TRACE(4, wall_clock64());
#endif
    return;
  }

  // GATEUP, in two passes over an LDS copy of the h tile:
  //  1. h = bf16(silu(g) * u) for intermediate column 64*wn + 32*jj + l32 of
  //     the tile (g in acc[.][jj], u in acc[.][jj+2]) -> LDS, row-major;
  //  2. h_tile_store: every thread takes 8 consecutive h of a row, the four
  //     threads of one 32-column E8M0 block (a quad) share their amax over
  //     DPP, then encode and store whole dwords of codes.
  constexpr int HR = BN / 2 + 8;
  static_assert(kMoeBM * HR * 2 <= (int)sizeof(sOp), "h tile fits the operand buffers");
  uint16_t* const sHb = reinterpret_cast<uint16_t*>(sA0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g2 + (r & 3);
      const uint32_t hp = cvt_pk_bf16(silu_mul(acc[i][0][r], acc[i][2][r]), silu_mul(acc[i][1][r], acc[i][3][r]));
      sHb[m * HR + 64 * wn + l32] = (uint16_t)hp;
      sHb[m * HR + 64 * wn + 32 + l32] = (uint16_t)(hp >> 16);
    }
  __syncthreads();
  h_tile_store<BN>(p, ti, sHb, tid);
#ifdef GBW_TILE_TRACE
  __syncthreads();
  GBW_TRACE(4, wall_clock64());
#endif
}

template <int WF>
int launch_moe_fp4(const MoeArgs& p, hipStream_t st) {
  constexpr int bn = 256;  // (128-row tiles, two workgroups per CU, were 4 % slower for the down stage)
  MoeArgs q = p;
  q.n_tiles = (int)(p.N / bn);
  int64_t grid = (cdiv(p.P, kMoeBM) + p.E) * q.n_tiles;
  grid = cdiv(grid, 8) * 8;
  if (grid > INT32_MAX) return fail(GBW_E_SHAPE, "moe_grouped_gemm: problem too large");
  q.total_tiles = (int)grid;
  hipLaunchKernelGGL((k_moe_fp4<WF, bn>), dim3((unsigned)grid), dim3(fp4_threads(bn)), 0, st, q);
  return check_launch("moe_grouped_gemm");
}

// ---------------------------------------------------------------------------
// E4M3-B16 experts: exact decode to fp16, fp16 MFMA
// ---------------------------------------------------------------------------
// An E4M3-B16 element is e2m1 * s with s an E4M3 block scale: at most 6
// significant bits and a magnitude in [2^-10, 2688], so it is exact in fp16
// (and in bf16); both operands are decoded once per tile into fp16 LDS tiles
// and contracted with v_mfma_f32_32x32x16_f16.  The two FP32 tensor scales
// are applied to the fp32 accumulators in the epilogue.  (There is no exact
// route through the FP4/FP8 scaled MFMA: its block scales are powers of two
// per 32 elements, an E4M3 scale carries a 3-bit mantissa per 16.)
//
// Decode: one dword of codes (8 elements, element 2i in the low nibble of
// byte i) -> four fp16x2 words in element order: v_cvt_scalef32_pk_f16_fp4
// with scale 1 gives the two E2M1 values of a byte exactly (the instruction
// applies only the exponent of its fp32 scale, so the E4M3 block scale cannot
// go there), then one packed fp16 multiply by the block scale (exact).
constexpr int kRowH = 144;  // LDS bytes per fp16 row per stage (64 elements + 16 pad)
constexpr int kE4Threads = 512, kE4BN = 256;
constexpr int kHRow8 = 136;  // bf16 per staged h row (128 + 8): rows 4 apart fall in different banks

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void e4m3_decode8(uint32_t w, uint32_t sc2, uint32_t (&o)[4]) {
  const v2h sv = __builtin_bit_cast(v2h, sc2);
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv);
}

// E5M3-B16: the four code bytes of a dword -> four bf16x2 words in element
// order.  v_cvt_scalef32_pk_f32_fp4 at scale 1 gives the two E2M1 values of a
// byte exactly; times the UE5M3 block scale in fp32 (exact: at most 6
// significant bits) and one v_cvt_pk_bf16_f32 (exact for the same reason).
// fp16 cannot hold these products (they reach 6 * 114688).
__device__ __forceinline__ void e5m3_decode8(uint32_t w, float sd, uint32_t (&o)[4]) {
  const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const v2f c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const v2f d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  o[0] = cvt_pk_bf16(a[0] * sd, a[1] * sd);
  o[1] = cvt_pk_bf16(b[0] * sd, b[1] * sd);
  o[2] = cvt_pk_bf16(c[0] * sd, c[1] * sd);
  o[3] = cvt_pk_bf16(d[0] * sd, d[1] * sd);
}

// E4M3 scale code -> fp16 bits duplicated into both halves (exact: an E4M3
// value has 4 significant bits and lies in [2^-9, 448])
__device__ __forceinline__ uint32_t e4m3_to_h2(uint32_t c) {
  const _Float16 h = (_Float16)e4m3_value(c & 0xFFu);
  const uint32_t b = __builtin_bit_cast(uint16_t, h);
  return b | (b << 16);
}

// 512 threads = 8 waves (4 x 2) of 64 x 128 over a 256 x 256 tile,
// v_mfma_f32_32x32x16_f16 (lane l: row l % 32, K elements [8*(l/32),
// 8*(l/32)+8) of the 16-element step; on gfx950 the 32x32 shape runs at about
// twice the 16x16 rate).  Stage = 64 K elements: threads 0..255 decode row tid
// of A, 256..511 row tid-256 of B, into fp16 LDS rows of 128 bytes + 16 of
// padding.  Same single-barrier pipeline as the FP4 kernel: stage s+1 is
// decoded into LDS before the MFMAs of stage s.  E5 = true: E5M3-B16 operands,
// decoded to bf16 and contracted with v_mfma_f32_32x32x16_bf16 (same layout).
//
// WL: the weight codes.  W16_NIB: packed E2M1 nibbles with a scale per 16.
// VQ ("MXCode: MX-Native Codebook Quantization", abstract; Table 2's E4M3-B16
// columns): 8-bit indices into the QBlock's 256-entry table of four E2M1
// codes, with the block scales per 16 along K (W16_VQ, PreScale), one per
// QBlock table (W16_VQ_POST, PostScale) or 8 at a time coded against a
// 256 x 8 table per expert (W16_VQ_PLUS, PreScale+).  A B-row thread expands
// its 16 indices of a stage through the tables of its 64-row band (in LDS,
// loaded one stage ahead) into the 32 code bytes the decode takes.  Every
// thread issues the same loads each stage (A threads' table load and B
// threads' second code load are spare), so the waits stay those of the
// plain kernel.
enum W16 { W16_NIB = 0, W16_VQ = 1, W16_VQ_POST = 2, W16_VQ_PLUS = 3 };

template <bool E5, int WL>
__global__ __launch_bounds__(kE4Threads) void k_moe_e4m3(const MoeArgs p) {
  constexpr bool VQ = WL != W16_NIB;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kMoeBM * kRowH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kE4BN * kRowH];
  __shared__ __attribute__((aligned(16))) uint16_t sLut[2][VQ ? 4 * 256 : 4];  // 4 bands of 64 B rows
  __shared__ uint32_t sScb[WL == W16_VQ_PLUS ? 512 : 1];                      // PreScale+: 256 x 8 scale codes
  __shared__ int scan[kMoeThreads];
  __shared__ int s_tok[kMoeBM];
  __shared__ float s_w[kMoeBM];

  TileInfo ti;
  if (!find_tile(p, ti, scan)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int64_t K = p.K;
  const int steps = (int)(K / 64);

  // per-row metadata: the token of each pair and, for the atomic down path
  // only, its routing weight
  for (int r = tid; r < kMoeBM; r += kE4Threads) {
    int tok = 0;
    float wt = 0.f;
    if (r < ti.rows) {
      const int pr = ti.row0 + r;
      tok = p.pair_token[pr];
      if (p.stage == GBW_MOE_DOWN_COMBINE && !p.slots)
        for (int j = 0; j < p.topk; ++j)
          if (p.pair_pos[(int64_t)tok * p.topk + j] == pr) wt = p.topk_w[(int64_t)tok * p.topk + j];
    }
    s_tok[r] = tok;
    s_w[r] = wt;
  }
  if (WL == W16_VQ_PLUS) {
    const uint32_t* scb = reinterpret_cast<const uint32_t*>(p.w_scb) + (int64_t)ti.e * 512;
    for (int i = tid; i < 512; i += kE4Threads) sScb[i] = scb[i];
  }
  __syncthreads();

  // thread tid stages one row: A row tid (tid < 256) or B row tid - 256
  const int row = tid & 255;
  const bool is_b = VQ && __builtin_amdgcn_readfirstlane(tid >> 6) >= 4;  // (whole waves)
  const uint8_t* rc;
  const uint8_t* rs;
  const uint16_t* cbase = nullptr;  // VQ: this thread's 8 bytes of its band's table, stage 0
  if (tid < 256) {
    const int rr = row < ti.rows ? row : ti.rows - 1;
    const int64_t src = p.stage == GBW_MOE_GATEUP_SWIGLU ? (int64_t)s_tok[rr] : (int64_t)(ti.row0 + rr);
    rc = p.a_codes + src * (K / 2);
    rs = p.a_scales + src * (K / 16);
  } else {
    const int64_t n = b_row<kE4BN>(p, ti.nt, row);
    const int64_t wr = (int64_t)ti.e * p.N + n;
    rc = p.w_codes + wr * (VQ ? K / 4 : K / 2);
    if (WL == W16_VQ_POST)
      rs = p.w_scales + ((int64_t)ti.e * (p.N >> p.qsh) + (n >> p.qsh)) * (K >> p.qsh);
    else if (WL == W16_VQ_PLUS)
      rs = p.w_scales + wr * (K / 128);
    else
      rs = p.w_scales + wr * (K / 16);
  }
  if (VQ) {
    // table loads: B thread t - 256 fetches 8 bytes of band (t - 256) / 64;
    // A threads fetch the same bytes (spare loads of valid memory)
    const int band = (row >> 6), bl = row & 63;
    const int64_t qrow = b_row<kE4BN>(p, ti.nt, band * 64) >> p.qsh;
    cbase = p.w_cb + ((int64_t)ti.e * (p.N >> p.qsh) + qrow) * (K >> p.qsh) * 256 + bl * 4;
  }
  // LDS row of this thread in buffer 0; buffer 1 is kMoeBM * kRowH bytes further
  uint8_t* const dst0 = tid < 256 ? &sA[0][row * kRowH] : &sB[0][row * kRowH];
  // packed codes: A rows past the tile's pairs are neither loaded nor
  // decoded, their LDS rows feed only output rows that are never stored (3 %
  // of the E4M3-B16 gate/up time, spent in the last, partly filled tile of
  // each expert; with VQ weights the same branch costs 8-10 %, so those keep
  // every row)
  const bool a_live = VQ || tid >= 256 || row < ti.rows;

  v4i pc[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
  uint32_t ps;
  uint2 pl;
  const int last = steps - 1;
  // table element offset of stage s (64 K per stage) within the band's QBlock row
  auto lut_off = [&](int s) __attribute__((always_inline)) { return (uint32_t)(((s * 64) >> p.qsh) << 8); };
  auto gload = [&](int s) __attribute__((always_inline)) {
    s = s < last ? s : last;
    if (!VQ) {
      if (a_live) {
        pc[0] = load16(rc + (int64_t)s * 32);
        pc[1] = load16(rc + (int64_t)s * 32 + 16);
        ps = *reinterpret_cast<const uint32_t*>(rs + (int64_t)s * 4);
      }
    } else {
      // A rows: 32 code bytes and 4 scale codes.  B rows: 16 indices (the
      // second load repeats them) and the stage's scale codes (PostScale:
      // the QBlock's code; PreScale+: the index of the 8-scale vector
      // covering stages 2(s/2), 2(s/2)+1)
      const int64_t c0 = is_b ? (int64_t)s * 16 : (int64_t)s * 32;
      pc[0] = load16(rc + c0);
      pc[1] = load16(rc + c0 + (is_b ? 0 : 16));
      if (is_b && WL == W16_VQ_POST)
        ps = rs[(s * 64) >> p.qsh];
      else if (is_b && WL == W16_VQ_PLUS)
        ps = rs[s >> 1];
      else
        ps = *reinterpret_cast<const uint32_t*>(rs + (int64_t)s * 4);
      const int sl = s + 1 < last ? s + 1 : last;  // tables run one stage ahead
      pl = *reinterpret_cast<const uint2*>(cbase + lut_off(sl));
    }
  };
  auto lstore = [&](int k) __attribute__((always_inline)) {
    if (!a_live) return;
    uint8_t* dst = dst0 + (k & 1) * (kMoeBM * kRowH);
    uint32_t cw[8];  // the 32 code bytes of this row's stage
    uint32_t sc = ps;  // its four block-scale codes
#pragma unroll
    for (int d = 0; d < 8; ++d) cw[d] = (uint32_t)pc[d >> 2][d & 3];
    if (VQ && is_b) {
      // store the next stage's table; expand this stage's 16 indices
      const int kk = k < last ? k : last;
      *reinterpret_cast<uint2*>(&sLut[(k + 1) & 1][(row >> 6) * 256 + (row & 63) * 4]) = pl;
      const uint16_t* lut = &sLut[k & 1][(row >> 6) * 256];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = (uint32_t)pc[0][q];
        cw[2 * q] = (uint32_t)lut[w & 0xFF] | ((uint32_t)lut[(w >> 8) & 0xFF] << 16);
        cw[2 * q + 1] = (uint32_t)lut[(w >> 16) & 0xFF] | ((uint32_t)lut[w >> 24] << 16);
      }
      if (WL == W16_VQ_POST) sc = (ps & 0xFFu) * 0x01010101u;
      if (WL == W16_VQ_PLUS) sc = sScb[((ps & 0xFFu) << 1) | (uint32_t)(kk & 1)];
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      // dword d of the 32 code bytes holds elements 8d..8d+7, scale block d/2
      uint32_t o[4];
      if constexpr (E5)
        e5m3_decode8(cw[d], ue5m3_value((sc >> (8 * (d >> 1))) & 0xFFu), o);
      else
        e4m3_decode8(cw[d], e4m3_to_h2(sc >> (8 * (d >> 1))), o);
      *reinterpret_cast<v4i*>(dst + 16 * d) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    }
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = p.stage == GBW_MOE_GATEUP_SWIGLU ? (j < 2 ? 64 * wn + 32 * j : 128 + 64 * wn + 32 * (j - 2))
                                               : 128 * wn + 32 * j;
  const int nband = band_count(ti.rows, wm);

  if (VQ) {
    // the tables of stage 0
    const uint2 t0 = *reinterpret_cast<const uint2*>(cbase);
    if (is_b) *reinterpret_cast<uint2*>(&sLut[0][(row >> 6) * 256 + (row & 63) * 4]) = t0;
    __syncthreads();
  }
  gload(0);
  lstore(0);
  gload(1);
  __syncthreads();
  auto mma = [&](int buf, auto nb) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb)::value;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // four 16-element MFMA steps per 64-element stage
      typedef typename std::conditional<E5, v8bf, v8h>::type frag;
      frag bf[4], af[2];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const frag*>(&sB[buf][(brow[j] + l32) * kRowH + 32 * ks + 16 * g2]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        af[i] = *reinterpret_cast<const frag*>(&sA[buf][(64 * wm + 32 * i + l32) * kRowH + 32 * ks + 16 * g2]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (E5)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
  };
  // Packed codes: waves 0-3 decode and store stage s+1 before the MFMAs of
  // stage s, waves 4-7 after them.  Wave w runs on SIMD w % 4, so each SIMD
  // holds one wave of each order, and one's decode overlaps the other's MFMAs
  // instead of the two decoding together between barriers (3 % faster; with
  // VQ weights, whose B rows also expand indices, 6-9 % slower, so those
  // keep one order; the FP4 kernel has no registers to spare for the two
  // orders).  The order inside a wave is free: the MFMAs read buffer s & 1,
  // the stores write buffer (s+1) & 1.  (The condition is left a vector
  // compare: made scalar, it changes the register allocation of the two
  // orders and the kernel spills.)
  const bool mfma_first = !VQ && wave >= 4;
  // (the last two stages peeled, as in the FP4 kernel)
  auto kloop = [&](auto nb) __attribute__((always_inline)) {
    int s = 0;
    for (; s < steps - 2; ++s) {
      if (mfma_first) {
        mma(s & 1, nb);
        lstore(s + 1);
        gload(s + 2);
      } else {
        lstore(s + 1);
        gload(s + 2);
        mma(s & 1, nb);
      }
      __syncthreads();
    }
    if (s == steps - 2) {
      if (mfma_first) {
        mma(s & 1, nb);
        lstore(s + 1);
      } else {
        lstore(s + 1);
        mma(s & 1, nb);
      }
      __syncthreads();
      ++s;
    }
    mma(s & 1, nb);
    __syncthreads();
  };
  if (nband == 2)
    kloop(IntC<2>{});
  else if (nband == 1)
    kloop(IntC<1>{});
  else
    kloop(IntC<0>{});

  const float sa = p.a_ts[0];
  if (p.stage == GBW_MOE_DOWN_COMBINE) {
    down_epilogue<kE4BN>(p, ti, acc, wm, wn, lane, sa * p.w_ts[(int64_t)ti.e * p.ts_per], &sA[0][0], s_tok, s_w);
    return;
  }
  // GATEUP: h = bf16(silu(g) * u), staged in LDS (the A buffers) for coalesced stores
  const float sg = sa * p.w_ts[(int64_t)ti.e * p.ts_per];
  const float su = sa * p.w_ts[(int64_t)ti.e * p.ts_per + (p.ts_per > 1 ? 1 : 0)];
  static_assert(kMoeBM * kHRow8 * 2 <= (int)sizeof(sA), "h tile fits the A buffers");
  uint16_t* sH = reinterpret_cast<uint16_t*>(&sA[0][0]);  // [256][kHRow8] bf16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g2 + (r & 3);
      const uint32_t hp = cvt_pk_bf16(silu_mul(acc[i][0][r] * sg, acc[i][2][r] * su),
                                      silu_mul(acc[i][1][r] * sg, acc[i][3][r] * su));
      sH[m * kHRow8 + 64 * wn + l32] = (uint16_t)hp;
      sH[m * kHRow8 + 64 * wn + 32 + l32] = (uint16_t)(hp >> 16);
    }
  __syncthreads();
  const int64_t I = p.N / 2;
  for (int c = tid; c < kMoeBM * 16; c += kE4Threads) {
    const int m = c >> 4, q = c & 15;
    if (m < ti.rows)
      *reinterpret_cast<v4i*>(p.h_bf16 + (int64_t)(ti.row0 + m) * I + (int64_t)ti.nt * 128 + 8 * q) =
          *reinterpret_cast<const v4i*>(&sH[m * kHRow8 + 8 * q]);
  }
}

template <bool E5>
static void launch_moe_b16(const MoeArgs& q, int wl, int grid, hipStream_t st) {
  switch (wl) {
    case W16_VQ: hipLaunchKernelGGL((k_moe_e4m3<E5, W16_VQ>), dim3((unsigned)grid), dim3(kE4Threads), 0, st, q); break;
    case W16_VQ_POST:
      hipLaunchKernelGGL((k_moe_e4m3<E5, W16_VQ_POST>), dim3((unsigned)grid), dim3(kE4Threads), 0, st, q);
      break;
    case W16_VQ_PLUS:
      hipLaunchKernelGGL((k_moe_e4m3<E5, W16_VQ_PLUS>), dim3((unsigned)grid), dim3(kE4Threads), 0, st, q);
      break;
    default: hipLaunchKernelGGL((k_moe_e4m3<E5, W16_NIB>), dim3((unsigned)grid), dim3(kE4Threads), 0, st, q); break;
  }
}

int launch_moe_bf16(const MoeArgs& p, const gbw_act* a, const gbw_weight* w, int grid, hipStream_t st) {
  MoeArgs q = p;
  q.a_ts = a->tensor_scale;
  q.w_ts = w->tensor_scale;
  q.ts_per = w->ts_per_expert;
  const int f = w->fmt;
  const int wl = (f == GBW_FMT_VQ4_E4M3 || f == GBW_FMT_VQ4_E5M3)             ? W16_VQ
                 : (f == GBW_FMT_VQ4_E4M3_POST || f == GBW_FMT_VQ4_E5M3_POST) ? W16_VQ_POST
                 : (f == GBW_FMT_VQ4_E4M3_PLUS || f == GBW_FMT_VQ4_E5M3_PLUS) ? W16_VQ_PLUS
                                                                                : W16_NIB;
  if (a->fmt == GBW_FMT_E5M3_B16)
    launch_moe_b16<true>(q, wl, grid, st);
  else
    launch_moe_b16<false>(q, wl, grid, st);
  return check_launch("moe_grouped_gemm(e4m3/e5m3)");
}

// y[t][n] = sum_j topk_w[t][j] * slots[pair_pos[t][j]][n], j = 0..topk-1 in
// order (a fixed summation order: bitwise repeatable), eight outputs per
// thread; the slot rows of a token are gathered whole-row by the pair index.
template <bool F32>
__global__ void k_moe_combine(const void* __restrict__ slots, const float* __restrict__ topk_w,
                              const int32_t* __restrict__ pair_pos, int topk, int64_t T, int64_t H,
                              float* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= T * H) return;
  const int64_t t = i / H, n = i % H;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const float w = topk_w[t * topk + j];
    const int64_t base = (int64_t)pair_pos[t * topk + j] * H + n;
    if (F32) {
      const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(slots) + base));
      const v4f b =
          __builtin_nontemporal_load(reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(slots) + base + 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] += w * a[q];
        acc[4 + q] += w * b[q];
      }
    } else {
      const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(slots) + base));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * bf16_to_f32((uint32_t)v[q] & 0xFFFFu);
        acc[2 * q + 1] += w * bf16_to_f32((uint32_t)v[q] >> 16);
      }
    }
  }
  __builtin_nontemporal_store(v4f{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<v4f*>(y + i));
  __builtin_nontemporal_store(v4f{acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<v4f*>(y + i + 4));
}

}  // namespace gbw

namespace gbw {

size_t ws_moe_gemm(int64_t P, int64_t N, int64_t f32) {
  // the down/combine stage: a pair-major [P][H] slot buffer, bf16 (fp32 with GBW_FP32_COMBINE)
  return P > 0 && N > 0 ? (size_t)P * N * (f32 ? sizeof(float) : sizeof(uint16_t)) : 0;
}

}  // namespace gbw

using namespace gbw;

extern "C" int moe_grouped_gemm(int32_t stage, int64_t T, int32_t topk, const int32_t* expert_offsets,
                                const int32_t* pair_token, const int32_t* pair_pos, const float* topk_w,
                                const gbw_act* a, const gbw_weight* w, const gbw_moe_out* out, int32_t flags,
                                void* ws, size_t ws_bytes, void* stream) {
  if (stage != GBW_MOE_GATEUP_SWIGLU && stage != GBW_MOE_DOWN_COMBINE)
    return fail(GBW_E_ARG, "moe_grouped_gemm: bad stage");
  if (T < 0 || topk < 1 || topk > 16) return fail(GBW_E_ARG, "moe_grouped_gemm: bad T/topk");
  if (!a || !w || !out) return fail(GBW_E_ARG, "moe_grouped_gemm: null descriptor");
  const int E = w->n_experts;
  if (E < 1 || E > kMaxMoeExperts) return fail(GBW_E_ARG, "moe_grouped_gemm: need 1 <= experts <= %d", kMaxMoeExperts);
  const int64_t K = w->K, N = w->N, P = T * topk;
  if (a->K != K) return fail(GBW_E_SHAPE, "moe_grouped_gemm: activation K %lld != weight K %lld", (long long)a->K,
                             (long long)K);
  if (K <= 0 || K % 128 || K > (int64_t(1) << 30))
    return fail(GBW_E_SHAPE, "moe_grouped_gemm: K must be a positive multiple of 128, at most 2^30");
  const int wf = w->fmt;
  const bool vq32 = wf == GBW_FMT_VQ4_E8M0 || wf == GBW_FMT_VQ4_POST || wf == GBW_FMT_VQ4_PLUS;
  const bool vq16e4 = wf == GBW_FMT_VQ4_E4M3 || wf == GBW_FMT_VQ4_E4M3_POST || wf == GBW_FMT_VQ4_E4M3_PLUS;
  const bool vq16e5 = wf == GBW_FMT_VQ4_E5M3 || wf == GBW_FMT_VQ4_E5M3_POST || wf == GBW_FMT_VQ4_E5M3_PLUS;
  const bool vq = vq32 || vq16e4 || vq16e5;
  const bool vq_plus = wf == GBW_FMT_VQ4_PLUS || wf == GBW_FMT_VQ4_E4M3_PLUS || wf == GBW_FMT_VQ4_E5M3_PLUS;
  const bool fp4 = (wf == GBW_FMT_E8M0_B32 || vq32) && a->fmt == GBW_FMT_E8M0_B32;
  // E4M3-B16 or E5M3-B16 (tensor-scaled, decoded exactly to fp16 / bf16), packed or VQ codes
  const bool e4m3 = ((wf == GBW_FMT_E4M3_B16 || vq16e4) && a->fmt == GBW_FMT_E4M3_B16) ||
                    ((wf == GBW_FMT_E5M3_B16 || vq16e5) && a->fmt == GBW_FMT_E5M3_B16);
  if (!fp4 && !e4m3) return fail(GBW_E_UNSUPPORTED, "moe_grouped_gemm: unsupported activation/weight formats");
  if (stage == GBW_MOE_GATEUP_SWIGLU) {
    if (N % 256) return fail(GBW_E_SHAPE, "moe_grouped_gemm: gate/up rows (2I) must be a multiple of 256");
    if (e4m3 && w->ts_per_expert != 2)
      return fail(GBW_E_ARG, "moe_grouped_gemm: E4M3/E5M3 gate/up needs two tensor scales per expert (gate, up)");
    if (a->rows < T) return fail(GBW_E_SHAPE, "moe_grouped_gemm: activation has fewer rows than tokens");
    // (with T = 0 nothing is written, and the outputs may be NULL)
    if (T > 0 && fp4 && (!out->h_codes || !out->h_scales) && !out->h_bf16)
      return fail(GBW_E_ARG, "moe_grouped_gemm: gate/up needs h_codes+h_scales or h_bf16");
    if (fp4 && (!out->h_codes) != (!out->h_scales))
      return fail(GBW_E_ARG, "moe_grouped_gemm: h_codes and h_scales go together");
    if (T > 0 && e4m3 && !out->h_bf16) return fail(GBW_E_ARG, "moe_grouped_gemm: E4M3/E5M3 gate/up writes h_bf16");
    if (out->h_tail < 0 || out->h_tail % 32 || out->h_tail > N / 2 || (out->h_tail && (e4m3 || !out->h_codes)))
      return fail(GBW_E_SHAPE, "moe_grouped_gemm: h_tail must be a multiple of 32, <= I, with E8M0 h codes");
  } else {
    if (N % 256) return fail(GBW_E_SHAPE, "moe_grouped_gemm: down rows (H) must be a multiple of 256");
    if (e4m3 && w->ts_per_expert != 1)
      return fail(GBW_E_ARG, "moe_grouped_gemm: E4M3/E5M3 down weights take one tensor scale per expert");
    if (a->rows < P) return fail(GBW_E_SHAPE, "moe_grouped_gemm: activation has fewer rows than pairs");
    if (T > 0 && !out->y) return fail(GBW_E_ARG, "moe_grouped_gemm: down needs y");
  }
  const int qb = vq && w->qblock ? w->qblock : 64;
  if (vq) {
    if (!w->codebook) return fail(GBW_E_ARG, "moe_grouped_gemm: VQ needs a codebook");
    if (qb != 64 && qb != 128 && qb != 256) return fail(GBW_E_ARG, "moe_grouped_gemm: QBlock edge must be 64, 128 or 256");
    if (N % qb || K % qb) return fail(GBW_E_SHAPE, "moe_grouped_gemm: N and K must be multiples of the QBlock edge");
    if ((wf == GBW_FMT_VQ4_POST || wf == GBW_FMT_VQ4_PLUS) && K > kXsMaxK)
      return fail(GBW_E_SHAPE, "moe_grouped_gemm: PostScale / PreScale+ weights need K <= %d", kXsMaxK);
    if (vq_plus) {
      if (K % (vq32 ? 256 : 128))
        return fail(GBW_E_SHAPE, "moe_grouped_gemm: PreScale+ needs K a multiple of 8 scale blocks");
      if (!w->scale_codebook) return fail(GBW_E_ARG, "moe_grouped_gemm: PreScale+ needs a scale codebook");
      if (reinterpret_cast<uintptr_t>(w->scale_codebook) & 3u)
        return fail(GBW_E_ALIGN, "moe_grouped_gemm: the scale codebook must be 4-byte aligned");
    }
  }
  if (e4m3 && (!w->tensor_scale || !a->tensor_scale || w->ts_per_expert < 1))
    return fail(GBW_E_ARG, "moe_grouped_gemm: E4M3/E5M3 needs tensor scales");
  if (T == 0) return GBW_OK;
  if (!expert_offsets || !pair_token || !pair_pos || !topk_w || !a->codes || !a->scales || !w->codes || !w->scales)
    return fail(GBW_E_ARG, "moe_grouped_gemm: null pointer");
  if (!aligned16(a->codes) || !aligned16(w->codes) || (w->codebook && !aligned16(w->codebook)) ||
      (reinterpret_cast<uintptr_t>(a->scales) & 3u) || (reinterpret_cast<uintptr_t>(w->scales) & 3u))
    return fail(GBW_E_ALIGN, "moe_grouped_gemm: codes/codebook must be 16-byte and scales 4-byte aligned");
  const bool f32c = (flags & GBW_FP32_COMBINE) != 0;
  const bool use_slots = stage == GBW_MOE_DOWN_COMBINE && ws != nullptr;
  if (stage == GBW_MOE_DOWN_COMBINE && (flags & GBW_DETERMINISTIC) && !ws)
    return fail(GBW_E_WORKSPACE, "moe_grouped_gemm: a deterministic combine needs the slot-buffer workspace");
  if (use_slots && ws_bytes < ws_moe_gemm(P, N, f32c))
    return fail(GBW_E_WORKSPACE, "moe_grouped_gemm: the combine needs %zu bytes of workspace", ws_moe_gemm(P, N, f32c));
  int st = check_device();
  if (st) return st;
  hipStream_t s = as_stream(stream);

  MoeArgs p{};
  p.stage = stage;
  p.topk = topk;
  p.E = E;
  p.T = T;
  p.P = P;
  p.off = expert_offsets;
  p.pair_token = pair_token;
  p.pair_pos = pair_pos;
  p.topk_w = topk_w;
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.K = K;
  p.w_codes = w->codes;
  p.w_scales = w->scales;
  p.w_cb = w->codebook;
  p.w_scb = vq_plus ? w->scale_codebook : nullptr;
  p.qsh = qb == 256 ? 8 : qb == 128 ? 7 : 6;
  p.N = N;
  p.h_bf16 = out->h_bf16;
  p.h_codes = out->h_codes;
  p.h_scales = out->h_scales;
  p.h_tail = stage == GBW_MOE_GATEUP_SWIGLU ? (int32_t)out->h_tail : 0;
  p.y = out->y;
  p.slots = use_slots ? ws : nullptr;
  p.slots_f32 = f32c ? 1 : 0;
  // (PostScale / PreScale+ weight scales are staged in LDS whatever this says)
  const bool w_row_scales = w->fmt != GBW_FMT_VQ4_POST && w->fmt != GBW_FMT_VQ4_PLUS;
  p.scales16 = (K % 512 == 0 && !(reinterpret_cast<uintptr_t>(a->scales) & 15u) &&
                (!w_row_scales || !(reinterpret_cast<uintptr_t>(w->scales) & 15u)))
                   ? 1
                   : 0;
  // every kernel below writes through these: refuse to launch without them
  if (stage == GBW_MOE_DOWN_COMBINE ? (!p.y || (use_slots && !p.slots)) : (!p.h_codes && !p.h_bf16))
    return fail(GBW_E_ARG, "moe_grouped_gemm: no output buffer");
  if (stage == GBW_MOE_DOWN_COMBINE && !use_slots) {
    if ((st = launch_fill_zero(out->y, T * N, s))) return st;
  }
  if (e4m3) {
    p.n_tiles = (int)(N / kE4BN);
    int64_t grid = (cdiv(P, kMoeBM) + E) * p.n_tiles;
    grid = cdiv(grid, 8) * 8;
    if (grid > INT32_MAX) return fail(GBW_E_SHAPE, "moe_grouped_gemm: problem too large");
    p.total_tiles = (int)grid;
    st = launch_moe_bf16(p, a, w, (int)grid, s);
  } else {
    // 256-row weight tiles for both stages: each expanded weight tile meets
    // the most pairs (for the down stage 4 % faster than 128-row tiles with
    // two workgroups per CU, measured at 65536 pairs, H 4096, I 1536)
    switch (w->fmt) {
      case GBW_FMT_VQ4_E8M0: st = launch_moe_fp4<W_VQ>(p, s); break;
      case GBW_FMT_VQ4_POST: st = launch_moe_fp4<W_VQ_POST>(p, s); break;
      case GBW_FMT_VQ4_PLUS: st = launch_moe_fp4<W_VQ_PLUS>(p, s); break;
      default: st = launch_moe_fp4<W_MX>(p, s); break;
    }
  }
  if (st) return st;
  if (use_slots) {
    const unsigned blocks = (unsigned)cdiv(cdiv(T * N, 8), 256);
    if (f32c)
      hipLaunchKernelGGL(k_moe_combine<true>, dim3(blocks), dim3(256), 0, s, ws, topk_w, pair_pos, topk, T, N, out->y);
    else
      hipLaunchKernelGGL(k_moe_combine<false>, dim3(blocks), dim3(256), 0, s, ws, topk_w, pair_pos, topk, T, N,
                         out->y);
    st = check_launch("moe_grouped_gemm(combine)");
  }
  return st;
}

#ifdef GBW_TILE_TRACE
// Copy the tile trace to host memory (bytes <= 16384 * 8 * 8), or with
// clear != 0 zero it.  Synchronous; only in the trace build.
extern "C" int gbw_tile_trace(void* host, size_t bytes, int clear) {
  static unsigned long long zero[gbw::kTraceBlocks * 8];
  if (clear) return (int)hipMemcpyToSymbol(HIP_SYMBOL(gbw::g_tile_trace), zero, sizeof(zero));
  if (bytes > sizeof(zero)) return (int)hipErrorInvalidValue;
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gbw::g_tile_trace), bytes);
}
#endif
