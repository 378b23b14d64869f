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
// Contraction: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands FP4 (E2M1)
// and one E8M0 scale per lane.  A lane (row r = lane % 16, group g = lane / 16)
// holds 32 consecutive K elements -- exactly one E8M0 block -- as 16 bytes, and
// that block's scale.  A and W use the same lane -> K mapping, so each lane's
// products pair the same K indices and the scale applies to its own block.
// The 16x16 fp32 result lives as lane l, register i = row 4*(l/16)+i, column l%16.
//
// Decode-shaped problems (M <= 128, N in the thousands) are bound by the weight
// stream from HBM: each wave streams its own 16*TN weight rows with 16-byte
// loads, the M side is covered in registers (TM tiles of 16 rows) and the K
// range is split across workgroups when the (N, M) tiles alone cannot fill
// 256 CUs; the split partial sums are combined with fp32 atomics.
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
  int32_t atomic;
};

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

template <int TM, int TN, int NW>
__global__ __launch_bounds__(64 * NW) void k_mx_gemm(const MxGemmArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.z * (16 * TM);
  const int64_t n0 = ((int64_t)blockIdx.x * NW + wave) * (16 * TN);
  if (n0 >= p.N) return;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int s_end = min(p.total_steps, s_begin + p.steps_per_split);

  const uint8_t* arow[TM];
  const uint8_t* asrow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t r = m0 + 16 * i + r16;
    r = r < p.M ? r : p.M - 1;
    arow[i] = p.a_codes + r * p.lda;
    asrow[i] = p.a_scales + r * p.ldas;
  }
  int64_t wrow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int64_t n = n0 + 16 * j + r16;
    wrow[j] = n < p.N ? n : p.N - 1;
  }

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s = s_begin; s < s_end; ++s) {
    const int si = s < p.seg[0].steps ? 0 : 1;
    const MxSeg& sg = p.seg[si];
    const int64_t kk = (int64_t)(s - (si ? p.seg[0].steps : 0)) * 128 + 32 * g;
    const bool valid = kk < sg.K;
    v4i af[TM], bf[TN];
    int as[TM], bs[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t ka = sg.a_k0 + kk;
      af[i] = valid ? load16(arow[i] + ka / 2) : v4i{0, 0, 0, 0};
      as[i] = valid ? (int)asrow[i][ka / 32] : 127;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      bf[j] = valid ? load16(sg.w_codes + wrow[j] * sg.ldw + kk / 2) : v4i{0, 0, 0, 0};
      bs[j] = valid ? (int)sg.w_scales[wrow[j] * sg.ldws + kk / 32] : 127;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(af[i]), widen(bf[j]), acc[i][j], 4, 4,
                                                                      0, as[i], 0, bs[j]);
  }

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
        float* dst = p.y + m * p.ldy + n;
        if (p.atomic)
          unsafeAtomicAdd(dst, acc[i][j][q]);
        else
          *dst = acc[i][j][q];
      }
    }
}

template <int TM, int TN, int NW>
static int launch_mx(MxGemmArgs& p, bool deterministic, hipStream_t st) {
  const int64_t n_tiles = cdiv(p.N, 16 * TN * NW);
  const int64_t m_tiles = cdiv(p.M, 16 * TM);
  const int64_t tiles = n_tiles * m_tiles;
  int splits = 1;
  if (!deterministic) {
    const int64_t want = 2 * (int64_t)device_cu_count();
    if (tiles < want) splits = (int)cdiv(want, tiles);
    if (splits > p.total_steps) splits = p.total_steps;
  }
  p.steps_per_split = (int)cdiv(p.total_steps, splits);
  splits = (int)cdiv(p.total_steps, p.steps_per_split);
  p.atomic = splits > 1;
  if (p.atomic) {
    int s = launch_fill_zero(p.y, p.M * p.ldy, st);
    if (s) return s;
  }
  hipLaunchKernelGGL((k_mx_gemm<TM, TN, NW>), dim3((unsigned)n_tiles, (unsigned)splits, (unsigned)m_tiles),
                     dim3(64 * NW), 0, st, p);
  return check_launch("mx_gemm");
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

static int run_mx(int64_t M, const gbw_act* a, const gbw_weight* w, const gbw_weight* r, int64_t tail, float* y,
                  int32_t flags, void* stream) {
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
  const bool det = (flags & GBW_DETERMINISTIC) != 0;
  hipStream_t st = as_stream(stream);
  if (M <= 16) return launch_mx<1, 1, 4>(p, det, st);
  if (M <= 32) return launch_mx<2, 1, 4>(p, det, st);
  if (M <= 64) return launch_mx<4, 1, 4>(p, det, st);
  return launch_mx<8, 1, 4>(p, det, st);
}

}  // namespace gbw

using namespace gbw;

extern "C" int mx_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, float* y, int32_t flags, void* stream) {
  if (M < 0) return fail(GBW_E_ARG, "mx_gemm: negative M");
  int st;
  if ((st = check_act(a, M, "mx_gemm"))) return st;
  if ((st = check_w(w, a->K, "mx_gemm"))) return st;
  if (M == 0 || w->N == 0) return GBW_OK;
  if (!y) return fail(GBW_E_ARG, "mx_gemm: null output");
  if ((st = check_device())) return st;
  return run_mx(M, a, w, nullptr, 0, y, flags, stream);
}

extern "C" int residual_tail_gemm(int64_t M, const gbw_act* a, const gbw_weight* w, const gbw_weight* r,
                                  int64_t tail, float* y, int32_t flags, void* stream) {
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
  return run_mx(M, a, w, tail > 0 ? r : nullptr, tail, y, flags, stream);
}
