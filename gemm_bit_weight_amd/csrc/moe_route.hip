// MoE routing: top-k experts per token, softmax weights over the chosen k,
// and the (expert, token)-sorted pair list the grouped GEMMs walk.
//
// The experts being routed are the quantized FFN experts of "CodeQuant:
// Unified Clustering and Quantization for Enhanced Outlier Smoothing in
// Low-Precision Mixture-of-Experts" (Fig. 1, Fig. 2) and the expert
// down-projections of "PRQuant: Permutation Residual Quantization for
// Low-Overhead Inference" (§4, §5.1).  The pages fix no routing rule; the one
// here is: the k largest logits (ties to the lower expert id; -0 ties +0,
// NaN ranks below every number), weights exp(l_j - l_max) / sum over the
// chosen k.
//
// Three kernels, no atomics on global memory, so the pair order is fixed:
//  1. k_route_topk: one thread per token keeps a sorted top-k in registers
//     while it scans the token's logits (k_route_topk16, for E <= 256: 16
//     lanes per token); a chunk of 64 tokens builds, in LDS, a 64-bit mask
//     per expert of the chunk's tokens that chose it and writes the
//     per-(chunk, expert) counts.
//  2. k_route_scan: exclusive scan of the counts in (expert, chunk) order ->
//     expert_offsets and the first pair slot of every (chunk, expert).
//  3. k_route_scatter: a token's pair index = its chunk's slot for the
//     expert + the number of earlier tokens of the chunk in that expert's
//     mask (a popcount).
// With at most kScanLds counts, 2 and 3 are one kernel, k_route_scan_scatter.
#include <mutex>

#include "common.hpp"

namespace gbw {

constexpr int kRouteThreads = 256;  // 4 chunks of 64 tokens per workgroup
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ int64_t n_chunks(int64_t T) { return (T + 63) / 64; }

// Every (logit, expert) as one 64-bit key that orders exactly as the routing
// rule does: the logit's bits made order-preserving as an unsigned integer in
// the high word (-0 counted as +0, so the two zeros tie; NaN below every
// number, where a stable sort of the negated logits puts it), 0xFFFF - expert
// in the low word (a tie goes to the lower id); 0 is "no entry".  Keys are
// distinct, so a top-k over keys needs no tie rule of its own.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
  uint32_t s = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // -inf -> 0x007FFFFF, +inf -> 0xFF800000
  s = nan ? 1u : s;
  return ((uint64_t)s << 32) | (uint32_t)(0xFFFF - e);
}

__device__ __forceinline__ float route_key_value(uint64_t k) {
  const uint32_t s = (uint32_t)(k >> 32);
  return __uint_as_float((s & 0x80000000u) ? (s & 0x7FFFFFFFu) : ~s);  // (s = 1, NaN: a NaN)
}

template <int K>
__global__ __launch_bounds__(kRouteThreads) void k_route_topk(const float* __restrict__ logits, int64_t T, int E,
                                                             int32_t* __restrict__ topk_ids,
                                                             float* __restrict__ topk_w,
                                                             int32_t* __restrict__ counts) {
  __shared__ unsigned long long mask[kRouteThreads / 64][kMaxExperts];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t chunk = (int64_t)blockIdx.x * (kRouteThreads / 64) + wv;
  const int64_t t = chunk * 64 + lane;
  for (int e = lane; e < E; e += 64) mask[wv][e] = 0ull;
  __syncthreads();

  uint64_t kk[K];  // descending route keys, 0 = empty
#pragma unroll
  for (int j = 0; j < K; ++j) kk[j] = 0ull;
  const bool live = t < T;
  if (live) {
    const float* row = logits + t * E;
    for (int e = 0; e < E; ++e) {
      // insertion: the candidate moves past every smaller key
      uint64_t c = route_key(row[e], e);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const uint64_t tk = kk[j];
        const bool gt = c > tk;
        kk[j] = gt ? c : tk;
        c = gt ? tk : c;
      }
    }
    float v[K];
    int id[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j] = route_key_value(kk[j]);
      id[j] = 0xFFFF - (int)(kk[j] & 0xFFFFu);
    }
    float ex[K], sum = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ex[j] = expf(v[j] - v[0]);
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      topk_ids[t * K + j] = id[j];
      topk_w[t * K + j] = ex[j] / sum;
      atomicOr(&mask[wv][id[j]], 1ull << lane);
    }
  }
  __syncthreads();
  if (chunk < n_chunks(T))
    for (int e = lane; e < E; e += 64) counts[chunk * E + e] = __popcll(mask[wv][e]);
}

// Same outputs for E <= 256 with 16 lanes per token: a workgroup of 1024
// threads is one chunk of 64 tokens; lane s of a token's group holds the
// logits of experts s, s + 16, ... (NV of them: 8 for E <= 128, else 16;
// coalesced loads), as route_key keys.  Round j takes the largest key below
// round j-1's: a lane-local pass over NV keys, then a 16-lane maximum over
// DPP row permutes -- no branches and nothing to remove from the lists.
template <int CTRL>
__device__ __forceinline__ uint64_t max_step(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)k, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, true);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// lanes ^1, ^2 (quad permutes), then the mirrors within 8 and 16 lanes:
// after the four steps every lane of the 16-lane row holds the row's maximum
__device__ __forceinline__ uint64_t row16_max(uint64_t k) {
  k = max_step<0xB1>(k);
  k = max_step<0x4E>(k);
  k = max_step<0x141>(k);
  return max_step<0x140>(k);
}

template <int K, int NV>
__global__ __launch_bounds__(1024) void k_route_topk16(const float* __restrict__ logits, int64_t T, int E,
                                                       int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                                                       int32_t* __restrict__ counts) {
  __shared__ unsigned long long mask[256];
  const int tid = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  const int tl = tid >> 4, sl = tid & 15;  // token of the chunk, lane of its group
  const int64_t t = chunk * 64 + tl;
  if (tid < E) mask[tid] = 0ull;
  __syncthreads();
  const bool live = t < T;
  const float* row = logits + (live ? t : 0) * E;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = sl + 16 * i;
    v[i] = live && e < E ? row[e] : 0.f;
  }
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = sl + 16 * i;
    key[i] = live && e < E ? route_key(v[i], e) : 0ull;
  }
  int ids[K];
  float vals[K];
  uint64_t bound = ~0ull;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint64_t c = key[i] < bound ? key[i] : 0ull;
      best = c > best ? c : best;
    }
    best = row16_max(best);
    bound = best;
    ids[j] = 0xFFFF - (int)(best & 0xFFFFu);
    vals[j] = route_key_value(best);
  }
  if (live) {
    float ex[K], sum = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ex[j] = expf(vals[j] - vals[0]);
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j == sl) {
        topk_ids[t * K + j] = ids[j];
        topk_w[t * K + j] = ex[j] / sum;
        atomicOr(&mask[ids[j]], 1ull << tl);
      }
  }
  __syncthreads();
  if (tid < E) counts[chunk * E + tid] = __popcll(mask[tid]);
}

// Single workgroup of 1024 threads (count tables larger than kScanLds; smaller
// ones go through k_route_scan_scatter): G = 1024 / E' threads per expert (E'
// = E rounded up to a power of two) each own a contiguous run of chunks;
// per-run sums, an exclusive scan over the runs of an expert, an inclusive
// scan over the expert totals, then each thread writes the bases of its own
// chunks.
constexpr int kScanLds = 16384;  // 64 KiB of counts
__global__ __launch_bounds__(kMaxExperts) void k_route_scan(const int32_t* __restrict__ counts, int64_t C, int E,
                                                           int32_t* __restrict__ base,
                                                           int32_t* __restrict__ expert_offsets) {
  __shared__ int32_t part[kMaxExperts];
  __shared__ int32_t tot[kMaxExperts];
  const int tid = threadIdx.x;
  const int32_t* const cnt = counts;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int G = kMaxExperts / Ep;
  const int e = tid / G, g = tid % G;
  const int64_t per = (C + G - 1) / G;
  const int64_t c0 = g * per, c1 = min(C, c0 + per);
  int32_t s = 0;
  if (e < E)
    for (int64_t c = c0; c < c1; ++c) s += cnt[c * E + e];
  part[tid] = s;
  __syncthreads();
  if (g == 0) {
    int32_t t = 0;
    for (int q = 0; q < G; ++q) t += part[e * G + q];
    tot[e] = e < E ? t : 0;
  }
  if (tid >= Ep) tot[tid] = 0;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {  // inclusive scan of the expert totals
    const int32_t add = tid >= o ? tot[tid - o] : 0;
    __syncthreads();
    tot[tid] += add;
    __syncthreads();
  }
  if (e < E) {
    int32_t run = (e ? tot[e - 1] : 0);
    for (int q = 0; q < g; ++q) run += part[e * G + q];
    if (g == 0) expert_offsets[e] = e ? tot[e - 1] : 0;
    if (e == E - 1 && g == 0) expert_offsets[E] = tot[E - 1];
    for (int64_t c = c0; c < c1; ++c) {
      base[c * E + e] = run;
      run += cnt[c * E + e];
    }
  }
}

template <int K>
__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const int32_t* __restrict__ topk_ids, int64_t T,
                                                                int E, const int32_t* __restrict__ base,
                                                                int32_t* __restrict__ pair_token,
                                                                int32_t* __restrict__ pair_pos) {
  __shared__ unsigned long long mask[kRouteThreads / 64][kMaxExperts];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t chunk = (int64_t)blockIdx.x * (kRouteThreads / 64) + wv;
  const int64_t t = chunk * 64 + lane;
  for (int e = lane; e < E; e += 64) mask[wv][e] = 0ull;
  __syncthreads();
  int id[K];
  const bool live = t < T;
  if (live) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      id[j] = topk_ids[t * K + j];
      atomicOr(&mask[wv][id[j]], 1ull << lane);
    }
  }
  __syncthreads();
  if (!live) return;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int32_t p = base[chunk * E + id[j]] + __popcll(mask[wv][id[j]] & below);
    pair_token[p] = (int32_t)t;
    pair_pos[t * K + j] = p;
  }
}

// Scan and scatter in one kernel when the [C][E] count table fits in LDS
// (C * E <= kScanLds): every workgroup (4 chunks, one wave each) copies the
// whole table with all loads in flight, forms for each expert the total over
// all chunks and the sum over the chunks before each of its own, scans the
// totals over the experts (expert_offsets, written by workgroup 0), and
// places its tokens' pairs as k_route_scatter does.  Same bases as the
// separate scan, without its single-workgroup pass and kernel boundary.
template <int K>
__global__ __launch_bounds__(kRouteThreads) void k_route_scan_scatter(const int32_t* __restrict__ counts,
                                                                     const int32_t* __restrict__ topk_ids, int64_t T,
                                                                     int E, int32_t* __restrict__ expert_offsets,
                                                                     int32_t* __restrict__ pair_token,
                                                                     int32_t* __restrict__ pair_pos) {
  constexpr int NW = kRouteThreads / 64;  // chunks per workgroup
  __shared__ int32_t stg[kScanLds];
  __shared__ unsigned long long mask[NW][kMaxExperts];
  __shared__ int32_t base[NW][kMaxExperts];  // expert_offsets[e] + pairs of e in earlier chunks
  __shared__ int32_t run[kRouteThreads];       // per-thread sums of the expert totals, then their scan
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t C = n_chunks(T);
  const int64_t c0 = (int64_t)blockIdx.x * NW;  // first chunk of this workgroup
  const int64_t chunk = c0 + wv;
  const int64_t t = chunk * 64 + lane;
  const int n = (int)(C * E);
#pragma unroll 16
  for (int i = tid; i < n; i += kRouteThreads) stg[i] = counts[i];
  for (int e = lane; e < E; e += 64) mask[wv][e] = 0ull;
  __syncthreads();
  int id[K];
  const bool live = t < T;
  if (live) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      id[j] = topk_ids[t * K + j];
      atomicOr(&mask[wv][id[j]], 1ull << lane);
    }
  }
  // experts are dealt to threads in runs of EPT consecutive ids; each thread
  // keeps, per expert of its run, the prefix over this workgroup's chunks in
  // base[w][e] and the total; the run sums are then scanned across threads
  const int EPT = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * EPT, e1 = min(E, e0 + EPT);
  int32_t rsum = 0;
  const int Ci = (int)C;
  const int w0 = (int)c0;
  for (int e = e0; e < e1; ++e) {
    int32_t acc = 0;
    int c = 0;
    for (; c + 8 <= Ci; c += 8) {  // eight LDS reads in flight per step
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = stg[(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = c + i - w0;
        if (w >= 0 && w < NW) base[w][e] = acc;
        acc += v[i];
      }
    }
    for (; c < Ci; ++c) {
      const int w = c - w0;
      if (w >= 0 && w < NW) base[w][e] = acc;
      acc += stg[c * E + e];
    }
    rsum += acc;
    stg[e] = acc;  // the total, over row 0 (only this thread reads column e)
  }
  run[tid] = rsum;
  __syncthreads();
  for (int o = 1; o < kRouteThreads; o <<= 1) {  // inclusive scan of the run sums
    const int32_t add = tid >= o ? run[tid - o] : 0;
    __syncthreads();
    run[tid] += add;
    __syncthreads();
  }
  int32_t off = tid ? run[tid - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    const int32_t tot = stg[e];
#pragma unroll
    for (int w = 0; w < NW; ++w) base[w][e] += off;
    if (blockIdx.x == 0) expert_offsets[e] = off;
    off += tot;
  }
  if (blockIdx.x == 0 && tid == kRouteThreads - 1) expert_offsets[E] = run[tid];
  __syncthreads();
  if (!live) return;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int32_t p = base[wv][id[j]] + __popcll(mask[wv][id[j]] & below);
    pair_token[p] = (int32_t)t;
    pair_pos[t * K + j] = p;
  }
}

size_t ws_moe_route(int64_t T, int64_t E) {
  if (T <= 0 || E <= 0) return 0;
  const int64_t C = (T + 63) / 64;
  return (size_t)2 * C * E * sizeof(int32_t);  // counts + bases
}

template <int K>
static int launch_route(const float* logits, int64_t T, int E, int32_t* ids, float* w, int32_t* off, int32_t* pt,
                        int32_t* pp, int32_t* ws, hipStream_t st) {
  const int64_t C = (T + 63) / 64;
  int32_t* counts = ws;
  int32_t* base = ws + C * E;
  const unsigned blocks = (unsigned)cdiv(C, kRouteThreads / 64);
  if (E <= 128)
    hipLaunchKernelGGL((k_route_topk16<K, 8>), dim3((unsigned)C), dim3(1024), 0, st, logits, T, E, ids, w, counts);
  else if (E <= 256)
    hipLaunchKernelGGL((k_route_topk16<K, 16>), dim3((unsigned)C), dim3(1024), 0, st, logits, T, E, ids, w, counts);
  else
    hipLaunchKernelGGL(k_route_topk<K>, dim3(blocks), dim3(kRouteThreads), 0, st, logits, T, E, ids, w, counts);
  int s = check_launch("moe_route(topk)");
  if (s) return s;
  if (C * E <= kScanLds) {
    hipLaunchKernelGGL(k_route_scan_scatter<K>, dim3(blocks), dim3(kRouteThreads), 0, st, counts, ids, T, E, off, pt,
                       pp);
    return check_launch("moe_route(scan + scatter)");
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kMaxExperts), 0, st, counts, C, E, base, off);
  if ((s = check_launch("moe_route(scan)"))) return s;
  hipLaunchKernelGGL(k_route_scatter<K>, dim3(blocks), dim3(kRouteThreads), 0, st, ids, T, E, base, pt, pp);
  return check_launch("moe_route(scatter)");
}

}  // namespace gbw

using namespace gbw;

namespace gbw {

// Validation and launches shared by moe_route and moe_route_noalloc; `ws`
// holds ws_moe_route(T, E) bytes (counts + bases), every byte written by the
// kernels before it is read.
static int route_checked(const char* who, const float* logits, int64_t T, int32_t E, int32_t topk,
                         int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* pair_token,
                         int32_t* pair_pos) {
  if (T < 0 || E <= 0 || E > kMaxExperts) return fail(GBW_E_ARG, "%s: need 0 < E <= %d", who, kMaxExperts);
  if (topk < 1 || topk > E || topk > kMaxTopk) return fail(GBW_E_ARG, "%s: need 1 <= topk <= min(E, 16)", who);
  if (!expert_offsets) return fail(GBW_E_ARG, "%s: null expert_offsets", who);
  if (T > 0 && (!logits || !topk_ids || !topk_w || !pair_token || !pair_pos))
    return fail(GBW_E_ARG, "%s: null pointer", who);
  if ((int64_t)T * topk > INT32_MAX) return fail(GBW_E_SHAPE, "%s: too many pairs for int32 indices", who);
  return GBW_OK;
}

static int route_launch(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids, float* topk_w,
                        int32_t* expert_offsets, int32_t* pair_token, int32_t* pair_pos, int32_t* w32,
                        hipStream_t s) {
  if (T == 0) {
    // no tokens: every expert offset is zero
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kMaxExperts), 0, s, (const int32_t*)nullptr, (int64_t)0, E,
                       (int32_t*)nullptr, expert_offsets);
    return check_launch("moe_route(empty)");
  }
  switch (topk) {
#define GBW_ROUTE_CASE(K) \
  case K:                 \
    return launch_route<K>(logits, T, E, topk_ids, topk_w, expert_offsets, pair_token, pair_pos, w32, s);
    GBW_ROUTE_CASE(1)
    GBW_ROUTE_CASE(2)
    GBW_ROUTE_CASE(3)
    GBW_ROUTE_CASE(4)
    GBW_ROUTE_CASE(5)
    GBW_ROUTE_CASE(6)
    GBW_ROUTE_CASE(7)
    GBW_ROUTE_CASE(8)
    GBW_ROUTE_CASE(9)
    GBW_ROUTE_CASE(10)
    GBW_ROUTE_CASE(11)
    GBW_ROUTE_CASE(12)
    GBW_ROUTE_CASE(13)
    GBW_ROUTE_CASE(14)
    GBW_ROUTE_CASE(15)
    GBW_ROUTE_CASE(16)
#undef GBW_ROUTE_CASE
    default:
      return fail(GBW_E_UNSUPPORTED, "moe_route: topk out of range");
  }
}

// ---------------------------------------------------------------------------
// Allocation-free routing: the counts and bases live in this file-scope
// device array (one copy per GPU, alive until the process ends) instead of
// a caller workspace.  Host code never passes `scratch` itself to a kernel:
// its device address on the current GPU is looked up once per device and
// kept in g_scratch[dev].
// ---------------------------------------------------------------------------
constexpr size_t kRouteScratchBytes = (size_t)1 << 20;  // counts + bases of C * E <= 131072 (chunks of 64 tokens)
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
int32_t* g_scratch[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
}  // namespace

static int32_t* route_scratch(int dev) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<int32_t*>(ptr) : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace gbw

extern "C" int moe_route(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids, float* topk_w,
                         int32_t* expert_offsets, int32_t* pair_token, int32_t* pair_pos, void* ws, size_t ws_bytes,
                         void* stream) {
  int st = route_checked("moe_route", logits, T, E, topk, topk_ids, topk_w, expert_offsets, pair_token, pair_pos);
  if (st) return st;
  if (T > 0 && (!ws || ws_bytes < ws_moe_route(T, E)))
    return fail(GBW_E_WORKSPACE, "moe_route: needs %zu bytes of workspace", ws_moe_route(T, E));
  if ((st = check_device())) return st;
  return route_launch(logits, T, E, topk, topk_ids, topk_w, expert_offsets, pair_token, pair_pos,
                      reinterpret_cast<int32_t*>(ws), as_stream(stream));
}

extern "C" int moe_route_noalloc(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids,
                                 float* topk_w, int32_t* expert_offsets, int32_t* pair_token, int32_t* pair_pos,
                                 void* stream) {
  int st = route_checked("moe_route_noalloc", logits, T, E, topk, topk_ids, topk_w, expert_offsets, pair_token,
                         pair_pos);
  if (st) return st;
  if (ws_moe_route(T, E) > kRouteScratchBytes)
    return fail(GBW_E_SHAPE, "moe_route_noalloc: %lld tokens x %d experts need %zu bytes of scratch, more than the "
                "fixed %zu (ceil(T / 64) * E must be <= %zu)", (long long)T, E, ws_moe_route(T, E),
                kRouteScratchBytes, kRouteScratchBytes / 8);
  if ((st = check_device())) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
    return fail(GBW_E_UNSUPPORTED, "moe_route_noalloc: no usable HIP device");
  int32_t* w32 = route_scratch(dev);
  if (!w32)
    return fail(GBW_E_LAUNCH, "moe_route_noalloc: scratch address lookup failed on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  return route_launch(logits, T, E, topk, topk_ids, topk_w, expert_offsets, pair_token, pair_pos, w32,
                      as_stream(stream));
}
