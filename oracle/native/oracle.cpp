// Plain CPU reference of the 4-bit-weight GEMM hot path, in C++17.
//
// TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
// CPU baseline call it; the HIP library never does, and this file shares no
// header, table or helper with it.
//
// Every operand is decoded to double from the closed forms of its format and
// every dot product is summed term by term in double with Neumaier's
// compensated summation; the naive double sum is kept beside it, and each call
// returns how many outputs the two disagree on.  For the block-scaled FP4
// formats a product e2m1*e2m1*2^(sa+sb-254) has at most 4 significant bits
// (E4M3 / UE5M3 block scales: at most 12), so when the sums span fewer than
// 53 bits the naive sum is exact and equal to the compensated one -- the
// value returned is then the exact value of the quantized GEMM.
//
// Sources (page titles):
//  * "MXCode: MX-Native Codebook Quantization" -- Table 1 (E8M0-B32, E4M3-B16
//    and E5M3-B16 FP4 block formats), abstract and Fig. 2-3 (PreScale VQ:
//    8-bit index per 4 weights into a 256-entry table per QBlock).
//  * "PRQuant: Permutation Residual Quantization for Low-Overhead Inference"
//    -- Sec. 4 Eq. (1) (gated MLP), Eq. (2) (offline residual), "Kernel
//    design for efficient inference" (one GEMM over the reduction C + k).
//  * "CodeQuant: Unified Clustering and Quantization for Enhanced Outlier
//    Smoothing in Low-Precision Mixture-of-Experts" -- Fig. 1 and Fig. 4
//    (weights as cluster indices into a per-group table of centroids).
// The E2M1 values {0, 0.5, 1, 1.5, 2, 3, 4, 6} are the OCP MX element type
// the PRQuant page cites for MXFP4.  Readings where the pages are silent:
// nibble 2i of a row in bits 3:0 of byte i; VQ key element i in bits 4i+3:4i;
// E8M0 scale = floor(log2 amax) - 2 (OCP rule), clamped at code 0; element
// rounding to nearest, ties to the even code, saturating at 6, sign kept;
// E4M3-B16 / E5M3-B16: S_T = amax / (6 * max scale), block scale =
// RNE(amax_blk / (6 S_T)), element = RNE(|x| / (scale * S_T)), fp32 steps in
// that order; routed-FFN h = bf16(silu(g) * u).
//
// Threads: std::thread over the outputs (GBWO_THREADS overrides the count);
// each output is one sequential sum, so the thread count never changes a
// result.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

enum { F_E8M0_B32 = 0, F_E4M3_B16 = 1, F_E5M3_B16 = 2 };

// ---------------------------------------------------------------- decoders
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double e2m1(unsigned c) { return (c & 8u) ? -kE2M1[c & 7u] : kE2M1[c & 7u]; }

// E8M0: 2^(e - 127)
double e8m0(unsigned e) { return std::ldexp(1.0, (int)e - 127); }

// E4M3 (fn), used unsigned: exponent field 0 gives (m/8) 2^-6, else (1 + m/8) 2^(e-7)
double e4m3(unsigned c) {
  const unsigned e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (m / 8.0) * std::ldexp(1.0, -6) : (1.0 + m / 8.0) * std::ldexp(1.0, (int)e - 7);
}

// UE5M3: 5 exponent bits with bias 15, 3 mantissa bits, unsigned
double ue5m3(unsigned c) {
  const unsigned e = (c >> 3) & 31u, m = c & 7u;
  return e == 0 ? (m / 8.0) * std::ldexp(1.0, -14) : (1.0 + m / 8.0) * std::ldexp(1.0, (int)e - 15);
}

// IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits
double fp16(uint16_t b) {
  const unsigned e = (b >> 10) & 31u, m = b & 1023u;
  double v;
  if (e == 0)
    v = m * std::ldexp(1.0, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = (1.0 + m / 1024.0) * std::ldexp(1.0, (int)e - 15);
  return (b & 0x8000u) ? -v : v;
}

// bfloat16: the top 16 bits of an fp32
double bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int block_of(int fmt) { return fmt == F_E8M0_B32 ? 32 : 16; }

double scale_value(unsigned code, int fmt) {
  return fmt == F_E8M0_B32 ? e8m0(code) : fmt == F_E4M3_B16 ? e4m3(code) : ue5m3(code);
}

unsigned nibble(const uint8_t* row, int64_t k) { return (row[k >> 1] >> (4 * (k & 1))) & 15u; }

// One row of packed codes + block scales -> doubles (no tensor scale).
void decode_row(const uint8_t* codes, const uint8_t* scales, int fmt, int64_t K, double* out) {
  const int bs = block_of(fmt);
  for (int64_t k = 0; k < K; ++k) out[k] = e2m1(nibble(codes, k)) * scale_value(scales[k / bs], fmt);
}

// ---------------------------------------------------------------- threads
int n_threads() {
  if (const char* s = std::getenv("GBWO_THREADS")) {
    const int v = std::atoi(s);
    if (v > 0) return v;
  }
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// fn(i) for i in [0, n), handed out in chunks to n_threads() threads
template <class F>
void parallel_for(int64_t n, F fn) {
  const int nt = n_threads();
  std::atomic<int64_t> next(0);
  const int64_t chunk = 16;
  auto work = [&]() {
    for (;;) {
      const int64_t i0 = next.fetch_add(chunk);
      if (i0 >= n) return;
      const int64_t i1 = i0 + chunk < n ? i0 + chunk : n;
      for (int64_t i = i0; i < i1; ++i) fn(i);
    }
  };
  std::vector<std::thread> th;
  for (int t = 1; t < nt && (int64_t)t * chunk < n; ++t) th.emplace_back(work);
  work();
  for (auto& t : th) t.join();
}

// ---------------------------------------------------------------- sums
struct Sum {
  double s = 0.0, c = 0.0, naive = 0.0;
  void add(double x) {
    naive += x;
    const double t = s + x;
    if (std::fabs(s) >= std::fabs(x))
      c += (s - t) + x;
    else
      c += (x - t) + s;
    s = t;
  }
  double value() const { return s + c; }
  bool exact() const { return naive == s + c; }
};

// out[r][n] = sum_k A[r][k] W[n][k] over decoded rows; returns the number of
// outputs whose naive and compensated sums differ
int64_t dot_all(int64_t R, int64_t N, int64_t K, const double* A, const double* W, double* out) {
  std::atomic<int64_t> inexact(0);
  parallel_for(R * N, [&](int64_t i) {
    const int64_t r = i / N, n = i % N;
    const double* a = A + r * K;
    const double* w = W + n * K;
    Sum s;
    for (int64_t k = 0; k < K; ++k) s.add(a[k] * w[k]);
    out[i] = s.value();
    if (!s.exact()) inexact.fetch_add(1);
  });
  return inexact.load();
}

// ---------------------------------------------------------------- rounding
// nearest entry of an increasing grid to v >= 0, ties to the even index,
// saturating at the last entry
unsigned round_to_grid(double v, const double* grid, unsigned n) {
  unsigned hi = 0;
  while (hi < n && grid[hi] < v) ++hi;  // first grid value >= v
  if (hi == 0) return 0;
  if (hi == n) return n - 1;
  const double dl = v - grid[hi - 1], dh = grid[hi] - v;
  if (dh < dl) return hi;
  if (dl < dh) return hi - 1;
  return (hi & 1u) ? hi - 1 : hi;
}

unsigned e2m1_rne(double v) { return round_to_grid(v, kE2M1, 8); }

struct Grids {
  double e4[127], e5[255];
  Grids() {
    for (unsigned c = 0; c < 127; ++c) e4[c] = e4m3(c);   // 0x00 .. 0x7E (0x7F is NaN)
    for (unsigned c = 0; c < 255; ++c) e5[c] = ue5m3(c);  // 0x00 .. 0xFE (0xFF reserved)
  }
};
const Grids kGrids;

float f32_of_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint32_t bits_of_f32(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// double -> bf16 bits, round to nearest, ties to even (finite inputs)
uint16_t bf16_rne(double v) {
  if (v == 0.0 || std::isnan(v)) return (uint16_t)(bits_of_f32((float)v) >> 16);
  double r;
  if (std::fabs(v) < std::ldexp(1.0, -126)) {
    r = std::ldexp(std::nearbyint(std::ldexp(v, 133)), -133);  // bf16 subnormal spacing 2^-133
  } else {
    int e;
    const double m = std::frexp(v, &e);                 // v = m 2^e, 0.5 <= |m| < 1
    r = std::ldexp(std::nearbyint(std::ldexp(m, 8)), e - 8);  // 8 significant bits
  }
  return (uint16_t)(bits_of_f32((float)r) >> 16);       // r is a bf16 value (or 2^128 -> inf)
}

}  // namespace

extern "C" {

int gbwo_threads(void) { return n_threads(); }

// The E2M1 magnitude code (0..7) of each |v[i]|: round to the nearest of
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating at 6 -- the
// rounding step every quantizer above applies to a scaled value.
void gbwo_e2m1_rne(int64_t n, const double* v, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)e2m1_rne(std::fabs(v[i]));
}

// Decode [rows][K] packed codes + block scales (fmt 0 E8M0-B32, 1 E4M3-B16,
// 2 E5M3-B16) to doubles, times `tensor_scale` (1 for E8M0-B32).
void gbwo_dequantize(int64_t rows, int64_t K, int fmt, const uint8_t* codes, const uint8_t* scales,
                     double tensor_scale, double* out) {
  const int bs = block_of(fmt);
  parallel_for(rows, [&](int64_t r) {
    decode_row(codes + r * (K / 2), scales + r * (K / bs), fmt, K, out + r * K);
    if (tensor_scale != 1.0)
      for (int64_t k = 0; k < K; ++k) out[r * K + k] *= tensor_scale;
  });
}

// Y[m][n] = S_Ta S_Tw sum_k (e2m1 s)_a[m][k] (e2m1 s)_w[n][k]; rows of A are
// a_rows[r] (NULL: r) of the code/scale arrays.  The tensor scales (1 for
// E8M0-B32) multiply the finished sum once.  Returns the inexact count.
int64_t gbwo_block_gemm(int64_t M, int64_t N, int64_t K, int fmt, const uint8_t* a_codes,
                        const uint8_t* a_scales, const int64_t* a_rows, double a_ts, const uint8_t* w_codes,
                        const uint8_t* w_scales, double w_ts, double* y) {
  const int bs = block_of(fmt);
  std::vector<double> A((size_t)(M * K)), W((size_t)(N * K));
  parallel_for(M, [&](int64_t r) {
    const int64_t src = a_rows ? a_rows[r] : r;
    decode_row(a_codes + src * (K / 2), a_scales + src * (K / bs), fmt, K, A.data() + r * K);
  });
  parallel_for(N, [&](int64_t n) {
    decode_row(w_codes + n * (K / 2), w_scales + n * (K / bs), fmt, K, W.data() + n * K);
  });
  const int64_t bad = dot_all(M, N, K, A.data(), W.data(), y);
  const double ts = a_ts * w_ts;  // two fp32 values: their product is exact in double
  if (ts != 1.0)
    for (int64_t i = 0; i < M * N; ++i) y[i] *= ts;
  return bad;
}

// PRQuant augmented GEMM (E8M0-B32): one sum over K + tail per output,
// Y = sum_k deq(A)[m][k] deq(W)[n][k] + sum_j deq(A)[m][K-tail+j] deq(R)[n][j].
int64_t gbwo_residual_tail_gemm(int64_t M, int64_t N, int64_t K, int64_t tail, const uint8_t* a_codes,
                                const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                const uint8_t* r_codes, const uint8_t* r_scales, double* y) {
  const int64_t KA = K + tail;
  std::vector<double> A((size_t)(M * KA)), W((size_t)(N * KA));
  parallel_for(M, [&](int64_t m) {
    double* a = A.data() + m * KA;
    decode_row(a_codes + m * (K / 2), a_scales + m * (K / 32), F_E8M0_B32, K, a);
    for (int64_t j = 0; j < tail; ++j) a[K + j] = a[K - tail + j];  // the tail read a second time
  });
  parallel_for(N, [&](int64_t n) {
    double* w = W.data() + n * KA;
    decode_row(w_codes + n * (K / 2), w_scales + n * (K / 32), F_E8M0_B32, K, w);
    if (tail) decode_row(r_codes + n * (tail / 2), r_scales + n * (tail / 32), F_E8M0_B32, tail, w + K);
  });
  return dot_all(M, N, KA, A.data(), W.data(), y);
}

// Codebook weights: Y[m][n] = sum_k bf16(x[m][k]) fp16(C[n][k / group][idx[n][k]]).
int64_t gbwo_lut_gemm(int64_t M, int64_t N, int64_t K, int64_t group, const uint16_t* x_bf16,
                      const uint8_t* idx, const uint16_t* cent_f16, double* y) {
  std::vector<double> A((size_t)(M * K)), W((size_t)(N * K));
  const int64_t G = K / group;
  parallel_for(M, [&](int64_t m) {
    for (int64_t k = 0; k < K; ++k) A[m * K + k] = bf16(x_bf16[m * K + k]);
  });
  parallel_for(N, [&](int64_t n) {
    for (int64_t k = 0; k < K; ++k)
      W[n * K + k] = fp16(cent_f16[(n * G + k / group) * 16 + nibble(idx + n * (K / 2), k)]);
  });
  return dot_all(M, N, K, A.data(), W.data(), y);
}

// MXCode PreScale decode to the E2M1 code stream: element 4j+i of row n is
// nibble i of key CB[n/qb][(4j)/qb][idx[n][j]].  codes [N][K/2].
void gbwo_vq_decode_codes(int64_t N, int64_t K, int64_t qb, const uint8_t* idx, const uint16_t* cb,
                          uint8_t* codes) {
  const int64_t KV = K / 4, QK = K / qb;
  parallel_for(N, [&](int64_t n) {
    uint8_t* out = codes + n * (K / 2);
    for (int64_t j = 0; j < KV; ++j) {
      const uint16_t key = cb[((n / qb) * QK + (4 * j) / qb) * 256 + idx[n * KV + j]];
      out[2 * j] = (uint8_t)(key & 0xFFu);          // elements 4j, 4j+1
      out[2 * j + 1] = (uint8_t)(key >> 8);         // elements 4j+2, 4j+3
    }
  });
}

// E8M0-B32 encoder, per block of 32 along K: amax (exact); scale code
// sc = max(0, E(amax) - 2) with E the fp32 biased exponent field; element
// code = sign(x) | RNE_sat(|x| 2^(127 - sc)) onto the E2M1 magnitudes.
void gbwo_quantize_e8m0_b32(int64_t rows, int64_t K, const float* x, uint8_t* codes, uint8_t* scales) {
  parallel_for(rows, [&](int64_t r) {
    const float* xr = x + r * K;
    for (int64_t b = 0; b < K / 32; ++b) {
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = std::fmax(amax, std::fabs(xr[32 * b + i]));
      const int E = (int)((bits_of_f32(amax) >> 23) & 0xFFu);
      const int sc = E > 2 ? E - 2 : 0;
      scales[r * (K / 32) + b] = (uint8_t)sc;
      for (int i = 0; i < 32; i += 2) {
        unsigned c[2];
        for (int h = 0; h < 2; ++h) {
          const float v = xr[32 * b + i + h];
          const unsigned mag = e2m1_rne(std::ldexp(std::fabs((double)v), 127 - sc));
          c[h] = mag | (std::signbit(v) ? 8u : 0u);
        }
        codes[r * (K / 2) + (32 * b + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  });
}

// E4M3-B16 (fmt 1) / E5M3-B16 (fmt 2) encoder with an FP32 tensor scale.
// tensor_amax < 0: A = max |x| over the tensor.  Every step an fp32
// operation, in order: S_T = A / (6 * max scale) (1 if A = 0); d = 6 S_T;
// s = amax_blk / d; sc = RNE_sat(s) onto the scale grid; sd = decode(sc);
// den = sd S_T; code = sign(x) | RNE_sat(|x| / den) (signed zeros if den = 0).
// Returns S_T.
float gbwo_quantize_b16(int fmt, int64_t rows, int64_t K, const float* x, double tensor_amax, uint8_t* codes,
                        uint8_t* scales) {
  float A = 0.0f;
  if (tensor_amax < 0.0) {
    for (int64_t i = 0; i < rows * K; ++i) A = std::fmax(A, std::fabs(x[i]));
  } else {
    A = (float)tensor_amax;
  }
  const float top = fmt == F_E4M3_B16 ? 2688.0f : 688128.0f;  // 6 * 448, 6 * 114688
  const float S_T = A == 0.0f ? 1.0f : A / top;
  const float d = 6.0f * S_T;
  const double* grid = fmt == F_E4M3_B16 ? kGrids.e4 : kGrids.e5;
  const unsigned gn = fmt == F_E4M3_B16 ? 127u : 255u;
  parallel_for(rows, [&](int64_t r) {
    const float* xr = x + r * K;
    for (int64_t b = 0; b < K / 16; ++b) {
      float amax = 0.0f;
      for (int i = 0; i < 16; ++i) amax = std::fmax(amax, std::fabs(xr[16 * b + i]));
      const float s = amax / d;
      const unsigned sc = round_to_grid((double)s, grid, gn);
      scales[r * (K / 16) + b] = (uint8_t)sc;
      const float sd = (float)(fmt == F_E4M3_B16 ? e4m3(sc) : ue5m3(sc));
      const float den = sd * S_T;
      for (int i = 0; i < 16; i += 2) {
        unsigned c[2];
        for (int h = 0; h < 2; ++h) {
          const float v = xr[16 * b + i + h];
          const unsigned mag = den > 0.0f ? e2m1_rne((double)(std::fabs(v) / den)) : 0u;
          c[h] = mag | (std::signbit(v) ? 8u : 0u);
        }
        codes[r * (K / 2) + (16 * b + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  });
  return S_T;
}

// h = bf16(silu(g) u), silu(z) = z / (1 + e^-z), in double, rounded once.
void gbwo_swiglu_bf16(int64_t n, const double* g, const double* u, uint16_t* h) {
  parallel_for(n, [&](int64_t i) {
    const double z = g[i];
    const double s = z > -700.0 ? z / (1.0 + std::exp(-z)) : z * std::exp(z) / (1.0 + std::exp(z));
    h[i] = bf16_rne(s * u[i]);
  });
}

// Routed combine: y[r][n] = sum_j w[t][j] o[pair_pos[t][j]][n] over the
// slots j of token t = tokens[r], in slot order; o rows are indexed through
// o_row[p] (the row of pair p in o, -1 if absent).
void gbwo_combine(int64_t R, int64_t topk, int64_t H, const int64_t* tokens, const int32_t* pair_pos,
                  const double* w, const int64_t* o_row, const double* o, double* y) {
  parallel_for(R * H, [&](int64_t i) {
    const int64_t r = i / H, n = i % H, t = tokens[r];
    Sum s;
    for (int64_t j = 0; j < topk; ++j) {
      const int64_t p = pair_pos[t * topk + j];
      s.add(w[t * topk + j] * o[o_row[p] * H + n]);
    }
    y[i] = s.value();
  });
}

// Top-k routing: per token the k largest logits (ties to the lower expert
// id; -0 ties +0; NaN after every number), weights exp(l_j - l_max) / sum
// over the k chosen in double; pairs listed by (expert, token): offsets
// [E+1], pair_token [T k], pair_pos [T][k].
void gbwo_route(int64_t T, int64_t E, int64_t k, const float* logits, int32_t* ids, double* w, int32_t* offsets,
                int32_t* pair_token, int32_t* pair_pos) {
  parallel_for(T, [&](int64_t t) {
    const float* l = logits + t * E;
    std::vector<int32_t> order((size_t)E);
    for (int64_t e = 0; e < E; ++e) order[e] = (int32_t)e;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      const float la = l[a], lb = l[b];
      return !std::isnan(la) && (std::isnan(lb) || la > lb);
    });
    double den = 0.0;
    const double lmax = l[order[0]];
    for (int64_t j = 0; j < k; ++j) {
      ids[t * k + j] = order[j];
      w[t * k + j] = std::exp((double)l[order[j]] - lmax);
      den += w[t * k + j];
    }
    for (int64_t j = 0; j < k; ++j) w[t * k + j] /= den;
  });
  std::vector<int64_t> count((size_t)E, 0);
  for (int64_t i = 0; i < T * k; ++i) ++count[ids[i]];
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + (int32_t)count[e];
  std::vector<int64_t> fill(offsets, offsets + E);
  for (int64_t t = 0; t < T; ++t)      // tokens ascending within each expert
    for (int64_t j = 0; j < k; ++j) {
      const int64_t p = fill[ids[t * k + j]]++;
      pair_token[p] = (int32_t)t;
      pair_pos[t * k + j] = (int32_t)p;
    }
}

}  // extern "C"
