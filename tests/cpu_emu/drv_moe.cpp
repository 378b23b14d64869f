// CPU emulation driver for moe_grouped_gemm (test infrastructure): every
// buffer is its own exact-size heap block, so AddressSanitizer reports any
// out-of-bounds access; usage: drv_moe T H I E topk fmt [h_bf16 [h_tail [qblock]]].
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdarg.h>
#include <random>
#include <algorithm>
#include "gbw.h"
thread_local emu_idx threadIdx, blockIdx, blockDim, gridDim;
thread_local std::barrier<>* emu_bar;
thread_local emu_wave emu_w;
std::mutex emu_atomic_mu;
namespace gbw {
size_t ws_moe_gemm(int64_t P, int64_t N, int64_t f32);
int fail(int status, const char* fmt, ...) {
  va_list ap; va_start(ap, fmt); fprintf(stderr, "fail: "); vfprintf(stderr, fmt, ap); fprintf(stderr, "\n"); va_end(ap);
  return status;
}
int check_device() { return 0; }
int check_launch(const char*) { return 0; }
int device_cu_count() { return 256; }
int launch_fill_zero(float* p, int64_t n, hipStream_t) { memset(p, 0, n * 4); return 0; }
int launch_splitk_reduce(const float*, int, int64_t, float*, hipStream_t) { return 0; }
}
template <class T> T* buf(size_t n, std::mt19937& g) {
  T* p = (T*)malloc(n * sizeof(T) ? n * sizeof(T) : 1);
  for (size_t i = 0; i < n * sizeof(T); ++i) ((uint8_t*)p)[i] = (uint8_t)g();
  return p;
}
int main(int argc, char** argv) {
  const int T = atoi(argv[1]), H = atoi(argv[2]), I = atoi(argv[3]), E = atoi(argv[4]), k = atoi(argv[5]);
  const int fmt = atoi(argv[6]);  // gbw.h GBW_FMT_* (0 .. 11)
  const int qb = argc > 9 ? atoi(argv[9]) : 64;   // VQ QBlock edge
  const int tail = argc > 8 ? atoi(argv[8]) : 0;  // E8M0 h: PRQuant tail copy, down over I + tail
  const int Ih = I + tail;                        // h code columns
  const int P = T * k;
  std::mt19937 g(1234);
  // routing: k distinct experts per token
  std::vector<std::vector<int>> ch(T);
  for (int t = 0; t < T; ++t) {
    std::vector<int> ex(E); for (int e = 0; e < E; ++e) ex[e] = e;
    std::shuffle(ex.begin(), ex.end(), g);
    ch[t].assign(ex.begin(), ex.begin() + k);
  }
  std::vector<std::pair<int,int>> pairs;  // (expert, token) with slot
  std::vector<int> slot_of;
  for (int t = 0; t < T; ++t) for (int j = 0; j < k; ++j) pairs.push_back({ch[t][j], t * k + j});
  std::sort(pairs.begin(), pairs.end());
  int32_t* off = (int32_t*)malloc((E + 1) * 4);
  int32_t* ptok = (int32_t*)malloc(P * 4);
  int32_t* ppos = (int32_t*)malloc(P * 4);
  float* tw = (float*)malloc(P * 4);
  for (int e = 0; e <= E; ++e) off[e] = 0;
  for (auto& q : pairs) off[q.first + 1]++;
  for (int e = 0; e < E; ++e) off[e + 1] += off[e];
  for (int p = 0; p < P; ++p) { ptok[p] = pairs[p].second / k; ppos[pairs[p].second] = p; }
  for (int i = 0; i < P; ++i) tw[i] = 1.0f / k;
  const bool e4 = fmt == 1 || fmt == 3 || fmt >= 6;  // tensor-scaled formats
  const int afmt = (fmt == 3 || fmt >= 9) ? 3 : e4 ? 1 : 0;  // activation format
  const int sdiv = e4 ? 16 : 32;
  const int lay = fmt == 4 ? 1 : fmt == 5 ? 2 : fmt >= 6 ? (fmt - 6) % 3 : 0;  // VQ scales: block / QBlock / table
  // gate/up
  gbw_weight wg{}, wd{};
  wg.fmt = fmt; wg.n_experts = E; wg.N = 2 * I; wg.K = H;
  wd.fmt = fmt; wd.n_experts = E; wd.N = H; wd.K = Ih;
  const bool vq = fmt == 2 || fmt == 4 || fmt == 5 || fmt >= 6;
  for (gbw_weight* w : {&wg, &wd}) {
    const size_t NK = (size_t)E * w->N * w->K;
    w->codes = vq ? buf<uint8_t>(NK / 4, g) : buf<uint8_t>(NK / 2, g);
    const size_t nsc = lay == 1 ? (size_t)E * (w->N / qb) * (w->K / qb) : lay == 2 ? NK / (8 * sdiv) : NK / sdiv;
    w->scales = buf<uint8_t>(nsc, g);
    if (vq) w->codebook = buf<uint16_t>((size_t)E * (w->N / qb) * (w->K / qb) * 256, g);
    if (vq) w->qblock = qb;
    if (lay == 2) w->scale_codebook = buf<uint8_t>((size_t)E * 2048, g);
    if (e4) { float* ts = (float*)malloc(E * 2 * 4); for (int i = 0; i < 2 * E; ++i) ts[i] = 1.f; w->tensor_scale = ts; w->ts_per_expert = w == &wg ? 2 : 1; }
  }
  float* ats = (float*)malloc(4); *ats = 1.f;
  gbw_act ax{}; ax.fmt = afmt; ax.rows = T; ax.K = H;
  ax.codes = buf<uint8_t>((size_t)T * H / 2, g); ax.scales = buf<uint8_t>((size_t)T * H / sdiv, g);
  ax.tensor_scale = e4 ? ats : nullptr;
  gbw_moe_out o{};
  uint8_t* hc = buf<uint8_t>((size_t)P * Ih / 2, g);
  uint8_t* hs = buf<uint8_t>((size_t)P * Ih / 32, g);
  o.h_tail = tail;
  uint16_t* hb = buf<uint16_t>((size_t)P * I, g);
  if (e4) o.h_bf16 = hb; else { o.h_codes = hc; o.h_scales = hs; o.h_bf16 = (argc > 7) ? hb : nullptr; }
  int st = moe_grouped_gemm(0, T, k, off, ptok, ppos, tw, &ax, &wg, &o, 0, nullptr, 0, nullptr);
  printf("gateup status %d\n", st);
  // down: activation = h
  gbw_act ah{}; ah.fmt = afmt; ah.rows = P; ah.K = Ih;
  uint8_t* hcodes = e4 ? buf<uint8_t>((size_t)P * I / 2, g) : hc;
  uint8_t* hsc = e4 ? buf<uint8_t>((size_t)P * I / 16, g) : hs;
  ah.codes = hcodes; ah.scales = hsc; ah.tensor_scale = e4 ? ats : nullptr;
  float* y = (float*)malloc((size_t)T * H * 4);
  gbw_moe_out od{}; od.y = y;
  for (int mode = 0; mode < 3; ++mode) {
    const int f32 = mode == 1;
    size_t wsb = gbw::ws_moe_gemm(P, H, f32);
    void* ws = mode == 2 ? nullptr : malloc(wsb);
    st = moe_grouped_gemm(1, T, k, off, ptok, ppos, tw, &ah, &wd, &od, f32 ? GBW_FP32_COMBINE : 0, ws, mode == 2 ? 0 : wsb, nullptr);
    printf("down mode %d status %d\n", mode, st);
    free(ws);
  }
  return 0;
}
