// CPU check of moe_route: bounds (ASan) and results against a sort-based reference.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdarg.h>
#include <random>
#include <numeric>
#include "gbw.h"
thread_local emu_idx threadIdx, blockIdx, blockDim, gridDim;
thread_local std::barrier<>* emu_bar;
thread_local emu_wave emu_w;
std::mutex emu_atomic_mu;
namespace gbw {
size_t ws_moe_route(int64_t T, int64_t E);
int fail(int status, const char* fmt, ...) {
  va_list ap; va_start(ap, fmt); fprintf(stderr, "fail: "); vfprintf(stderr, fmt, ap); fprintf(stderr, "\n"); va_end(ap);
  return status;
}
int check_device() { return 0; }
int check_launch(const char*) { return 0; }
int device_cu_count() { return 256; }
}
int main(int argc, char** argv) {
  const int64_t T = atoll(argv[1]); const int E = atoi(argv[2]), K = atoi(argv[3]);
  const std::string mode = argc > 4 ? argv[4] : "";  // "ties": values 0, 1, 2; "special": +-0, +-1, +-inf, NaN
  std::mt19937 g(3); std::normal_distribution<float> nd;
  const float sp[8] = {0.f, -0.f, 1.f, -1.f, INFINITY, -INFINITY, NAN, -NAN};
  float* l = (float*)malloc(T * E * 4);
  for (int64_t i = 0; i < T * E; ++i) l[i] = mode == "ties" ? (float)(g() % 3) : mode == "special" ? sp[g() % 8] : nd(g);
  int32_t* ids = (int32_t*)malloc(T * K * 4); float* w = (float*)malloc(T * K * 4);
  int32_t* off = (int32_t*)malloc((E + 1) * 4); int32_t* pt = (int32_t*)malloc(T * K * 4); int32_t* pp = (int32_t*)malloc(T * K * 4);
  size_t wsb = gbw::ws_moe_route(T, E); void* ws = malloc(wsb);
  int st = moe_route(l, T, E, K, ids, w, off, pt, pp, ws, wsb, nullptr);
  long bad = 0;
  for (int64_t t = 0; t < T; ++t) {
    std::vector<int> o(E); std::iota(o.begin(), o.end(), 0);
    // descending, NaN after every number, equal values (and the two zeros) in id order
    std::stable_sort(o.begin(), o.end(), [&](int a, int b) {
      const float x = l[t * E + a], y = l[t * E + b];
      if (std::isnan(x)) return false;
      if (std::isnan(y)) return true;
      return x > y;
    });
    for (int j = 0; j < K; ++j) bad += ids[t * K + j] != o[j];
  }
  // pair list: (expert, token) order; offsets = exclusive prefix of the counts
  long badp = 0;
  std::vector<long> cnt(E + 1, 0);
  for (int64_t i = 0; i < T * K; ++i) cnt[ids[i] + 1]++;
  for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
  for (int e = 0; e <= E; ++e) badp += off[e] != cnt[e];
  std::vector<long> fill(cnt.begin(), cnt.end() - 1);
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const long p = fill[ids[t * K + j]]++;  // tokens ascend within an expert
      badp += pp[t * K + j] != p;
      badp += pt[p] != t;
    }
  printf("route T=%lld E=%d K=%d status %d mismatched ids %ld mismatched pairs %ld off[E]=%d\n", (long long)T, E, K,
         st, bad, badp, off[E]);
  // the allocation-free entry point (scratch in the library's fixed array):
  // the same outputs, in bounds of that array
  int32_t* ids2 = (int32_t*)malloc(T * K * 4); float* w2 = (float*)malloc(T * K * 4);
  int32_t* off2 = (int32_t*)malloc((E + 1) * 4); int32_t* pt2 = (int32_t*)malloc(T * K * 4);
  int32_t* pp2 = (int32_t*)malloc(T * K * 4);
  const int st2 = moe_route_noalloc(l, T, E, K, ids2, w2, off2, pt2, pp2, nullptr);
  long diff = 0;
  if (st2 == 0) {
    diff += memcmp(ids, ids2, T * K * 4) != 0;
    diff += memcmp(off, off2, (E + 1) * 4) != 0;
    diff += memcmp(pt, pt2, T * K * 4) != 0;
    diff += memcmp(pp, pp2, T * K * 4) != 0;
  }
  printf("noalloc status %d differing outputs %ld\n", st2, diff);
  return 0;
}
