// CPU bounds check of lut_gemm (every buffer an exact-size heap block): the
// call with the full workspace twice (the arrival counters must be back at
// zero after each call), then with a workspace one byte short (the no-split
// path).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdarg.h>
#include <random>
#include "gbw.h"
thread_local emu_idx threadIdx, blockIdx, blockDim, gridDim;
thread_local std::barrier<>* emu_bar;
thread_local emu_wave emu_w;
std::mutex emu_atomic_mu;
namespace gbw {
size_t ws_lut_gemm(int64_t M, int64_t N, int64_t K);
int fail(int status, const char* fmt, ...) {
  va_list ap; va_start(ap, fmt); fprintf(stderr, "fail: "); vfprintf(stderr, fmt, ap); fprintf(stderr, "\n"); va_end(ap);
  return status;
}
int check_device() { return 0; }
int check_launch(const char*) { return 0; }
int device_cu_count() { return 256; }
int launch_fill_zero(float* p, int64_t n, hipStream_t) { memset(p, 0, n * 4); return 0; }
int launch_splitk_reduce(const float* part, int splits, int64_t mn, float* y, hipStream_t) {
  for (int64_t i = 0; i < mn; ++i) { float s = 0; for (int k = 0; k < splits; ++k) s += part[k * mn + i]; y[i] = s; }
  return 0;
}
}
int main(int argc, char** argv) {
  const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
  const int group = atoi(argv[4]);
  std::mt19937 g(7);
  auto mk = [&](size_t bytes) { uint8_t* p = (uint8_t*)malloc(bytes ? bytes : 1); for (size_t i = 0; i < bytes; ++i) p[i] = (uint8_t)g(); return p; };
  uint16_t* x = (uint16_t*)mk(M * K * 2);
  uint8_t* idx = mk(N * K / 2);
  uint16_t* cent = (uint16_t*)mk(N * (K / group) * 16 * 2);
  float* y = (float*)mk(M * N * 4);
  const size_t wsb = gbw::ws_lut_gemm(M, N, K);
  uint8_t* ws = wsb ? (uint8_t*)calloc(wsb, 1) : nullptr;
  for (int rep = 0; rep < 2; ++rep) {
    int st = lut_gemm(M, N, K, group, x, idx, cent, y, 0, ws, wsb, nullptr);
    size_t nonzero = 0;
    // the counters sit at the front of the workspace, one dword per tile
    const size_t tiles = (size_t)((N + 63) / 64) * ((M + 63) / 64);
    for (size_t i = 0; wsb && i < tiles; ++i) nonzero += ((uint32_t*)ws)[i] != 0;
    printf("lut M=%lld N=%lld K=%lld g=%d ws=%zu status %d counters left %zu\n", (long long)M, (long long)N,
           (long long)K, group, wsb, st, nonzero);
  }
  if (wsb) {
    uint8_t* shortws = (uint8_t*)calloc(wsb - 1, 1);
    int st = lut_gemm(M, N, K, group, x, idx, cent, y, 0, shortws, wsb - 1, nullptr);
    printf("short workspace status %d\n", st);
    free(shortws);
  }
  return 0;
}
