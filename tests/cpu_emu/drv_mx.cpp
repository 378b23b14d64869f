// CPU bounds check of mx_gemm / residual_tail_gemm (exact-size buffers under ASan).
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
size_t ws_mx_gemm(int64_t M, int64_t N, int64_t Ktot);
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
  const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]), tail = atoll(argv[4]);
  std::mt19937 g(5);
  auto mk = [&](size_t bytes) { uint8_t* p = (uint8_t*)malloc(bytes ? bytes : 1); for (size_t i = 0; i < bytes; ++i) p[i] = (uint8_t)(g() & 0x77); return p; };
  gbw_act a{}; a.fmt = GBW_FMT_E8M0_B32; a.rows = M; a.K = K; a.codes = mk(M * K / 2); a.scales = mk(M * K / 32);
  gbw_weight w{}; w.fmt = GBW_FMT_E8M0_B32; w.n_experts = 1; w.N = N; w.K = K; w.codes = mk(N * K / 2); w.scales = mk(N * K / 32);
  gbw_weight r{}; r.fmt = GBW_FMT_E8M0_B32; r.n_experts = 1; r.N = N; r.K = tail; r.codes = mk(N * tail / 2 + (tail ? 0 : 16)); r.scales = mk(N * tail / 32 + 1);
  float* y = (float*)malloc(M * N * 4);
  // no workspace, then one zeroed workspace for two calls in a row: the
  // arrival counters at its front (64 KiB) must be back at zero after each
  for (int wsmode = 0; wsmode < 2; ++wsmode) {
    size_t wsb = wsmode ? gbw::ws_mx_gemm(M, N, K + tail) : 0;
    uint8_t* ws = wsb ? (uint8_t*)calloc(wsb, 1) : nullptr;
    for (int rep = 0; rep < (wsmode ? 2 : 1); ++rep) {
      int st = tail ? residual_tail_gemm(M, &a, &w, &r, tail, y, 0, ws, wsb, nullptr) : mx_gemm(M, &a, &w, y, 0, ws, wsb, nullptr);
      size_t left = 0;
      for (size_t i = 0; wsb && i < 65536 / 4; ++i) left += ((uint32_t*)ws)[i] != 0;
      printf("mx M=%lld N=%lld K=%lld tail=%lld ws=%zu status %d counters left %zu\n", (long long)M, (long long)N,
             (long long)K, (long long)tail, wsb, st, left);
    }
    free(ws);
  }
  return 0;
}
