// Host plumbing shared by every entry point: status strings, the per-thread
// error message, the gfx950 device check, launch checks, workspace sizes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace gbw {

static thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_is_gfx950[kMaxDevices];
int g_cus[kMaxDevices];
}  // namespace

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(GBW_E_UNSUPPORTED, "no HIP device available");
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      g_is_gfx950[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0;
      g_cus[dev] = p.multiProcessorCount;
    }
  });
  if (!g_is_gfx950[dev]) return fail(GBW_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return GBW_OK;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  return g_cus[dev] > 0 ? g_cus[dev] : 256;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GBW_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return GBW_OK;
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

// Sum split-K partials [splits][mn] in split order (a fixed order, so the
// result is bitwise repeatable), four outputs per thread.
__global__ void k_splitk_reduce(const float* __restrict__ part, int splits, int64_t mn, float* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= mn) return;
  if (i + 4 <= mn) {
    v4f acc = *reinterpret_cast<const v4f*>(part + i);
    for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const v4f*>(part + (int64_t)s * mn + i);
    *reinterpret_cast<v4f*>(y + i) = acc;
  } else {
    for (int64_t j = i; j < mn; ++j) {
      float a = part[j];
      for (int s = 1; s < splits; ++s) a += part[(int64_t)s * mn + j];
      y[j] = a;
    }
  }
}

int launch_splitk_reduce(const float* part, int splits, int64_t mn, float* y, hipStream_t st) {
  if (mn <= 0) return GBW_OK;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)cdiv(cdiv(mn, 4), 256)), dim3(256), 0, st, part, splits, mn, y);
  return check_launch("splitk_reduce");
}

int launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return GBW_OK;
  int64_t blocks = cdiv(n, 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return check_launch("fill_zero");
}

}  // namespace gbw

// workspace sizes of the individual ops live next to their kernels
namespace gbw {
size_t ws_quantize(int64_t rows, int64_t K, int32_t fmt);
size_t ws_moe_route(int64_t T, int64_t E);
size_t ws_moe_gemm(int64_t P, int64_t N, int64_t f32);
size_t ws_lut_gemm(int64_t M, int64_t N, int64_t K);
size_t ws_mx_gemm(int64_t M, int64_t N, int64_t Ktot);
}  // namespace gbw

extern "C" {

const char* gbw_status_string(int status) {
  switch (status) {
    case GBW_OK: return "ok";
    case GBW_E_ARG: return "invalid argument";
    case GBW_E_SHAPE: return "invalid shape";
    case GBW_E_ALIGN: return "misaligned pointer";
    case GBW_E_UNSUPPORTED: return "unsupported";
    case GBW_E_WORKSPACE: return "workspace too small";
    case GBW_E_LAUNCH: return "launch failed";
    default: return "unknown status";
  }
}

const char* gbw_last_error(void) { return gbw::g_err; }

size_t gbw_workspace_size(int32_t op, int64_t d0, int64_t d1, int64_t d2, int32_t fmt) {
  switch (op) {
    case GBW_OP_QUANTIZE: return gbw::ws_quantize(d0, d1, fmt);
    case GBW_OP_MX_GEMM: return gbw::ws_mx_gemm(d0, d1, d2);
    case GBW_OP_LUT_GEMM: return gbw::ws_lut_gemm(d0, d1, d2);
    case GBW_OP_MOE_ROUTE: return gbw::ws_moe_route(d0, d1);
    case GBW_OP_MOE_GEMM: return gbw::ws_moe_gemm(d0, d1, d2);
    default: return 0;
  }
}

}  // extern "C"
