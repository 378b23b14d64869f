// Measurement aid, not part of the library's API: the time a plain streaming
// read of a buffer takes on this device, and the time of an empty kernel, so
// a memory-bound kernel's time can be set beside what merely reading its
// bytes costs when launched the same way (one kernel per call, cold caches).
//
// k_stream_read: 1024 workgroups of 256 threads (or fewer for small
// buffers); each thread loads 4 x 16 bytes per round, grid-stride, folds
// them with XOR and each workgroup writes one word, so no load is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256, kUnroll = 4;

__global__ __launch_bounds__(kThreads) void k_stream_read(const v4u* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += step) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kThreads;
      v[u] = i < n16 ? p[i] : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kThreads; ++i) r ^= s[i];
    out[blockIdx.x] = r;
  }
}

__global__ void k_empty(uint32_t* out) {
  if (threadIdx.x == 0) out[0] = 0;
}

}  // namespace

// Reads `bytes` (a multiple of 16) at the 16-byte aligned device address p;
// `out` holds at least 1024 words.  Returns 0, or 1 for bad arguments, 2 if
// the launch failed.
extern "C" int gbw_floor_stream_read(const void* p, int64_t bytes, uint32_t* out, void* stream) {
  if (!p || !out || bytes <= 0 || (bytes & 15) || ((uintptr_t)p & 15)) return 1;
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  blocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const v4u*)p, n16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// One single-wave kernel that writes one word of `out`.
extern "C" int gbw_floor_empty(uint32_t* out, void* stream) {
  if (!out) return 1;
  hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
