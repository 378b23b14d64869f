// Measurement aid, not part of the library's API: the rate at which this
// device retires one MFMA shape when nothing else runs (operands in
// registers, no memory traffic in the loop), so a kernel's MFMA rate can be
// set beside what the matrix cores sustain under load, clock included.
//
// k_mfma_rate<KIND>: every wave keeps eight independent accumulators and
// issues `iters` rounds of eight MFMAs; the operands are built from the lane
// index (any byte is a valid E2M1 pair; fp16 operands are small, so no sum
// overflows), and each lane writes one float of its accumulators, so no
// MFMA is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// KIND: 0 = FP4 32x32x64 (scaled), 1 = FP4 16x16x128 (scaled),
//       2 = fp16 32x32x16,        3 = fp16 16x16x32
template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_rate(int iters, float* __restrict__ out) {
  constexpr bool big = KIND == 0 || KIND == 2;
  typedef typename std::conditional<big, v16f, v4f>::type acc_t;
  const int lane = threadIdx.x & 63;
  acc_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = acc_t{};
  v8i a8 = v8i{}, b8 = v8i{};
  v8h ah, bh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a8[i] = (int)(0x9E3779B9u * (uint32_t)(lane + 64 * i + 1));
    b8[i] = (int)(0x85EBCA6Bu * (uint32_t)(lane + 64 * i + 7));
    ah[i] = (_Float16)(0.0009765625f * (float)((lane + i) & 7));
    bh[i] = (_Float16)(0.0009765625f * (float)((lane + 3 * i) & 7));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (KIND == 0)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 4, 4, 0, 127, 0, 127);
      else if constexpr (KIND == 1)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[c], 4, 4, 0, 127, 0, 127);
      else if constexpr (KIND == 2)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads of shape `kind` (0..3, above),
// each wave running `iters` rounds of eight MFMAs; `out` holds blocks * 256
// floats.  Flops per wave and round: 8 * 2 * (32*32*64, 16*16*128,
// 32*32*16, 16*16*32).  Returns 0, 1 for bad arguments, 2 if the launch
// failed.
extern "C" int gbw_floor_mfma_rate(int kind, int blocks, int iters, float* out, void* stream) {
  if (!out || blocks < 1 || iters < 1 || kind < 0 || kind > 3) return 1;
  const hipStream_t st = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_mfma_rate<0>, dim3(blocks), dim3(256), 0, st, iters, out); break;
    case 1: hipLaunchKernelGGL(k_mfma_rate<1>, dim3(blocks), dim3(256), 0, st, iters, out); break;
    case 2: hipLaunchKernelGGL(k_mfma_rate<2>, dim3(blocks), dim3(256), 0, st, iters, out); break;
    default: hipLaunchKernelGGL(k_mfma_rate<3>, dim3(blocks), dim3(256), 0, st, iters, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
