// Shared device codecs and host plumbing for the gfx950 kernels.
//
// Device codecs follow the block formats of "MXCode: MX-Native Codebook
// Quantization", Table 1 (E2M1 elements, E8M0 and E4M3 block scales) and the
// OCP MX element type that "PRQuant: Permutation Residual Quantization for
// Low-Overhead Inference" cites for MXFP4 (§1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gbw.h"

namespace gbw {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// E2M1
// ---------------------------------------------------------------------------

// Round a non-negative magnitude (already divided by the block scale) onto
// the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest value, ties to the even
// code, saturating at 6.  Each comparison counts one grid step crossed; the
// closed/open choice at each midpoint encodes ties-to-even.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
         (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
         (uint32_t)(v > 5.0f);
}

// E2M1 code -> float from its bit fields (1 sign, 2 exponent with bias 1, 1 mantissa).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = (e == 0) ? 0.5f * (float)m : __uint_as_float((uint32_t)(e + 126) << 23) * (1.0f + 0.5f * (float)m);
  return (c & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// E8M0 and E4M3 block scales
// ---------------------------------------------------------------------------

// 2^(127 - sc) as an fp32, sc in [0, 252]: the reciprocal of an E8M0 scale.
__device__ __forceinline__ float e8m0_inv(uint32_t sc) { return __uint_as_float((254u - sc) << 23); }

// E8M0 scale value 2^(sc - 127), sc in [1, 254]; sc = 0 gives 2^-127 (subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t sc) {
  return sc == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(sc << 23);
}

// OCP MX shared-scale rule for E2M1 elements: floor(log2 amax) - 2, biased,
// clamped at 0 (zero and subnormal blocks get code 0).
__device__ __forceinline__ uint32_t e8m0_scale_code(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(E > 2 ? E - 2 : 0);
}

// Non-negative fp32 -> E4M3 ("fn") code, round to nearest even, saturating
// at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(s);
  const int e = (int)((b >> 23) & 0xFFu) - 127;
  if (e < -6) {
    // subnormal range: multiples of 2^-9; an exact power-of-two product, then RNE
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  const uint32_t m = b & 0x7FFFFFu;
  const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;  // 0..8, 8 carries into the exponent
  return ((uint32_t)(e + 7) << 3) + r;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Non-negative fp32 -> UE5M3 code (5 exponent bits with bias 15, 3 mantissa
// bits, no sign), round to nearest even, saturating at 114688 (0xFE; the
// all-ones code is reserved).
__device__ __forceinline__ uint32_t ue5m3_rne_sat(float s) {
  if (!(s < 114688.0f)) return 0xFEu;
  const uint32_t b = __float_as_uint(s);
  const int e = (int)((b >> 23) & 0xFFu) - 127;
  if (e < -14) {
    // subnormal range: multiples of 2^-17; an exact power-of-two product, then RNE
    return (uint32_t)__builtin_rintf(s * 131072.0f);
  }
  const uint32_t m = b & 0x7FFFFFu;
  const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;  // 0..8, 8 carries into the exponent
  return ((uint32_t)(e + 15) << 3) + r;
}

__device__ __forceinline__ float ue5m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0x1Fu, m = c & 7u;
  if (e == 0) return (float)m * 7.62939453125e-06f;  // m * 2^-17
  return __uint_as_float(((e + 112u) << 23) | (m << 20));
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (a in the low half), round to nearest even, in one
// v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// silu(g) * u = g / (1 + e^-g) * u from the hardware exp2 and reciprocal
// (a few fp32 ulp; the result is rounded to bf16 next)
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// eight bf16 (four dwords, element 2i in the low half of dword i) -> eight
// E2M1 codes (element 2i in the low nibble of byte i) of x / scale, round to
// nearest even, saturating at 6, sign kept (v_cvt_scalef32_pk_fp4_f32 divides
// by `scale`; every scale here is a power of two, so the quotient is exact).
// The bf16 are widened to fp32 first (exact): the bf16-source form of the
// instruction is not used.
__device__ __forceinline__ uint32_t e2m1x8_from_bf16(v4i w, float scale) {
#define GBW_CVT_PAIR(c, d) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, __uint_as_float((uint32_t)w[d] << 16), \
                                           __uint_as_float((uint32_t)w[d] & 0xFFFF0000u), scale, d)
  uint32_t c = 0;
  c = GBW_CVT_PAIR(c, 0);
  c = GBW_CVT_PAIR(c, 1);
  c = GBW_CVT_PAIR(c, 2);
  c = GBW_CVT_PAIR(c, 3);
#undef GBW_CVT_PAIR
  return c;
}

// largest |x| of eight bf16 (as above), as the bf16 magnitude bits
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(v4i w) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  const v2u16 a = __builtin_bit_cast(v2u16, (uint32_t)w[0] & 0x7FFF7FFFu);
  const v2u16 b = __builtin_bit_cast(v2u16, (uint32_t)w[1] & 0x7FFF7FFFu);
  const v2u16 c = __builtin_bit_cast(v2u16, (uint32_t)w[2] & 0x7FFF7FFFu);
  const v2u16 d = __builtin_bit_cast(v2u16, (uint32_t)w[3] & 0x7FFF7FFFu);
  const v2u16 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// max over the four lanes of a quad (lanes 4k..4k+3), by two DPP quad permutes
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));  // lanes ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));  // lanes ^ 2
  return v;
}

// ---------------------------------------------------------------------------
// misc
// ---------------------------------------------------------------------------

__device__ __forceinline__ v4i load16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

// Direct global -> LDS load of 16 bytes per lane (lane l's bytes land at
// lds + 16 l; `lds` must be the same in every lane of the wave): a weight
// segment is copied into LDS one contiguous kilobyte of a row per
// instruction, with no registers in between.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
// `stream`: the non-temporal cache policy (bit 1 of the instruction's cache
// policy field), for data read once per call such as a decode GEMV's weights.
template <bool stream = false>
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 16, 0, stream ? 2 : 0);
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K GEMM workspaces (mx_gemm, residual_tail_gemm, lut_gemm) start with
// this many bytes of per-tile arrival counters (one uint32 per output tile,
// at most kWsCounterBytes / 4 tiles); the partial tiles follow.  The counters
// are zero before a workspace's first use and every call leaves them zero,
// so one zeroed workspace serves any sequence of these GEMMs.
constexpr size_t kWsCounterBytes = 65536;
constexpr int64_t kWsMaxTiles = (int64_t)(kWsCounterBytes / 4);

// Partial tiles that the workgroups of one split-K launch hand to each other
// are written and read with relaxed agent-scope atomics: those are coherent
// across every CU of the GPU (they bypass the per-CU and per-XCD caches)
// without the whole-L2 write-back and invalidate that an agent-scope fence
// costs.  Ordering comes from the hardware: a thread waits until its stores
// have completed (vmcnt counts stores on this chip) before the workgroup
// counts its arrival, and the last arrival's loads are issued only after
// the counter has told it so.
__device__ __forceinline__ void store_shared_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same accesses 16 bytes at a time: buffer loads and stores with the
// cache policy the compiler gives agent-scope atomics (sc1), through a raw
// buffer resource over `nbytes` at `base` (word 3 0x00020000: the raw
// 32-bit format of this chip family; out-of-range accesses read 0 and write
// nothing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t shared_tile_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}
constexpr int kCpolAgentCoherent = 16;  // sc1
__device__ __forceinline__ void store_shared_v4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, v4f v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)byte_off, 0, kCpolAgentCoherent);
}
__device__ __forceinline__ v4f load_shared_v4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCpolAgentCoherent));
}
// every memory operation this thread issued has completed
__device__ __forceinline__ void wait_all_memory() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("" ::: "memory");
}
// Arrival of this workgroup at its tile's counter, after every thread's
// partial-tile stores: true in the last of `splits` workgroups, which then
// resets the counter (with an atomic store) for the next call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int splits, int* s_flag) {
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(splits - 1);
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last && threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

}  // namespace gbw

// ---------------------------------------------------------------------------
// host plumbing (defined in api.hip)
// ---------------------------------------------------------------------------
namespace gbw {
int fail(int status, const char* fmt, ...);
int check_device();                       // GBW_OK on gfx950, GBW_E_UNSUPPORTED otherwise
int check_launch(const char* what);       // maps hipGetLastError to GBW_E_LAUNCH
int device_cu_count();
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int launch_fill_zero(float* p, int64_t n, hipStream_t st);
// y[i] = sum_s part[s][i] over s = 0..splits-1, in that order
int launch_splitk_reduce(const float* part, int splits, int64_t mn, float* y, hipStream_t st);
}  // namespace gbw
