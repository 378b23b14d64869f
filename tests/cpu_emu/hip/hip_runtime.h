// Test infrastructure: a CPU emulation of the HIP runtime surface the kernels
// use, so that the kernel sources compile as host C++ under AddressSanitizer.
// Every GPU thread runs as an OS thread; __syncthreads is a std::barrier per
// workgroup (a barrier-count mismatch deadlocks, which the test's timeout
// catches); DPP row/quad permutes exchange through a per-wave array; the
// fp4 -> fp16 conversion is emulated; the matrix and other conversion
// builtins return placeholder data (no address depends on them).  Every
// device buffer is a separate exact-size host allocation, so an out-of-bounds
// access is an ASan report.
#pragma once
#include <stdint.h>
#include <math.h>
#include <string.h>
#include <algorithm>
#include <barrier>
#include <thread>
#include <vector>
#include <mutex>
#include <functional>
#include <stdio.h>
#include <stdlib.h>
#include <memory>
#include <atomic>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static

struct dim3 {
  unsigned x = 1, y = 1, z = 1;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct emu_idx { unsigned x, y, z; };
extern thread_local emu_idx threadIdx, blockIdx, blockDim, gridDim;
extern thread_local std::barrier<>* emu_bar;
inline void __syncthreads() { emu_bar->arrive_and_wait(); }

typedef void* hipStream_t;
typedef int hipError_t;
#define hipSuccess 0
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }
inline const char* hipGetErrorString(hipError_t) { return "emulated"; }
struct uint2 { unsigned x, y; };

template <class A, class B> inline auto min(A a, B b) { return a < b ? a : b; }
template <class A, class B> inline auto max(A a, B b) { return a > b ? a : b; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline int __float_as_int(float f) { int u; memcpy(&u, &f, 4); return u; }
inline float __int_as_float(int u) { float f; memcpy(&f, &u, 4); return f; }
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
extern std::mutex emu_atomic_mu;
inline void unsafeAtomicAdd(float* p, float v) { std::lock_guard<std::mutex> g(emu_atomic_mu); *p += v; }
inline unsigned long long atomicOr(unsigned long long* p, unsigned long long v) { std::lock_guard<std::mutex> g(emu_atomic_mu); auto o = *p; *p |= v; return o; }
template <class T> inline T __shfl_xor(T v, int) { return v; }
inline unsigned atomicAdd(unsigned* p, unsigned v) { std::lock_guard<std::mutex> g(emu_atomic_mu); auto o = *p; *p += v; return o; }
inline void __threadfence() { std::atomic_thread_fence(std::memory_order_seq_cst); }
#define __HIP_MEMORY_SCOPE_AGENT 3
template <class T, class V> inline void emu_atomic_store(T* p, V v) { T t = (T)v; __atomic_store(p, &t, __ATOMIC_SEQ_CST); }
template <class T> inline T emu_atomic_load(T* p) { T t; __atomic_load(p, &t, __ATOMIC_SEQ_CST); return t; }
#define __hip_atomic_store(p, v, order, scope) emu_atomic_store((p), (v))
#define __hip_atomic_load(p, order, scope) emu_atomic_load((p))
#define __hip_atomic_fetch_add(p, v, order, scope) __atomic_fetch_add((p), (v), __ATOMIC_SEQ_CST)
// raw buffer resources: a base and a byte count; accesses past the count read
// zero and write nothing, as on the hardware (within the count, ASan checks
// the access against the real allocation)
struct emu_rsrc { char* base; uint32_t n; };
typedef emu_rsrc __amdgpu_buffer_rsrc_t;
#define __builtin_amdgcn_make_buffer_rsrc(p, stride, num, flags) emu_rsrc{(char*)(p), (uint32_t)(num)}
typedef unsigned int emu_v4u __attribute__((ext_vector_type(4)));
inline void emu_buf_store(emu_v4u v, emu_rsrc r, int off) {
  if ((uint32_t)off + 16 > r.n) return;
  std::lock_guard<std::mutex> g(emu_atomic_mu);
  memcpy(r.base + off, &v, 16);
}
inline emu_v4u emu_buf_load(emu_rsrc r, int off) {
  emu_v4u v = {0, 0, 0, 0};
  if ((uint32_t)off + 16 > r.n) return v;
  std::lock_guard<std::mutex> g(emu_atomic_mu);
  memcpy(&v, r.base + off, 16);
  return v;
}
#define __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, aux) emu_buf_store((v), (r), (off) + (soff))
#define __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, aux) emu_buf_load((r), (off) + (soff))

#define __builtin_amdgcn_readfirstlane(x) (x)
// DPP: the 64 lanes of a wave exchange through a per-wave array (all lanes
// of the wave must reach the call together, as on the hardware)
struct emu_wave { std::barrier<>* bar; int* buf; };
extern thread_local emu_wave emu_w;
inline int emu_dpp_src(int lane, int ctrl) {
  const int row = lane & ~15, r = lane & 15;
  if (ctrl <= 0xFF) return (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);     // quad_perm
  if (ctrl == 0x140) return row | (15 - r);                                      // row_mirror
  if (ctrl == 0x141) return row | ((r & 8) | (7 - (r & 7)));                     // row_half_mirror
  if (ctrl > 0x120 && ctrl <= 0x12F) return row | ((r - (ctrl - 0x120)) & 15);   // row_ror:n
  fprintf(stderr, "emu: unsupported dpp ctrl %x\n", ctrl); abort();
}
inline int emu_dpp(int v, int ctrl) {
  const int lane = threadIdx.x & 63;
  emu_w.buf[lane] = v;
  emu_w.bar->arrive_and_wait();
  const int r = emu_w.buf[emu_dpp_src(lane, ctrl)];
  emu_w.bar->arrive_and_wait();
  return r;
}
#define __builtin_amdgcn_mov_dpp(v, ctrl, ...) emu_dpp((v), (ctrl))
#define __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, ...) ((void)(a), (void)(b), (c))
#define __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, ...) ((void)(a), (void)(b), (c))
#define __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, ...) ((void)(a), (void)(b), (c))
#define __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, ...) ((void)(a), (void)(b), (c))
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
#define __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, sel) ((old) | ((uint32_t)(((a) != (b)) & 1) << (8 * (sel))))
typedef _Float16 emu_v2h __attribute__((ext_vector_type(2)));
inline emu_v2h emu_cvt_f16_fp4(uint32_t w, float s, int sel) {
  static const float m[8] = {0, .5f, 1, 1.5f, 2, 3, 4, 6};
  const uint32_t b = (w >> (8 * sel)) & 255;
  const float lo = ((b & 8) ? -m[b & 7] : m[b & 7]) * s, hi = ((b & 128) ? -m[(b >> 4) & 7] : m[(b >> 4) & 7]) * s;
  return emu_v2h{(_Float16)lo, (_Float16)hi};
}
#define __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, sel) emu_cvt_f16_fp4((w), (s), (sel))
typedef float emu_v2f __attribute__((ext_vector_type(2)));
inline emu_v2f emu_cvt_f32_fp4(uint32_t w, float s, int sel) {
  static const float m[8] = {0, .5f, 1, 1.5f, 2, 3, 4, 6};
  const uint32_t b = (w >> (8 * sel)) & 255;
  return emu_v2f{((b & 8) ? -m[b & 7] : m[b & 7]) * s, ((b & 128) ? -m[(b >> 4) & 7] : m[(b >> 4) & 7]) * s};
}
#define __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, sel) emu_cvt_f32_fp4((w), (s), (sel))
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, ...) ((void)(a), (void)(b), (c))
#define __builtin_amdgcn_perm(a, b, s) ((uint32_t)(a) ^ (uint32_t)(b) ^ (uint32_t)(s))
#define __builtin_amdgcn_s_waitcnt(x) ((void)0)
#define __builtin_amdgcn_s_barrier() __syncthreads()
// direct-to-LDS load: lane l of the wave writes `size` bytes at dst + off + l * size
#define __builtin_amdgcn_global_load_lds(src, dst, size, off, aux) \
  memcpy((char*)(void*)(dst) + (off) + (threadIdx.x & 63) * (size), (const void*)(src), (size))
#define __builtin_amdgcn_wave_barrier() ((void)0)
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_s_setprio(x) ((void)0)
#define __builtin_amdgcn_sched_group_barrier(a, b, c) ((void)0)

template <class K, class... A>
void emu_launch(K kernel, dim3 g, dim3 b, A... args) {
  const unsigned nt = b.x * b.y * b.z;
  for (unsigned bz = 0; bz < g.z; ++bz)
    for (unsigned by = 0; by < g.y; ++by)
      for (unsigned bx = 0; bx < g.x; ++bx) {
        std::barrier<> bar((std::ptrdiff_t)nt);
        const unsigned nw = (nt + 63) / 64;
        std::vector<std::unique_ptr<std::barrier<>>> wbar;
        std::vector<int> wbuf(nw * 64);
        for (unsigned w = 0; w < nw; ++w) wbar.emplace_back(new std::barrier<>((std::ptrdiff_t)std::min(64u, nt - 64 * w)));
        std::vector<std::thread> th;
        th.reserve(nt);
        for (unsigned t = 0; t < nt; ++t)
          th.emplace_back([&, t]() {
            threadIdx = {t % b.x, (t / b.x) % b.y, t / (b.x * b.y)};
            blockIdx = {bx, by, bz};
            blockDim = {b.x, b.y, b.z};
            gridDim = {g.x, g.y, g.z};
            emu_bar = &bar;
            emu_w = {wbar[t / 64].get(), &wbuf[(t / 64) * 64]};
            kernel(args...);
            bar.arrive_and_drop();
            wbar[t / 64]->arrive_and_drop();
          });
        for (auto& x : th) x.join();
      }
}
#define hipLaunchKernelGGL(k, g, b, shm, st, ...) emu_launch(k, dim3(g), dim3(b), __VA_ARGS__)
