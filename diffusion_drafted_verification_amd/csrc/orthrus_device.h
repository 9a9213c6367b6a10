// Device-side building blocks shared by the gfx950 kernels: vector types,
// 16-byte memory moves and the 32x32 MFMA step for bf16 and fp32 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kPage = 16;  // tokens per cache page

// Eight consecutive elements of the storage type: the per-lane A/B operand
// of one 32x32 MFMA k-step of 16 (two lane halves x 8 elements).
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; static constexpr int bytes = 16; };
template <> struct Vec8<float> { typedef f32x8 type; static constexpr int bytes = 32; };

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// D(32x32, fp32) += A(32 x 16) * B(16 x 32) for one lane's operands.  Lane l
// supplies row (l % 32) of A / column (l % 32) of B, elements 8*(l/32)+e of
// the contracted dimension.  Only the pairing of A's and B's k-slots matters
// for the contraction, and it is the same for both operands by construction.
__device__ __forceinline__ f32x16 mfma_step(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp32 storage: eight 32x32x2 steps, step e contracting element e of both halves.
__device__ __forceinline__ f32x16 mfma_step(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// max of x over lanes l and l ^ 32: v_permlane32_swap exchanges the two
// 32-lane halves between two registers (no LDS round trip)
__device__ __forceinline__ float wave_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


#define ORTHRUS_LDS __attribute__((address_space(3)))

// One wave instruction of the LDS-DMA path: lane l copies 16 bytes from its
// global address to LDS address (dst + 16 l).  Written as inline assembly so
// that the compiler does not track these LDS writes: the kernel orders them
// itself (s_waitcnt vmcnt + barrier before any wave reads the data).  The
// instruction has no register result; M0 holds the wave-uniform LDS base
// (one wait state after writing M0 before the load reads it).
__device__ __forceinline__ void dma16(const void* src, char* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((ORTHRUS_LDS char*)dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// The same with the nontemporal hint, for data a call reads exactly once: it
// streams past the caches (measured on the Qwen3-8B attention shape: 9 %
// faster at batch 1, a few % at batch 4 to 16; slower where the data is
// re-read, as across the chunks of a prefill).
__device__ __forceinline__ void dma16_nt(const void* src, char* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((ORTHRUS_LDS char*)dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds) : "memory");
}

// one DMA instruction either way (hand-placed vmcnt counts do not change);
// `once` is uniform (a kernel argument)
__device__ __forceinline__ void dma16_kv(const void* src, char* dst, int once) {
  if (once)
    dma16_nt(src, dst);
  else
    dma16(src, dst);
}

// The same with 4 bytes per lane (lane l writes dst + 4 l).
__device__ __forceinline__ void dma4(const void* src, char* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((ORTHRUS_LDS char*)dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Wait until at most N of this wave's vector memory loads are outstanding
// (they complete in issue order).  Inline assembly, like the DMA itself: the
// compiler does not count the DMA loads, so kernels place these waits by hand
// where only LDS-DMA loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace orthrus
