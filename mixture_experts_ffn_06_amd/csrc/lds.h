// Device helpers for the LDS rings of the expert kernels: direct loads to
// LDS (through a buffer resource, or global_load_lds), waits, barriers, plain
// LDS loads, and grouped LDS reads that wait for themselves.
#pragma once
#include "common.h"
#include <type_traits>

namespace moe {

// A value known to be equal on all lanes, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Direct global -> LDS loads of 16 or 4 bytes per lane (global_load_lds_
// dwordx4 / _dword): lane l's bytes land at lds_dst + 16 l (or 4 l).
// Completion is counted by the issuing wave's vmcnt.
__device__ __forceinline__ void dma16_to_lds(const void *src, void *lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void *src, void *lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 4, 0, 0);
}

// A buffer resource over `bytes` bytes from base (raw, stride 0): offsets at
// or past `bytes` read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Direct loads of 16 or 4 bytes per lane from a buffer resource to LDS
// (buffer_load_dwordx4 / _dword ... lds): lane l's bytes land at lds_dst +
// 16 l (or 4 l).  Completion is counted by the issuing wave's vmcnt.
__device__ __forceinline__ void buf16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void buf4_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_dst, 4, off, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (expcnt and lgkmcnt left unconstrained).  The empty asm
// statements keep the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Wait until at most N LDS (and scalar memory) operations of this wave are
// outstanding; vmcnt and expcnt left unconstrained.
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (N << 8) | (0x3 << 14));
  asm volatile("" ::: "memory");
}

// A plain load of a T from LDS (p points into a __shared__ array): the
// compiler places the wait for it before the value's first use.
template <typename T>
__device__ __forceinline__ T lds_load(const uint8_t *p) {
  return *reinterpret_cast<const T *>(p);
}

// Block barrier for the LDS ring.  __syncthreads() also releases memory at
// workgroup scope, which on this target waits for every outstanding load --
// including the direct-to-LDS loads of the stages still in flight.  The ring
// only needs the execution barrier: each wave waits for its own loads with
// wait_vm<>() first, and LDS reads of a slot are complete (their values are
// in registers) before a wave reaches the barrier that frees the slot.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// The LDS byte address a as a pointer (the inverse of lds_off).
__device__ __forceinline__ void *lds_ptr(uint32_t a) {
  return (void *)(__attribute__((address_space(3))) void *)(static_cast<uintptr_t>(a));
}

__device__ __forceinline__ uint32_t lds_off(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void *)p));
}

// Grouped 16-byte LDS reads in one asm statement that ends with the wait
// for them (the streaming kernel reads a stage's operand pieces together):
// four at p0 + O0, p1 + O1, p2 + O2, p3 + O3.
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read4(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                          u32x4_t &v0, u32x4_t &v1, u32x4_t &v2, u32x4_t &v3) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n"
      "ds_read_b128 %1, %5 offset:%9\n"
      "ds_read_b128 %2, %6 offset:%10\n"
      "ds_read_b128 %3, %7 offset:%11\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "i"(O0), "i"(O1), "i"(O2), "i"(O3));
}

// Two 16-byte reads at p0 + O0, p1 + O1.
template <int O0, int O1>
__device__ __forceinline__ void lds_read2(uint32_t p0, uint32_t p1, u32x4_t &v0, u32x4_t &v1) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n"
      "ds_read_b128 %1, %3 offset:%5\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1)
      : "v"(p0), "v"(p1), "i"(O0), "i"(O1));
}

}  // namespace moe
