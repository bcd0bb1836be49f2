// Device helpers of the direct-load matrix-core kernels (mfma_dl.hip, mfma_big.hip):
// waits, the direct global -> LDS loads, the activation-row swizzle and small bit
// tricks.  Both kernels stage the same activation rows and superblocks.
#pragma once

#include <type_traits>
#include <utility>

#include "qgemm_internal.hpp"

namespace qg {
namespace dl {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ uint32_t as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte direct global -> LDS load of this lane (gfx950 global_load_lds_dwordx4:
// lane l's bytes land at LDS address m0 + 16 l).  Written as inline assembly so
// that the compiler, which cannot tell the ring slots apart, does not make every
// later LDS read wait for all of these loads; m0 is saved and restored inside.
// Completion is waited for explicitly (s_waitcnt vmcnt + s_barrier) before a
// slot is read.  No register receives data from these loads.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// The same load in its scalar-base form: 64-bit wave-uniform base in SGPRs plus a
// 32-bit offset per lane, so no per-lane 64-bit address is formed.  The LDS base
// is an operand bound to m0, so the compiler writes m0 once per load and knows it
// holds the value (no save and restore around the load).
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds_base) : "memory");
}

// (x & m) | c in one VALU op (masks that are not inline constants go in registers)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// position (in 16-byte units) of chunk c of activation row r.  Only r mod 16
// enters, so rows that are 16 apart share one pattern and a fragment read's lane
// addresses differ between sub-tiles by a constant offset.  A fragment read
// (ds_read_b128) has lanes 16 q + j read row j at chunk c(q): chunks 4 t + q for
// fp16 / int8, (q & 1) * 4 + 2 t + (q >> 1) for the packed formats.  The patterns
// keep every 16 lanes on distinct 16-byte slots of 256 bytes, every 32 lanes on
// distinct slots of 512 bytes and all 64 on distinct slots of 1 KiB (the LDS of
// gfx950 serves a 16-byte read in passes of 32 lanes: with rows 128 bytes long an
// XOR by (r ^ r >> 3) & 7, distinct only per 16 lanes, stalled the fp16 16384^3
// product on bank conflicts for 17 % of its cycles).
template <int ROWB, bool PACKED>
__device__ __forceinline__ int swz(int r, int c) {
  r &= 15;
  if constexpr (ROWB == 64) return c ^ (((r >> 1) ^ (r >> 2)) & 3);
  else if constexpr (PACKED) return c ^ (((r >> 2) & 3) | (((r >> 1) & 1) << 2));
  else return c ^ ((r >> 1) & 7);
}

template <int... T, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, T...>, F&& f) {
  (f(std::integral_constant<int, T>{}), ...);
}

}  // namespace dl
}  // namespace qg
