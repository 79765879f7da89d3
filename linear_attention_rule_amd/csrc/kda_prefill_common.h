// Shared by the two prefill kernels: MFMA operand types, the key-channel order of the
// state's accumulator layout, and the MFMA wrappers.
#pragma once

#include "kda_internal.h"

namespace kda {
namespace prefill {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Key/value channel held by lane group g in element e of k-step s (pairs of
// 16-row accumulator blocks 2s and 2s+1 form one 32-deep k-step).
__device__ __forceinline__ constexpr int kperm(int s, int g, int e) {
  return 32 * s + 16 * (e >> 2) + 4 * g + (e & 3);
}

__device__ __forceinline__ f32x4 mfma_f16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS (no VGPR staging):
// lane l's bytes land at LDS address lds + 16 l.  The global address is a
// wave-uniform base (SGPR pair) plus a per-lane 32-bit byte offset.  Issued as
// inline asm so the compiler does not track it: the caller orders these copies
// itself with an explicit s_waitcnt vmcnt (and a barrier where other waves read
// the data).
__device__ __forceinline__ void lds_dma16(uint64_t gbase, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(lane_off), "s"(gbase)
               : "memory", "m0");
}

// 4 bytes per lane, same addressing (lane l writes lds + 4 l).
__device__ __forceinline__ void lds_dma4(uint64_t gbase, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(lane_off), "s"(gbase)
               : "memory", "m0");
}

__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// LDS byte address of a __shared__ object (computed once; no per-use cast).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)p)));
}

}  // namespace prefill
}  // namespace kda
