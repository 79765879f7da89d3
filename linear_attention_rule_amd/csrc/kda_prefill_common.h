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

}  // namespace prefill
}  // namespace kda
