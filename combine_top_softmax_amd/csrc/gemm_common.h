// Device helpers shared by the bf16 MFMA GEMM kernels (forward and backward).
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// XOR swizzle of the 16-byte chunk index of a K-contiguous LDS row (CH chunks
// per row), chosen so that a wave's direct load writes whole rows
// contiguously and the fragment reads of 16 consecutive rows (one chunk each)
// touch 16 distinct 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (CH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}

#define MOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace moe
