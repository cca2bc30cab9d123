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

// Direct global -> LDS loads (lane l's SZ bytes land at LDS byte address
// lds + SZ * l; lds wave-uniform). Written as inline asm rather than the
// compiler builtin: the compiler counts the builtin as an LDS event of its own
// kind, which turns every wait for the fragment reads (ds_read) into a full
// lgkmcnt(0); the asm form leaves those waits exact. The loads are then
// invisible to the compiler's own vmcnt bookkeeping: the kernels order them
// with explicit wait_vmcnt + s_barrier (and wait_vmcnt<0> before any other
// use of the LDS they write).
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void *gptr, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)MOE_LDS(p);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Order in which a sub-step's fragments are read: the order of their first
// use by the MFMA sequence (A0 B0 B1 A1 A2 A3 for 4 x 2 tiles), so that the
// MFMAs at the start of a sub-step wait only for the oldest reads.
template <int TM, int TN>
struct FragOrder {
  int q[TM + TN];
  constexpr FragOrder() : q() {
    bool seen[TM + TN] = {};
    int n = 0;
    for (int m = 0; m < TM * TN; ++m) {
      const int a = m / TN, b = TM + m % TN;
      if (!seen[a]) { seen[a] = true; q[n++] = a; }
      if (!seen[b]) { seen[b] = true; q[n++] = b; }
    }
  }
};

// Row-grouped GEMM tiles from the device offsets of the local experts: the
// grid is sized from the capacity bound, every block recomputes the
// per-expert m-tile counts (tm rows each) with a wave scan and maps itself to
// (expert, m-tile, n-tile) or exits. XCD-aware order: blocks are dealt to the
// 8 XCDs round-robin, so block b takes tile (b % 8) * q + b / 8 and each XCD
// walks a contiguous run of tiles. Wave-uniform result.
struct RowTile {
  int expert, row0, row_end, n_idx;
  bool valid;
};

__device__ __forceinline__ RowTile find_row_tile(const int32_t *__restrict__ off, int E_L, int tm,
                                                 int n_tiles_n) {
  const int lane = threadIdx.x & 63;
  RowTile tl;
  tl.valid = false;
  int total_m = 0;
  for (int c = 0; c < E_L; c += 64) {
    const int j = c + lane;
    const int n = (j < E_L) ? off[j + 1] - off[j] : 0;
    const int incl = wave_incl_scan((n + tm - 1) / tm);
    total_m += __shfl(incl, 63, 64);
  }
  const int total = total_m * n_tiles_n;
  const int q = (total + kNumXcd - 1) / kNumXcd;
  const int b = blockIdx.x;
  const int slot = b / kNumXcd;
  const int L = (b % kNumXcd) * q + slot;
  if (slot >= q || L >= total) return tl;
  const int m_glob = L / n_tiles_n;
  tl.n_idx = L - m_glob * n_tiles_n;
  int run = 0;
  for (int c = 0; c < E_L; c += 64) {
    const int j = c + lane;
    const int n = (j < E_L) ? off[j + 1] - off[j] : 0;
    const int mt = (n + tm - 1) / tm;
    const int incl = wave_incl_scan(mt);
    const int tot = __shfl(incl, 63, 64);
    if (m_glob < run + tot) {
      const uint64_t hit = __ballot(m_glob < run + incl);
      const int first = __builtin_ctzll(hit);
      const int excl = __shfl(incl - mt, first, 64);
      const int e = c + first;
      tl.expert = e;
      tl.row0 = off[e] + (m_glob - run - excl) * tm;
      tl.row_end = off[e + 1];
      tl.valid = true;
      return tl;
    }
    run += tot;
  }
  return tl;
}

}  // namespace moe
