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
  static_assert(CH == 8, "rows of 8 chunks (64 bf16 or 128 fp8 elements)");
  return (r & 7) ^ ((r >> 3) & 1);
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

// 64 local experts as the lanes of a wave hold them: lane j has expert c + j's
// buffer rows [o0, o1), its count of bm-row m-tiles and the inclusive scan of
// those counts over the chunk; tot is the chunk's total (wave-uniform).
struct ExpertChunk {
  int o0, o1, mt, incl, tot;
};

// Offsets are clamped into the buffer, [0, rows], with o1 >= o0, so that
// offsets from any source keep every tile inside the row buffers.
__device__ __forceinline__ ExpertChunk expert_chunk(const int32_t *__restrict__ off, int E_L, int c,
                                                    int bm, int rows) {
  const int j = c + (threadIdx.x & 63);
  ExpertChunk ch;
  ch.o0 = 0;
  ch.o1 = 0;
  if (j < E_L) {
    ch.o0 = min(max(off[j], 0), rows);
    ch.o1 = min(max(off[j + 1], ch.o0), rows);
  }
  ch.mt = (max(ch.o1 - ch.o0, 0) + bm - 1) / bm;
  ch.incl = wave_incl_scan_dpp(ch.mt);
  ch.tot = __builtin_amdgcn_readlane(ch.incl, 63);
  return ch;
}

// Grouped GEMM tiles from the device offsets of the local experts: the grid is
// sized from the capacity bound, every block counts the experts' m-tiles (bm
// rows each) and maps itself to tile L of the XCD-aware order, or exits.
// Blocks are dealt to the 8 XCDs round-robin, so block b takes tile
// (b % 8) * q + b / 8 and each XCD walks a contiguous run of tiles; tiles are
// numbered expert by expert (n_tiles_n per m-tile). The offsets are read once
// (one load per lane for up to 64 experts) and everything after is register
// work. The result is wave-uniform and, whatever the scan returns, names an
// expert below E_L with at least one row and an m-tile inside it, so every
// address the kernels form from it stays inside that expert's rows.
struct ExpertTile {
  int L;          // this block's tile index
  int e;          // expert
  int mstart;     // index of the expert's first m-tile among all m-tiles
  int M;          // m-tiles of the expert
  int row_begin;  // the expert's buffer rows [row_begin, row_end)
  int row_end;
  bool valid;
};

// m-tiles (bm rows each) of all local experts: the tile count is this times
// the n-tiles. The c0 chunk (experts 0..63) is returned for reuse.
__device__ __forceinline__ int count_m_tiles(const int32_t *__restrict__ off, int E_L, int bm,
                                             int rows, ExpertChunk &c0) {
  c0 = expert_chunk(off, E_L, 0, bm, rows);
  int total_m = c0.tot;
  for (int c = 64; c < E_L; c += 64) total_m += expert_chunk(off, E_L, c, bm, rows).tot;
  return total_m;
}

// Tile L (< total) of the expert-by-expert numbering: its expert, the
// expert's m-tile run and rows. c0: the first chunk, as count_m_tiles read it.
__device__ __forceinline__ ExpertTile expert_tile_at(const int32_t *__restrict__ off, int E_L,
                                                     int bm, int rows, int n_tiles_n, int L,
                                                     const ExpertChunk &c0) {
  ExpertTile t;
  t.valid = false;
  const int m_glob = L / n_tiles_n;
  int run = 0;
  for (int c = 0; c < E_L; c += 64) {
    const ExpertChunk ch = (c == 0) ? c0 : expert_chunk(off, E_L, c, bm, rows);
    if (m_glob < run + ch.tot) {
      const uint64_t hit = __ballot(m_glob < run + ch.incl);
      if (hit == 0) return t;
      const int first = __builtin_ctzll(hit);
      const int M = __builtin_amdgcn_readlane(ch.mt, first);
      const int mstart = run + __builtin_amdgcn_readlane(ch.incl, first) - M;
      if (c + first >= E_L || M <= 0 || m_glob < mstart || m_glob >= mstart + M) return t;
      t.L = L;
      t.e = c + first;
      t.M = M;
      t.mstart = mstart;
      t.row_begin = __builtin_amdgcn_readlane(ch.o0, first);
      t.row_end = __builtin_amdgcn_readlane(ch.o1, first);
      t.valid = true;
      return t;
    }
    run += ch.tot;
  }
  return t;
}

__device__ __forceinline__ ExpertTile find_expert_tile(const int32_t *__restrict__ off, int E_L,
                                                       int bm, int rows, int n_tiles_n) {
  ExpertTile t;
  t.valid = false;
  ExpertChunk c0;
  const int total = count_m_tiles(off, E_L, bm, rows, c0) * n_tiles_n;
  const int q = (total + kNumXcd - 1) / kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int L = (blockIdx.x % kNumXcd) * q + slot;
  if (slot >= q || L >= total) return t;
  return expert_tile_at(off, E_L, bm, rows, n_tiles_n, L, c0);
}

// Row-mode tiles: m-tile by m-tile, its n_tiles_n n-tiles consecutive.
struct RowTile {
  int expert, row0, row_end, n_idx;
  bool valid;
};

__device__ __forceinline__ RowTile find_row_tile(const int32_t *__restrict__ off, int E_L, int tm,
                                                 int rows, int n_tiles_n) {
  RowTile tl;
  const ExpertTile x = find_expert_tile(off, E_L, tm, rows, n_tiles_n);
  tl.valid = x.valid;
  if (!x.valid) return tl;
  const int m_glob = x.L / n_tiles_n;
  tl.expert = x.e;
  tl.row0 = x.row_begin + (m_glob - x.mstart) * tm;
  tl.row_end = x.row_end;
  tl.n_idx = x.L - m_glob * n_tiles_n;
  return tl;
}

}  // namespace moe
