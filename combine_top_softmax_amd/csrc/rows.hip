// Rowwise dispatch and weighted combine: HBM-bound row movement.
//
// Olmo-core MoE report, Sec. 05 "Expert Parallelism", Sec. 5.6 and Table 8:
// dispatch forward pushes x_t into the capacity row of each selected expert
// (one read of the source row, fan-out to up to K destinations; negative
// destinations are skipped); combine forward gathers the K selected expert
// rows of a token, multiplies them by the router weights and sums them in
// token order (invalid entries gather zero).
//
// One wave per token row. A row is moved in 16-byte vectors (dwordx4), 64
// lanes side by side, so every wave access is a contiguous 1 KiB segment.
// Dispatch loads the source row once into registers and stores it to each
// local destination. Combine accumulates in fp32, k ascending, and writes each
// output row exactly once (no atomics, deterministic). With no weights it is
// the dispatch backward: the plain sum of a token's route rows (Sec. 5.6,
// Table 8, dispatch backward).
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 4;   // 4 waves = 4 token rows per 256-thread block

// Segment of a row: up to 64*NV 16-byte vectors handled per pass. The
// token's route metadata is read once (lane k: route k) and a ballot marks the
// local routes. FULL: the row is a whole number of segments.
template <int NV, bool FULL>
__global__ __launch_bounds__(256) void k_dispatch(
    const u32x4_t *__restrict__ x, const int32_t *__restrict__ dest_rank,
    const int32_t *__restrict__ dest_row, u32x4_t *__restrict__ buf, int T, int K,
    int nvec, int ep_rank, int rows) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6));
  if (t >= T) return;
  const size_t q0 = (size_t)t * K;
  int m_rank = -1, m_row = 0;
  if (lane < K) {
    m_rank = dest_rank[q0 + lane];
    m_row = dest_row[q0 + lane];
  }
  // a local route whose row lies outside the buffer is skipped
  const uint64_t local = __ballot(m_rank == ep_rank && (unsigned)m_row < (unsigned)rows);
  if (local == 0) return;
  const u32x4_t *src = x + (size_t)t * nvec;
  for (int seg = 0; seg < nvec; seg += 64 * NV) {
    u32x4_t r[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = seg + i * 64 + lane;
      if (FULL || c < nvec) r[i] = __builtin_nontemporal_load(src + c);
    }
    for (uint64_t rest = local; rest != 0; rest &= rest - 1) {
      const int k = __builtin_ctzll(rest);
      u32x4_t *dst = buf + (size_t)__builtin_amdgcn_readlane(m_row, k) * nvec;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = seg + i * 64 + lane;
        if (FULL || c < nvec) dst[c] = r[i];
      }
    }
  }
}

// Combine. Element type: bf16 (8 per vector) or fp32 (4 per vector). The
// token's route metadata is read once, lane k holding route k; a ballot
// marks the local routes, taken two at a time in k order: both rows are
// loaded before either is accumulated, so two rows per wave are in flight and
// the sum still runs k ascending. FULL: the row is a whole number of
// 64*NV-vector segments (no per-vector bounds test).
template <bool BF16, int NV, bool FULL>
__global__ __launch_bounds__(256) void k_combine(
    const u32x4_t *__restrict__ y, const int32_t *__restrict__ dest_rank,
    const int32_t *__restrict__ dest_row, const float *__restrict__ w,
    u32x4_t *__restrict__ out, int T, int K, int nvec, int ep_rank, int rows) {
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6));
  if (t >= T) return;
  const size_t q0 = (size_t)t * K;
  int m_rank = -1, m_row = 0;
  float m_w = 1.0f;                  // NULL weights: unit weights
  if (lane < K) {
    m_rank = dest_rank[q0 + lane];
    m_row = dest_row[q0 + lane];
    if (w != nullptr) m_w = w[q0 + lane];
  }
  // a local route whose row lies outside the buffer gathers nothing
  const uint64_t local = __ballot(m_rank == ep_rank && (unsigned)m_row < (unsigned)rows);
  auto accumulate = [&](float (&acc)[NV][EPV], const u32x4_t (&v)[NV], float wk) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t u[4] = {v[i][0], v[i][1], v[i][2], v[i][3]};
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][2 * e] = fmaf(wk, bf16_lo(u[e]), acc[i][2 * e]);
          acc[i][2 * e + 1] = fmaf(wk, bf16_hi(u[e]), acc[i][2 * e + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(wk, __uint_as_float(u[e]), acc[i][e]);
      }
    }
  };
  for (int seg = 0; seg < nvec; seg += 64 * NV) {
    float acc[NV][EPV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[i][e] = 0.f;
    for (uint64_t rest = local; rest != 0;) {
      const int ka = __builtin_ctzll(rest);
      rest &= rest - 1;
      const bool hb = rest != 0;
      const int kb = hb ? __builtin_ctzll(rest) : ka;
      if (hb) rest &= rest - 1;
      const u32x4_t *sa = y + (size_t)__builtin_amdgcn_readlane(m_row, ka) * nvec;
      const u32x4_t *sb = y + (size_t)__builtin_amdgcn_readlane(m_row, kb) * nvec;
      u32x4_t va[NV], vb[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = seg + i * 64 + lane;
        if (FULL || c < nvec) {
          // each expert row is read once: nontemporal, so that the gather
          // does not evict what the next kernels reuse (9% faster combine on
          // the skewed layer than with plain loads)
          va[i] = __builtin_nontemporal_load(sa + c);
          if (hb) vb[i] = __builtin_nontemporal_load(sb + c);
        }
      }
      accumulate(acc, va, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, m_w), ka)));
      if (hb)
        accumulate(acc, vb, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                          __builtin_bit_cast(int, m_w), kb)));
    }
    u32x4_t *dst = out + (size_t)t * nvec;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = seg + i * 64 + lane;
      if (!FULL && c >= nvec) continue;
      u32x4_t o;
      if constexpr (BF16) {
        o[0] = pack_bf16x2(acc[i][0], acc[i][1]);
        o[1] = pack_bf16x2(acc[i][2], acc[i][3]);
        o[2] = pack_bf16x2(acc[i][4], acc[i][5]);
        o[3] = pack_bf16x2(acc[i][6], acc[i][7]);
      } else {
        o[0] = __float_as_uint(acc[i][0]);
        o[1] = __float_as_uint(acc[i][1]);
        o[2] = __float_as_uint(acc[i][2]);
        o[3] = __float_as_uint(acc[i][3]);
      }
      __builtin_nontemporal_store(o, dst + c);
    }
  }
}

// Vectors-per-lane per pass: the smallest of 1,2,4,8 that covers the row.
inline int pick_nv(int nvec) {
  const int per_lane = (int)ceil_div(nvec, 64);
  return per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
}

}  // namespace

int launch_dispatch(const moe_shape_t &s, const void *x, const int32_t *dest_rank,
                    const int32_t *dest_row, void *buf, hipStream_t st) {
  const int nvec = s.d * elem_bytes(s.dtype) / 16;
  const int rows = (int)buffer_rows(s);
  const dim3 grid((unsigned)ceil_div(s.T, kRowsPerBlock)), block(256);
  const u32x4_t *xv = static_cast<const u32x4_t *>(x);
  u32x4_t *bv = static_cast<u32x4_t *>(buf);
  const int nv = pick_nv(nvec);
  if (nvec % (64 * nv) == 0) {
    switch (nv) {
      case 1: hipLaunchKernelGGL((k_dispatch<1, true>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      case 2: hipLaunchKernelGGL((k_dispatch<2, true>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      case 4: hipLaunchKernelGGL((k_dispatch<4, true>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      default: hipLaunchKernelGGL((k_dispatch<8, true>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
    }
  } else {
    switch (nv) {
      case 1: hipLaunchKernelGGL((k_dispatch<1, false>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      case 2: hipLaunchKernelGGL((k_dispatch<2, false>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      case 4: hipLaunchKernelGGL((k_dispatch<4, false>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
      default: hipLaunchKernelGGL((k_dispatch<8, false>), grid, block, 0, st, xv, dest_rank, dest_row, bv, s.T, s.K, nvec, s.ep_rank, rows); break;
    }
  }
  return launch_status();
}

template <bool BF16, bool FULL>
static void combine_nv(int nv, dim3 grid, hipStream_t st, const u32x4_t *y, const int32_t *dr,
                       const int32_t *drow, const float *w, u32x4_t *o, const moe_shape_t &s,
                       int nvec) {
  const int rows = (int)buffer_rows(s);
  switch (nv) {
    case 1: hipLaunchKernelGGL((k_combine<BF16, 1, FULL>), grid, dim3(256), 0, st, y, dr, drow, w, o, s.T, s.K, nvec, s.ep_rank, rows); break;
    case 2: hipLaunchKernelGGL((k_combine<BF16, 2, FULL>), grid, dim3(256), 0, st, y, dr, drow, w, o, s.T, s.K, nvec, s.ep_rank, rows); break;
    case 4: hipLaunchKernelGGL((k_combine<BF16, 4, FULL>), grid, dim3(256), 0, st, y, dr, drow, w, o, s.T, s.K, nvec, s.ep_rank, rows); break;
    default: hipLaunchKernelGGL((k_combine<BF16, 8, FULL>), grid, dim3(256), 0, st, y, dr, drow, w, o, s.T, s.K, nvec, s.ep_rank, rows); break;
  }
}

int launch_combine(const moe_shape_t &s, const void *y, const int32_t *dest_rank,
                   const int32_t *dest_row, const float *w, void *out, hipStream_t st) {
  const int nvec = s.d * elem_bytes(s.dtype) / 16;
  const dim3 grid((unsigned)ceil_div(s.T, kRowsPerBlock));
  const u32x4_t *yv = static_cast<const u32x4_t *>(y);
  u32x4_t *ov = static_cast<u32x4_t *>(out);
  const int nv = pick_nv(nvec);
  const bool full = nvec % (64 * nv) == 0;
  if (s.dtype == MOE_BF16) {
    if (full) combine_nv<true, true>(nv, grid, st, yv, dest_rank, dest_row, w, ov, s, nvec);
    else combine_nv<true, false>(nv, grid, st, yv, dest_rank, dest_row, w, ov, s, nvec);
  } else {
    if (full) combine_nv<false, true>(nv, grid, st, yv, dest_rank, dest_row, w, ov, s, nvec);
    else combine_nv<false, false>(nv, grid, st, yv, dest_rank, dest_row, w, ov, s, nvec);
  }
  return launch_status();
}

}  // namespace moe
