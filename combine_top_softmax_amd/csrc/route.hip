// Top-K softmax gating and the route-map builder, without atomics.
//
// Olmo-core MoE report, Sec. 05 "Expert Parallelism", Sec. 5.4 and Fig. 16: the
// route-map builder gives every route its destination rank and row, where the
// row is the expert's offset on its rank plus the number of EARLIER accepted
// routes for that expert; the capacity decision is applied before movement and
// the counts stay on the device (Sec. 08 "Synchronization-Free Training",
// Sec. 8.5).
//
// "Earlier" is token order, so a route's position p in its expert is
//   p = (routes to e in earlier 64-token tiles) + (earlier lanes of this tile
//       that route to e).
// Three kernels compute it without atomics and without a host round trip:
//   k_route_tile   one wave per 64-token tile (one lane per token): top-K in
//                  registers, fp64 softmax over the K winners, then per expert
//                  a wave ballot of "my token routes to e"; the ballot masks go
//                  to LDS, popcount(mask) is the tile histogram and
//                  popcount(mask & lanes-below) the in-tile rank.
//   k_tile_scan    one block per expert: exclusive scan of its tile histogram
//                  column -> tile bases; the total is counts[e].
//   k_assign       one wave per tile: every block rebuilds the exclusive scan
//                  of min(counts, C) over experts in LDS, then p = base + rank,
//                  keep iff p < C, row = offset of e on its rank + p.
//
// Workspace: hist/base [N][ntiles] int32, then rank [T*K] uint8.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

// Insert (x, i) into a list sorted by (value desc, index asc); the smallest
// element falls off the end. Elements arrive in ascending index, so a strict
// '>' keeps the earlier (lower) id ahead on ties; IEEE '>' treats -0.0 and +0.0
// as equal. Once the new element has been placed, every later slot shifts.
template <int KM>
__device__ __forceinline__ void topk_insert(float (&v)[KM], int (&ix)[KM], float x, int i) {
  bool placed = false;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const bool sw = placed || (x > v[j]);
    const float tv = v[j];
    const int ti = ix[j];
    v[j] = sw ? x : tv;
    ix[j] = sw ? i : ti;
    x = sw ? tv : x;
    i = sw ? ti : i;
    placed = sw;
  }
}

template <int KM, bool FROM_LOGITS>
__global__ __launch_bounds__(64) void k_route_tile(
    const float *__restrict__ logits, const int32_t *__restrict__ ids_in,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ hist, uint8_t *__restrict__ rank_ws,
    int T, int N, int K, int ntiles) {
  __shared__ uint64_t s_mask[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int t = tile * kRouteTile + lane;
  const bool active = t < T;

  int ix[KM];
  if constexpr (FROM_LOGITS) {
    float v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) { v[j] = -INFINITY; ix[j] = -1; }
    if (active) {
      const float *row = logits + (size_t)t * N;
      if ((N & 3) == 0) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t *row4 = reinterpret_cast<const f32x4_t *>(row);
        for (int q = 0; q < (N >> 2); ++q) {
          const f32x4_t f = __builtin_nontemporal_load(row4 + q);
          topk_insert<KM>(v, ix, f.x, 4 * q + 0);
          topk_insert<KM>(v, ix, f.y, 4 * q + 1);
          topk_insert<KM>(v, ix, f.z, 4 * q + 2);
          topk_insert<KM>(v, ix, f.w, 4 * q + 3);
        }
      } else {
        for (int e = 0; e < N; ++e) topk_insert<KM>(v, ix, row[e], e);
      }
      // softmax over the K selected logits, in fp64, rounded once to fp32
      const double m = (double)v[0];
      double ex[KM];
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        ex[j] = (j < K) ? exp((double)v[j] - m) : 0.0;
        sum += ex[j];
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < K) {
          topk_idx[(size_t)t * K + j] = ix[j];
          topk_w[(size_t)t * K + j] = (float)(ex[j] / sum);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j) ix[j] = (active && j < K) ? ids_in[(size_t)t * K + j] : -1;
  }

  // Per chunk of 64 experts: a ballot per expert; lane j keeps the mask of
  // expert (64*chunk + j), stores it to LDS and writes the tile histogram.
  const int nchunks = (N + kWave - 1) / kWave;
  for (int c = 0; c < nchunks; ++c) {
    uint64_t mine_bits = 0;  // which experts of this chunk my token routes to
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = ix[j];
      const bool in = (j < K) && e >= 0 && e < N && (e >> 6) == c;
      mine_bits |= in ? (1ull << (e & 63)) : 0ull;
    }
    uint32_t mlo = 0, mhi = 0;
#pragma unroll
    for (int j = 0; j < kWave; ++j) {
      const uint64_t b = __ballot((mine_bits >> j) & 1ull);
      mlo = (lane == j) ? (uint32_t)b : mlo;
      mhi = (lane == j) ? (uint32_t)(b >> 32) : mhi;
    }
    const int e = c * kWave + lane;
    if (e < N) {
      const uint64_t m = ((uint64_t)mhi << 32) | mlo;
      s_mask[e] = m;
      hist[(size_t)e * ntiles + tile] = __popcll(m);
    }
  }
  __syncthreads();
  if (active) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        const int e = ix[j];
        const int r = (e >= 0 && e < N) ? __popcll(s_mask[e] & below) : 0;
        rank_ws[(size_t)t * K + j] = (uint8_t)r;
      }
    }
  }
}

// Exclusive scan of hist[e][0..ntiles) in place; counts[e] = the column total.
__global__ __launch_bounds__(256) void k_tile_scan(int32_t *__restrict__ hist,
                                                   int32_t *__restrict__ counts, int ntiles) {
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  int32_t *col = hist + (size_t)e * ntiles;
  const int tid = threadIdx.x;
  const int per = (ntiles + 255) / 256;
  const int beg = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (beg + i < ntiles) local += col[beg + i];
  const int incl = wave_incl_scan(local);
  const int w = tid >> 6, lane = tid & 63;
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int i = 0; i < w; ++i) wave_base += s_wave[i];
  int run = wave_base + incl - local;
  for (int i = 0; i < per; ++i) {
    if (beg + i < ntiles) {
      const int h = col[beg + i];
      col[beg + i] = run;
      run += h;
    }
  }
  if (tid == 255) counts[e] = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
}

__global__ __launch_bounds__(64) void k_assign(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ base,
    const uint8_t *__restrict__ rank_ws, const int32_t *__restrict__ counts,
    int32_t *__restrict__ dest_rank, int32_t *__restrict__ dest_row,
    uint8_t *__restrict__ drop_mask, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_src, int T, int N, int K, int C, int E_L, int ep_size,
    int ep_rank, int ntiles) {
  __shared__ int s_g[MOE_MAX_EXPERTS + 1];  // exclusive scan of min(counts, C)
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  {
    const int per = (N + kWave - 1) / kWave;
    const int beg = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (beg + i < N) local += min(counts[beg + i], C);
    const int incl = wave_incl_scan(local);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      if (beg + i < N) {
        s_g[beg + i] = run;
        run += min(counts[beg + i], C);
      }
    }
    if (lane == 63) s_g[N] = incl;
  }
  __syncthreads();
  if (tile == 0) {
    const int n_off = ep_size * (E_L + 1);
    for (int i = lane; i < n_off; i += kWave) {
      const int r = i / (E_L + 1), j = i % (E_L + 1);
      offsets[i] = s_g[r * E_L + j] - s_g[r * E_L];
    }
  }
  const int t = tile * kRouteTile + lane;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const size_t q = (size_t)t * K + k;
      const int e = ids[q];
      int drk = -1, drw = -1;
      uint8_t drop = 0;
      if (e >= 0 && e < N) {
        const int p = base[(size_t)e * ntiles + tile] + (int)rank_ws[q];
        if (p < C) {
          const int r = e / E_L;
          drk = r;
          drw = s_g[e] - s_g[r * E_L] + p;
          if (row_src != nullptr && r == ep_rank) row_src[drw] = (int32_t)q;
        } else {
          drop = 1;
        }
      }
      dest_rank[q] = drk;
      dest_row[q] = drw;
      drop_mask[q] = drop;
    }
  }
  if (row_src != nullptr) {
    const int used = s_g[(ep_rank + 1) * E_L] - s_g[ep_rank * E_L];
    const int64_t rows = (int64_t)E_L * C;
    for (int64_t r = used + (int64_t)tile * kWave + lane; r < rows; r += (int64_t)ntiles * kWave)
      row_src[r] = -1;
  }
}

template <int KM>
void launch_tile(const moe_shape_t &s, const float *logits, const int32_t *ids_in,
                 const moe_route_out_t &o, int32_t *hist, uint8_t *rank_ws, int ntiles,
                 hipStream_t st) {
  if (logits != nullptr)
    hipLaunchKernelGGL((k_route_tile<KM, true>), dim3(ntiles), dim3(64), 0, st, logits,
                       nullptr, o.topk_idx, o.topk_w, hist, rank_ws, s.T, s.N, s.K, ntiles);
  else
    hipLaunchKernelGGL((k_route_tile<KM, false>), dim3(ntiles), dim3(64), 0, st, nullptr,
                       ids_in, nullptr, nullptr, hist, rank_ws, s.T, s.N, s.K, ntiles);
}

}  // namespace

int launch_route(const moe_shape_t &s, const float *logits, const int32_t *ids_in,
                 const moe_route_out_t &o, void *ws, hipStream_t st) {
  const int ntiles = route_tiles(s);
  int32_t *hist = static_cast<int32_t *>(ws);
  uint8_t *rank_ws = reinterpret_cast<uint8_t *>(hist + (size_t)s.N * ntiles);
  if (s.K <= 2) launch_tile<2>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  else if (s.K <= 4) launch_tile<4>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  else if (s.K <= 8) launch_tile<8>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  else launch_tile<16>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  if (launch_status() != MOE_OK) return MOE_EHIP;
  hipLaunchKernelGGL(k_tile_scan, dim3(s.N), dim3(256), 0, st, hist, o.counts, ntiles);
  if (launch_status() != MOE_OK) return MOE_EHIP;
  const int32_t *ids = logits != nullptr ? o.topk_idx : ids_in;
  const int E_L = s.N / s.ep_size;
  hipLaunchKernelGGL(k_assign, dim3(ntiles), dim3(64), 0, st, ids, hist, rank_ws, o.counts,
                     o.dest_rank, o.dest_row, o.drop_mask, o.offsets, o.row_src, s.T, s.N,
                     s.K, s.capacity, E_L, s.ep_size, s.ep_rank, ntiles);
  return launch_status();
}

}  // namespace moe
