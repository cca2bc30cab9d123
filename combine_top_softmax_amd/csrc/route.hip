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
//   k_route_tile   one 4-wave block per 64-token tile: top-K selection with
//                  one DPP quad of 4 lanes per token (sorted 64-bit keys per
//                  lane, K rounds of a quad-wide max), fp64 softmax over the K
//                  winners, then per expert a wave ballot of "my token routes
//                  to e" (lane = token); the ballot masks go to LDS,
//                  popcount(mask) is the tile histogram and
//                  popcount(mask & lanes-below) the in-tile rank.
//   k_tile_scan    one block per expert: exclusive scan of its tile histogram
//                  column -> tile bases; the total is counts[e].
//   k_assign       one wave per tile: every block rebuilds the exclusive scan
//                  of min(counts, C) over experts in LDS, then p = base + rank,
//                  keep iff p < C, row = offset of e on its rank + p.
// Small route maps (N <= 256, <= 256 tiles, N * tiles <= 16384) take two kernels:
// k_assign_scan does the work of the last two, each block summing the
// histogram columns itself.
//
// Workspace: hist/base [N][ntiles] int32, then rank [T*K] uint8.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kRouteWaves = 4;    // waves per 64-token routing tile
constexpr int kTokLanes = 4;      // lanes per token while selecting (one DPP quad)

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Sort key of (logit x, expert id) for the order "logit descending, id
// ascending" that a stable sort of -logit gives: IEEE comparison, so -0.0 and
// +0.0 are one value; -inf is the smallest number; NaN after every number,
// NaNs in id order. High word: the value's rank (0 for NaN); low word: ~id.
// Key 0 is an empty slot. Keys of distinct ids are distinct.
__device__ __forceinline__ uint64_t route_key(float x, int id) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;                            // -0.0 -> +0.0
  uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if ((u & 0x7fffffffu) > 0x7f800000u) hi = 0u;             // NaN
  return ((uint64_t)hi << 32) | (uint32_t)~(uint32_t)id;
}

__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  if (hi == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}

__device__ __forceinline__ int route_key_id(uint64_t key) {
  return key == 0 ? -1 : (int)~(uint32_t)key;
}

// Insert x into k[] kept in descending order; the smallest key falls off.
template <int KM>
__device__ __forceinline__ void key_insert(uint64_t (&k)[KM], uint64_t x) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const uint64_t a = k[j];
    const bool sw = x > a;
    k[j] = sw ? x : a;
    x = sw ? a : x;
  }
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf,
                                                            false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL,
                                                            0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}

// Largest key over the 4 lanes of each quad (quad_perm [1,0,3,2], [2,3,0,1]).
__device__ __forceinline__ uint64_t quad_max_key(uint64_t v) {
  uint64_t o = dpp_u64<0xb1>(v);
  v = o > v ? o : v;
  o = dpp_u64<0x4e>(v);
  return o > v ? o : v;
}

// Quad lane L's value, in every lane of the quad (quad_perm [L,L,L,L]).
template <int L>
__device__ __forceinline__ double quad_bcast(double v) {
  return __builtin_bit_cast(double, dpp_u64<L * 0x55>(__builtin_bit_cast(uint64_t, v)));
}

// Route tile: 64 tokens, 4 waves. Selection (from logits): wave w takes
// tokens 16w .. 16w+15, one DPP quad of 4 lanes each; lane s of a quad keeps
// the sorted top keys of logits 4s..4s+3 (+ 16 r), then K rounds take the
// quad's largest head key (the lane that held it drops it), so every lane of
// the quad sees the K winners in order; lane s owns slots s, s+4, s+8, s+12.
// Softmax: each owner forms exp(l_j - m) in fp64, every lane of the quad sums
// the K terms in slot order (quad broadcasts), weights rounded once to fp32.
// Ballots (lane = token): wave w builds the masks of experts 16w .. 16w+15 of
// each 64-expert chunk; ranks: wave w takes the slots j with j % 4 == w.
template <int KM, bool FROM_LOGITS>
__global__ __launch_bounds__(64 * kRouteWaves) void k_route_tile(
    const float *__restrict__ logits, const int32_t *__restrict__ ids_in,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int32_t *__restrict__ hist, uint8_t *__restrict__ rank_ws,
    int T, int N, int K, int ntiles) {
  constexpr int TPW = kWave / kTokLanes;                 // tokens per wave
  constexpr int SPL = (KM + kTokLanes - 1) / kTokLanes;  // slots per lane
  static_assert(kRouteTile == TPW * kRouteWaves, "route tile layout");
  __shared__ uint64_t s_mask[MOE_MAX_EXPERTS];
  __shared__ int32_t s_ix[KM * kRouteTile];   // slot-major: s_ix[j * 64 + token]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;
  const int t0 = tile * kRouteTile;

  if constexpr (FROM_LOGITS) {
    const int s = lane & (kTokLanes - 1);
    const int tt = TPW * wv + lane / kTokLanes;   // token within the tile
    const int t = t0 + tt;
    uint64_t key[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) key[j] = 0;
    if (t < T) {
      const float *row = logits + (size_t)t * N;
      if ((N & 3) == 0) {
        // up to 4 vector loads in flight per lane (all of a 64-expert row)
        constexpr int LPI = 4;
        for (int b0 = 4 * s; b0 < N; b0 += 4 * kTokLanes * LPI) {
          f32x4_t f[LPI];
#pragma unroll
          for (int u = 0; u < LPI; ++u) {
            const int e0 = b0 + 4 * kTokLanes * u;
            if (e0 < N)
              f[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(row + e0));
          }
#pragma unroll
          for (int u = 0; u < LPI; ++u) {
            const int e0 = b0 + 4 * kTokLanes * u;
            if (e0 < N) {
              key_insert<KM>(key, route_key(f[u].x, e0 + 0));
              key_insert<KM>(key, route_key(f[u].y, e0 + 1));
              key_insert<KM>(key, route_key(f[u].z, e0 + 2));
              key_insert<KM>(key, route_key(f[u].w, e0 + 3));
            }
          }
        }
      } else {
        for (int e = s; e < N; e += kTokLanes) key_insert<KM>(key, route_key(row[e], e));
      }
    }
    uint64_t first = 0;   // slot 0's key
    uint64_t mine[SPL];   // slot s + 4 i's key
#pragma unroll
    for (int i = 0; i < SPL; ++i) mine[i] = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        const uint64_t m = quad_max_key(key[0]);
        if (key[0] == m) {          // this lane held the winner: drop it
#pragma unroll
          for (int i = 0; i + 1 < KM; ++i) key[i] = key[i + 1];
          key[KM - 1] = 0;
        }
        if (j == 0) first = m;
        if (s == j % kTokLanes) mine[j / kTokLanes] = m;
      }
    }
    // softmax over the K selected logits, in fp64, rounded once to fp32
    const double mx = (double)route_key_value(first);
    double ex[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i)
      ex[i] = (s + kTokLanes * i < K) ? exp((double)route_key_value(mine[i]) - mx) : 0.0;
    double sum = 0.0;             // ex_0 + ex_1 + ... in slot order
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        double o;
        switch (j % kTokLanes) {
          case 0: o = quad_bcast<0>(ex[j / kTokLanes]); break;
          case 1: o = quad_bcast<1>(ex[j / kTokLanes]); break;
          case 2: o = quad_bcast<2>(ex[j / kTokLanes]); break;
          default: o = quad_bcast<3>(ex[j / kTokLanes]); break;
        }
        sum += o;
      }
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int j = s + kTokLanes * i;
      if (j < KM) {
        const int id = route_key_id(mine[i]);
        if (j < K && t < T) {
          topk_idx[(size_t)t * K + j] = id;
          topk_w[(size_t)t * K + j] = (float)(ex[i] / sum);
        }
        s_ix[j * kRouteTile + tt] = (j < K && t < T) ? id : -1;
      }
    }
  } else {
    for (int q = tid; q < KM * kRouteTile; q += 64 * kRouteWaves) {
      const int j = q / kRouteTile, tt = q % kRouteTile, t = t0 + tt;
      s_ix[q] = (j < K && t < T) ? ids_in[(size_t)t * K + j] : -1;
    }
  }
  __syncthreads();

  // lane = token from here on
  const int t = t0 + lane;
  int ix[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) ix[j] = s_ix[j * kRouteTile + lane];

  // Per chunk of 64 experts: a ballot per expert; wave w keeps the masks of
  // experts 16w .. 16w+15 of the chunk (in those lanes), stores them to LDS
  // and writes the tile histogram.
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
    for (int jj = 0; jj < kWave / kRouteWaves; ++jj) {
      const int j = wv * (kWave / kRouteWaves) + jj;
      const uint64_t b = __ballot((mine_bits >> j) & 1ull);
      mlo = (lane == j) ? (uint32_t)b : mlo;
      mhi = (lane == j) ? (uint32_t)(b >> 32) : mhi;
    }
    const int e = c * kWave + lane;
    if (lane / (kWave / kRouteWaves) == wv && e < N) {
      const uint64_t m = ((uint64_t)mhi << 32) | mlo;
      s_mask[e] = m;
      hist[(size_t)e * ntiles + tile] = __popcll(m);
    }
  }
  __syncthreads();
  if (t < T) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K && (j % kRouteWaves) == wv) {
        const int e = ix[j];
        const int r = (e >= 0 && e < N) ? __popcll(s_mask[e] & below) : 0;
        rank_ws[(size_t)t * K + j] = (uint8_t)r;
      }
    }
  }
}

// Exclusive scan of hist[e][0..ntiles) in place; counts[e] = the column total.
// Thread i takes a run of `per` consecutive tiles; the first kScanRegs values
// of the run stay in registers between the read and the write.
constexpr int kScanRegs = 8;

__global__ __launch_bounds__(256) void k_tile_scan(int32_t *__restrict__ hist,
                                                   int32_t *__restrict__ counts, int ntiles) {
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  int32_t *col = hist + (size_t)e * ntiles;
  const int tid = threadIdx.x;
  const int per = (ntiles + 255) / 256;
  const int beg = tid * per;
  int v[kScanRegs];
  int local = 0;
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) {
    v[i] = (i < per && beg + i < ntiles) ? col[beg + i] : 0;
    local += v[i];
  }
  for (int i = kScanRegs; i < per; ++i)
    if (beg + i < ntiles) local += col[beg + i];
  const int incl = wave_incl_scan_dpp(local);
  const int w = tid >> 6, lane = tid & 63;
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int i = 0; i < w; ++i) wave_base += s_wave[i];
  int run = wave_base + incl - local;
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) {
    if (i < per && beg + i < ntiles) {
      col[beg + i] = run;
      run += v[i];
    }
  }
  for (int i = kScanRegs; i < per; ++i) {
    if (beg + i < ntiles) {
      const int h = col[beg + i];
      col[beg + i] = run;
      run += h;
    }
  }
  if (tid == 255) counts[e] = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
}

template <int KM>
__global__ __launch_bounds__(64) void k_assign(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ base,
    const uint8_t *__restrict__ rank_ws, const int32_t *__restrict__ counts,
    int32_t *__restrict__ dest_rank, int32_t *__restrict__ dest_row,
    uint8_t *__restrict__ drop_mask, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_src, int T, int N, int K, int C, int E_L, int ep_size,
    int ep_rank, int ntiles, int rows) {
  __shared__ int s_g[MOE_MAX_EXPERTS + 1];  // exclusive scan of min(counts, C)
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int t = tile * kRouteTile + lane;
  // this token's experts and in-tile ranks, loaded ahead of the scan
  int e[KM];
  uint8_t rk[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    e[k] = -1;
    rk[k] = 0;
    if (k < K && t < T) {
      e[k] = ids[(size_t)t * K + k];
      rk[k] = rank_ws[(size_t)t * K + k];
    }
  }
  {
    const int per = (N + kWave - 1) / kWave;
    const int beg = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (beg + i < N) local += min(counts[beg + i], C);
    const int incl = wave_incl_scan_dpp(local);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      if (beg + i < N) {
        s_g[beg + i] = run;
        run += min(counts[beg + i], C);
      }
    }
    if (lane == 63) s_g[N] = incl;
  }
  // position of each route in its expert: tile base + in-tile rank
  int p[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k)
    p[k] = (e[k] >= 0 && e[k] < N) ? base[(size_t)e[k] * ntiles + tile] + (int)rk[k] : -1;
  __syncthreads();
  if (tile == 0) {
    const int n_off = ep_size * (E_L + 1);
    for (int i = lane; i < n_off; i += kWave) {
      const int r = i / (E_L + 1), j = i % (E_L + 1);
      offsets[i] = s_g[r * E_L + j] - s_g[r * E_L];
    }
  }
  if (t < T) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k >= K) continue;
      const size_t q = (size_t)t * K + k;
      int drk = -1, drw = -1;
      uint8_t drop = 0;
      if (p[k] >= 0) {
        if (p[k] < C) {
          const int r = e[k] / E_L;
          drk = r;
          drw = s_g[e[k]] - s_g[r * E_L] + p[k];
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
    for (int64_t r = used + (int64_t)tile * kWave + lane; r < rows; r += (int64_t)ntiles * kWave)
      row_src[r] = -1;
  }
}

// k_assign with the tile scan folded in, for small route maps (N <= 256, at
// most 256 tiles and N * ntiles <= kFusedScanMax, i.e. at most 64 KiB of histogram per
// block and 16 MiB of L2 reads in all): every block reads the whole histogram
// and forms its own tile's bases and the expert totals, which saves the
// k_tile_scan launch and its round trip. The histogram is only read,
// so the blocks do not race. 4 waves: G = 256 / N (a power of two, <= 64)
// threads per expert sum interleaved tiles; partial sums meet in LDS; wave 0
// scans min(count, C) over the experts; then lane = token, wave w writes the
// slots k with k % 4 == w.
constexpr int kFusedScanMax = 16384;

template <int KM>
__global__ __launch_bounds__(256) void k_assign_scan(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ hist,
    const uint8_t *__restrict__ rank_ws, int32_t *__restrict__ counts,
    int32_t *__restrict__ dest_rank, int32_t *__restrict__ dest_row,
    uint8_t *__restrict__ drop_mask, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_src, int T, int N, int K, int C, int E_L, int ep_size,
    int ep_rank, int ntiles, int rows, int G) {
  __shared__ int s_below[256], s_tot[256];     // partial sums, one per thread
  __shared__ int s_base[MOE_MAX_EXPERTS];     // routes to e in the tiles before this one
  __shared__ int s_g[MOE_MAX_EXPERTS + 1];    // exclusive scan of min(counts, C)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;
  const int t = tile * kRouteTile + lane;
  // this token's experts and in-tile ranks, loaded ahead of the scan
  int e[KM];
  uint8_t rk[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    e[k] = -1;
    rk[k] = 0;
    if (k < K && (k & 3) == wv && t < T) {
      e[k] = ids[(size_t)t * K + k];
      rk[k] = rank_ws[(size_t)t * K + k];
    }
  }
  {
    // thread (expert ex, part q) sums tiles q, q + G, ... of column ex
    const int ex = tid / G, q = tid - ex * G;
    int below = 0, tot = 0;
    if (ex < N) {
      const int32_t *col = hist + (size_t)ex * ntiles;
#pragma unroll 8
      for (int tt = q; tt < ntiles; tt += G) {
        const int v = col[tt];
        tot += v;
        below += tt < tile ? v : 0;
      }
    }
    s_below[tid] = below;
    s_tot[tid] = tot;
  }
  __syncthreads();
  if (wv == 0) {
    // per lane a run of experts: totals from the partial sums, then the scan
    const int per = (N + kWave - 1) / kWave;
    const int beg = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int ex = beg + i;
      if (ex < N) {
        int b = 0, c = 0;
        for (int j = 0; j < G; ++j) {
          b += s_below[ex * G + j];
          c += s_tot[ex * G + j];
        }
        s_base[ex] = b;
        s_tot[ex * G] = c;           // the expert's total, in its first slot
        if (tile == 0) counts[ex] = c;
        local += min(c, C);
      }
    }
    const int incl = wave_incl_scan_dpp(local);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int ex = beg + i;
      if (ex < N) {
        s_g[ex] = run;
        run += min(s_tot[ex * G], C);
      }
    }
    if (lane == 63) s_g[N] = incl;
  }
  __syncthreads();
  if (tile == 0) {
    const int n_off = ep_size * (E_L + 1);
    for (int i = tid; i < n_off; i += 256) {
      const int r = i / (E_L + 1), j = i % (E_L + 1);
      offsets[i] = s_g[r * E_L + j] - s_g[r * E_L];
    }
  }
  if (t < T) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k >= K || (k & 3) != wv) continue;
      const size_t qi = (size_t)t * K + k;
      const int p = (e[k] >= 0 && e[k] < N) ? s_base[e[k]] + (int)rk[k] : -1;
      int drk = -1, drw = -1;
      uint8_t drop = 0;
      if (p >= 0) {
        if (p < C) {
          const int r = e[k] / E_L;
          drk = r;
          drw = s_g[e[k]] - s_g[r * E_L] + p;
          if (row_src != nullptr && r == ep_rank) row_src[drw] = (int32_t)qi;
        } else {
          drop = 1;
        }
      }
      dest_rank[qi] = drk;
      dest_row[qi] = drw;
      drop_mask[qi] = drop;
    }
  }
  if (row_src != nullptr) {
    const int used = s_g[(ep_rank + 1) * E_L] - s_g[ep_rank * E_L];
    for (int64_t r = used + (int64_t)tile * 256 + tid; r < rows; r += (int64_t)ntiles * 256)
      row_src[r] = -1;
  }
}

template <int KM>
int launch_route_km(const moe_shape_t &s, const float *logits, const int32_t *ids_in,
                    const moe_route_out_t &o, int32_t *hist, uint8_t *rank_ws, int ntiles,
                    hipStream_t st) {
  if (logits != nullptr)
    hipLaunchKernelGGL((k_route_tile<KM, true>), dim3(ntiles), dim3(64 * kRouteWaves), 0, st,
                       logits, nullptr, o.topk_idx, o.topk_w, hist, rank_ws, s.T, s.N, s.K,
                       ntiles);
  else
    hipLaunchKernelGGL((k_route_tile<KM, false>), dim3(ntiles), dim3(64 * kRouteWaves), 0, st,
                       nullptr, ids_in, nullptr, nullptr, hist, rank_ws, s.T, s.N, s.K, ntiles);
  if (launch_status() != MOE_OK) return MOE_EHIP;
  const int32_t *ids = logits != nullptr ? o.topk_idx : ids_in;
  const int E_L = s.N / s.ep_size;
  if (s.N <= 256 && ntiles <= 256 && s.N * ntiles <= kFusedScanMax) {
    // threads per expert: the largest power of two <= min(64, 256 / N), so that
    // the N * G partial sums fit the block's 256 threads
    int G = 1;
    while (G < 64 && 2 * G * s.N <= 256) G *= 2;
    hipLaunchKernelGGL((k_assign_scan<KM>), dim3(ntiles), dim3(256), 0, st, ids, hist, rank_ws,
                       o.counts, o.dest_rank, o.dest_row, o.drop_mask, o.offsets, o.row_src,
                       s.T, s.N, s.K, s.capacity, E_L, s.ep_size, s.ep_rank, ntiles,
                       (int)buffer_rows(s), G);
    return launch_status();
  }
  hipLaunchKernelGGL(k_tile_scan, dim3(s.N), dim3(256), 0, st, hist, o.counts, ntiles);
  if (launch_status() != MOE_OK) return MOE_EHIP;
  hipLaunchKernelGGL((k_assign<KM>), dim3(ntiles), dim3(64), 0, st, ids, hist, rank_ws, o.counts,
                     o.dest_rank, o.dest_row, o.drop_mask, o.offsets, o.row_src, s.T, s.N,
                     s.K, s.capacity, E_L, s.ep_size, s.ep_rank, ntiles, (int)buffer_rows(s));
  return launch_status();
}

}  // namespace

int launch_route(const moe_shape_t &s, const float *logits, const int32_t *ids_in,
                 const moe_route_out_t &o, void *ws, hipStream_t st) {
  const int ntiles = route_tiles(s);
  int32_t *hist = static_cast<int32_t *>(ws);
  uint8_t *rank_ws = reinterpret_cast<uint8_t *>(hist + (size_t)s.N * ntiles);
  if (s.K <= 2) return launch_route_km<2>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  if (s.K <= 4) return launch_route_km<4>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  if (s.K <= 8) return launch_route_km<8>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
  return launch_route_km<16>(s, logits, ids_in, o, hist, rank_ws, ntiles, st);
}

}  // namespace moe
