// Grouped expert SwiGLU FFN over the packed prefix of the capacity buffer.
//
// Olmo-core MoE report, Sec. 05, Sec. 5.7: the local experts' rows are packed
// back to back from row 0 and one unwritten tail follows, so the grouped GEMM
// receives the real per-expert offsets and skips the tail; Sec. 08
// "Synchronization-Free Training", Sec. 8.5: the grouped GEMM consumes an
// int32 device cumulative-offset tensor (no host loop over experts) and the
// SwiGLU is applied to the valid prefix only.
//
// Two kernels per layer:
//   up   : H[r, :] = silu(X[r] W_gate^T) * (X[r] W_up^T), SwiGLU fused into the
//          epilogue (gate and up columns of the same H column are computed by
//          the same lanes), H stored in the layer dtype;
//   down : Y[r, :] = H[r] W_d^T.
// Both are "NT" products: every operand is K-contiguous (x and H rows, and
// the [out, in] weight rows), so each lane loads 16-byte runs along K.
//
// Scheduling from device offsets: the grid is sized from the capacity bound
// (sum_j ceil(n_j/BM) <= ceil(E_L*C/BM) + E_L m-tiles); every block recomputes
// the per-expert m-tile counts from the offsets with a wave scan, maps its
// block id to a real tile and exits if there is none. The block id -> tile map
// is XCD-aware: blocks are dealt to the 8 XCDs round-robin, so block b gets
// tile (b % 8) * q + b / 8 (q = ceil(tiles / 8)) and each XCD walks a
// contiguous run of tiles (n-tiles of one m-tile, m-tiles of one expert),
// which keeps the shared A rows and expert weights in that XCD's L2.
//
// bf16 path: 128 x 128 block tile, K step 64, 4 waves of 64 x 64, each a 2 x 2
// grid of v_mfma_f32_32x32x16_bf16, LDS double buffer (rows padded by 16 bytes
// so the 16-byte fragment reads of 16 lanes cover all 64 banks once).
// fp32 path: a plain LDS-tiled SIMT kernel (64 x 64 tile, 4 x 4 per thread).
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct Tile {
  int expert;
  int row0;     // first buffer row of this m-tile
  int row_end;  // one past the expert's last valid row
  int n_idx;    // output column tile
  bool valid;
};

// Map this block to a (expert, m-tile, n-tile) from the local offsets.
// Executed redundantly by every wave of the block; the result is wave-uniform.
__device__ __forceinline__ Tile find_tile(const int32_t *__restrict__ off, int E_L, int bm,
                                          int n_tiles_n) {
  const int lane = threadIdx.x & 63;
  Tile tl;
  tl.valid = false;
  int total_m = 0;
  for (int c = 0; c < E_L; c += 64) {
    const int j = c + lane;
    const int n = (j < E_L) ? off[j + 1] - off[j] : 0;
    const int incl = wave_incl_scan((n + bm - 1) / bm);
    total_m += __shfl(incl, 63, 64);
  }
  const int total = total_m * n_tiles_n;
  const int q = (total + kNumXcd - 1) / kNumXcd;
  const int b = blockIdx.x;
  const int slot = b / kNumXcd;
  const int L = (b % kNumXcd) * q + slot;
  if (slot >= q || L >= total) return tl;
  const int m_idx = L / n_tiles_n;
  tl.n_idx = L - m_idx * n_tiles_n;
  int run = 0;
  for (int c = 0; c < E_L; c += 64) {
    const int j = c + lane;
    const int n = (j < E_L) ? off[j + 1] - off[j] : 0;
    const int mt = (n + bm - 1) / bm;
    const int incl = wave_incl_scan(mt);
    const int tot = __shfl(incl, 63, 64);
    if (m_idx < run + tot) {
      const uint64_t hit = __ballot(m_idx < run + incl);
      const int first = __builtin_ctzll(hit);
      const int excl = __shfl(incl - mt, first, 64);
      const int e = c + first;
      const int o0 = off[e];
      tl.expert = e;
      tl.row0 = o0 + (m_idx - run - excl) * bm;
      tl.row_end = off[e + 1];
      tl.valid = true;
      return tl;
    }
    run += tot;
  }
  return tl;
}

// ------------------------------------------------------------------ bf16 MFMA
constexpr int kBM = 128;        // rows per block tile
constexpr int kBW = 128;        // weight rows per block tile
constexpr int kBK = 64;         // K per main-loop step
constexpr int kLds = kBK + 8;   // padded LDS row (elements)

template <bool GATE_UP>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const int32_t *__restrict__ off, uint16_t *__restrict__ Out, int E_L, int Kdim,
    int Nout, int n_tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBW * kLds];

  const Tile tl = find_tile(off, E_L, kBM, n_tiles_n);
  if (!tl.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int Nw = GATE_UP ? 2 * Nout : Nout;
  const uint16_t *Wj = W + (size_t)tl.expert * Nw * Kdim;
  const int kv = tid & 7;            // 16-byte vector within a 64-element K step
  const int n0 = tl.n_idx * (GATE_UP ? kBW / 2 : kBW);

  const uint16_t *a_ptr[4];
  const uint16_t *b_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int grow = min(tl.row0 + r, tl.row_end - 1);  // rows past the expert: clamped, discarded
    a_ptr[i] = A + (size_t)grow * Kdim + kv * 8;
    int wrow;
    if (GATE_UP)
      wrow = (r < kBW / 2) ? min(n0 + r, Nout - 1) : Nout + min(n0 + r - kBW / 2, Nout - 1);
    else
      wrow = min(n0 + r, Nout - 1);
    b_ptr[i] = Wj + (size_t)wrow * Kdim + kv * 8;
  }

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const bool ok = k0 + kv * 8 < Kdim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ok ? *reinterpret_cast<const uint4 *>(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = ok ? *reinterpret_cast<const uint4 *>(b_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4 *>(&sA[s][r * kLds + kv * 8]) = ra[i];
      *reinterpret_cast<uint4 *>(&sB[s][r * kLds + kv * 8]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (Kdim + kBK - 1) / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 31;          // fragment row within a 32-row MFMA tile
  const int fk = (lane >> 5) * 8;    // fragment K offset within a 16-wide K step
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nk) gload((kb + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        a[ms] = *reinterpret_cast<const bf16x8_t *>(
            &sA[cur][(wm * 64 + ms * 32 + fr) * kLds + ks * 16 + fk]);
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        const int brow = GATE_UP ? (ns * (kBW / 2) + wn * 32) : (wn * 64 + ns * 32);
        b[ns] = *reinterpret_cast<const bf16x8_t *>(&sB[cur][(brow + fr) * kLds + ks * 16 + fk]);
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ms], b[ns], acc[ms][ns], 0, 0, 0);
    }
    if (kb + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue. 32x32 MFMA result layout: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 tile.
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row_l = wm * 64 + ms * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const int grow = tl.row0 + row_l;
      if (grow >= tl.row_end) continue;
      uint16_t *orow = Out + (size_t)grow * Nout;
      if (GATE_UP) {
        const int col = n0 + wn * 32 + fr;
        const float g = acc[ms][0][r], u = acc[ms][1][r];
        const float hv = g / (1.0f + __expf(-g)) * u;
        if (col < Nout) orow[col] = f2bf(hv);
      } else {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const int col = n0 + wn * 64 + ns * 32 + fr;
          if (col < Nout) orow[col] = f2bf(acc[ms][ns][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 SIMT
constexpr int kFM = 64, kFW = 64, kFK = 16;

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_gemm_f32(
    const float *__restrict__ A, const float *__restrict__ W, const int32_t *__restrict__ off,
    float *__restrict__ Out, int E_L, int Kdim, int Nout, int n_tiles_n) {
  __shared__ float sA[kFK][kFM + 1];
  __shared__ float sB[kFK][kFW + 1];
  const Tile tl = find_tile(off, E_L, kFM, n_tiles_n);
  if (!tl.valid) return;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int Nw = GATE_UP ? 2 * Nout : Nout;
  const float *Wj = W + (size_t)tl.expert * Nw * Kdim;
  const int n0 = tl.n_idx * (GATE_UP ? kFW / 2 : kFW);
  const int lr = tid >> 2, kq = (tid & 3) * 4;
  const float *a_ptr = A + (size_t)min(tl.row0 + lr, tl.row_end - 1) * Kdim + kq;
  int wrow;
  if (GATE_UP)
    wrow = (lr < kFW / 2) ? min(n0 + lr, Nout - 1) : Nout + min(n0 + lr - kFW / 2, Nout - 1);
  else
    wrow = min(n0 + lr, Nout - 1);
  const float *b_ptr = Wj + (size_t)wrow * Kdim + kq;
  int wsel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wsel[j] = GATE_UP ? ((j < 2) ? tx * 2 + j : kFW / 2 + tx * 2 + (j - 2)) : tx * 4 + j;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kdim; k0 += kFK) {
    const bool ok = k0 + kq < Kdim;
    const float4 av = ok ? *reinterpret_cast<const float4 *>(a_ptr + k0) : make_float4(0, 0, 0, 0);
    const float4 bv = ok ? *reinterpret_cast<const float4 *>(b_ptr + k0) : make_float4(0, 0, 0, 0);
    __syncthreads();
    sA[kq + 0][lr] = av.x; sA[kq + 1][lr] = av.y; sA[kq + 2][lr] = av.z; sA[kq + 3][lr] = av.w;
    sB[kq + 0][lr] = bv.x; sB[kq + 1][lr] = bv.y; sB[kq + 2][lr] = bv.z; sB[kq + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][wsel[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = tl.row0 + ty * 4 + i;
    if (grow >= tl.row_end) continue;
    float *orow = Out + (size_t)grow * Nout;
    if (GATE_UP) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = n0 + tx * 2 + c;
        const float g = acc[i][c], u = acc[i][c + 2];
        if (col < Nout) orow[col] = g / (1.0f + expf(-g)) * u;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = n0 + tx * 4 + c;
        if (col < Nout) orow[col] = acc[i][c];
      }
    }
  }
}

// Grid: every possible m-tile times the n-tiles, rounded up to the XCD count.
inline unsigned grid_blocks(const moe_shape_t &s, int bm, int n_tiles_n) {
  const int E_L = s.N / s.ep_size;
  const int64_t max_m = ceil_div((int64_t)E_L * s.capacity, bm) + E_L;
  return (unsigned)(ceil_div(max_m * n_tiles_n, kNumXcd) * kNumXcd);
}

}  // namespace

int launch_expert_up(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                     const void *w_gu, void *h, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  if (s.dtype == MOE_BF16) {
    const int ntn = (int)ceil_div(s.F, kBW / 2);
    hipLaunchKernelGGL(k_gemm_bf16<true>, dim3(grid_blocks(s, kBM, ntn)), dim3(256), 0, st,
                       static_cast<const uint16_t *>(buf), static_cast<const uint16_t *>(w_gu),
                       off, static_cast<uint16_t *>(h), E_L, s.d, s.F, ntn);
  } else {
    const int ntn = (int)ceil_div(s.F, kFW / 2);
    hipLaunchKernelGGL(k_gemm_f32<true>, dim3(grid_blocks(s, kFM, ntn)), dim3(256), 0, st,
                       static_cast<const float *>(buf), static_cast<const float *>(w_gu), off,
                       static_cast<float *>(h), E_L, s.d, s.F, ntn);
  }
  return launch_status();
}

int launch_expert_down(const moe_shape_t &s, const void *h, const int32_t *offsets,
                       const void *w_d, void *y, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  if (s.dtype == MOE_BF16) {
    const int ntn = (int)ceil_div(s.d, kBW);
    hipLaunchKernelGGL(k_gemm_bf16<false>, dim3(grid_blocks(s, kBM, ntn)), dim3(256), 0, st,
                       static_cast<const uint16_t *>(h), static_cast<const uint16_t *>(w_d), off,
                       static_cast<uint16_t *>(y), E_L, s.F, s.d, ntn);
  } else {
    const int ntn = (int)ceil_div(s.d, kFW);
    hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid_blocks(s, kFM, ntn)), dim3(256), 0, st,
                       static_cast<const float *>(h), static_cast<const float *>(w_d), off,
                       static_cast<float *>(y), E_L, s.F, s.d, ntn);
  }
  return launch_status();
}

}  // namespace moe
