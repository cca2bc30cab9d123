// Backward of the MoE layer.
//
// Olmo-core MoE report, Sec. 05 "Expert Parallelism", Sec. 5.6 Table 8: the
// backward reverses each forward movement with the same saved route map --
// combine backward pushes each router-weighted output gradient to the
// expert-output-gradient row of its route, dispatch backward pulls the route
// gradients and sums them into the token's gradient, and the router-weight
// gradient uses the gathered expert outputs with the token-output gradient of
// the same accepted routes. Sec. 5.7: the expert GEMMs of the backward run over
// the valid prefix only (the unwritten tail is skipped).
//
// Kernels:
//   k_combine_bwd  wave per token: reads dOut[t] once per row segment, writes
//                  w * dOut[t] to the dY row of each kept local route and the
//                  dot <dOut[t], Y[row]> (a DPP wave sum) as that route's
//                  weight gradient (0 for every other route).
//   k_route_bwd    wave per token: logit gradient through the softmax over the
//                  K selected logits, zero on the experts not selected.
//   k_gemm_bwd     (bf16, MFMA) / k_gemm_bwd_f32 (fp32, SIMT): one grouped
//                  GEMM for the four products of the expert backward:
//                    DH: dH = dY W_d per expert over its rows, fused with the
//                        SwiGLU backward on G, U -> [dG dU]
//                    DX: dX = [dG dU] W_gu per expert over its rows
//                    WG: dW = P^T Q per expert, contracted over the expert's
//                        rows (dW_d = dY^T H, dW_gu = [dG dU]^T X), fp32 out;
//                        an expert without rows gets zeros.
//                  The weights are N-contiguous in these products and the
//                  weight-gradient left operand is M-contiguous; the bf16
//                  kernel transposes those tiles while writing them to LDS, so
//                  every MFMA operand is read K-contiguous.
// G, U are recomputed by the forward NT GEMM (no activation, 2F columns), or
// taken from the rows the up GEMM kept during the forward;
// dispatch backward is the forward combine kernel with unit weights.
#include <type_traits>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 4;   // 4 waves = 4 token rows per 256-thread block

// v plus the DPP-moved value of v (lanes without a source add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// Sum of v over the 64 lanes, returned to every lane: the DPP inclusive scan
// (shifts by 1, 2, 4, 8 inside each row of 16, then the row-15 and row-31
// broadcasts) leaves the total in lane 63. All lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v = add_dpp<0x111, 0xf>(v);   // row_shr:1
  v = add_dpp<0x112, 0xf>(v);   // row_shr:2
  v = add_dpp<0x114, 0xf>(v);   // row_shr:4
  v = add_dpp<0x118, 0xf>(v);   // row_shr:8
  v = add_dpp<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = add_dpp<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// ------------------------------------------------------------ combine backward
// The token's route metadata is read once (lane k: route k) and a ballot marks
// the kept local routes, taken two at a time in k order with both Y rows loaded
// before either is used. FULL: the row is a whole number of segments.
template <bool BF16, int NV, bool FULL>
__global__ __launch_bounds__(256) void k_combine_bwd(
    const u32x4_t *__restrict__ dout, const u32x4_t *__restrict__ y,
    const int32_t *__restrict__ dest_rank, const int32_t *__restrict__ dest_row,
    const float *__restrict__ w, u32x4_t *__restrict__ dy, float *__restrict__ dw, int T, int K,
    int nvec, int ep_rank, int rows) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6));
  if (t >= T) return;
  const size_t q0 = (size_t)t * K;
  int m_rank = -1, m_row = 0;
  float m_w = 0.f;
  if (lane < K) {
    m_rank = dest_rank[q0 + lane];
    m_row = dest_row[q0 + lane];
    m_w = w[q0 + lane];
  }
  // a local route whose row lies outside the buffer is skipped (dw = 0)
  const uint64_t local = __ballot(m_rank == ep_rank && (unsigned)m_row < (unsigned)rows);
  float dw_mine = 0.f;   // lane k < K accumulates route k's weight gradient
  // dY row segment = w * dOut; returns this lane's part of <dOut, Y[row]>
  auto route = [&](const u32x4_t (&g)[NV], const u32x4_t (&yv)[NV], size_t row, float wk,
                   int seg) {
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = seg + i * 64 + lane;
      if (!FULL && c >= nvec) continue;
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
          const float g0 = bf16_lo(g[i][e]), g1 = bf16_hi(g[i][e]);
          dot = fmaf(g0, bf16_lo(yv[i][e]), dot);
          dot = fmaf(g1, bf16_hi(yv[i][e]), dot);
          o[e] = pack_bf16x2(wk * g0, wk * g1);
        } else {
          const float g0 = __uint_as_float(g[i][e]);
          dot = fmaf(g0, __uint_as_float(yv[i][e]), dot);
          o[e] = __float_as_uint(wk * g0);
        }
      }
      dy[row * nvec + c] = o;
    }
    return dot;
  };
  for (int seg = 0; seg < nvec; seg += 64 * NV) {
    u32x4_t g[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = seg + i * 64 + lane;
      g[i] = (FULL || c < nvec) ? __builtin_nontemporal_load(dout + (size_t)t * nvec + c)
                                : u32x4_t{0, 0, 0, 0};
    }
    for (uint64_t rest = local; rest != 0;) {
      const int ka = __builtin_ctzll(rest);
      rest &= rest - 1;
      const bool hb = rest != 0;
      const int kb = hb ? __builtin_ctzll(rest) : ka;
      if (hb) rest &= rest - 1;
      const size_t ra = (size_t)__builtin_amdgcn_readlane(m_row, ka);
      const size_t rb = (size_t)__builtin_amdgcn_readlane(m_row, kb);
      u32x4_t ya[NV], yb[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = seg + i * 64 + lane;
        if (FULL || c < nvec) {   // read once: nontemporal (as the forward combine)
          ya[i] = __builtin_nontemporal_load(y + ra * nvec + c);
          if (hb) yb[i] = __builtin_nontemporal_load(y + rb * nvec + c);
        }
      }
      const float da = wave_sum(route(g, ya, ra, __builtin_bit_cast(float,
                                __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_w), ka)), seg));
      if (lane == ka) dw_mine += da;
      if (hb) {
        const float db = wave_sum(route(g, yb, rb, __builtin_bit_cast(float,
                                  __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_w), kb)), seg));
        if (lane == kb) dw_mine += db;
      }
    }
  }
  if (lane < K) dw[q0 + lane] = dw_mine;
}

// ------------------------------------------------------------ router backward
// dl[t, idx[t,k]] = w[t,k] * (dw[t,k] - sum_j w[t,j] dw[t,j]); 0 elsewhere.
__global__ __launch_bounds__(256) void k_route_bwd(const int32_t *__restrict__ idx,
                                                   const float *__restrict__ w,
                                                   const float *__restrict__ dw,
                                                   float *__restrict__ dl, int T, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6));
  if (t >= T) return;
  const size_t base = (size_t)t * K;
  float inner = 0.f;
  for (int k = 0; k < K; ++k) inner = fmaf(w[base + k], dw[base + k], inner);
  for (int e = lane; e < N; e += 64) {
    float v = 0.f;
    for (int k = 0; k < K; ++k)
      if (idx[base + k] == e) v = w[base + k] * (dw[base + k] - inner);
    dl[(size_t)t * N + e] = v;
  }
}

// ------------------------------------------------------------ grouped GEMMs
enum { BW_DH = 0, BW_DX = 1, BW_WG = 2 };

// Problem of one block: expert, output tile origin, valid rows, contraction range.
struct Work {
  int expert, m0, m_end, n0, kbeg, kend;
};

// Arguments shared by both element types.
//   A(m, k) = A[m*lda + k] (DH, DX: rows of the expert)   or
//   A(m, k) = A[(kbeg+k)*lda + m] (WG: M-contiguous rows of the expert)
//   B(k, n) = Bj[(kbeg+k)*ldb + n], Bj = B + expert * b_expert_stride
//   DH: N = F, K = d;  DX: N = d, K = 2F;  WG: M x N per expert, K = its rows
struct GemmArgs {
  const void *A;
  int lda;
  const void *B;
  int ldb;
  int64_t b_expert_stride;
  const int32_t *off;
  int E_L, M, N, Kdim;
  int rows;         // buffer rows: offsets are clamped into [0, rows]
  const void *gu;   // DH: pre-activation [G U] rows (recomputed or saved), [rows, 2F]
  int F;
  void *Out;
  int ldo;
  int64_t out_expert_stride;   // WG
  int n_tiles_n, m_tiles;
};

template <int MODE>
__device__ __forceinline__ bool get_work(const GemmArgs &p, int tm, int tn, Work &w) {
  if constexpr (MODE == BW_WG) {
    // tiles numbered expert by expert (n fastest); XCD-aware order as above,
    // so each XCD works through whole experts and their rows stay in its L2
    const int total = p.E_L * p.m_tiles * p.n_tiles_n;
    const int q = (total + kNumXcd - 1) / kNumXcd;
    const int slot = blockIdx.x / kNumXcd;
    const int b = (blockIdx.x % kNumXcd) * q + slot;
    if (slot >= q || b >= total) return false;
    w.expert = b / (p.m_tiles * p.n_tiles_n);
    w.m0 = ((b / p.n_tiles_n) % p.m_tiles) * tm;
    w.n0 = (b % p.n_tiles_n) * tn;
    w.m_end = p.M;
    w.kbeg = min(max(p.off[w.expert], 0), p.rows);
    w.kend = min(max(p.off[w.expert + 1], w.kbeg), p.rows);
    return true;
  } else {
    const RowTile tl = find_row_tile(p.off, p.E_L, tm, p.rows, p.n_tiles_n);
    if (!tl.valid) return false;
    w.expert = tl.expert;
    w.m0 = tl.row0;
    w.m_end = tl.row_end;
    w.n0 = tl.n_idx * tn;
    w.kbeg = 0;
    w.kend = p.Kdim;
    return true;
  }
}

// One output element: SwiGLU backward (DH), a dX row element (DX) or a
// weight-gradient element (WG). T is the element type of the row tensors.
template <int MODE, typename T>
__device__ __forceinline__ void store_elem(const GemmArgs &p, const Work &w, int row, int col,
                                           float v) {
  if constexpr (MODE == BW_DH) {
    const T *gr = static_cast<const T *>(p.gu) + (size_t)row * 2 * p.F;
    T *o = static_cast<T *>(p.Out) + (size_t)row * p.ldo;
    float g, u;
    if constexpr (sizeof(T) == 2) {
      g = __uint_as_float((uint32_t)gr[col] << 16);
      u = __uint_as_float((uint32_t)gr[p.F + col] << 16);
    } else {
      g = gr[col];
      u = gr[p.F + col];
    }
    const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
    const float dg = v * u * s * (1.0f + g * (1.0f - s));
    const float du = v * g * s;
    if constexpr (sizeof(T) == 2) {
      o[col] = f2bf(dg);
      o[p.F + col] = f2bf(du);
    } else {
      o[col] = dg;
      o[p.F + col] = du;
    }
  } else if constexpr (MODE == BW_DX) {
    T *o = static_cast<T *>(p.Out) + (size_t)row * p.ldo;
    if constexpr (sizeof(T) == 2) o[col] = f2bf(v);
    else o[col] = v;
  } else {
    static_cast<float *>(p.Out)[w.expert * p.out_expert_stride + (int64_t)row * p.ldo + col] = v;
  }
}

// ---- bf16: 128 x 128 tile, K step 32, 4 waves of 64 x 64 (2 x 2 MFMA 32x32x16)
constexpr int kT = 128;
constexpr int kK = 32;
constexpr int kLd = kK + 8;   // LDS row: 40 bf16 = 80 bytes (16-byte aligned, skewed banks)

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_bwd(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kT * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kT * kLd];
  constexpr bool A_MCONTIG = MODE == BW_WG;
  Work wk;
  if (!get_work<MODE>(p, kT, kT, wk)) return;
  const uint16_t *A = static_cast<const uint16_t *>(p.A);
  const uint16_t *Bj = static_cast<const uint16_t *>(p.B) +
                       (MODE == BW_WG ? 0 : (int64_t)wk.expert * p.b_expert_stride);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  u32x4_t ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i;
      if constexpr (!A_MCONTIG) {
        const int m = v >> 2, kv = v & 3;
        const int mg = min(wk.m0 + m, wk.m_end - 1);   // rows past the expert: discarded
        const int k = k0 + kv * 8;
        ra[i] = (k < wk.kend) ? *reinterpret_cast<const u32x4_t *>(A + (size_t)mg * p.lda + k)
                              : u32x4_t{0, 0, 0, 0};
      } else {
        const int kk = v >> 4, mv = v & 15;
        const int r = wk.kbeg + k0 + kk;
        const int m = wk.m0 + mv * 8;
        ra[i] = (r < wk.kend && m < p.M)
                    ? *reinterpret_cast<const u32x4_t *>(A + (size_t)r * p.lda + m)
                    : u32x4_t{0, 0, 0, 0};
      }
      const int kk = v >> 4, nv = v & 15;
      const int kr = wk.kbeg + k0 + kk;
      const int n = wk.n0 + nv * 8;
      rb[i] = (kr < wk.kend && n < p.N)
                  ? *reinterpret_cast<const u32x4_t *>(Bj + (size_t)kr * p.ldb + n)
                  : u32x4_t{0, 0, 0, 0};
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + 256 * i;
      if constexpr (!A_MCONTIG) {
        const int m = v >> 2, kv = v & 3;
        *reinterpret_cast<u32x4_t *>(&sA[m * kLd + kv * 8]) = ra[i];
      } else {
        const int kk = v >> 4, mv = v & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sA[(mv * 8 + 2 * e) * kLd + kk] = (uint16_t)(ra[i][e] & 0xffff);
          sA[(mv * 8 + 2 * e + 1) * kLd + kk] = (uint16_t)(ra[i][e] >> 16);
        }
      }
      const int kk = v >> 4, nv = v & 15;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sB[(nv * 8 + 2 * e) * kLd + kk] = (uint16_t)(rb[i][e] & 0xffff);
        sB[(nv * 8 + 2 * e + 1) * kLd + kk] = (uint16_t)(rb[i][e] >> 16);
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (wk.kend - wk.kbeg + kK - 1) / kK;
  const int fr = lane & 31, khalf = lane >> 5;
  if (nk > 0) {
    gload(0);
    sstore();
    __syncthreads();
  }
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) gload((kb + 1) * kK);
#pragma unroll
    for (int ks = 0; ks < kK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        a[ms] = *reinterpret_cast<const bf16x8_t *>(
            &sA[(wm * 64 + ms * 32 + fr) * kLd + ks * 16 + khalf * 8]);
#pragma unroll
      for (int ns = 0; ns < 2; ++ns)
        b[ns] = *reinterpret_cast<const bf16x8_t *>(
            &sB[(wn * 64 + ns * 32 + fr) * kLd + ks * 16 + khalf * 8]);
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ms], b[ns], acc[ms][ns], 0, 0, 0);
    }
    __syncthreads();
    if (kb + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wk.m0 + wm * 64 + ms * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
        const int col = wk.n0 + wn * 64 + ns * 32 + fr;
        if (row < wk.m_end && col < p.N) store_elem<MODE, uint16_t>(p, wk, row, col, acc[ms][ns][r]);
      }
}

// ---- bf16 big tiles: the forward's pipeline for operands of any layout.
// 256 x 256 block tile, K step 64, two LDS stages, 8 waves of 128 x 64 (4 x 2
// MFMA 32x32x16 tiles each),
// operands loaded global -> LDS directly and the
// loads of step k+1 issued between the MFMAs of step k (as in the forward).
// Two LDS tile layouts per stage (32 KiB per operand):
//   K-contiguous (A of DH, DX): 256 rows of 64 k (128 B), chunk-swizzled as in
//     the forward, fragments read with ds_read_b128;
//   MN-contiguous (B always, A of WG): 64 k-rows of 256 m or n (512 B); the
//     16-byte chunk c of k-row r is stored at c ^ 4*(r % 4). Fragments are read
//     with the LDS transpose read ds_read_b64_tr_b16: in each 16-lane group,
//     lane 4j+a points at k-row j, columns 4a..4a+3 of the group's 16
//     columns, and lane i receives column i of the four k-rows. Two such reads
//     (k-rows +0..3, +4..7) give a lane its 8 k-values; the swizzle puts the
//     4 k-rows x 4 chunks that two 16-lane groups read at once in 16 distinct
//     16-byte bank groups.
// Weight gradients contract over a ragged row range: loads clamp the row to
// the expert's last one (in bounds, finite) and the last partial step zeroes
// the B rows past the range in LDS before its MFMAs.
// Waves per block: 8 (128 x 64 wave tiles) measured 3-4% faster here than 4
// (128 x 128), the reverse of the forward kernel.
namespace bt {
constexpr int BM = 256, BN = 256, BK = 64, NW = 8, NT = 64 * NW;
constexpr int WAVES_N = NW / 2;        // 2 wave rows of 128 x WAVES_N wave columns
constexpr int WTN = BN / WAVES_N;      // output columns per wave
constexpr int TM = 4, TN = WTN / 32;   // 32 x 32 MFMA tiles per wave
constexpr int KROW = BK * 2;           // bytes per row of a K-contiguous tile
constexpr int MNROW = 256 * 2;         // bytes per k-row of an MN-contiguous tile
constexpr int TILE = 32768;            // bytes per operand tile
constexpr int A_STAGES = 2;            // LDS stages of the A tile
constexpr int B_BASE = A_STAGES * TILE;     // B stages follow the A stages
// LDS stages of the B tile: 3 for the weight gradients (measured 2-4% faster
// than 2 there), 2 for dH and dX (3 measured between 1% faster and 2.5% slower)
template <int MODE>
constexpr int b_stages() { return MODE == 2 ? 3 : 2; }
constexpr int LPW = 32 / NW;           // direct loads per wave per operand per step
constexpr int KS = BK / 16;            // MFMA K sub-steps per step
}  // namespace bt

struct BigCtx {
  const uint16_t *A, *Bj;
  int lda, ldb, kbeg, kend;
  uint32_t a_off[bt::LPW];   // K-contiguous A: element offset of (clamped row, chunk)
  int a_col[bt::LPW];        // MN-contiguous A: column (clamped)
  int b_col[bt::LPW];        // B: column (clamped)
  int krow[bt::LPW];         // MN-contiguous tiles: k-row of each load within the step
  int fa[bt::TM], fb[bt::TN];
  int sw;
  uint32_t a_skip;           // K-contiguous A loads that feed only rows past the valid ones
};

__device__ __forceinline__ bf16x8_t tr_pair(const uint8_t *p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * bt::MNROW));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int MODE>
__device__ __forceinline__ const uint16_t *big_a_src(const BigCtx &c, int i, int k0) {
  if constexpr (MODE == BW_WG) {
    const int row = min(c.kbeg + k0 + c.krow[i], c.kend - 1);
    return c.A + (size_t)row * c.lda + c.a_col[i];
  } else {
    return c.A + c.a_off[i] + k0;
  }
}

template <int MODE>
__device__ __forceinline__ const uint16_t *big_b_src(const BigCtx &c, int i, int k0) {
  int row = c.kbeg + k0 + c.krow[i];
  if constexpr (MODE == BW_WG) row = min(row, c.kend - 1);
  return c.Bj + (size_t)row * c.ldb + c.b_col[i];
}

template <int MODE>
__device__ __forceinline__ void big_issue_a(const BigCtx &c, int k0, int wv, uint32_t stage) {
#pragma unroll
  for (int i = 0; i < bt::LPW; ++i)
    if (!((c.a_skip >> i) & 1))
      dma16(big_a_src<MODE>(c, i, k0), stage + (wv * bt::LPW + i) * 1024);
}

template <int MODE>
__device__ __forceinline__ void big_issue_b(const BigCtx &c, int k0, int wv, uint32_t stage) {
#pragma unroll
  for (int i = 0; i < bt::LPW; ++i)
    dma16(big_b_src<MODE>(c, i, k0), stage + (wv * bt::LPW + i) * 1024);
}

// One main-loop step (see the forward's big_step): MFMAs of this step from
// `rda` / `rdb`, one direct load every other MFMA over the first half -- the
// A tile of the next step (at ka) into `lda`, then the B tile of the step
// after it (at kb) into `ldb` -- and fragments double-buffered across the K
// sub-steps. Every A load of a step is issued before its B loads, so waiting
// until only the last step's B loads are in flight is exact. VT: this wave's
// 32-row MFMA tiles that hold valid rows (fewer than TM on a ragged last
// tile: the others' MFMAs and A fragment reads are dropped).
template <int MODE, int VT, bool LOAD_A = true, bool LOAD_B = true>
__device__ __forceinline__ void big_step(const BigCtx &c, int ka, int kb, int wv, uint32_t lda,
                                         uint32_t ldb, const uint8_t *__restrict__ rda,
                                         const uint8_t *__restrict__ rdb, int khalf,
                                         f32x16_t (&acc)[bt::TM][bt::TN]) {
  constexpr int MF = bt::KS * bt::TM * bt::TN;   // MFMAs per step
  constexpr int L = 2 * bt::LPW;                 // direct loads per step
  constexpr int GAP = MF / (2 * L);
  constexpr FragOrder<bt::TM, bt::TN> ord{};     // fragment reads in first-use order
  auto issue_one = [&](int d) {
    if (d < bt::LPW) {
      if (LOAD_A && (VT == bt::TM || !((c.a_skip >> d) & 1)))
        dma16(big_a_src<MODE>(c, d, ka), lda + (wv * bt::LPW + d) * 1024);
    } else if (LOAD_B) {
      dma16(big_b_src<MODE>(c, d - bt::LPW, kb), ldb + (wv * bt::LPW + d - bt::LPW) * 1024);
    }
  };
  bf16x8_t fra[2][bt::TM], frb[2][bt::TN];
  auto read_frag = [&](int buf, int ks, int r) {
    const int q = ord.q[r];
    if (q < bt::TM) {
      if (q >= VT) return;
      if constexpr (MODE == BW_WG)
        fra[buf][q] = tr_pair(rda + c.fa[q] + ks * 16 * bt::MNROW);
      else
        fra[buf][q] = *reinterpret_cast<const bf16x8_t *>(
            rda + c.fa[q] + (((ks * 2 + khalf) ^ c.sw) << 4));
    } else {
      frb[buf][q - bt::TM] = tr_pair(rdb + c.fb[q - bt::TM] + ks * 16 * bt::MNROW);
    }
  };
#pragma unroll
  for (int q = 0; q < bt::TM + bt::TN; ++q) read_frag(0, 0, q);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < bt::KS; ++ks) {
    const int cur = ks & 1;
#pragma unroll
    for (int q = 0; q < bt::TM * bt::TN; ++q) {
      const int g = ks * bt::TM * bt::TN + q;
      const int i = q / bt::TN, j = q % bt::TN;
      if (i < VT)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fra[cur][i], frb[cur][j], acc[i][j],
                                                            0, 0, 0);
      if (ks + 1 < bt::KS && q < bt::TM + bt::TN) read_frag(cur ^ 1, ks + 1, q);
      if (g % GAP == 0 && g / GAP < L) issue_one(g / GAP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(bt::NT, 1) void k_gemm_bwd_big(GemmArgs p) {
  constexpr int NSB = bt::b_stages<MODE>();
  __shared__ __attribute__((aligned(1024))) uint8_t smem[bt::B_BASE + NSB * bt::TILE];
  Work wk;
  if (!get_work<MODE>(p, bt::BM, bt::BN, wk)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / bt::WAVES_N, wn = wv % bt::WAVES_N;
  const int khalf = lane >> 5, fr = lane & 31;

  BigCtx c;
  // K-contiguous A rows are addressed from the tile's first row (64-bit
  // base), so the 32-bit offsets stay below BM * lda wherever the tile lies
  c.A = static_cast<const uint16_t *>(p.A) +
        (MODE == BW_WG ? (size_t)0 : (size_t)wk.m0 * p.lda);
  c.Bj = static_cast<const uint16_t *>(p.B) +
         (MODE == BW_WG ? 0 : (int64_t)wk.expert * p.b_expert_stride);
  c.lda = p.lda;
  c.ldb = p.ldb;
  c.kbeg = wk.kbeg;
  c.kend = wk.kend;
  const int a_cols = MODE == BW_WG ? p.M : 0;
  {
    // MN-contiguous loads: 2 k-rows of 32 chunks per instruction
    const int pch = lane & 31;
#pragma unroll
    for (int i = 0; i < bt::LPW; ++i) {
      const int kr = 2 * (wv * bt::LPW + i) + (lane >> 5);
      const int cl = pch ^ (4 * (kr & 3));
      c.krow[i] = kr;
      c.b_col[i] = min(wk.n0 + 8 * cl, p.N - 8);
      c.a_col[i] = min(wk.m0 + 8 * cl, a_cols - 8);
    }
    // K-contiguous A: 8 rows of 8 chunks per instruction
    const int lrow = lane >> 3, kch = lane & 7;
#pragma unroll
    for (int i = 0; i < bt::LPW; ++i) {
      const int r = (wv * bt::LPW + i) * 8 + lrow;
      const int tr = min(r, wk.m_end - 1 - wk.m0);   // clamped rows are discarded
      c.a_off[i] = (uint32_t)tr * (uint32_t)p.lda + ((kch ^ chunk_swz<8>(r)) << 3);
    }
  }
  {
    // transpose-read fragment offsets: lane 4j+a of 16-lane group g
    const int g = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    auto mn_off = [&](int col0) {
      const int cl = ((col0 + (g & 1) * 16 + 4 * a) >> 3) ^ (4 * j);
      return ((g >> 1) * 8 + j) * bt::MNROW + cl * 16 + (a & 1) * 8;
    };
#pragma unroll
    for (int t = 0; t < bt::TN; ++t) c.fb[t] = mn_off(wn * bt::WTN + t * 32);
#pragma unroll
    for (int t = 0; t < bt::TM; ++t)
      c.fa[t] = MODE == BW_WG ? mn_off(wm * 128 + t * 32) : (wm * 128 + t * 32 + fr) * bt::KROW;
    c.sw = chunk_swz<8>(fr);
  }

  f32x16_t acc[bt::TM][bt::TN];
#pragma unroll
  for (int i = 0; i < bt::TM; ++i)
#pragma unroll
    for (int j = 0; j < bt::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int klen = wk.kend - wk.kbeg;
  const int nk = (klen + bt::BK - 1) / bt::BK;
  const int rem = klen % bt::BK;
  // valid output rows of the tile, this wave's valid 32-row MFMA tiles, and
  // the K-contiguous A loads that feed only rows past them (wave-uniform)
  const int nvalid = MODE == BW_WG ? min(bt::BM, p.M - wk.m0) : min(bt::BM, wk.m_end - wk.m0);
  const int vt = __builtin_amdgcn_readfirstlane(min(bt::TM, max(0, (nvalid - wm * 128 + 31) / 32)));
  c.a_skip = 0;
  if (MODE != BW_WG) {
#pragma unroll
    for (int i = 0; i < bt::LPW; ++i)
      if ((wv * bt::LPW + i) * 8 >= ((nvalid + 31) / 32) * 32) c.a_skip |= 1u << i;
  }
  c.a_skip = __builtin_amdgcn_readfirstlane(c.a_skip);
  const uint32_t smem_l = lds_addr(smem);
  // prologue: A of step 0, B of steps 0 .. NSB-2 (A before B: exact waits)
  if (nk > 0) {
    big_issue_a<MODE>(c, 0, wv, smem_l);
    big_issue_b<MODE>(c, 0, wv, smem_l + bt::B_BASE);
    if (NSB == 3 && nk > 1) big_issue_b<MODE>(c, bt::BK, wv, smem_l + bt::B_BASE + bt::TILE);
  }
  // one main loop per count of valid 32-row tiles of this wave. Step kb loads
  // A(kb+1) and B(kb+NSB-1) while they exist (so the last NSB-1 steps are
  // peeled: with 3 B stages step nk-2 loads only A(nk-1); the last step loads
  // nothing), and no load is left to drain before the epilogue. At the top of
  // a step, A(kb) and B(kb) must have landed: with 3 B stages B(kb+1) may
  // still fly (its loads were issued last), except before the last step.
  auto main_loop = [&](auto vt_tag) {
    constexpr int VT = decltype(vt_tag)::value;
    auto step = [&](int kb, auto load_a, auto load_b) {
      if (NSB == 3 && kb + 1 < nk) wait_vmcnt<bt::LPW>();   // ... this wave's loads of step kb
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();                           // ... and every wave's landed
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // A stage (kb+1)&1 and B stage (kb+NSB-1)%NSB were read in earlier steps: free now
      const uint32_t lda = smem_l + ((kb + 1) & 1) * bt::TILE;
      const uint32_t ldb = smem_l + bt::B_BASE + ((kb + NSB - 1) % NSB) * bt::TILE;
      const uint8_t *rda = smem + (kb & 1) * bt::TILE;
      uint8_t *rdb = smem + bt::B_BASE + (kb % NSB) * bt::TILE;
      if (MODE == BW_WG && kb == nk - 1 && rem != 0) {
        // rows past the expert's range contribute nothing: zero them in B
        const u32x4_t z = {0, 0, 0, 0};
        for (int o = rem * bt::MNROW + tid * 16; o < bt::TILE; o += bt::NT * 16)
          *reinterpret_cast<u32x4_t *>(rdb + o) = z;
        __syncthreads();
      }
      big_step<MODE, VT, decltype(load_a)::value, decltype(load_b)::value>(
          c, (kb + 1) * bt::BK, (kb + NSB - 1) * bt::BK, wv, lda, ldb, rda, rdb, khalf, acc);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int kb = 0;
    for (; kb + NSB - 1 < nk; ++kb) step(kb, T_{}, T_{});
    if (NSB == 3 && kb + 1 < nk) step(kb++, T_{}, F_{});
    if (kb < nk) step(kb, F_{}, F_{});
  };
  switch (vt) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }
  wait_vmcnt<0>();   // no direct load still in flight into the stages

  // ---- epilogues. MFMA result layout: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of its 32 x 32 tile.
  if constexpr (MODE == BW_WG) {
    float *O = static_cast<float *>(p.Out) + wk.expert * p.out_expert_stride;
#pragma unroll
    for (int tm = 0; tm < bt::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < bt::TN; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wk.m0 + wm * 128 + tm * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
          const int col = wk.n0 + wn * bt::WTN + tn * 32 + fr;
          if (row < p.M && col < p.N) O[(size_t)row * p.ldo + col] = acc[tm][tn][r];
        }
  } else if constexpr (MODE == BW_DX) {
    // bf16 rows through LDS, 16-byte stores (the forward's epilogue): lanes
    // swap one value with their DPP partner so each writes two adjacent
    // columns of one row as a dword; chunk c of LDS row r sits at c ^ 4*q(r),
    // q(r) = bit0(r) | bit2(r) << 1
    constexpr int ROWB = bt::BN * 2;
    __syncthreads();
    auto stage_off = [](int row, int colb) {
      const int q = (row & 1) | (((row >> 2) & 1) << 1);
      return row * ROWB + ((((colb >> 4) ^ (q << 2))) << 4) + (colb & 15);
    };
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int tm = 0; tm < bt::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < bt::TN; ++tn) {
        const int colb0 = (wn * bt::WTN + tn * 32) * 2;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float v0 = acc[tm][tn][r], v1 = acc[tm][tn][r + 1];
          const float send = odd ? v0 : v1;
          const float recv = __int_as_float(
              __builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
          const int row = wm * 128 + tm * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3) + (odd ? 1 : 0);
          const int colb = colb0 + (fr & ~1) * 2;
          const uint32_t packed = odd ? pack_bf16x2(recv, v1) : pack_bf16x2(v0, recv);
          *reinterpret_cast<uint32_t *>(smem + stage_off(row, colb)) = packed;
        }
      }
    __syncthreads();
    constexpr int CPR = ROWB / 16;
    const int ncols = min(bt::BN, p.N - wk.n0);
    const int nrows = min(bt::BM, wk.m_end - wk.m0);
    uint16_t *O = static_cast<uint16_t *>(p.Out);
#pragma unroll 4
    for (int idx = tid; idx < bt::BM * CPR; idx += bt::NT) {
      const int row = idx / CPR, ch = idx % CPR;
      if (row < nrows && ch * 8 < ncols) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + stage_off(row, ch * 16));
        *reinterpret_cast<u32x4_t *>(O + (size_t)(wk.m0 + row) * p.ldo + wk.n0 + ch * 8) = v;
      }
    }
  } else {
    // DH: dH stays fp32; it goes through LDS in two halves of 128 columns
    // (row pitch 512 B, 16-byte chunk c of row r at c ^ 8*bit2(r)). Each
    // thread then takes 8 columns of a row, reads G and U of those columns as
    // 16-byte vectors and writes dG and dU the same way.
    const int ncols = min(bt::BN, p.N - wk.n0);
    const int nrows = min(bt::BM, wk.m_end - wk.m0);
    const uint16_t *GU = static_cast<const uint16_t *>(p.gu);
    uint16_t *DGU = static_cast<uint16_t *>(p.Out);
    const size_t ld2 = (size_t)2 * p.F;
    auto sw_off = [](int row, int col) {   // byte offset of fp32 (row, col) in the half
      return row * 512 + ((((col >> 2) ^ (((row >> 2) & 1) << 3))) << 4) + (col & 3) * 4;
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      if ((wn * bt::WTN) / 128 == h) {
#pragma unroll
        for (int tm = 0; tm < bt::TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < bt::TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = wm * 128 + tm * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
              const int col = (wn * bt::WTN) % 128 + tn * 32 + fr;
              *reinterpret_cast<float *>(smem + sw_off(row, col)) = acc[tm][tn][r];
            }
      }
      __syncthreads();
      for (int idx = tid; idx < bt::BM * 16; idx += bt::NT) {
        const int row = idx >> 4, c8 = idx & 15;
        const int lcol = h * 128 + c8 * 8;
        if (row >= nrows || lcol >= ncols) continue;
        const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(smem + sw_off(row, c8 * 8));
        const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(smem + sw_off(row, c8 * 8 + 4));
        const size_t base = (size_t)(wk.m0 + row) * ld2 + wk.n0 + lcol;
        const u32x4_t gv = *reinterpret_cast<const u32x4_t *>(GU + base);
        const u32x4_t uv = *reinterpret_cast<const u32x4_t *>(GU + base + p.F);
        u32x4_t dg, du;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o[2][2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float dh = (e < 2) ? lo[2 * e + hh] : hi[2 * (e - 2) + hh];
            const float g = hh ? bf16_hi(gv[e]) : bf16_lo(gv[e]);
            const float u = hh ? bf16_hi(uv[e]) : bf16_lo(uv[e]);
            const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
            o[0][hh] = dh * u * s * (1.0f + g * (1.0f - s));
            o[1][hh] = dh * g * s;
          }
          dg[e] = pack_bf16x2(o[0][0], o[0][1]);
          du[e] = pack_bf16x2(o[1][0], o[1][1]);
        }
        *reinterpret_cast<u32x4_t *>(DGU + base) = dg;
        *reinterpret_cast<u32x4_t *>(DGU + base + p.F) = du;
      }
    }
  }
}

// ---- fp32: 64 x 64 tile, K step 16, 4 x 4 outputs per thread
constexpr int kFT = 64;
constexpr int kFK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_bwd_f32(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) float sA[kFK][kFT + 4];
  __shared__ __attribute__((aligned(16))) float sB[kFK][kFT + 4];
  Work wk;
  if (!get_work<MODE>(p, kFT, kFT, wk)) return;
  const float *A = static_cast<const float *>(p.A);
  const float *Bj = static_cast<const float *>(p.B) +
                    (MODE == BW_WG ? 0 : (int64_t)wk.expert * p.b_expert_stride);
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  const int klen = wk.kend - wk.kbeg;
  for (int k0 = 0; k0 < klen; k0 += kFK) {
    if constexpr (MODE != BW_WG) {
      const int m = tid >> 2, kq = (tid & 3) * 4;
      const int mg = min(wk.m0 + m, wk.m_end - 1);
      const int k = k0 + kq;
      const f32x4_t v = (k < wk.kend) ? *reinterpret_cast<const f32x4_t *>(A + (size_t)mg * p.lda + k)
                                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[kq + e][m] = v[e];
    } else {
      const int kk = tid >> 4, mq = (tid & 15) * 4;
      const int r = wk.kbeg + k0 + kk;
      const int m = wk.m0 + mq;
      const f32x4_t v = (r < wk.kend && m < p.M)
                            ? *reinterpret_cast<const f32x4_t *>(A + (size_t)r * p.lda + m)
                            : f32x4_t{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4_t *>(&sA[kk][mq]) = v;
    }
    {
      const int kk = tid >> 4, nq = (tid & 15) * 4;
      const int kr = wk.kbeg + k0 + kk;
      const int n = wk.n0 + nq;
      const f32x4_t v = (kr < wk.kend && n < p.N)
                            ? *reinterpret_cast<const f32x4_t *>(Bj + (size_t)kr * p.ldb + n)
                            : f32x4_t{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4_t *>(&sB[kk][nq]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t *>(&sA[kk][ty * 4]);
      const f32x4_t b = *reinterpret_cast<const f32x4_t *>(&sB[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wk.m0 + ty * 4 + i, col = wk.n0 + tx * 4 + j;
      if (row < wk.m_end && col < p.N) store_elem<MODE, float>(p, wk, row, col, acc[i][j]);
    }
}

// Grid of a grouped GEMM launch: the capacity bound of row tiles (row modes)
// or every expert's fixed tiles (WG), times the n-tiles, rounded up to the
// XCD count.
inline dim3 gemm_grid(int mode, const moe_shape_t &s, int tile, const GemmArgs &p) {
  const int E_L = s.N / s.ep_size;
  int64_t tiles;
  if (mode == BW_WG)
    tiles = (int64_t)E_L * p.m_tiles * p.n_tiles_n;
  else
    tiles = (ceil_div(buffer_rows(s), tile) + E_L) * p.n_tiles_n;
  return dim3((unsigned)(ceil_div(tiles, kNumXcd) * kNumXcd));
}

// One grouped product. bf16: the pipelined 256 x 256 kernel when the
// contraction of a row mode is a multiple of its K step (the weight-gradient
// contraction may have any length), else the 128 x 128 kernel; fp32: SIMT.
template <int MODE>
void launch_mode(const moe_shape_t &s, GemmArgs p, hipStream_t st) {
  const bool bf16 = s.dtype == MOE_BF16;
  const bool big = bf16 && (MODE == BW_WG || p.Kdim % bt::BK == 0);
  const int tile = big ? bt::BM : bf16 ? kT : kFT;
  p.n_tiles_n = (int)ceil_div(p.N, tile);
  p.m_tiles = MODE == BW_WG ? (int)ceil_div(p.M, tile) : 0;
  const dim3 grid = gemm_grid(MODE, s, tile, p);
  if (big) hipLaunchKernelGGL(k_gemm_bwd_big<MODE>, grid, dim3(bt::NT), 0, st, p);
  else if (bf16) hipLaunchKernelGGL(k_gemm_bwd<MODE>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_gemm_bwd_f32<MODE>, grid, dim3(256), 0, st, p);
}

template <bool BF16, bool FULL>
void combine_bwd_nv(int nv, dim3 grid, hipStream_t st, const u32x4_t *g, const u32x4_t *y,
                    const int32_t *dr, const int32_t *drow, const float *w, u32x4_t *o,
                    float *dw, const moe_shape_t &s, int nvec) {
  const int rows = (int)buffer_rows(s);
  switch (nv) {
    case 1: hipLaunchKernelGGL((k_combine_bwd<BF16, 1, FULL>), grid, dim3(256), 0, st, g, y, dr, drow, w, o, dw, s.T, s.K, nvec, s.ep_rank, rows); break;
    case 2: hipLaunchKernelGGL((k_combine_bwd<BF16, 2, FULL>), grid, dim3(256), 0, st, g, y, dr, drow, w, o, dw, s.T, s.K, nvec, s.ep_rank, rows); break;
    case 4: hipLaunchKernelGGL((k_combine_bwd<BF16, 4, FULL>), grid, dim3(256), 0, st, g, y, dr, drow, w, o, dw, s.T, s.K, nvec, s.ep_rank, rows); break;
    default: hipLaunchKernelGGL((k_combine_bwd<BF16, 8, FULL>), grid, dim3(256), 0, st, g, y, dr, drow, w, o, dw, s.T, s.K, nvec, s.ep_rank, rows); break;
  }
}

}  // namespace

int launch_combine_bwd(const moe_shape_t &s, const void *dout, const void *y,
                       const int32_t *dest_rank, const int32_t *dest_row, const float *w, void *dy,
                       float *dw, hipStream_t st) {
  const int nvec = s.d * elem_bytes(s.dtype) / 16;
  const int per_lane = (int)ceil_div(nvec, 64);
  const int nv = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : 8;
  const dim3 grid((unsigned)ceil_div(s.T, kRowsPerBlock));
  const u32x4_t *g = static_cast<const u32x4_t *>(dout);
  const u32x4_t *yv = static_cast<const u32x4_t *>(y);
  u32x4_t *o = static_cast<u32x4_t *>(dy);
  const bool full = nvec % (64 * nv) == 0;
  if (s.dtype == MOE_BF16) {
    if (full) combine_bwd_nv<true, true>(nv, grid, st, g, yv, dest_rank, dest_row, w, o, dw, s, nvec);
    else combine_bwd_nv<true, false>(nv, grid, st, g, yv, dest_rank, dest_row, w, o, dw, s, nvec);
  } else {
    if (full) combine_bwd_nv<false, true>(nv, grid, st, g, yv, dest_rank, dest_row, w, o, dw, s, nvec);
    else combine_bwd_nv<false, false>(nv, grid, st, g, yv, dest_rank, dest_row, w, o, dw, s, nvec);
  }
  return launch_status();
}

int launch_route_bwd(const moe_shape_t &s, const int32_t *idx, const float *w, const float *dw,
                     float *dlogits, hipStream_t st) {
  hipLaunchKernelGGL(k_route_bwd, dim3((unsigned)ceil_div(s.T, kRowsPerBlock)), dim3(256), 0, st,
                     idx, w, dw, dlogits, s.T, s.N, s.K);
  return launch_status();
}

int launch_expert_ffn_bwd_data(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                               const void *w_gu, const void *w_down, const void *dy, void *gu,
                               void *dgu, void *dx_rows, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  // [G U] = X W_gu^T over the prefix rows (forward NT GEMM, no activation)
  const int rc = launch_gemm_nt(s, buf, w_gu, off, gu, s.d, 2 * s.F, st);
  if (rc != MOE_OK) return rc;
  return launch_expert_ffn_bwd_data_gu(s, offsets, w_gu, w_down, dy, gu, dgu, dx_rows, st);
}

int launch_expert_ffn_bwd_data_gu(const moe_shape_t &s, const int32_t *offsets, const void *w_gu,
                                  const void *w_down, const void *dy, const void *gu, void *dgu,
                                  void *dx_rows, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int d = s.d, F = s.F;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  int rc;
  GemmArgs p{};
  p.off = off;
  p.E_L = E_L;
  p.rows = (int)buffer_rows(s);
  p.F = F;
  // dH = dY W_d (K = d, N = F), SwiGLU backward on [G U] in the epilogue -> [dG dU]
  p.A = dy; p.lda = d; p.B = w_down; p.ldb = F; p.b_expert_stride = (int64_t)d * F;
  p.N = F; p.Kdim = d; p.gu = gu; p.Out = dgu; p.ldo = 2 * F;
  launch_mode<BW_DH>(s, p, st);
  if ((rc = launch_status()) != MOE_OK) return rc;
  // then dX = [dG dU] W_gu (K = 2F, N = d)
  p.A = dgu; p.lda = 2 * F; p.B = w_gu; p.ldb = d; p.b_expert_stride = (int64_t)2 * F * d;
  p.N = d; p.Kdim = 2 * F; p.gu = nullptr; p.Out = dx_rows; p.ldo = d;
  launch_mode<BW_DX>(s, p, st);
  return launch_status();
}

int launch_expert_ffn_bwd_weight(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                                 const void *h, const void *dy, const void *dgu, float *dw_gu,
                                 float *dw_down, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int d = s.d, F = s.F;
  GemmArgs p{};
  p.off = offsets + (size_t)s.ep_rank * (E_L + 1);
  p.E_L = E_L;
  p.rows = (int)buffer_rows(s);
  p.F = F;
  // 4. dW_d[j] = dY^T H over the expert's rows (M = d, N = F), fp32
  p.A = dy; p.lda = d; p.B = h; p.ldb = F;
  p.M = d; p.N = F; p.Out = dw_down; p.ldo = F; p.out_expert_stride = (int64_t)d * F;
  launch_mode<BW_WG>(s, p, st);
  int rc = launch_status();
  if (rc != MOE_OK) return rc;
  // 5. dW_gu[j] = [dG dU]^T X over the expert's rows (M = 2F, N = d), fp32
  p.A = dgu; p.lda = 2 * F; p.B = buf; p.ldb = d;
  p.M = 2 * F; p.N = d; p.Out = dw_gu; p.ldo = d; p.out_expert_stride = (int64_t)2 * F * d;
  launch_mode<BW_WG>(s, p, st);
  return launch_status();
}

}  // namespace moe
