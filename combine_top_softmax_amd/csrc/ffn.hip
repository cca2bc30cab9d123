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
// (sum_j ceil(n_j/BM) <= ceil(R/BM) + E_L m-tiles, R the buffer rows); every block recomputes
// the per-expert m-tile counts from the offsets with a wave scan, maps its
// block id to a real tile and exits if there is none. The block id -> tile map
// is XCD-aware: blocks are dealt to the 8 XCDs round-robin, so block b gets
// tile (b % 8) * q + b / 8 (q = ceil(tiles / 8)) and each XCD walks a
// contiguous run of tiles (the m-tiles of one expert for one weight panel,
// then the next panel), which keeps the shared A rows and expert weights in
// that XCD's L2.
//
// bf16 paths (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   k_gemm_bf16_big (K % 64 == 0): 256 x 256 block tile, 4 waves of 128 x 128
//     (one per SIMD), operands loaded global -> LDS directly,
//     XOR-swizzled LDS rows, two A and three weight LDS stages, loads and
//     fragment reads interleaved with the MFMAs (details at the kernel);
//   k_gemm_bf16 (any K % 8 == 0): 128 x 128 block tile, 4 waves of 64 x 64,
//     register-staged LDS double buffer with 16-byte row padding.
// fp32 path: a plain LDS-tiled SIMT kernel (64 x 64 tile, 4 x 4 per thread).
#include <type_traits>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace {


struct Tile {
  int expert;
  int row0;     // first buffer row of this m-tile
  int row_end;  // one past the expert's last valid row
  int n_idx;    // output column tile
  bool valid;
};

// Map this block to a (expert, m-tile, n-tile) from the local offsets (the
// shared lookup above; wave-uniform). Inside an expert with M m-tiles, the
// tiles of one weight panel come first: all M m-tiles of n-tile 0, then of
// n-tile 1, ..., so the tiles that run at the same time on one XCD share their
// weight panel and the expert's A rows in L2 (equal or best on every named
// workload among groups of 1, 2, 4 and 8 n-tiles and "all n-tiles of an
// m-tile first").
__device__ __forceinline__ Tile find_tile(const int32_t *__restrict__ off, int E_L, int bm,
                                          int rows, int n_tiles_n) {
  Tile tl;
  const ExpertTile x = find_expert_tile(off, E_L, bm, rows, n_tiles_n);
  tl.valid = x.valid;
  if (!x.valid) return tl;
  const int li = x.L - x.mstart * n_tiles_n;   // tile index inside the expert, < M * n_tiles_n
  const int n = li / x.M;                      // n-tile
  tl.expert = x.e;
  tl.row0 = x.row_begin + (li - n * x.M) * bm;
  tl.row_end = x.row_end;
  tl.n_idx = n;
  return tl;
}


// ------------------------------------------------------------------ bf16 MFMA
constexpr int kBM = 128;        // rows per block tile
constexpr int kBW = 128;        // weight rows per block tile
constexpr int kBK = 64;         // K per main-loop step
constexpr int kLds = kBK + 8;   // padded LDS row (elements)

// silu(g) * u of the fused up epilogue (the same expression wherever H is
// formed from the accumulators, so H does not depend on the epilogue variant).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <bool GATE_UP>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const int32_t *__restrict__ off, uint16_t *__restrict__ Out, int E_L, int rows, int Kdim,
    int Nout, int n_tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBW * kLds];

  const Tile tl = find_tile(off, E_L, kBM, rows, n_tiles_n);
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
        const float hv = swiglu(g, u);
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

// ------------------------------------------------------------ bf16 MFMA, big tiles
// Block tile 256 rows x 256 weight rows, K step 64, two LDS stages for the A
// rows and three for the weight rows, 4 waves: 2 x 2 waves of 128 x 128 (4 x
// 4 MFMA tiles, 256 accumulators each, one wave per SIMD). Square wave tiles
// read a third fewer LDS bytes per flop than 8 waves of 128 x 64, and the
// kernel runs power-limited (the shader clock drops to ~1.3-1.6 GHz in its
// main loop), so the 4-wave layout measured 2-5% faster on every named
// workload; 128-row tiles and 32-wide K steps measured slower.
// Operands go global -> LDS directly (global_load_lds_dwordx4, no VGPR
// staging). Step k, right after its opening barrier, issues the A loads of
// step k + 1 and then the weight loads of step k + 2: the weight rows
// (each read from HBM once per expert, shared by fewer tiles than the A rows)
// get two steps of MFMA work to land, the A rows one (2 x 32 KiB + 3 x 32
// KiB fill the 160 KiB of LDS). The barrier is a plain s_barrier preceded by
// a wait for this wave's loads of the step about to be read (s_waitcnt
// vmcnt(N) with N = the younger weight loads still allowed in flight), not a
// full fence that would drain every outstanding load.
// LDS rows are BK bf16 (BK/8 16-byte chunks); chunk c of row r is stored at
// c ^ swz(r), chosen so that a wave's direct load writes whole rows
// contiguously and the fragment reads of 16 consecutive rows (one chunk each)
// touch 16 distinct 16-byte bank groups. Requires K % BK == 0.
struct BigTile {
  static constexpr int BM = 256;                 // rows per block
  static constexpr int BK = 64;                  // K per main-loop step
  static constexpr int NS = 3;                   // LDS stages of the weight rows
  static constexpr int NW = 4;                   // waves per block
  static constexpr int BW = 256;                 // weight rows per block
  static constexpr int WAVES_M = BM / 128;
  static constexpr int WAVES_N = NW / WAVES_M;
  static constexpr int WTN = BW / WAVES_N;       // weight rows per wave
  static constexpr int TM = 4;                   // 32-row MFMA tiles per wave
  static constexpr int TN = WTN / 32;            // 32-col MFMA tiles per wave
  static constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
  static constexpr int ROW_B = BK * 2;           // bytes per LDS row
  static constexpr int RPI = 64 / CH;            // rows per direct-load instruction
  static constexpr int NA = BM / RPI / NW;       // A direct loads per wave per step
  static constexpr int NB = BW / RPI / NW;       // B direct loads per wave per step
  static constexpr int L = NA + NB;
  static constexpr int KS = BK / 16;             // MFMA K sub-steps per step
  static constexpr int A_BYTES = BM * ROW_B;     // one A stage
  static constexpr int B_BYTES = BW * ROW_B;     // one B stage
};


// Issue the direct global -> LDS loads of one K step into `stage`.
__device__ __forceinline__ void big_issue(const uint16_t *__restrict__ A,
                                          const uint16_t *__restrict__ Wj, const uint32_t *a_off,
                                          const uint32_t *b_off, int ka, int kb, int wv,
                                          uint32_t sa, uint32_t sb, bool do_a) {
  using P = BigTile;
  if (do_a) {
#pragma unroll
    for (int i = 0; i < P::NA; ++i) dma16(A + a_off[i] + ka, sa + (wv * P::NA + i) * 1024);
  }
#pragma unroll
  for (int i = 0; i < P::NB; ++i) dma16(Wj + b_off[i] + kb, sb + (wv * P::NB + i) * 1024);
}

// One main-loop step: run the MFMAs of this K step from `rd` while issuing
// the direct loads of a later K step into `ld`. The stages are restrict
// pointers so that, once inlined, the compiler does not wait for the loads
// into `ld` before the reads of `rd`; the ordering the pipeline needs comes
// from wait_vmcnt + s_barrier at the top of each step.
//
// Issue order inside a step is fixed with scheduling fences:
//   * one direct load every (MFMAs per step / loads per step) MFMAs, so the
//     address path is fed steadily instead of stalling issue at step start;
//   * fragments double-buffered across the K sub-steps: each read of
//     sub-step ks+1 follows one MFMA of sub-step ks, so it lands while the
//     remaining MFMAs of ks execute; reads go in first-use order, and the
//     direct loads are inline asm (dma16), so each MFMA waits only for the
//     reads it needs.
//
// VT < TM (the last m-tile of an expert): only this wave's first VT 32-row
// MFMA tiles hold valid rows; the MFMAs and A fragment reads of the others are
// dropped at compile time, and the A direct loads in a_skip (bit d: load d
// feeds only rows past the last valid 32-row group) are not issued. Full
// tiles take VT = TM.
template <bool GATE_UP, int VT = BigTile::TM>
__device__ __forceinline__ void big_step(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ Wj, const uint32_t *a_off,
    const uint32_t *b_off, int ka, int kb, int wv, uint32_t lda, uint32_t ldb,
    const uint8_t *__restrict__ rda, const uint8_t *__restrict__ rdb, const int *fa,
    const int *fb, int khalf, int sw,
    f32x16_t (&acc)[BigTile::TM][BigTile::TN], bf16x8_t (&fra)[2][BigTile::TM],
    bf16x8_t (&frb)[2][BigTile::TN],
    uint32_t a_skip = 0) {
  using P = BigTile;
  constexpr bool PARTIAL = VT < P::TM;
  constexpr int MF = P::KS * P::TM * P::TN;      // MFMAs per step
  constexpr int MS = P::TM * P::TN;              // MFMAs per sub-step
  // MFMAs between two direct loads: spread over the whole step
  constexpr int GAP = MF / P::L;
  static_assert(GAP >= 1 && GAP * P::L <= MF, "load spacing");
  constexpr FragOrder<P::TM, P::TN> ord{};
  auto issue_one = [&](int d) {
    if (d < P::NA) {
      if (!PARTIAL || !((a_skip >> d) & 1))
        dma16(A + a_off[d] + ka, lda + (wv * P::NA + d) * 1024);
    } else
      dma16(Wj + b_off[d - P::NA] + kb, ldb + (wv * P::NB + (d - P::NA)) * 1024);
  };
  auto read_frag = [&](int buf, int ks, int r) {
    const int q = ord.q[r];
    const int cb = ((ks * 2 + khalf) ^ sw) << 4;
    if (q < P::TM) {
      if (q < VT)
        fra[buf][q] = *reinterpret_cast<const bf16x8_t *>(rda + fa[q] + cb);
    } else
      frb[buf][q - P::TM] = *reinterpret_cast<const bf16x8_t *>(rdb + fb[q - P::TM] + cb);
  };
  auto mfma = [&](int buf, int q) {
    const int i = q / P::TN, j = q % P::TN;
    if (i < VT)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frb[buf][j], fra[buf][i], acc[i][j],
                                                          0, 0, 0);   // transposed tile
  };
#pragma unroll
  for (int r = 0; r < P::TM + P::TN; ++r) read_frag(0, 0, r);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < P::KS; ++ks) {
    const int cur = ks & 1;
#pragma unroll
    for (int q = 0; q < MS; ++q) {
      const int g = ks * MS + q;
      mfma(cur, q);
      if (ks + 1 < P::KS && q < P::TM + P::TN) read_frag(cur ^ 1, ks + 1, q);
      if (g % GAP == 0 && g / GAP < P::L) issue_one(g / GAP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Epilogue of the big-tile kernels (every wave past its last MFMA, every
// direct load drained, the stages free).
template <bool GATE_UP, bool SAVE>
__device__ __forceinline__ void big_epilogue(
    const f32x16_t (&acc)[BigTile::TM][BigTile::TN],
    uint8_t *__restrict__ smem, const Tile &tl, uint16_t *__restrict__ Out,
    uint16_t *__restrict__ GU, int Nout, int n0, int wm, int wn) {
  using P = BigTile;
  constexpr int BM = P::BM, NW = P::NW;
  static_assert(!SAVE || GATE_UP, "only the gate/up product has a [G U] tile to keep");
  // Epilogue, staged through LDS so that global stores are whole 16-byte
  // vectors along output rows. The MFMAs take the weight fragment as their
  // first operand, so each 32x32 accumulator tile holds the transposed tile:
  // register r of lane l is row l%32, column 8*(r/4) + 4*(l/32) + r%4 of the
  // output tile, i.e. every lane owns four runs of four adjacent columns of
  // one row. Each run is converted to four bf16 (two packed conversions) and
  // written as one 8-byte LDS store; then every thread copies 16-byte chunks
  // of the tile to global memory, skipping rows past the expert's last valid
  // row and columns past Nout.
  // LDS rows are OUTC bf16; 16-byte chunk c of row r sits at c ^ (r % CPR)
  // (CPR chunks per row), so the 16 consecutive rows that one 16-lane group
  // of a store instruction writes land in 16 distinct chunks.
  constexpr int OUTC = GATE_UP ? P::BW / 2 : P::BW;    // output columns per block
  constexpr int ROWB = OUTC * 2;                       // bytes per staged row
  constexpr int CPR = ROWB / 16;                       // 16-byte chunks per row
  static_assert(BM * ROWB <= 2 * P::A_BYTES + 2 * P::B_BYTES, "epilogue tile fits the stages");
  const int tid = threadIdx.x, lane = tid & 63, fr = lane & 31, khalf = lane >> 5;
  auto stage_off = [](int row, int chunk) {   // byte offset of 16-byte chunk `chunk` of `row`
    return row * ROWB + ((chunk ^ (row & (CPR - 1))) << 4);
  };
  if constexpr (SAVE) {
    // H and the pre-activation G, U of the same columns (G from weight rows
    // 0..BW/2-1 of the block, U from BW/2..BW-1), all rounded from the same
    // accumulators, in two passes over half the rows (the wave's 32-row
    // tiles 2p and 2p+1), so that every accumulator is read once: a pass
    // stages [G U] rows (BW columns) and H rows (OUTC columns) of BM/2 block
    // rows in the swizzled layout, then copies them out with 16-byte stores
    // to GU[row, n0 + c] (gate half), GU[row, Nout + n0 + c] (up half) and
    // Out[row, n0 + c].
    constexpr int GROWB = P::BW * 2;
    constexpr int GCPR = GROWB / 16;
    constexpr int SR = BM / 2;                     // block rows staged per pass
    constexpr int H_BASE = SR * GROWB;
    static_assert(H_BASE + SR * ROWB <= 2 * P::A_BYTES + 2 * P::B_BYTES, "pass fits the stages");
    auto gstage_off = [](int row, int chunk) {
      return row * GROWB + ((chunk ^ (row & (GCPR - 1))) << 4);
    };
    const int nrows = min(BM, tl.row_end - tl.row0);
    const int ncols = min(OUTC, Nout - n0);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int tm = 2 * pass + t;
        const int srow = wm * 64 + t * 32 + fr;    // staged row
#pragma unroll
        for (int tn = 0; tn < P::TN / 2; ++tn) {
          const int col0 = wn * (P::WTN / 2) + tn * 32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float gv[4], uv[4], hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              gv[e] = acc[tm][tn][4 * g + e];
              uv[e] = acc[tm][tn + P::TN / 2][4 * g + e];
              hv[e] = swiglu(gv[e], uv[e]);
            }
            const int cb = (col0 + 8 * g + 4 * khalf) * 2;
            uint2 w;
            w.x = pack2_bf16(gv[0], gv[1]);
            w.y = pack2_bf16(gv[2], gv[3]);
            *reinterpret_cast<uint2 *>(smem + gstage_off(srow, cb >> 4) + (cb & 15)) = w;
            w.x = pack2_bf16(uv[0], uv[1]);
            w.y = pack2_bf16(uv[2], uv[3]);
            *reinterpret_cast<uint2 *>(smem + gstage_off(srow, (GROWB / 2 + cb) >> 4) +
                                       (cb & 15)) = w;
            w.x = pack2_bf16(hv[0], hv[1]);
            w.y = pack2_bf16(hv[2], hv[3]);
            *reinterpret_cast<uint2 *>(smem + H_BASE + stage_off(srow, cb >> 4) + (cb & 15)) = w;
          }
        }
      }
      __syncthreads();
      // staged row r holds block row (r / 64) * 128 + 64 * pass + r % 64
      constexpr int HALF = GCPR / 2;   // chunks per gate or up half row
#pragma unroll 4
      for (int idx = tid; idx < SR * GCPR; idx += 64 * NW) {
        const int r = idx / GCPR, ch = idx % GCPR;
        const int row = (r / 64) * 128 + 64 * pass + r % 64;
        const int c = (ch % HALF) * 8;
        if (row < nrows && c < ncols) {
          const uint4 v = *reinterpret_cast<const uint4 *>(smem + gstage_off(r, ch));
          *reinterpret_cast<uint4 *>(GU + (size_t)(tl.row0 + row) * (2 * Nout) +
                                     (ch < HALF ? 0 : Nout) + n0 + c) = v;
        }
      }
#pragma unroll 4
      for (int idx = tid; idx < SR * CPR; idx += 64 * NW) {
        const int r = idx / CPR, ch = idx % CPR;
        const int row = (r / 64) * 128 + 64 * pass + r % 64;
        if (row < nrows && ch * 8 < ncols) {
          const uint4 v = *reinterpret_cast<const uint4 *>(smem + H_BASE + stage_off(r, ch));
          *reinterpret_cast<uint4 *>(Out + (size_t)(tl.row0 + row) * Nout + n0 + ch * 8) = v;
        }
      }
      __syncthreads();   // the stage is read out before the next pass reuses it
    }
    return;
  }
#pragma unroll
  for (int tm = 0; tm < P::TM; ++tm) {
    const int row = wm * 128 + tm * 32 + fr;
#pragma unroll
    for (int tn = 0; tn < (GATE_UP ? P::TN / 2 : P::TN); ++tn) {
      const int col0 = (GATE_UP ? wn * (P::WTN / 2) : wn * P::WTN) + tn * 32;  // tile column
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          if (GATE_UP) {
            v[e] = swiglu(acc[tm][tn][r], acc[tm][tn + P::TN / 2][r]);
          } else {
            v[e] = acc[tm][tn][r];
          }
        }
        const int cb = (col0 + 8 * g + 4 * khalf) * 2;   // byte column of the run
        uint2 w;
        w.x = pack2_bf16(v[0], v[1]);
        w.y = pack2_bf16(v[2], v[3]);
        *reinterpret_cast<uint2 *>(smem + stage_off(row, cb >> 4) + (cb & 15)) = w;
      }
    }
  }
  __syncthreads();
  const int ncols = min(OUTC, Nout - n0);               // multiple of 8
  const int nrows = min(BM, tl.row_end - tl.row0);
#pragma unroll 4
  for (int idx = tid; idx < BM * CPR; idx += 64 * NW) {
    const int row = idx / CPR, ch = idx % CPR;
    if (row < nrows && ch * 8 < ncols) {
      const uint4 v = *reinterpret_cast<const uint4 *>(smem + stage_off(row, ch));
      *reinterpret_cast<uint4 *>(Out + (size_t)(tl.row0 + row) * Nout + n0 + ch * 8) = v;
    }
  }
}

// SAVE (gate/up product only): also keep the pre-activation [G U] rows in GU
// ([rows, 2 Nout], gate columns then up columns) for the backward.
template <bool GATE_UP, bool SAVE>
__global__ __launch_bounds__(64 * BigTile::NW, 1) void k_gemm_bf16_big(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const int32_t *__restrict__ off, uint16_t *__restrict__ Out, uint16_t *__restrict__ GU,
    int E_L, int rows, int Kdim, int Nout, int n_tiles_n) {
  using P = BigTile;
  constexpr int BM = P::BM, BK = P::BK, NS = P::NS;
  // two A stages, NS = 3 B stages: the weight rows, which miss to HBM more
  // often, get two steps to land
  constexpr int B_BASE = 2 * P::A_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[B_BASE + NS * P::B_BYTES];

  const uint32_t smem_l = lds_addr(smem);
  const Tile tl = find_tile(off, E_L, BM, rows, n_tiles_n);
  if (!tl.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / P::WAVES_N, wn = wv % P::WAVES_N;
  const int Nw = GATE_UP ? 2 * Nout : Nout;
  const uint16_t *Wj = W + (size_t)tl.expert * Nw * Kdim;
  const int n0 = tl.n_idx * (GATE_UP ? P::BW / 2 : P::BW);

  // direct-load sources (element offsets): lane -> row RPI*instr + lane/CH,
  // physical chunk lane%CH. The A rows are addressed from the tile's first
  // row At (64-bit), so an offset stays below BM * Kdim however far into the
  // buffer the tile lies; weight rows stay below 2F * d < 2^31 elements of
  // the expert's matrix (checked on the host).
  const uint16_t *At = A + (size_t)tl.row0 * Kdim;
  uint32_t a_off[P::NA], b_off[P::NB];
  {
    const int lrow = lane / P::CH, pch = lane % P::CH;
#pragma unroll
    for (int i = 0; i < P::NA; ++i) {
      const int r = (wv * P::NA + i) * P::RPI + lrow;
      const int tr = min(r, tl.row_end - 1 - tl.row0);   // clamped rows are discarded
      a_off[i] = (uint32_t)tr * (uint32_t)Kdim + ((pch ^ chunk_swz<P::CH>(r)) << 3);
    }
#pragma unroll
    for (int i = 0; i < P::NB; ++i) {
      const int r = (wv * P::NB + i) * P::RPI + lrow;
      int wrow;
      if (GATE_UP)
        wrow = (r < P::BW / 2) ? min(n0 + r, Nout - 1) : Nout + min(n0 + r - P::BW / 2, Nout - 1);
      else
        wrow = min(n0 + r, Nout - 1);
      b_off[i] = (uint32_t)wrow * (uint32_t)Kdim + ((pch ^ chunk_swz<P::CH>(r)) << 3);
    }
  }
  // fragment read offsets (bytes within a stage)
  const int fr = lane & 31;
  const int sw = chunk_swz<P::CH>(fr);
  const int khalf = lane >> 5;
  int fa[P::TM], fb[P::TN];
#pragma unroll
  for (int t = 0; t < P::TM; ++t) fa[t] = (wm * 128 + t * 32 + fr) * P::ROW_B;
#pragma unroll
  for (int t = 0; t < P::TN; ++t) {
    int brow;
    if (GATE_UP)
      brow = (t < P::TN / 2) ? wn * (P::WTN / 2) + t * 32
                             : P::BW / 2 + wn * (P::WTN / 2) + (t - P::TN / 2) * 32;
    else
      brow = wn * P::WTN + t * 32;
    fb[t] = (brow + fr) * P::ROW_B;
  }

  f32x16_t acc[P::TM][P::TN];
#pragma unroll
  for (int i = 0; i < P::TM; ++i)
#pragma unroll
    for (int j = 0; j < P::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = Kdim / BK;
  // valid 32-row MFMA tiles of this wave, and the A loads that feed only rows
  // past the last valid 32-row group of the tile (wave-uniform)
  const int nvalid = min(BM, tl.row_end - tl.row0);
  const int vt = __builtin_amdgcn_readfirstlane(min(P::TM, max(0, (nvalid - wm * 128 + 31) / 32)));
  uint32_t a_skip = 0;
#pragma unroll
  for (int i = 0; i < P::NA; ++i)
    if ((wv * P::NA + i) * P::RPI >= ((nvalid + 31) / 32) * 32) a_skip |= 1u << i;
  a_skip = __builtin_amdgcn_readfirstlane(a_skip);
  // prologue: A step 0, B steps 0 .. NS-2 (in this order: the waits below
  // rely on every A load of a step being issued before that step's B loads)
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    big_issue(At, Wj, a_off, b_off, 0, min(s, nk - 1) * BK, wv, smem_l,
                              smem_l + B_BASE + s * P::B_BYTES, s == 0);
  // one main loop per count of valid 32-row tiles of this wave (TM for full
  // tiles; fewer on an expert's last m-tile), each with a single inlined step
  bf16x8_t fra[2][P::TM], frb[2][P::TN];
  auto main_loop = [&](auto vt_tag) {
    constexpr int VT = decltype(vt_tag)::value;
    for (int kb = 0; kb < nk; ++kb) {
      // step j issues A(j+1) then B(j+NS-1): A(kb) and B(kb) have landed once
      // at most the NS-2 younger B steps' loads are in flight; after the
      // barrier, every wave's have
      wait_vmcnt<(NS - 2) * P::NB>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // stages read in step kb-1 are free after the barrier; the last steps
      // reload the last K step into free stages, so every step issues the
      // same loads (no branch around them)
      const uint32_t lda = smem_l + ((kb + 1) & 1) * P::A_BYTES;
      const uint32_t ldb = smem_l + B_BASE + ((kb + NS - 1) % NS) * P::B_BYTES;
      const uint8_t *rda = smem + (kb & 1) * P::A_BYTES;
      const uint8_t *rdb = smem + B_BASE + (kb % NS) * P::B_BYTES;
      big_step<GATE_UP, VT>(At, Wj, a_off, b_off, min(kb + 1, nk - 1) * BK,
                            min(kb + NS - 1, nk - 1) * BK, wv, lda, ldb, rda, rdb, fa, fb, khalf,
                            sw, acc, fra, frb, a_skip);
    }
  };
  static_assert(P::TM == 4, "main-loop variants");
  switch (vt) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }

  wait_vmcnt<0>();   // no direct load still in flight into the stages
  __syncthreads();   // every wave is done reading the last stage
  big_epilogue<GATE_UP, SAVE>(acc, smem, tl, Out, GU, Nout, n0, wm, wn);
}

// ------------------------------------------------------------------ fp32 SIMT
constexpr int kFM = 64, kFW = 64, kFK = 16;

template <bool GATE_UP>
__global__ __launch_bounds__(256) void k_gemm_f32(
    const float *__restrict__ A, const float *__restrict__ W, const int32_t *__restrict__ off,
    float *__restrict__ Out, int E_L, int rows, int Kdim, int Nout, int n_tiles_n) {
  __shared__ float sA[kFK][kFM + 1];
  __shared__ float sB[kFK][kFW + 1];
  const Tile tl = find_tile(off, E_L, kFM, rows, n_tiles_n);
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
  const int64_t max_m = ceil_div(buffer_rows(s), bm) + E_L;
  return (unsigned)(ceil_div(max_m * n_tiles_n, kNumXcd) * kNumXcd);
}

// Which bf16 kernel runs: the big-tile kernel (256 x 256 tiles, K step 64)
// when K % 64 == 0, else the 128 x 128 register-staged kernel (any
// K % 8 == 0).
template <bool GATE_UP>
int launch_bf16(const moe_shape_t &s, const uint16_t *A, const uint16_t *W, const int32_t *off,
                uint16_t *Out, int Kdim, int Nout, hipStream_t st, uint16_t *GU = nullptr) {
  const int E_L = s.N / s.ep_size;
  const int rows = (int)buffer_rows(s);
  if (Kdim % 64 == 0) {
    using P = BigTile;
    const int ntn = (int)ceil_div(Nout, GATE_UP ? P::BW / 2 : P::BW);
    const dim3 grid(grid_blocks(s, P::BM, ntn)), block(64 * P::NW);
    if (GATE_UP && GU != nullptr)
      hipLaunchKernelGGL((k_gemm_bf16_big<true, true>), grid, block, 0, st, A, W, off, Out, GU,
                         E_L, rows, Kdim, Nout, ntn);
    else
      hipLaunchKernelGGL((k_gemm_bf16_big<GATE_UP, false>), grid, block, 0, st, A, W, off, Out,
                         nullptr, E_L, rows, Kdim, Nout, ntn);
  } else {
    const int ntn = (int)ceil_div(Nout, GATE_UP ? kBW / 2 : kBW);
    hipLaunchKernelGGL(k_gemm_bf16<GATE_UP>, dim3(grid_blocks(s, kBM, ntn)), dim3(256), 0, st,
                       A, W, off, Out, E_L, rows, Kdim, Nout, ntn);
  }
  return launch_status();
}

}  // namespace

int launch_expert_up(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                     const void *w_gu, void *h, hipStream_t st, void *gu) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  if (gu != nullptr && !(s.dtype == MOE_BF16 && s.d % 64 == 0)) {
    // kernels without a [G U] epilogue: the plain product, then the usual up
    const int rc = launch_gemm_nt(s, buf, w_gu, off, gu, s.d, 2 * s.F, st);
    if (rc != MOE_OK) return rc;
    gu = nullptr;
  }
  if (s.dtype == MOE_BF16)
    return launch_bf16<true>(s, static_cast<const uint16_t *>(buf),
                             static_cast<const uint16_t *>(w_gu), off, static_cast<uint16_t *>(h),
                             s.d, s.F, st, static_cast<uint16_t *>(gu));
  const int ntn = (int)ceil_div(s.F, kFW / 2);
  hipLaunchKernelGGL(k_gemm_f32<true>, dim3(grid_blocks(s, kFM, ntn)), dim3(256), 0, st,
                     static_cast<const float *>(buf), static_cast<const float *>(w_gu), off,
                     static_cast<float *>(h), E_L, (int)buffer_rows(s), s.d, s.F, ntn);
  return launch_status();
}

int launch_gemm_nt(const moe_shape_t &s, const void *A, const void *W, const int32_t *off,
                   void *Out, int Kdim, int Nout, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  if (s.dtype == MOE_BF16)
    return launch_bf16<false>(s, static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(W),
                              off, static_cast<uint16_t *>(Out), Kdim, Nout, st);
  const int ntn = (int)ceil_div(Nout, kFW);
  hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid_blocks(s, kFM, ntn)), dim3(256), 0, st,
                     static_cast<const float *>(A), static_cast<const float *>(W), off,
                     static_cast<float *>(Out), E_L, (int)buffer_rows(s), Kdim, Nout, ntn);
  return launch_status();
}

int launch_expert_down(const moe_shape_t &s, const void *h, const int32_t *offsets,
                       const void *w_d, void *y, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  if (s.dtype == MOE_BF16)
    return launch_bf16<false>(s, static_cast<const uint16_t *>(h),
                              static_cast<const uint16_t *>(w_d), off, static_cast<uint16_t *>(y),
                              s.F, s.d, st);
  const int ntn = (int)ceil_div(s.d, kFW);
  hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid_blocks(s, kFM, ntn)), dim3(256), 0, st,
                     static_cast<const float *>(h), static_cast<const float *>(w_d), off,
                     static_cast<float *>(y), E_L, (int)buffer_rows(s), s.F, s.d, ntn);
  return launch_status();
}

}  // namespace moe
