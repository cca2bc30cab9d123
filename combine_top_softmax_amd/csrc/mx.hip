// MXFP8 forward: quantize-on-dispatch and the grouped expert GEMMs on
// E4M3 data with E8M0 block scales.
//
// Olmo-core MoE report, Sec. 05 "Expert Parallelism": Sec. 5.5 (rows are
// quantized during dispatch and the expert grouped GEMM consumes the
// quantized data and scales directly), Sec. 5.8 (an MXFP8 route carries a
// qdata row and a scale row that follow the same destination indices and
// validity mask), Sec. 5.9 (E4M3 data with E8M0 scales on forward dispatch,
// MXFP8 expert GEMMs, forward combine in BF16). Block format: the OCP
// microscaling format the report cites -- 32 consecutive elements along the
// contraction dimension share the scale 2^(floor(log2 amax) - 8) (8 = the
// exponent of E4M3's largest normal, 448), stored as a biased E8M0 code, and
// each element is its value over the scale rounded to the nearest E4M3 value
// (ties to the even code), saturating at 448; an all-zero block gets code 0.
//
// Kernels:
//   k_quant_rows<true>   quantize-on-dispatch: wave per token, each lane one
//                        16-byte vector (8 bf16), four lanes per block
//                        (amax reduced across them), qdata and scale bytes
//                        written to every kept local route's row;
//   k_quant_rows<false>  the same quantizer over plain rows (expert weights,
//                        which are quantized once along their contraction
//                        dimension);
//   k_gemm_mx<GATE_UP>   grouped GEMM on v_mfma_scale_f32_32x32x64_f8f6f4:
//                        the forward bf16 kernel's schedule (device-offset
//                        tiles, XCD-aware order, 256 x 256 block tile, 8 waves
//                        of 128 x 64, two direct-load LDS stages, loads
//                        interleaved with the MFMAs) with 128-byte K steps
//                        (4 blocks); up: SwiGLU in the epilogue, H rounded to
//                        bf16 and MX-quantized along F on its way out; down:
//                        bf16 Y.
// MFMA operand layout (checked on the device): lane l holds row (or column)
// l % 32 of the 64-wide K slice, bytes 0..15 from the slice's first 32-element
// block and bytes 16..31 from its second (any order inside a block, the same
// for A and B); lane l's scale operand is the E8M0 code of block l / 32 of that
// row. Here lane l takes 16-byte chunks g and 2 + g (g = l / 32) of the slice.
#include <type_traits>

#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ MX encoding
// Shared exponent of a block: floor(log2 amax) - 8, clamped to the E8M0 range.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int e;
  (void)frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1)
  return max(-127, min(127, e - 1 - 8));
}

// E4M3 codes of v already divided by the block scale: nearest value, ties to
// the even code, saturating at 448, the sign bit from v's sign. The hardware
// fp32 -> fp8 conversion (OCP E4M3, round to nearest even) does the rounding
// once v is clamped to [-448, 448] (med3 keeps -0.0); checked on the device
// bit for bit against a direct encoding of that rule over every finite bf16
// value and shared exponents -140 .. 147. Codes of (a, b) land in bytes
// 2*HI and 2*HI + 1 of the result; the other bytes come from `old`.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t old) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, (int)old, HI);
}

// Codes of 8 bf16 values (two packed per dword) over the scale 2^se.
__device__ __forceinline__ u32x2_t quant8(const u32x4_t v, int se) {
  u32x2_t o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w =
        e4m3_pair<false>(ldexpf(bf16_lo(v[2 * h]), -se), ldexpf(bf16_hi(v[2 * h]), -se), 0u);
    o[h] = e4m3_pair<true>(ldexpf(bf16_lo(v[2 * h + 1]), -se), ldexpf(bf16_hi(v[2 * h + 1]), -se),
                           w);
  }
  return o;
}

__device__ __forceinline__ float amax8(const u32x4_t v) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[e])), fabsf(bf16_hi(v[e]))));
  return m;
}

// ------------------------------------------------------------ quantize rows
// ROUTED: row t of x goes to every route with dest_rank == ep_rank, at
// dest_row; else row r goes to row r (n_src rows). Row length d (bf16),
// d % 32 == 0. Scale rows are mx_scale_row_bytes(d) bytes apart (the d / 32
// scales, then pad bytes that are not written).
template <bool ROUTED>
__global__ __launch_bounds__(256) void k_quant_rows(
    const u32x4_t *__restrict__ x, const int32_t *__restrict__ dest_rank,
    const int32_t *__restrict__ dest_row, uint8_t *__restrict__ qdata,
    uint8_t *__restrict__ scales, int64_t n_src, int K, int d, int ep_rank, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= n_src) return;
  const int nvec = d >> 3;                 // 16-byte vectors per row
  const int nblk = mx_scale_row_bytes(d);  // scale row stride
  const u32x4_t *src = x + t * nvec;
  for (int seg = 0; seg < nvec; seg += 64) {
    const int c = seg + lane;
    const bool act = c < nvec;             // whole blocks: nvec % 4 == 0
    const u32x4_t v = act ? __builtin_nontemporal_load(src + c) : u32x4_t{0, 0, 0, 0};
    float am = amax8(v);
    am = fmaxf(am, __shfl_xor(am, 1, 64));
    am = fmaxf(am, __shfl_xor(am, 2, 64));
    const int se = mx_shared_exp(am);
    const u32x2_t q = quant8(v, se);
    const uint8_t sc = (uint8_t)(se + 127);
    if (!act) continue;
    if constexpr (ROUTED) {
      for (int k = 0; k < K; ++k) {
        const int64_t qk = t * K + k;
        const int64_t row = dest_row[qk];
        if (dest_rank[qk] != ep_rank || row < 0 || row >= rows) continue;   // outside: skipped
        *reinterpret_cast<u32x2_t *>(qdata + row * d + (int64_t)c * 8) = q;
        if ((c & 3) == 0) scales[row * nblk + (c >> 2)] = sc;
      }
    } else {
      *reinterpret_cast<u32x2_t *>(qdata + t * d + (int64_t)c * 8) = q;
      if ((c & 3) == 0) scales[t * nblk + (c >> 2)] = sc;
    }
  }
}

// ------------------------------------------------------------ MX grouped GEMM
// Waves per MX block: 8 (two per SIMD, 128 x 64 wave tiles). 4 waves (one per
// SIMD, 128 x 128 wave tiles, a third fewer LDS fragment bytes per flop)
// measured 1-5% slower on the named workloads: with two LDS stages and a full
// wait per step, a second wave per SIMD covers more of the stalls.
namespace mxg {
constexpr int BM = 256, BW = 256, BK = 128, NW = 8, NT = 64 * NW;
constexpr int WAVES_N = NW / 2, WTN = BW / WAVES_N;   // weight rows per wave
constexpr int TM = 4, TN = WTN / 32;             // 4 x TN MFMA tiles per wave
constexpr int SPW = 8 / NW;                      // scale-dword loads per wave and step
constexpr int ROW_B = BK;                        // bytes per LDS row
constexpr int RPI = 8;                           // rows per direct-load instruction
constexpr int NA = BM / RPI / NW, NB = BW / RPI / NW, L = NA + NB;
constexpr int KS = BK / 64;                      // MFMA K sub-steps per step
constexpr int A_BYTES = BM * ROW_B;
constexpr int SC_OFF = (BM + BW) * ROW_B;        // scale dwords: BM for A, then BW for B
constexpr int STAGE = SC_OFF + (BM + BW) * 4;
}  // namespace mxg

struct MxCtx {
  const uint8_t *A, *W;
  const uint8_t *S[mxg::SPW];   // this wave's scale sources (A's or the expert's W scales)
  uint32_t a_off[mxg::NA], b_off[mxg::NB];
  uint32_t s_off[mxg::SPW];     // byte offset of this lane's scale row (step 0)
  int s_dst[mxg::SPW];          // LDS byte offset of this wave's scale dwords
  int fa[mxg::TM], fb[mxg::TN];
  int sa_lds[mxg::TM], sb_lds[mxg::TN];
  int sw;
  uint32_t a_skip;            // A loads that feed only rows past the valid ones
  int kdim;                   // K (bytes of a qdata row)
  // half K step: bytes to take off a load's offset so that it reads chunk
  // (logical chunk & 3), one of the 64 valid bytes: 64 if the load's logical
  // chunk pch ^ swz(r) is 4..7, else 0. With 8 rows per load instruction, bit
  // 2 of swz(r) is bit 2 of the lane's row in the instruction, so the value
  // is the same for every A and B load of the lane.
  uint32_t hadj;
};

__device__ __forceinline__ void mx_issue(const MxCtx &c, int k0, int wv, uint32_t stage) {
  const uint32_t hm = k0 + mxg::BK > c.kdim ? ~0u : 0u;   // a half step's loads
#pragma unroll
  for (int j = 0; j < mxg::SPW; ++j)
    dma4(c.S[j] + (uint32_t)(c.s_off[j] + (k0 >> 5)), stage + c.s_dst[j]);
#pragma unroll
  for (int i = 0; i < mxg::NA; ++i)
    if (!((c.a_skip >> i) & 1))
      dma16(c.A + (uint32_t)(c.a_off[i] + k0 - (c.hadj & hm)),
            stage + (wv * mxg::NA + i) * 1024);
#pragma unroll
  for (int i = 0; i < mxg::NB; ++i)
    dma16(c.W + (uint32_t)(c.b_off[i] + k0 - (c.hadj & hm)),
          stage + mxg::A_BYTES + (wv * mxg::NB + i) * 1024);
}

// One main-loop step: 2 x 8 scaled MFMAs from `rd`, the direct loads of the
// next step into `ld` one every MFMA over the first half. Fragments are 8
// dwords (32 fp8 values): B fragments are double-buffered across the two K
// sub-steps, each A fragment is reloaded for the next sub-step right after
// its last MFMA of this one (6 MFMAs before it is needed again), which keeps
// the fragments at 64 VGPRs. sa/sb: this step's scale dwords (the 4 blocks of
// the row of the lane's fragment).
// VT: this wave's 32-row MFMA tiles that hold valid rows (fewer than TM on an
// expert's last m-tile: the others' MFMAs and A fragment reads are dropped).
// KSE: the K sub-steps this step runs (1 for a half step); LOADS: whether it
// issues the next step's loads (a half step is the last one and issues none).
template <int VT, int KSE = mxg::KS, bool LOADS = true>
__device__ __forceinline__ void mx_step(const MxCtx &c, int k0, int wv,
                                        uint32_t ld, const uint8_t *__restrict__ rd,
                                        int g, f32x16_t (&acc)[mxg::TM][mxg::TN]) {
  constexpr int MF = mxg::KS * mxg::TM * mxg::TN;   // 16
  constexpr int L = mxg::L + mxg::SPW;              // + the scale loads
  constexpr int GAP = MF / (2 * L) > 0 ? MF / (2 * L) : 1;
  // k0: the K offset (bytes) of the step loaded into `ld` (the caller repeats
  // the last step on the last iteration: no branch inside the step)
  const uint32_t hm = k0 + mxg::BK > c.kdim ? ~0u : 0u;   // loads of a half step
  auto issue_one = [&](int d) {
    if (d < mxg::NA) {
      if (VT == mxg::TM || !((c.a_skip >> d) & 1))
        dma16(c.A + (uint32_t)(c.a_off[d] + k0 - (c.hadj & hm)),
              ld + (wv * mxg::NA + d) * 1024);
    } else if (d < mxg::L)
      dma16(c.W + (uint32_t)(c.b_off[d - mxg::NA] + k0 - (c.hadj & hm)),
            ld + mxg::A_BYTES + (wv * mxg::NB + (d - mxg::NA)) * 1024);
    else {
      const int j = d - mxg::L;
      dma4(c.S[j] + (uint32_t)(c.s_off[j] + (k0 >> 5)), ld + c.s_dst[j]);
    }
  };
  // chunks g and 2 + g of the 64-byte K slice ks of LDS row `off`
  auto frag = [&](int off, int ks) {
    const int c0 = ((ks * 4 + g) ^ c.sw) << 4, c1 = ((ks * 4 + 2 + g) ^ c.sw) << 4;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(rd + off + c0);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(rd + off + c1);
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // scale dwords of the fragments' rows (the step's 4 blocks, one byte each),
  // shifted by one byte in lanes 32-63: lane group g needs blocks g (first
  // K slice) and 2 + g (second), now bytes 0 and 2 for both groups, which the
  // MFMA selects with op_sel
  // Read in the order of first use by the MFMA sequence (each fragment with
  // its rows' scale dword: A0 B0 B1 A1 A2 A3), so that the first MFMAs of the
  // step wait only for the oldest reads instead of for all of them.
  uint32_t sa[mxg::TM], sb[mxg::TN];
  const int gsh = 8 * g;
  i32x8_t fra[mxg::TM], frb[2][mxg::TN];
  constexpr FragOrder<mxg::TM, mxg::TN> ord{};
#pragma unroll
  for (int n = 0; n < mxg::TM + mxg::TN; ++n) {
    const int f = ord.q[n];
    if (f < mxg::TM) {
      sa[f] = *reinterpret_cast<const uint32_t *>(rd + c.sa_lds[f]) >> gsh;
      if (f < VT) fra[f] = frag(c.fa[f], 0);
    } else {
      const int j = f - mxg::TM;
      sb[j] = *reinterpret_cast<const uint32_t *>(rd + c.sb_lds[j]) >> gsh;
      frb[0][j] = frag(c.fb[j], 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KSE; ++ks) {
    const int cur = ks & 1;
#pragma unroll
    for (int q = 0; q < mxg::TM * mxg::TN; ++q) {
      const int gi = ks * mxg::TM * mxg::TN + q;
      const int i = q / mxg::TN, j = q % mxg::TN;
      if (i < VT) {
        if (ks == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fra[i], frb[cur][j], acc[i][j], 0, 0, 0, (int)sa[i], 0, (int)sb[j]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fra[i], frb[cur][j], acc[i][j], 0, 0, 2, (int)sa[i], 2, (int)sb[j]);
      }
      if (ks + 1 < KSE) {
        if (q < mxg::TN) frb[cur ^ 1][q] = frag(c.fb[q], ks + 1);
        if (j == mxg::TN - 1 && i < VT) fra[i] = frag(c.fa[i], ks + 1);
      }
      if (LOADS && gi % GAP == 0 && gi / GAP < L) issue_one(gi / GAP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// A: qdata rows [rows, Kdim] with scales As [rows, SK]; W: expert weights
// [E_L, Nw, Kdim] (Nw = 2 Nout for GATE_UP: gate rows then up rows) with
// scales Ws [E_L, Nw, SK]; SK = mx_scale_row_bytes(Kdim). GATE_UP: H =
// silu(G) * U (Nout = F columns) rounded to bf16, written as qdata OutQ
// [rows, Nout] and scales OutS [rows, mx_scale_row_bytes(Nout)]; else
// Y = A W^T in bf16 (OutY [rows, Nout]). Kdim % 64 == 0: when Kdim % 128 ==
// 64 the last K step is half a step (one 64-wide MFMA sub-step); its loads
// read only the 64 valid bytes of each row (the other lanes load a valid
// chunk again, into LDS bytes no MFMA reads) and the scale dword it reads
// ends in two pad bytes of the scale row.
template <bool GATE_UP>
__global__ __launch_bounds__(mxg::NT, 1) void k_gemm_mx(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const uint8_t *__restrict__ W,
    const uint8_t *__restrict__ Ws, const int32_t *__restrict__ off, uint8_t *__restrict__ OutQ,
    uint8_t *__restrict__ OutS, uint16_t *__restrict__ OutY, int E_L, int rows, int Kdim,
    int Nout, int n_tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * mxg::STAGE];
  RowTile tl = find_row_tile(off, E_L, mxg::BM, rows, n_tiles_n);
  if (!tl.valid) return;
  // wave-uniform: keep the tile in scalar registers (scalar load bases)
  tl.expert = __builtin_amdgcn_readfirstlane(tl.expert);
  tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
  tl.row_end = __builtin_amdgcn_readfirstlane(tl.row_end);
  tl.n_idx = __builtin_amdgcn_readfirstlane(tl.n_idx);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / mxg::WAVES_N, wn = wv % mxg::WAVES_N;
  const int fr = lane & 31, g = lane >> 5;
  const int Nw = GATE_UP ? 2 * Nout : Nout;
  const int n0 = tl.n_idx * (GATE_UP ? mxg::BW / 2 : mxg::BW);
  const int kb32 = mx_scale_row_bytes(Kdim);   // scale row stride

  MxCtx c;
  // A rows and their scale rows are addressed from the tile's first row
  // (64-bit bases), so the 32-bit offsets stay below BM * Kdim
  c.A = A + (size_t)tl.row0 * Kdim;
  c.W = W + (size_t)tl.expert * Nw * Kdim;
  auto wrow_of = [&](int r) {               // block weight row r -> weight row
    if (GATE_UP)
      return (r < mxg::BW / 2) ? min(n0 + r, Nout - 1) : Nout + min(n0 + r - mxg::BW / 2, Nout - 1);
    return min(n0 + r, Nout - 1);
  };
  {
    const int lrow = lane >> 3, pch = lane & 7;
#pragma unroll
    for (int i = 0; i < mxg::NA; ++i) {
      const int r = (wv * mxg::NA + i) * mxg::RPI + lrow;
      const int tr = min(r, tl.row_end - 1 - tl.row0);   // clamped rows are discarded
      c.a_off[i] = (uint32_t)tr * (uint32_t)Kdim + ((pch ^ chunk_swz<8>(r)) << 4);
    }
#pragma unroll
    for (int i = 0; i < mxg::NB; ++i) {
      const int r = (wv * mxg::NB + i) * mxg::RPI + lrow;
      c.b_off[i] = (uint32_t)wrow_of(r) * (uint32_t)Kdim + ((pch ^ chunk_swz<8>(r)) << 4);
    }
    static_assert(mxg::RPI == 8, "bit 2 of swz(r) is bit 2 of lrow");
    c.hadj = ((pch ^ lrow) & 4) << 4;
  }
  c.kdim = Kdim;
  c.sw = chunk_swz<8>(fr);
  // scale dwords of one step (4 blocks per row) through LDS, one dword per
  // lane: scale load u = wv * SPW + j takes A's rows 64u .. 64u+63 for u < 4,
  // else the block's weight rows 64(u-4) .. 64(u-4)+63
#pragma unroll
  for (int j = 0; j < mxg::SPW; ++j) {
    const int u = wv * mxg::SPW + j;
    const int r = (u & 3) * 64 + lane;
    if (u < 4) {
      c.S[j] = As + (size_t)tl.row0 * kb32;
      c.s_off[j] = (uint32_t)min(r, tl.row_end - 1 - tl.row0) * (uint32_t)kb32;
      c.s_dst[j] = mxg::SC_OFF + (u & 3) * 256;
    } else {
      c.S[j] = Ws + (size_t)tl.expert * Nw * kb32;
      c.s_off[j] = (uint32_t)wrow_of(r) * (uint32_t)kb32;
      c.s_dst[j] = mxg::SC_OFF + mxg::BM * 4 + (u & 3) * 256;
    }
  }
  // fragment rows and the LDS scale dwords that go with them
#pragma unroll
  for (int t = 0; t < mxg::TM; ++t) {
    const int r = wm * 128 + t * 32 + fr;
    c.fa[t] = r * mxg::ROW_B;
    c.sa_lds[t] = mxg::SC_OFF + r * 4;
  }
#pragma unroll
  for (int t = 0; t < mxg::TN; ++t) {
    int brow;
    if (GATE_UP)
      brow = (t < mxg::TN / 2) ? wn * (mxg::WTN / 2) + t * 32
                               : mxg::BW / 2 + wn * (mxg::WTN / 2) + (t - mxg::TN / 2) * 32;
    else
      brow = wn * mxg::WTN + t * 32;
    c.fb[t] = mxg::A_BYTES + (brow + fr) * mxg::ROW_B;
    c.sb_lds[t] = mxg::SC_OFF + mxg::BM * 4 + (brow + fr) * 4;
  }

  f32x16_t acc[mxg::TM][mxg::TN];
#pragma unroll
  for (int i = 0; i < mxg::TM; ++i)
#pragma unroll
    for (int j = 0; j < mxg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (Kdim + mxg::BK - 1) / mxg::BK;
  const int nfull = Kdim / mxg::BK;           // nk - 1 when the last step is a half step
  // this wave's valid 32-row MFMA tiles and the A loads that feed only rows
  // past the last valid 32-row group of the tile (wave-uniform)
  const int nvalid = min(mxg::BM, tl.row_end - tl.row0);
  const int vt = __builtin_amdgcn_readfirstlane(min(mxg::TM, max(0, (nvalid - wm * 128 + 31) / 32)));
  c.a_skip = 0;
#pragma unroll
  for (int i = 0; i < mxg::NA; ++i)
    if ((wv * mxg::NA + i) * mxg::RPI >= ((nvalid + 31) / 32) * 32) c.a_skip |= 1u << i;
  c.a_skip = __builtin_amdgcn_readfirstlane(c.a_skip);
  const uint32_t smem_l = lds_addr(smem);
  mx_issue(c, 0, wv, smem_l);
  auto main_loop = [&](auto vt_tag) {
    constexpr int VT = decltype(vt_tag)::value;
    for (int kb = 0; kb < nfull; ++kb) {
      wait_vmcnt<0>();                    // this wave's loads of step kb have landed ...
      __builtin_amdgcn_s_barrier();       // ... and every wave's
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ld = smem_l + ((kb + 1) & 1) * mxg::STAGE;
      const uint8_t *rd = smem + (kb & 1) * mxg::STAGE;
      // the next step's loads; the last step, when it is a full one, reloads
      // its own step into the idle stage (in bounds, never read; drained
      // before the epilogue)
      mx_step<VT>(c, min(kb + 1, nk - 1) * mxg::BK, wv, ld, rd, g, acc);
    }
    if (nfull < nk) {                     // the half step: loads nothing
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mx_step<VT, 1, false>(c, nfull * mxg::BK, wv, smem_l, smem + (nfull & 1) * mxg::STAGE, g,
                            acc);
    }
  };
  switch (vt) {
    case 4: main_loop(std::integral_constant<int, 4>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    default: main_loop(std::integral_constant<int, 0>{}); break;
  }
  wait_vmcnt<0>();   // no direct load still in flight into the stages

  // Epilogue through LDS (the forward's): neighbouring lanes swap one value
  // (DPP) so each writes two adjacent columns of one row as a bf16x2 dword;
  // chunk c of LDS row r sits at c ^ 4*q(r), q(r) = bit0(r) | bit2(r) << 1.
  constexpr int OUTC = GATE_UP ? mxg::BW / 2 : mxg::BW;
  constexpr int ROWB = OUTC * 2;
  __syncthreads();
  auto stage_off = [](int row, int colb) {
    const int q = (row & 1) | (((row >> 2) & 1) << 1);
    return row * ROWB + ((((colb >> 4) ^ (q << 2))) << 4) + (colb & 15);
  };
  const bool odd = (lane & 1) != 0;
#pragma unroll
  for (int tm = 0; tm < mxg::TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < (GATE_UP ? mxg::TN / 2 : mxg::TN); ++tn) {
      const int colb0 = (GATE_UP ? wn * (mxg::WTN / 2) : wn * mxg::WTN) * 2 + tn * 64;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float v0, v1;
        if (GATE_UP) {
          const float g0 = acc[tm][tn][r], u0 = acc[tm][tn + mxg::TN / 2][r];
          const float g1 = acc[tm][tn][r + 1], u1 = acc[tm][tn + mxg::TN / 2][r + 1];
          v0 = g0 * __builtin_amdgcn_rcpf(1.0f + __expf(-g0)) * u0;
          v1 = g1 * __builtin_amdgcn_rcpf(1.0f + __expf(-g1)) * u1;
        } else {
          v0 = acc[tm][tn][r];
          v1 = acc[tm][tn][r + 1];
        }
        const float send = odd ? v0 : v1;
        const float recv = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
        const int row = wm * 128 + tm * 32 + (r >> 2) * 8 + g * 4 + (r & 3) + (odd ? 1 : 0);
        const int colb = colb0 + (fr & ~1) * 2;
        const uint32_t packed = odd ? pack_bf16x2(recv, v1) : pack_bf16x2(v0, recv);
        *reinterpret_cast<uint32_t *>(smem + stage_off(row, colb)) = packed;
      }
    }
  }
  __syncthreads();
  const int ncols = min(OUTC, Nout - n0);               // multiple of 32
  const int nrows = min(mxg::BM, tl.row_end - tl.row0);
  if constexpr (GATE_UP) {
    // H (bf16 in LDS) quantized along F: one 32-column block of a row per task
    const int nblk_row = mx_scale_row_bytes(Nout);
    for (int idx = tid; idx < mxg::BM * (OUTC / 32); idx += mxg::NT) {
      const int row = idx / (OUTC / 32), blk = idx % (OUTC / 32);
      if (row >= nrows || blk * 32 >= ncols) continue;
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = *reinterpret_cast<const u32x4_t *>(smem + stage_off(row, blk * 64 + q * 16));
      const float am = fmaxf(fmaxf(amax8(v[0]), amax8(v[1])), fmaxf(amax8(v[2]), amax8(v[3])));
      const int se = mx_shared_exp(am);
      const size_t grow = (size_t)(tl.row0 + row);
      uint8_t *dst = OutQ + grow * Nout + n0 + blk * 32;
      const u32x2_t q0 = quant8(v[0], se), q1 = quant8(v[1], se);
      const u32x2_t q2 = quant8(v[2], se), q3 = quant8(v[3], se);
      *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{q0[0], q0[1], q1[0], q1[1]};
      *reinterpret_cast<u32x4_t *>(dst + 16) = u32x4_t{q2[0], q2[1], q3[0], q3[1]};
      OutS[grow * nblk_row + (n0 >> 5) + blk] = (uint8_t)(se + 127);
    }
  } else {
    constexpr int CPR = ROWB / 16;
#pragma unroll 4
    for (int idx = tid; idx < mxg::BM * CPR; idx += mxg::NT) {
      const int row = idx / CPR, ch = idx % CPR;
      if (row < nrows && ch * 8 < ncols) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + stage_off(row, ch * 16));
        *reinterpret_cast<u32x4_t *>(OutY + (size_t)(tl.row0 + row) * Nout + n0 + ch * 8) = v;
      }
    }
  }
}

inline unsigned mx_grid(const moe_shape_t &s, int ntn) {
  const int E_L = s.N / s.ep_size;
  const int64_t max_m = ceil_div(buffer_rows(s), mxg::BM) + E_L;
  return (unsigned)(ceil_div(max_m * ntn, kNumXcd) * kNumXcd);
}

}  // namespace

int launch_quantize_rows(int64_t rows, int cols, const void *src, uint8_t *qdata, uint8_t *scales,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_quant_rows<false>, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, st,
                     static_cast<const u32x4_t *>(src), nullptr, nullptr, qdata, scales, rows, 1,
                     cols, 0, rows);
  return launch_status();
}

int launch_dispatch_mx(const moe_shape_t &s, const void *x, const int32_t *dest_rank,
                       const int32_t *dest_row, uint8_t *qbuf, uint8_t *sbuf, hipStream_t st) {
  hipLaunchKernelGGL(k_quant_rows<true>, dim3((unsigned)ceil_div(s.T, 4)), dim3(256), 0, st,
                     static_cast<const u32x4_t *>(x), dest_rank, dest_row, qbuf, sbuf,
                     (int64_t)s.T, s.K, s.d, s.ep_rank, buffer_rows(s));
  return launch_status();
}

int launch_expert_up_mx(const moe_shape_t &s, const uint8_t *qbuf, const uint8_t *sbuf,
                        const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                        uint8_t *h_q, uint8_t *h_s, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  const int ntn = (int)ceil_div(s.F, mxg::BW / 2);
  hipLaunchKernelGGL(k_gemm_mx<true>, dim3(mx_grid(s, ntn)), dim3(mxg::NT), 0, st, qbuf, sbuf,
                     w_gu_q, w_gu_s, off, h_q, h_s, nullptr, E_L, (int)buffer_rows(s), s.d, s.F,
                     ntn);
  return launch_status();
}

int launch_expert_down_mx(const moe_shape_t &s, const uint8_t *h_q, const uint8_t *h_s,
                          const int32_t *offsets, const uint8_t *w_d_q, const uint8_t *w_d_s,
                          void *y, hipStream_t st) {
  const int E_L = s.N / s.ep_size;
  const int32_t *off = offsets + (size_t)s.ep_rank * (E_L + 1);
  const int ntn = (int)ceil_div(s.d, mxg::BW);
  hipLaunchKernelGGL(k_gemm_mx<false>, dim3(mx_grid(s, ntn)), dim3(mxg::NT), 0, st, h_q, h_s,
                     w_d_q, w_d_s, off, nullptr, nullptr, static_cast<uint16_t *>(y), E_L,
                     (int)buffer_rows(s), s.F, s.d, ntn);
  return launch_status();
}

}  // namespace moe
