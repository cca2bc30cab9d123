// Internal declarations shared by the HIP translation units of libmoe_hip.
// Not part of the public C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kRouteTile = 64;     // tokens per routing tile (one lane per token in its ballots)
constexpr int kNumXcd = 8;         // MI355X: 8 accelerator complex dies, each with its own L2

// ---- host-side helpers -----------------------------------------------------
inline int elem_bytes(moe_dtype_t dt) { return dt == MOE_F32 ? 4 : 2; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// at least one tile, so an empty batch still writes counts, offsets and row_src
inline int route_tiles(const moe_shape_t &s) {
  return s.T > 0 ? (int)ceil_div(s.T, kRouteTile) : 1;
}
// Rows of every capacity-shaped buffer (moe_buffer_rows): the kept local
// routes never exceed E_L*C, nor max(T,1)*min(K, E_L) (a token's K experts
// are distinct, so at most min(K, E_L) of its routes are local).
inline int64_t buffer_rows(const moe_shape_t &s) {
  const int64_t E_L = s.N / s.ep_size;
  const int64_t per_tok = s.K < E_L ? s.K : E_L;
  const int64_t by_tok = (int64_t)(s.T > 0 ? s.T : 1) * per_tok;
  return E_L * s.capacity < by_tok ? E_L * s.capacity : by_tok;
}

// Bytes between consecutive MX scale rows of `cols` elements: the cols / 32
// block scales rounded up to a multiple of 4, so that every row's scales
// start 4-byte aligned (the GEMMs load them as dwords).
__host__ __device__ inline int mx_scale_row_bytes(int cols) { return ((cols >> 5) + 3) & ~3; }

// Launchers (return MOE_OK or MOE_EHIP). Shapes are already validated.
int launch_route(const moe_shape_t &s, const float *logits, const int32_t *ids_in,
                 const moe_route_out_t &o, void *ws, hipStream_t st);
int launch_dispatch(const moe_shape_t &s, const void *x, const int32_t *dest_rank,
                    const int32_t *dest_row, void *buf, hipStream_t st);
int launch_combine(const moe_shape_t &s, const void *y, const int32_t *dest_rank,
                   const int32_t *dest_row, const float *w, void *out, hipStream_t st);
// gu != nullptr: also write the pre-activation [G U] rows ([rows, 2F]), equal
// bit for bit to launch_gemm_nt(buf, w_gu) over the same rows.
int launch_expert_up(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                     const void *w_gu, void *h, hipStream_t st, void *gu = nullptr);
int launch_expert_down(const moe_shape_t &s, const void *h, const int32_t *offsets,
                       const void *w_d, void *y, hipStream_t st);
// Out[r, :] = A[r] W[j]^T over the rows [off[j], off[j+1]) of each local expert
// j (off already offset to this rank), W[j] = [Nout, Kdim]; no activation.
int launch_gemm_nt(const moe_shape_t &s, const void *A, const void *W, const int32_t *off,
                   void *Out, int Kdim, int Nout, hipStream_t st);
// Backward.
int launch_combine_bwd(const moe_shape_t &s, const void *dout, const void *y,
                       const int32_t *dest_rank, const int32_t *dest_row, const float *w, void *dy,
                       float *dw, hipStream_t st);
int launch_route_bwd(const moe_shape_t &s, const int32_t *idx, const float *w, const float *dw,
                     float *dlogits, hipStream_t st);
// MXFP8 forward.
int launch_quantize_rows(int64_t rows, int cols, const void *src, uint8_t *qdata, uint8_t *scales,
                         hipStream_t st);
int launch_dispatch_mx(const moe_shape_t &s, const void *x, const int32_t *dest_rank,
                       const int32_t *dest_row, uint8_t *qbuf, uint8_t *sbuf, hipStream_t st);
int launch_expert_up_mx(const moe_shape_t &s, const uint8_t *qbuf, const uint8_t *sbuf,
                        const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                        uint8_t *h_q, uint8_t *h_s, hipStream_t st);
int launch_expert_down_mx(const moe_shape_t &s, const uint8_t *h_q, const uint8_t *h_s,
                          const int32_t *offsets, const uint8_t *w_d_q, const uint8_t *w_d_s,
                          void *y, hipStream_t st);
int launch_expert_ffn_bwd_data(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                               const void *w_gu, const void *w_down, const void *dy, void *gu,
                               void *dgu, void *dx_rows, hipStream_t st);
// The data half from [G U] rows already in gu (no recompute).
int launch_expert_ffn_bwd_data_gu(const moe_shape_t &s, const int32_t *offsets, const void *w_gu,
                                  const void *w_down, const void *dy, const void *gu, void *dgu,
                                  void *dx_rows, hipStream_t st);
int launch_expert_ffn_bwd_weight(const moe_shape_t &s, const void *buf, const int32_t *offsets,
                                 const void *h, const void *dy, const void *dgu, float *dw_gu,
                                 float *dw_down, hipStream_t st);

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// ---- device-side helpers ---------------------------------------------------
// bfloat16 <-> float. The float -> bf16 conversion of __bf16 rounds to nearest
// even (the gfx950 hardware conversion).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
// Same result as pack_bf16x2 (round to nearest even) in one packed conversion.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Wave-wide inclusive prefix sum over the 64 lanes in DPP moves (no LDS round
// trip): shifts by 1, 2, 4 and 8 lanes inside each row of 16 lanes (lanes
// with no source add 0), then lane 15 of rows 0 and 2 added into rows 1 and 3,
// then lane 31 added into the upper half. All 64 lanes must be active.
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}


}  // namespace moe
