/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer (forward and
 * backward).
 *
 * The layer runs in four stream-ordered calls, the rowwise path of the
 * Olmo-core MoE report (Sec. 05 "Expert Parallelism", Sec. 5.4 and Fig. 16):
 *
 *   moe_route          top-K gating + route metadata (counts, offsets, route map)
 *   moe_dispatch_rows  each kept route's token row copied into its capacity row
 *   moe_expert_ffn     grouped SwiGLU expert FFN over each expert's valid rows
 *   moe_combine        router-weighted gather back to token order
 *
 * General conventions (apply to every call):
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the moe_shape_t / moe_route_out_t structs themselves and the size_t
 *     out-parameter of moe_route_workspace_size, which are host memory.
 *   - Sizes are element counts; matrices are row-major and dense.
 *   - Every call is enqueued on `stream` (0 = the null stream) and returns
 *     without waiting. Outputs are valid once the stream reaches that point.
 *     The library never copies device data to the host, never synchronizes,
 *     never allocates and keeps no state between calls (Olmo-core MoE report,
 *     Sec. 08 "Synchronization-Free Training", Sec. 8.5: route metadata stays
 *     on the device; capacity-shaped buffers are fixed before the loop).
 *     The one exception is moe_route_noalloc, whose scratch is a static
 *     device array whose address is looked up once per device.
 *   - Only host arguments are validated. Return value 0 = success, otherwise
 *     one of the negative MOE_E* codes below; nothing is enqueued on error.
 *   - Device-data preconditions that are NOT checked (checking would need a
 *     device-to-host read): moe_route_map ids lie in
 *     [-1, N) and the valid ids of one token are distinct; buf, h, y and out
 *     do not alias each other or the inputs. Route maps and offsets that
 *     reach the row calls and the GEMMs are bounded on the device instead:
 *     rows outside [0, Rmax) are skipped and offsets are clamped into
 *     [0, Rmax] (see moe_route_out_t and moe_expert_ffn).
 *   - Expert placement is contiguous: rank r owns global experts
 *     [r*E_L, (r+1)*E_L), E_L = N / ep_size; this GPU is rank ep_rank and
 *     holds only its E_L experts (AWS Neuron vLLM "Expert Parallelism (EP)"
 *     design, weight layout across ranks).
 *   - Capacity C is per expert; an expert keeps its first C routes in token
 *     order and drops the rest. The caller computes C (normally
 *     ceil(T*K*cf/N)) and sizes the buffers with it.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* Return codes. */
#define MOE_OK          0
#define MOE_EINVAL     -1  /* a size or index is out of range                      */
#define MOE_EDTYPE     -2  /* unknown dtype                                         */
#define MOE_EALIGN     -3  /* a data pointer is NULL or not 16-byte aligned         */
#define MOE_EWORKSPACE -4  /* workspace NULL or smaller than moe_route_workspace_size */
#define MOE_EHIP       -5  /* the HIP runtime rejected a kernel launch              */
#define MOE_ESCRATCH   -6  /* the shape needs more than MOE_NOALLOC_SCRATCH_BYTES   */

/* Limits of this implementation (MOE_EINVAL beyond them). */
#define MOE_MAX_K        16     /* top-K                     */
#define MOE_MAX_EXPERTS  1024   /* N                         */
#define MOE_MAX_WIDTH    (1 << 20)  /* d and F                */

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Layer shape. T tokens, hidden d, N global experts, top-K, expert SwiGLU
 * width F, ep_size expert shards of which this GPU is ep_rank, per-expert
 * capacity C, and the dtype of x / buf / weights / h / y / out.
 * Validated: T >= 0 and every other size >= 1, K <= N, K <= MOE_MAX_K,
 * N <= MOE_MAX_EXPERTS, N % ep_size == 0, 0 <= ep_rank < ep_size, d and F
 * multiples of 8 and at most MOE_MAX_WIDTH, T*K < 2^31, 2*F*d < 2^31 (one
 * expert's weight matrix; the GEMMs address a weight row and a tile's rows
 * with 32-bit offsets from 64-bit bases), and the grouped-GEMM tile count
 * (ceil(Rmax/64) + E_L) * ceil(max(2F, d)/32) < 2^31. Any capacity C >= 1 is valid; C >= T keeps
 * every route (no expert can receive more than T routes): the dropless mode,
 * with buffers of the upper-bound size Rmax below and no host-visible count.
 * An empty batch (T == 0) is valid: moe_route / moe_route_map write zero
 * counts and offsets and a row_src of -1 (their [T,K] pointers may be NULL),
 * moe_expert_ffn finds no row, and moe_dispatch_rows / moe_combine return
 * MOE_OK without touching memory. */
typedef struct {
  int32_t T, d, N, K, F, ep_size, ep_rank, capacity;
  moe_dtype_t dtype;
} moe_shape_t;

/* Rows Rmax of every capacity-shaped buffer of a rank (buf, h, y, gu, dgu, dy,
 * dx_rows, row_src and the MXFP8 qbuf, sbuf, h_q, h_s; "[Rmax, ...]" below):
 *   Rmax = min(E_L*C, max(T,1) * min(K, E_L)),
 * the most kept local routes there can be: each local expert keeps at most C,
 * and a token's K experts are distinct, so at most min(K, E_L) of its routes
 * are local (max(T,1): an empty batch still gets one-row buffers). Only the
 * packed prefix (offsets[ep_rank*(E_L+1)+E_L] rows) is ever read or written.
 * With C >= T this is the preallocated upper-bound buffer of a sync-free
 * dropless layer (Olmo-core MoE report, Section 23: Related MoE Systems Make
 * Different Trade-offs, Sec. 23.3: dispatch into preallocated upper-bound
 * buffers with device-side grouped GEMM instead of a host sync on counts);
 * with a smaller C it is the fixed capacity envelope of Sec. 8.5 (report
 * Section 08), which may drop routes. Returns Rmax, or a negative MOE_E* code
 * for an invalid shape. */
int64_t moe_buffer_rows(const moe_shape_t *shape);

/* Outputs of moe_route / moe_route_map (all device pointers).
 *   topk_idx  [T,K] int32  expert ids, logit-descending, ties -> lower id
 *   topk_w    [T,K] fp32   softmax over the K selected logits
 *   dest_rank [T,K] int32  owning rank of each kept route, -1 dropped/invalid
 *   dest_row  [T,K] int32  row in that rank's capacity buffer, -1 dropped/invalid
 *   drop_mask [T,K] uint8  1 = valid route dropped at capacity, else 0
 *   counts    [N]   int32  routes per global expert before the capacity cut
 *   offsets   [ep_size*(E_L+1)] int32  per rank r, entry r*(E_L+1)+j is the
 *             number of kept rows of r's local experts j' < j (j = 0..E_L):
 *             the cumulative offsets the grouped FFN consumes
 *   row_src   [Rmax] int32 or NULL   for rank ep_rank: t*K+k of the route
 *             stored in each row, -1 on every row after the packed prefix
 * Olmo-core MoE report Sec. 5.4: two [T,K] tensors give destination rank and
 * destination row, negative entries mark invalid or capacity-dropped routes;
 * the row is the expert's offset on its rank plus the number of earlier
 * accepted routes for that expert.
 * The row calls (moe_dispatch_rows, moe_combine, moe_combine_bwd,
 * moe_dispatch_bwd, moe_dispatch_rows_mx) take route (t,k) as local when
 * dest_rank[t,k] == ep_rank and 0 <= dest_row[t,k] < Rmax; a route of this
 * rank whose row lies outside that range is skipped (nothing read or written
 * for it, dw[t,k] = 0), so a route map from any source keeps them inside
 * their buffers. moe_route and moe_route_map never produce such a route. */
typedef struct {
  int32_t *topk_idx;
  float   *topk_w;
  int32_t *dest_rank;
  int32_t *dest_row;
  uint8_t *drop_mask;
  int32_t *counts;
  int32_t *offsets;
  int32_t *row_src;
} moe_route_out_t;

/* Bytes of device workspace moe_route / moe_route_map need for `shape`.
 * Returns MOE_EINVAL/MOE_EDTYPE for an invalid shape. */
int moe_route_workspace_size(const moe_shape_t *shape, size_t *bytes);

/* Top-K softmax gating and the route-map builder.
 * logits [T,N] fp32 (device). For each token: the K largest logits (ties ->
 * lower expert id, -0.0 == +0.0; -inf ranks below every number and NaN after
 * every number, so any input selects K distinct experts; weights that meet
 * inf - inf or NaN come out NaN), their softmax weights (Olmo-core MoE report
 * Sec. 05 Fig. 15: K ids and K weights per token, descending, summing to one),
 * then counts, capacity admission in token order, offsets and the route map
 * (Sec. 5.4, Fig. 16). All outputs except row_src are required; ws/ws_bytes
 * is a device workspace of at least moe_route_workspace_size bytes (its
 * contents on entry do not matter). */
int moe_route(const moe_shape_t *shape, const float *logits, const moe_route_out_t *out,
              void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_route without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES held by the library on every GPU it runs on until
 * the process ends; the call allocates nothing and frees nothing. Outputs,
 * validation and kernels are those of moe_route, and the results are equal
 * bit for bit. The first call on a device (with that device current) looks
 * up the array's address with hipGetSymbolAddress, so make one call outside
 * a graph capture before capturing. Returns MOE_ESCRATCH when
 * moe_route_workspace_size(shape) exceeds MOE_NOALLOC_SCRATCH_BYTES (the
 * workspace is 4*N/64 + K bytes per token: with N = 256 and K = 8 up to about
 * 699,000 tokens fit), MOE_EHIP when
 * the address lookup fails. Every call on one GPU shares the array: calls
 * that may run concurrently on one GPU (different streams without ordering,
 * or different host threads) race and give undefined results; calls ordered
 * on one stream do not. Nothing in the array has to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_route_noalloc(const moe_shape_t *shape, const float *logits, const moe_route_out_t *out,
                      hipStream_t stream);

/* The route-map builder alone (Olmo-core MoE report Sec. 5.4): as moe_route
 * but from given ids. topk_idx_in [T,K] int32, -1 = invalid route (gets
 * dest_rank = dest_row = -1 and drop_mask = 0). out->topk_idx and
 * out->topk_w are ignored and may be NULL. */
int moe_route_map(const moe_shape_t *shape, const int32_t *topk_idx_in,
                  const moe_route_out_t *out, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* Rowwise dispatch (Olmo-core MoE report Sec. 5.6, Table 8, dispatch forward:
 * the token source pushes x_t to the capacity row of the selected expert;
 * negative destinations are skipped). buf[dest_row[t,k]] = x[t] for every
 * route with dest_rank[t,k] == ep_rank. x [T,d], buf [Rmax, d] in dtype.
 * Rows of buf after the packed prefix are neither read nor written. */
int moe_dispatch_rows(const moe_shape_t *shape, const void *x, const int32_t *dest_rank,
                      const int32_t *dest_row, void *buf, hipStream_t stream);

/* Grouped expert SwiGLU FFN over the packed prefix (Olmo-core MoE report
 * Sec. 5.7: experts packed back to back from row 0, grouped GEMM skips the
 * tail; Sec. 08, Sec. 8.5: int32 device cumulative offsets, tail-aware
 * SwiGLU). For each local expert j with rows [o_j, o_{j+1}) where
 * o = offsets + ep_rank*(E_L+1):
 *   G = X W_gu[j][0:F]^T,  U = X W_gu[j][F:2F]^T,  H = silu(G) * U,
 *   Y = H W_d[j]^T
 * buf [Rmax, d], w_gu [E_L, 2F, d] (rows 0..F-1 gate, F..2F-1 up),
 * w_down [E_L, d, F], h [Rmax, F] (caller-owned scratch), y [Rmax, d];
 * all in dtype. Accumulation is fp32; H and Y are stored in dtype with
 * round-to-nearest-even. Only prefix rows of h and y are written.
 * Every grouped GEMM here and below (forward, backward, MXFP8) reads each
 * expert's range as [min(max(o_j,0),Rmax), min(max(o_{j+1},start),Rmax)),
 * so offsets from any source keep it inside the row buffers; offsets that
 * are not non-decreasing give overlapping experts and unspecified values. */
int moe_expert_ffn(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                   const void *w_gu, const void *w_down, void *h, void *y,
                   hipStream_t stream);

/* The two halves of moe_expert_ffn, same arguments and layouts:
 * moe_expert_up writes h = silu(X W_gate^T) * (X W_up^T) for the prefix rows;
 * moe_expert_down writes y = h W_d^T for the prefix rows. */
int moe_expert_up(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                  const void *w_gu, void *h, hipStream_t stream);
int moe_expert_down(const moe_shape_t *shape, const void *h, const int32_t *offsets,
                    const void *w_down, void *y, hipStream_t stream);

/* Training forward of the up half: moe_expert_up, and in the same pass the
 * pre-activation rows [G U] = X W_gu[j]^T that the expert backward reads
 * (the [G U] of moe_expert_ffn_bwd), so that moe_expert_ffn_bwd_data_saved_gu
 * can skip recomputing them. gu [Rmax, 2F] in dtype, caller-owned: only the
 * prefix rows are written, gate columns 0..F-1 then up columns F..2F-1, each
 * value the fp32 accumulator rounded to nearest even. h is the same as
 * moe_expert_up writes, and gu the same, bit for bit, as the recompute inside
 * moe_expert_ffn_bwd_data writes for the same rows. */
int moe_expert_up_save_gu(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                          const void *w_gu, void *h, void *gu, hipStream_t stream);

/* Weighted combine (Olmo-core MoE report Sec. 5.6, Table 8, combine forward:
 * the token source pulls the selected expert rows and performs the
 * router-weighted reduction; invalid entries gather zero). For every token t:
 *   out[t] = sum over k ascending with dest_rank[t,k] == ep_rank of
 *            topk_w[t,k] * y[dest_row[t,k]]
 * accumulated in fp32 and stored in dtype; a token with no kept local route
 * gets an exact zero row. On an expert shard this is the shard's partial
 * output; the sum over all ranks is the full layer output (AWS Neuron EP
 * design, "Why a single all-reduce works"). y [Rmax, d], out [T,d]. */
int moe_combine(const moe_shape_t *shape, const void *y, const int32_t *dest_rank,
                const int32_t *dest_row, const float *topk_w, void *out,
                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward. The adjoint of the forward calls for an output gradient dout,
 * reusing the forward's saved route map and buffers (Olmo-core MoE report
 * Sec. 5.6, Table 8: combine backward, dispatch backward and the
 * router-weight gradient run on the same destination rank/row indices as the
 * forward; Sec. 5.7: the expert backward GEMMs cover the packed prefix only).
 * Order: moe_combine_bwd, moe_expert_ffn_bwd, moe_dispatch_bwd, moe_route_bwd;
 * or, with the expert backward in its two halves: moe_combine_bwd,
 * moe_expert_ffn_bwd_data, moe_dispatch_bwd, moe_route_bwd,
 * moe_expert_ffn_bwd_weight.
 * On an expert shard each call yields the shard's contribution; dx and dlogits
 * of the whole layer are the sums over the ranks.
 * ------------------------------------------------------------------------ */

/* Combine backward (Table 8: the weighted output gradient is pushed to each
 * accepted route's expert-output row; the router-weight gradient uses the
 * gathered expert output with the same token's output gradient).
 * dout [T,d] and y [Rmax,d] (the forward's expert outputs) in dtype,
 * topk_w [T,K] fp32. For every route with dest_rank[t,k] == ep_rank:
 *   dy[dest_row[t,k]] = topk_w[t,k] * dout[t]      (stored in dtype)
 *   dw[t,k]           = <dout[t], y[dest_row[t,k]]> (fp32 accumulation)
 * every other route gets dw[t,k] = 0. dy [Rmax,d]: exactly the packed prefix
 * rows are written; dw [T,K] fp32 is fully written. T == 0: MOE_OK, nothing
 * touched. */
int moe_combine_bwd(const moe_shape_t *shape, const void *dout, const void *y,
                    const int32_t *dest_rank, const int32_t *dest_row, const float *topk_w,
                    void *dy, float *dw, hipStream_t stream);

/* Expert FFN backward over each local expert j's rows [o_j, o_{j+1})
 * (o = offsets + ep_rank*(E_L+1), as in moe_expert_ffn), with X = buf rows,
 * H = h rows (the forward's) and dY = dy rows (from moe_combine_bwd):
 *   [G U] = X W_gu[j]^T                          recomputed, stored in gu
 *   dH = dY W_d[j],  s = sigmoid(G)
 *   dG = dH * U * s * (1 + G*(1 - s)),  dU = dH * G * s   stored in dgu = [dG dU]
 *   dx_rows = [dG dU] W_gu[j]
 *   dw_down[j] = dY^T H,  dw_gu[j] = [dG dU]^T X     (fp32)
 * gu, dgu [Rmax, 2F] and dx_rows [Rmax, d] in dtype: caller-owned, only the
 * prefix rows are written; dgu may be the same buffer as gu (gu is then
 * overwritten). Accumulation is fp32; row results are stored in dtype with
 * round-to-nearest-even. dw_gu [E_L,2F,d] and dw_down [E_L,d,F] fp32 are fully
 * overwritten (not accumulated into); an expert with no row gets zeros. */
int moe_expert_ffn_bwd(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                       const void *w_gu, const void *w_down, const void *h, const void *dy,
                       void *gu, void *dgu, void *dx_rows, float *dw_gu, float *dw_down,
                       hipStream_t stream);

/* The two halves of moe_expert_ffn_bwd, same arguments and layouts:
 * moe_expert_ffn_bwd_data writes gu, dgu and dx_rows (the row gradients, what
 * moe_dispatch_bwd needs next); moe_expert_ffn_bwd_weight writes dw_gu and
 * dw_down from buf, h, dy and the dgu the first half wrote. Issuing the data
 * half, then moe_dispatch_bwd, then the weight half reads dx_rows while it is
 * still in cache. */
int moe_expert_ffn_bwd_data(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                            const void *w_gu, const void *w_down, const void *dy, void *gu,
                            void *dgu, void *dx_rows, hipStream_t stream);
int moe_expert_ffn_bwd_weight(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                              const void *h, const void *dy, const void *dgu, float *dw_gu,
                              float *dw_down, hipStream_t stream);

/* moe_expert_ffn_bwd_data when the forward kept [G U] (moe_expert_up_save_gu):
 * gu is read, not recomputed, so buf is not needed; dgu and dx_rows are
 * written as by moe_expert_ffn_bwd_data, bit for bit. dgu may be the same
 * buffer as gu (gu is then overwritten). */
int moe_expert_ffn_bwd_data_saved_gu(const moe_shape_t *shape, const int32_t *offsets,
                                     const void *w_gu, const void *w_down, const void *dy,
                                     const void *gu, void *dgu, void *dx_rows,
                                     hipStream_t stream);

/* Dispatch backward (Table 8: each token pulls its route gradients and sums
 * them): dx[t] = sum over k ascending with dest_rank[t,k] == ep_rank of
 * dx_rows[dest_row[t,k]], accumulated in fp32 and stored in dtype; a token
 * with no kept local route gets an exact zero row. dx_rows [Rmax,d],
 * dx [T,d]. T == 0: MOE_OK, nothing touched. */
int moe_dispatch_bwd(const moe_shape_t *shape, const void *dx_rows, const int32_t *dest_rank,
                     const int32_t *dest_row, void *dx, hipStream_t stream);

/* Router backward: the gradient of the logits through the softmax over the
 * K selected logits that produced topk_w (Sec. 05, Fig. 15); the selection
 * itself is piecewise constant and passes no gradient:
 *   dlogits[t, topk_idx[t,k]] = topk_w[t,k] * (dw[t,k] - sum_j topk_w[t,j] dw[t,j])
 * and 0 on every expert token t did not select. topk_idx, topk_w as moe_route
 * wrote them, dw from moe_combine_bwd; dlogits [T,N] fp32 is fully written.
 * T == 0: MOE_OK, nothing touched. */
int moe_route_bwd(const moe_shape_t *shape, const int32_t *topk_idx, const float *topk_w,
                  const float *dw, float *dlogits, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MXFP8 forward of a bf16 layer (Olmo-core MoE report Sec. 5.5: rows are
 * quantized during dispatch and the expert grouped GEMM consumes the
 * quantized data and scales directly; Sec. 5.8: a route's qdata row and scale
 * row follow the same destination indices and validity mask; Sec. 5.9: E4M3
 * data with E8M0 scales, MXFP8 expert GEMMs, forward combine in BF16 --
 * moe_combine on the bf16 y).
 * Format (the OCP microscaling format the report cites): a row of n values is
 * stored as qdata [n] uint8 E4M3 codes (OCP "E4M3FN": bias 7, max 448, no
 * infinities) and n/32 uint8 E8M0 scale codes (value 2^(code - 127)), one
 * per 32 consecutive elements. A block's scale is 2^(floor(log2 amax) - 8);
 * each element is its value over the scale rounded to the nearest E4M3 value,
 * ties to the even code, saturating at 448, sign bit from the value's sign;
 * an all-zero block gets scale code 0. Scale arrays hold one row of
 * SC(n) = 4*ceil(n/128) bytes per qdata row: the n/32 scales, then (when n is
 * not a multiple of 128) two pad bytes that are never written and never
 * affect a result, so that every scale row starts 4-byte aligned. Below,
 * "[R, SC(n)]" is such an array. Requirements of the MX calls
 * (MOE_EDTYPE / MOE_EINVAL otherwise): dtype MOE_BF16, d and F multiples of
 * 64 (whole 64-element K slices of the scaled MFMA; a contraction with
 * K % 128 == 64 ends in a half K step). Alignment: bf16 sources and qdata
 * 16 bytes, scale arrays 4 bytes.
 * ------------------------------------------------------------------------ */

/* MX-quantize `rows` rows of `cols` bf16 values (cols % 32 == 0) along the row:
 * src [rows, cols] -> qdata [rows, cols], scales [rows, SC(cols)]. Used once per
 * weight refresh for the expert weights, along their contraction dimension:
 * W_gu as rows = E_L*2F, cols = d; W_d as rows = E_L*d, cols = F. */
int moe_mx_quantize_rows(int64_t rows, int32_t cols, const void *src, uint8_t *qdata,
                         uint8_t *scales, hipStream_t stream);

/* Quantize-on-dispatch: token row x[t] (bf16, [T,d]) MX-quantized along d;
 * its qdata and scale rows are written to row dest_row[t,k] of qbuf
 * [Rmax, d] and sbuf [Rmax, SC(d)] for every route with dest_rank[t,k] ==
 * ep_rank. Rows after the packed prefix are not written. T == 0: MOE_OK. */
int moe_dispatch_rows_mx(const moe_shape_t *shape, const void *x, const int32_t *dest_rank,
                         const int32_t *dest_row, uint8_t *qbuf, uint8_t *sbuf,
                         hipStream_t stream);

/* MXFP8 grouped expert FFN over the packed prefix (offsets as moe_expert_ffn):
 * up:   H = silu(X W_gate^T) * (X W_up^T) from qbuf/sbuf and the quantized
 *       W_gu (w_gu_q [E_L,2F,d], w_gu_s [E_L,2F,SC(d)]); fp32 accumulation, H
 *       rounded to bf16 and MX-quantized along F into h_q [Rmax, F] and
 *       h_s [Rmax, SC(F)];
 * down: Y = H W_d^T from h_q/h_s and the quantized W_d (w_d_q [E_L,d,F],
 *       w_d_s [E_L,d,SC(F)]); Y [Rmax, d] bf16 (round to nearest even).
 * Only prefix rows are written. */
int moe_expert_up_mx(const moe_shape_t *shape, const uint8_t *qbuf, const uint8_t *sbuf,
                     const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                     uint8_t *h_q, uint8_t *h_s, hipStream_t stream);
int moe_expert_down_mx(const moe_shape_t *shape, const uint8_t *h_q, const uint8_t *h_s,
                       const int32_t *offsets, const uint8_t *w_d_q, const uint8_t *w_d_s,
                       void *y, hipStream_t stream);
int moe_expert_ffn_mx(const moe_shape_t *shape, const uint8_t *qbuf, const uint8_t *sbuf,
                      const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                      const uint8_t *w_d_q, const uint8_t *w_d_s, uint8_t *h_q, uint8_t *h_s,
                      void *y, hipStream_t stream);

/* Human-readable text of a return code (static storage, never NULL). */
const char *moe_strerror(int code);

/* Validate a shape without enqueuing anything: MOE_OK or the error code the
 * other calls would return for it. */
int moe_validate_shape(const moe_shape_t *shape);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
