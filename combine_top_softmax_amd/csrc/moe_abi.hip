// C ABI entry points of libmoe_hip (declared in include/moe.h).
//
// Host-only validation, then stream-ordered kernel launches. Nothing here
// reads device memory, synchronizes or allocates (Olmo-core MoE report,
// Sec. 08 "Synchronization-Free Training", Sec. 8.5: device-resident route
// metadata, capacity-shaped buffers fixed before the loop).
#include "moe_internal.h"

#include <mutex>

// Workspace of moe_route_noalloc: one static array per GPU, alive until the
// process ends. Host code never uses the symbol itself as an address (on the
// host it only names the array); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::ceil_div;

constexpr int64_t kLim31 = (int64_t)1 << 31;

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

int check_shape(const moe_shape_t *s) {
  if (s == nullptr) return MOE_EINVAL;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_EDTYPE;
  if (s->T < 0 || s->d < 1 || s->N < 1 || s->K < 1 || s->F < 1 || s->ep_size < 1 ||
      s->capacity < 1)
    return MOE_EINVAL;
  if (s->K > s->N || s->K > MOE_MAX_K || s->N > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (s->N % s->ep_size != 0 || s->ep_rank < 0 || s->ep_rank >= s->ep_size) return MOE_EINVAL;
  if (s->d % 8 != 0 || s->F % 8 != 0) return MOE_EINVAL;
  // the buffer rows, the offsets and every row index stay below T*K (or
  // min(K, E_L) for an empty batch), whatever the capacity
  if ((int64_t)s->T * s->K >= kLim31) return MOE_EINVAL;
  // 32-bit offsets inside the GEMMs: a tile's A rows are addressed from its
  // first row (at most 256 rows of d or 2F elements past a 64-bit base), and
  // a weight row inside one expert's matrix (fewer than 2F*d elements)
  if (s->d > MOE_MAX_WIDTH || s->F > MOE_MAX_WIDTH) return MOE_EINVAL;
  if ((int64_t)2 * s->F * s->d >= kLim31) return MOE_EINVAL;
  // tile counts of the grouped GEMMs (the smallest tiles: 64 rows, 32 output
  // columns) fit a signed 32-bit grid index
  const int64_t E_L = s->N / s->ep_size;
  const int64_t m_tiles = moe::ceil_div(moe::buffer_rows(*s), 64) + E_L;
  const int64_t n_tiles = moe::ceil_div(2 * (int64_t)s->F > s->d ? 2 * (int64_t)s->F : s->d, 32);
  if (m_tiles * n_tiles >= kLim31) return MOE_EINVAL;
  return MOE_OK;
}

size_t route_ws_bytes(const moe_shape_t &s) {
  const size_t hist = (size_t)s.N * moe::route_tiles(s) * sizeof(int32_t);
  const size_t rank = (size_t)s.T * s.K;
  return ((hist + rank) + 255) / 256 * 256;
}

int check_route_out(const moe_shape_t &s, const moe_route_out_t *o, bool need_topk) {
  if (o == nullptr) return MOE_EINVAL;
  // the [T,K] arrays are not touched when T == 0 (they may then be NULL)
  if (s.T > 0) {
    if (need_topk && (!aligned4(o->topk_idx) || !aligned4(o->topk_w))) return MOE_EALIGN;
    if (!aligned4(o->dest_rank) || !aligned4(o->dest_row) || o->drop_mask == nullptr)
      return MOE_EALIGN;
  }
  if (!aligned4(o->counts) || !aligned4(o->offsets)) return MOE_EALIGN;
  if (o->row_src != nullptr && !aligned4(o->row_src)) return MOE_EALIGN;
  return MOE_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

int scratch_address(void **addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();   // do not leave the error for the next launch check
      return MOE_EHIP;
    }
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_validate_shape(const moe_shape_t *shape) { return check_shape(shape); }

int64_t moe_buffer_rows(const moe_shape_t *shape) {
  const int rc = check_shape(shape);
  return rc != MOE_OK ? rc : moe::buffer_rows(*shape);
}

const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid size or index argument";
    case MOE_EDTYPE: return "unknown dtype";
    case MOE_EALIGN: return "data pointer is NULL or misaligned (16 bytes for rows, 4 for int32/fp32 arrays)";
    case MOE_EWORKSPACE: return "workspace is NULL or smaller than moe_route_workspace_size";
    case MOE_EHIP: return "HIP kernel launch failed";
    case MOE_ESCRATCH:
      return "the shape's route workspace exceeds the static no-allocation scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int moe_route_workspace_size(const moe_shape_t *shape, size_t *bytes) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (bytes == nullptr) return MOE_EINVAL;
  *bytes = route_ws_bytes(*shape);
  return MOE_OK;
}

int moe_route(const moe_shape_t *shape, const float *logits, const moe_route_out_t *out,
              void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T > 0 && !aligned16(logits)) return MOE_EALIGN;
  if ((rc = check_route_out(*shape, out, true)) != MOE_OK) return rc;
  if (!aligned4(ws) || ws_bytes < route_ws_bytes(*shape)) return MOE_EWORKSPACE;
  return moe::launch_route(*shape, logits, nullptr, *out, ws, stream);
}

int moe_route_noalloc(const moe_shape_t *shape, const float *logits, const moe_route_out_t *out,
                      hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T > 0 && !aligned16(logits)) return MOE_EALIGN;
  if ((rc = check_route_out(*shape, out, true)) != MOE_OK) return rc;
  const size_t need = route_ws_bytes(*shape);
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws)) != MOE_OK) return rc;
  return moe::launch_route(*shape, logits, nullptr, *out, ws, stream);
}

int moe_route_map(const moe_shape_t *shape, const int32_t *topk_idx_in,
                  const moe_route_out_t *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T > 0 && !aligned4(topk_idx_in)) return MOE_EALIGN;
  if ((rc = check_route_out(*shape, out, false)) != MOE_OK) return rc;
  if (!aligned4(ws) || ws_bytes < route_ws_bytes(*shape)) return MOE_EWORKSPACE;
  return moe::launch_route(*shape, nullptr, topk_idx_in, *out, ws, stream);
}

int moe_dispatch_rows(const moe_shape_t *shape, const void *x, const int32_t *dest_rank,
                      const int32_t *dest_row, void *buf, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;   // no token, nothing to move
  if (!aligned16(x) || !aligned16(buf) || !aligned4(dest_rank) || !aligned4(dest_row))
    return MOE_EALIGN;
  return moe::launch_dispatch(*shape, x, dest_rank, dest_row, buf, stream);
}

int moe_expert_up(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                  const void *w_gu, void *h, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(w_gu) || !aligned16(h) || !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_up(*shape, buf, offsets, w_gu, h, stream);
}

int moe_expert_up_save_gu(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                          const void *w_gu, void *h, void *gu, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(w_gu) || !aligned16(h) || !aligned16(gu) ||
      !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_up(*shape, buf, offsets, w_gu, h, stream, gu);
}

int moe_expert_down(const moe_shape_t *shape, const void *h, const int32_t *offsets,
                    const void *w_down, void *y, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(y) || !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_down(*shape, h, offsets, w_down, y, stream);
}

int moe_expert_ffn(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                   const void *w_gu, const void *w_down, void *h, void *y, hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(w_gu) || !aligned16(w_down) || !aligned16(h) ||
      !aligned16(y) || !aligned4(offsets))
    return MOE_EALIGN;
  if ((rc = moe::launch_expert_up(*shape, buf, offsets, w_gu, h, stream)) != MOE_OK) return rc;
  return moe::launch_expert_down(*shape, h, offsets, w_down, y, stream);
}

int moe_combine(const moe_shape_t *shape, const void *y, const int32_t *dest_rank,
                const int32_t *dest_row, const float *topk_w, void *out, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;   // no token, no output row
  if (!aligned16(y) || !aligned16(out) || !aligned4(dest_rank) || !aligned4(dest_row) ||
      !aligned4(topk_w))
    return MOE_EALIGN;
  return moe::launch_combine(*shape, y, dest_rank, dest_row, topk_w, out, stream);
}

int moe_combine_bwd(const moe_shape_t *shape, const void *dout, const void *y,
                    const int32_t *dest_rank, const int32_t *dest_row, const float *topk_w,
                    void *dy, float *dw, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;
  if (!aligned16(dout) || !aligned16(y) || !aligned16(dy) || !aligned4(dest_rank) ||
      !aligned4(dest_row) || !aligned4(topk_w) || !aligned4(dw))
    return MOE_EALIGN;
  return moe::launch_combine_bwd(*shape, dout, y, dest_rank, dest_row, topk_w, dy, dw, stream);
}

int moe_expert_ffn_bwd_data(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                            const void *w_gu, const void *w_down, const void *dy, void *gu,
                            void *dgu, void *dx_rows, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(w_gu) || !aligned16(w_down) || !aligned16(dy) ||
      !aligned16(gu) || !aligned16(dgu) || !aligned16(dx_rows) || !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_ffn_bwd_data(*shape, buf, offsets, w_gu, w_down, dy, gu, dgu, dx_rows,
                                         stream);
}

int moe_expert_ffn_bwd_data_saved_gu(const moe_shape_t *shape, const int32_t *offsets,
                                     const void *w_gu, const void *w_down, const void *dy,
                                     const void *gu, void *dgu, void *dx_rows,
                                     hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(w_gu) || !aligned16(w_down) || !aligned16(dy) || !aligned16(gu) ||
      !aligned16(dgu) || !aligned16(dx_rows) || !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_ffn_bwd_data_gu(*shape, offsets, w_gu, w_down, dy, gu, dgu, dx_rows,
                                            stream);
}

int moe_expert_ffn_bwd_weight(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                              const void *h, const void *dy, const void *dgu, float *dw_gu,
                              float *dw_down, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(h) || !aligned16(dy) || !aligned16(dgu) ||
      !aligned16(dw_gu) || !aligned16(dw_down) || !aligned4(offsets))
    return MOE_EALIGN;
  return moe::launch_expert_ffn_bwd_weight(*shape, buf, offsets, h, dy, dgu, dw_gu, dw_down,
                                           stream);
}

int moe_expert_ffn_bwd(const moe_shape_t *shape, const void *buf, const int32_t *offsets,
                       const void *w_gu, const void *w_down, const void *h, const void *dy,
                       void *gu, void *dgu, void *dx_rows, float *dw_gu, float *dw_down,
                       hipStream_t stream) {
  int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(buf) || !aligned16(w_gu) || !aligned16(w_down) || !aligned16(h) ||
      !aligned16(dy) || !aligned16(gu) || !aligned16(dgu) || !aligned16(dx_rows) ||
      !aligned16(dw_gu) || !aligned16(dw_down) || !aligned4(offsets))
    return MOE_EALIGN;
  rc = moe::launch_expert_ffn_bwd_data(*shape, buf, offsets, w_gu, w_down, dy, gu, dgu, dx_rows,
                                       stream);
  if (rc != MOE_OK) return rc;
  return moe::launch_expert_ffn_bwd_weight(*shape, buf, offsets, h, dy, dgu, dw_gu, dw_down,
                                           stream);
}

int moe_dispatch_bwd(const moe_shape_t *shape, const void *dx_rows, const int32_t *dest_rank,
                     const int32_t *dest_row, void *dx, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;
  if (!aligned16(dx_rows) || !aligned16(dx) || !aligned4(dest_rank) || !aligned4(dest_row))
    return MOE_EALIGN;
  // the combine kernel with unit weights
  return moe::launch_combine(*shape, dx_rows, dest_rank, dest_row, nullptr, dx, stream);
}

int moe_route_bwd(const moe_shape_t *shape, const int32_t *topk_idx, const float *topk_w,
                  const float *dw, float *dlogits, hipStream_t stream) {
  const int rc = check_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;
  if (!aligned4(topk_idx) || !aligned4(topk_w) || !aligned4(dw) || !aligned4(dlogits))
    return MOE_EALIGN;
  return moe::launch_route_bwd(*shape, topk_idx, topk_w, dw, dlogits, stream);
}

static int check_mx_shape(const moe_shape_t *s) {
  const int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (s->dtype != MOE_BF16) return MOE_EDTYPE;
  // whole 64-element MFMA K slices in both GEMMs (d and F are each the
  // contraction of one of them)
  if (s->d % 64 != 0 || s->F % 64 != 0) return MOE_EINVAL;
  return MOE_OK;
}

int moe_mx_quantize_rows(int64_t rows, int32_t cols, const void *src, uint8_t *qdata,
                         uint8_t *scales, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || rows >= ((int64_t)1 << 31)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!aligned16(src) || !aligned16(qdata) || scales == nullptr) return MOE_EALIGN;
  return moe::launch_quantize_rows(rows, cols, src, qdata, scales, stream);
}

int moe_dispatch_rows_mx(const moe_shape_t *shape, const void *x, const int32_t *dest_rank,
                         const int32_t *dest_row, uint8_t *qbuf, uint8_t *sbuf,
                         hipStream_t stream) {
  const int rc = check_mx_shape(shape);
  if (rc != MOE_OK) return rc;
  if (shape->T == 0) return MOE_OK;
  if (!aligned16(x) || !aligned16(qbuf) || !aligned4(sbuf) || !aligned4(dest_rank) ||
      !aligned4(dest_row))
    return MOE_EALIGN;
  return moe::launch_dispatch_mx(*shape, x, dest_rank, dest_row, qbuf, sbuf, stream);
}

int moe_expert_up_mx(const moe_shape_t *shape, const uint8_t *qbuf, const uint8_t *sbuf,
                     const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                     uint8_t *h_q, uint8_t *h_s, hipStream_t stream) {
  const int rc = check_mx_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(qbuf) || !aligned4(sbuf) || !aligned4(offsets) || !aligned16(w_gu_q) ||
      !aligned4(w_gu_s) || !aligned16(h_q) || !aligned4(h_s))
    return MOE_EALIGN;
  return moe::launch_expert_up_mx(*shape, qbuf, sbuf, offsets, w_gu_q, w_gu_s, h_q, h_s, stream);
}

int moe_expert_down_mx(const moe_shape_t *shape, const uint8_t *h_q, const uint8_t *h_s,
                       const int32_t *offsets, const uint8_t *w_d_q, const uint8_t *w_d_s,
                       void *y, hipStream_t stream) {
  const int rc = check_mx_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!aligned16(h_q) || !aligned4(h_s) || !aligned4(offsets) || !aligned16(w_d_q) ||
      !aligned4(w_d_s) || !aligned16(y))
    return MOE_EALIGN;
  return moe::launch_expert_down_mx(*shape, h_q, h_s, offsets, w_d_q, w_d_s, y, stream);
}

int moe_expert_ffn_mx(const moe_shape_t *shape, const uint8_t *qbuf, const uint8_t *sbuf,
                      const int32_t *offsets, const uint8_t *w_gu_q, const uint8_t *w_gu_s,
                      const uint8_t *w_d_q, const uint8_t *w_d_s, uint8_t *h_q, uint8_t *h_s,
                      void *y, hipStream_t stream) {
  int rc = moe_expert_up_mx(shape, qbuf, sbuf, offsets, w_gu_q, w_gu_s, h_q, h_s, stream);
  if (rc != MOE_OK) return rc;
  return moe_expert_down_mx(shape, h_q, h_s, offsets, w_d_q, w_d_s, y, stream);
}

}  // extern "C"
