// C ABI of libqlinear (declared and documented in include/qlinear.h): host-side argument
// checks, workspace carving and dispatch to the gfx950 kernels.  No device memory is
// allocated here; every buffer and workspace comes from the caller.  Every limit a kernel
// has is checked here, so that a call either launches or returns an argument error
// having enqueued nothing.
#include "../../include/qlinear.h"

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

constexpr size_t kAlign = 256;
static_assert(QLINEAR_WS_RESERVED_BYTES == ql::kWsReserved, "reserved region size");

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Largest token counts served by the few-token (streaming) kernels.
constexpr int64_t kG16MaxM = 64;

bool elems_ok(int64_t n, int64_t k) {
  return n > 0 && k > 0 && n <= QLINEAR_MAX_ELEMS / k;
}

bool is_fp8(int32_t format) { return format == QL_FP8_BLOCK128 || format == QL_FP8_POW2; }

qlinear_status check_qweight(const qlinear_qweight* w) {
  if (!w) return QL_ERR_NULL;
  if (w->format != QL_NVFP4 && !is_fp8(w->format)) return QL_ERR_FORMAT;
  if (!w->codes || !w->scales) return QL_ERR_NULL;
  if (!elems_ok(w->n, w->k)) return QL_ERR_SHAPE;
  if (w->format == QL_NVFP4) {
    if (!w->tensor_scale) return QL_ERR_NULL;
    if (w->k % 16) return QL_ERR_SHAPE;
    if (!aligned16(w->codes) || !aligned16(w->scales) || !aligned16(w->tensor_scale)) return QL_ERR_ALIGN;
  } else {
    if (w->n % 128 || w->k % 128) return QL_ERR_SHAPE;
    if (!aligned16(w->codes) || !aligned16(w->scales)) return QL_ERR_ALIGN;
  }
  return QL_OK;
}

// Effective LoRA rank (0 when there is no adapter or its scale is zero).
int32_t lora_rank(const uint16_t* a, const uint16_t* b, int32_t rank, float scale) {
  return (rank > 0 && a && b && scale != 0.0f) ? rank : 0;
}

// FP8 activation codes and their scales (float32, or E8M0 bytes with power-of-two scales).
size_t fp8_act_bytes(int32_t format, int64_t m, int64_t k) {
  const size_t sb = format == QL_FP8_POW2 ? 1 : 4;
  return up((size_t)m * (size_t)k) + up((size_t)m * (size_t)(k / 128) * sb);
}

// The NVFP4 path for m > 64: the f16 pre-pass GEMM when K allows it, else the generic one.
bool nvfp4_f16_path(int64_t k) { return k % 64 == 0 && k < ql::kNvF16MaxK; }

qlinear_status hip_status(hipError_t e) { return e == hipSuccess ? QL_OK : QL_ERR_HIP; }

// Scratch bytes (after the reserved region) of a forward call; SIZE_MAX when the shape is
// beyond what the kernels can run.
size_t forward_scratch(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank, bool prequant) {
  if (format == QL_NVFP4) {
    if (m <= kG16MaxM) {
      const ql::G16Plan p = ql::plan_g16(m, n, k, rank);
      return ql::g16_plan_ok(p, m) ? up(ql::g16_workspace(p, m)) : SIZE_MAX;
    }
    if (nvfp4_f16_path(k)) return up(ql::gemm_nvfp4_f16_workspace(m, n, k, rank));
    return up(ql::lora_down_bytes(m, k, rank));
  }
  if (is_fp8(format)) {
    if (k >= ql::kFp8MaxK) return SIZE_MAX;
    return (prequant ? 0 : fp8_act_bytes(format, m, k)) + up(ql::lora_down_bytes(m, k, rank));
  }
  return SIZE_MAX;
}

}  // namespace

extern "C" {

const char* qlinear_status_string(qlinear_status s) {
  switch (s) {
    case QL_OK: return "ok";
    case QL_ERR_NULL: return "required pointer is NULL";
    case QL_ERR_SHAPE: return "invalid shape";
    case QL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QL_ERR_FORMAT: return "unknown format or output type";
    case QL_ERR_WORKSPACE: return "workspace missing or too small";
    case QL_ERR_HIP: return "HIP launch failed";
    case QL_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

int32_t* qlinear_status_word(void* ws) { return ql::ws_status(ws); }

// ------------------------------------------------------------------ quantizers

size_t qlinear_quantize_workspace(int32_t format, int64_t n, int64_t k) {
  (void)n;
  (void)k;
  return format == QL_NVFP4 ? (size_t)ql::kAmaxParts * sizeof(uint32_t) : 0;
}

qlinear_status qlinear_quantize_nvfp4(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      uint8_t* scales, float* tensor_scale, int32_t* status_word,
                                      void* ws, size_t ws_bytes, void* stream) {
  if (!w || !codes || !scales || !tensor_scale) return QL_ERR_NULL;
  if (!elems_ok(n, k) || k % 16) return QL_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(tensor_scale) ||
      (status_word && ((uintptr_t)status_word & 3)))
    return QL_ERR_ALIGN;
  if (!ws || ws_bytes < qlinear_quantize_workspace(QL_NVFP4, n, k)) return QL_ERR_WORKSPACE;
  if (!aligned16(ws)) return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_nvfp4_quantize(w, n, k, codes, scales, tensor_scale, status_word,
                                              (uint32_t*)ws, (hipStream_t)stream));
}

qlinear_status qlinear_quantize_fp8_block(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                          float* scales, int32_t* status_word, void* stream) {
  if (!w || !codes || !scales) return QL_ERR_NULL;
  if (!elems_ok(n, k) || n % 128 || k % 128) return QL_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) ||
      (status_word && ((uintptr_t)status_word & 3)))
    return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_fp8_weight_quantize(w, n, k, codes, scales, false, status_word,
                                                   (hipStream_t)stream));
}

qlinear_status qlinear_quantize_fp8_pow2(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                         uint8_t* scales, int32_t* status_word, void* stream) {
  if (!w || !codes || !scales) return QL_ERR_NULL;
  if (!elems_ok(n, k) || n % 128 || k % 128) return QL_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) ||
      (status_word && ((uintptr_t)status_word & 3)))
    return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_fp8_weight_quantize(w, n, k, codes, scales, true, status_word,
                                                   (hipStream_t)stream));
}

qlinear_status qlinear_quantize_act_fp8(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                        float* sx, void* stream) {
  if (!x || !xq || !sx) return QL_ERR_NULL;
  if (!elems_ok(m, k) || k % 128) return QL_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(sx)) return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_fp8_act_quantize(x, m, k, xq, sx, false, (hipStream_t)stream));
}

qlinear_status qlinear_quantize_act_fp8_pow2(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                             uint8_t* sx, void* stream) {
  if (!x || !xq || !sx) return QL_ERR_NULL;
  if (!elems_ok(m, k) || k % 128) return QL_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(sx)) return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_fp8_act_quantize(x, m, k, xq, sx, true, (hipStream_t)stream));
}

// --------------------------------------------------------------------- forward

size_t qlinear_forward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank) {
  if (m <= 0 || n <= 0 || k <= 0 || rank < 0 || rank > QLINEAR_MAX_RANK) return 0;
  const size_t s = forward_scratch(format, m, n, k, rank, false);
  return s == SIZE_MAX ? 0 : ql::kWsReserved + s;
}

size_t qlinear_forward_prequant_workspace(int64_t m, int64_t n, int64_t k, int32_t rank) {
  if (m <= 0 || n <= 0 || k <= 0 || rank < 0 || rank > QLINEAR_MAX_RANK) return 0;
  const size_t s = forward_scratch(QL_FP8_BLOCK128, m, n, k, rank, true);
  return s == SIZE_MAX ? 0 : ql::kWsReserved + s;
}

static qlinear_status check_forward_common(const qlinear_qweight* w, int64_t m,
                                           const uint16_t* lora_a, const uint16_t* lora_b,
                                           int32_t rank, void* y, int32_t out_dtype) {
  qlinear_status st = check_qweight(w);
  if (st != QL_OK) return st;
  if (!y) return QL_ERR_NULL;
  if (m <= 0 || m > QLINEAR_MAX_M || !elems_ok(m, w->k) || !elems_ok(m, w->n)) return QL_ERR_SHAPE;
  if (rank < 0 || rank > QLINEAR_MAX_RANK) return QL_ERR_ARG;
  if (out_dtype != QL_OUT_BF16 && out_dtype != QL_OUT_F32) return QL_ERR_FORMAT;
  if (!aligned16(y) || (lora_a && !aligned16(lora_a)) || (lora_b && !aligned16(lora_b))) return QL_ERR_ALIGN;
  return QL_OK;
}

// Workspace check shared by both forward entry points: present, large enough, aligned, and
// the shape within what the kernels run.
static qlinear_status check_forward_ws(const qlinear_qweight* w, int64_t m, int32_t r, bool prequant,
                                       void* ws, size_t ws_bytes) {
  const size_t s = forward_scratch(w->format, m, w->n, w->k, r, prequant);
  if (s == SIZE_MAX) return QL_ERR_SHAPE;
  if (!ws || ws_bytes < ql::kWsReserved + s) return QL_ERR_WORKSPACE;
  if (!aligned16(ws)) return QL_ERR_ALIGN;
  return QL_OK;
}

}  // extern "C"

// The body of qlinear_forward, also behind the allocation-free variant (noalloc.hip).
qlinear_status ql::forward_impl(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                                const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                                float lora_scale, void* y, int32_t out_dtype, void* ws,
                                size_t ws_bytes, void* stream) {
  qlinear_status st = check_forward_common(w, m, lora_a, lora_b, rank, y, out_dtype);
  if (st != QL_OK) return st;
  if (!x) return QL_ERR_NULL;
  if (!aligned16(x)) return QL_ERR_ALIGN;
  const int32_t r = lora_rank(lora_a, lora_b, rank, lora_scale);
  st = check_forward_ws(w, m, r, false, ws, ws_bytes);
  if (st != QL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const int out_f32 = out_dtype == QL_OUT_F32;
  char* scratch = ql::ws_scratch(ws);
  ql::clear_hip_error();

  if (w->format == QL_NVFP4) {
    const uint8_t* codes = (const uint8_t*)w->codes;
    const uint8_t* scales = (const uint8_t*)w->scales;
    if (m <= kG16MaxM) {
      const ql::G16Plan p = ql::plan_g16(m, w->n, w->k, r);
      return hip_status(ql::launch_g16(p, x, m, w->n, w->k, codes, scales, w->tensor_scale, lora_a,
                                       lora_b, r, lora_scale, y, out_f32, ws, s));
    }
    if (nvfp4_f16_path(w->k))
      return hip_status(ql::launch_gemm_nvfp4_f16(x, m, w->n, w->k, codes, scales, w->tensor_scale,
                                                  lora_a, lora_b, r, lora_scale, y, out_f32, scratch, s));
    uint16_t* t = nullptr;
    if (r > 0 && ql::launch_lora_down(x, m, w->k, lora_a, r, lora_scale, scratch, &t, s) != hipSuccess)
      return QL_ERR_HIP;
    return hip_status(ql::launch_gemm_nvfp4(x, m, w->n, w->k, codes, scales, w->tensor_scale, t,
                                            lora_b, r, y, out_f32, s));
  }

  // FP8: quantize activations per 1x128 segment, then the block-scaled GEMM.
  const bool pow2 = w->format == QL_FP8_POW2;
  uint8_t* xq = (uint8_t*)scratch;
  void* sx = scratch + up((size_t)m * (size_t)w->k);
  char* rest = scratch + fp8_act_bytes(w->format, m, w->k);
  if (ql::launch_fp8_act_quantize(x, m, w->k, xq, sx, pow2, s) != hipSuccess) return QL_ERR_HIP;
  uint16_t* t = nullptr;
  if (r > 0 && ql::launch_lora_down(x, m, w->k, lora_a, r, lora_scale, rest, &t, s) != hipSuccess)
    return QL_ERR_HIP;
  return hip_status(ql::launch_gemm_fp8(xq, sx, m, w->n, w->k, (const uint8_t*)w->codes, w->scales, pow2, t,
                                        lora_b, r, y, out_f32, s));
}

extern "C" {

qlinear_status qlinear_forward(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                               const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                               float lora_scale, void* y, int32_t out_dtype, void* ws,
                               size_t ws_bytes, void* stream) {
  return ql::forward_impl(w, x, m, lora_a, lora_b, rank, lora_scale, y, out_dtype, ws, ws_bytes, stream);
}

qlinear_status qlinear_forward_fp8_prequant(const qlinear_qweight* w, const uint8_t* xq,
                                            const void* sx, int64_t m, const uint16_t* x,
                                            const uint16_t* lora_a, const uint16_t* lora_b,
                                            int32_t rank, float lora_scale, void* y,
                                            int32_t out_dtype, void* ws, size_t ws_bytes,
                                            void* stream) {
  qlinear_status st = check_forward_common(w, m, lora_a, lora_b, rank, y, out_dtype);
  if (st != QL_OK) return st;
  if (!is_fp8(w->format)) return QL_ERR_FORMAT;
  if (!xq || !sx) return QL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(sx)) return QL_ERR_ALIGN;
  const int32_t r = lora_rank(lora_a, lora_b, rank, lora_scale);
  if (r > 0 && !x) return QL_ERR_NULL;
  if (x && !aligned16(x)) return QL_ERR_ALIGN;
  st = check_forward_ws(w, m, r, true, ws, ws_bytes);
  if (st != QL_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  ql::clear_hip_error();
  uint16_t* t = nullptr;
  if (r > 0 && ql::launch_lora_down(x, m, w->k, lora_a, r, lora_scale, ql::ws_scratch(ws), &t, s) != hipSuccess)
    return QL_ERR_HIP;
  return hip_status(ql::launch_gemm_fp8(xq, sx, m, w->n, w->k, (const uint8_t*)w->codes, w->scales,
                                        w->format == QL_FP8_POW2, t, lora_b, r, y, out_dtype == QL_OUT_F32, s));
}

// ---------------------------------------------------------- layers sharing x

static_assert(QLINEAR_MAX_GROUP == ql::kNvMaxSeg, "group size");

// Whether a group runs fused (one pre-pass, one GEMM) rather than layer by layer.
static bool group_fused(int32_t count, int64_t m, int64_t k, int32_t r) {
  return count > 1 && m > kG16MaxM && nvfp4_f16_path(k) && r % 32 == 0 && count * r <= 128;
}

size_t qlinear_forward_group_workspace(int64_t m, int64_t k, const int64_t* n, int32_t count, int32_t rank) {
  if (!n || count < 1 || count > QLINEAR_MAX_GROUP || m <= 0 || k <= 0 || rank < 0 || rank > QLINEAR_MAX_RANK)
    return 0;
  for (int32_t i = 0; i < count; ++i)
    if (n[i] <= 0) return 0;
  size_t s = 0;
  if (group_fused(count, m, k, rank)) {
    s = up(ql::gemm_nvfp4_f16_layers_workspace(m, k, n, count, rank));
  } else {
    for (int32_t i = 0; i < count; ++i) {
      const size_t si = forward_scratch(QL_NVFP4, m, n[i], k, rank, false);
      if (si == SIZE_MAX) return 0;
      if (si > s) s = si;
    }
  }
  return ql::kWsReserved + s;
}

qlinear_status qlinear_forward_group(const qlinear_group_layer* layers, int32_t count, const uint16_t* x,
                                     int64_t m, int32_t rank, float lora_scale, int32_t out_dtype,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (!layers) return QL_ERR_NULL;
  if (count < 1 || count > QLINEAR_MAX_GROUP) return QL_ERR_ARG;
  if (!x) return QL_ERR_NULL;
  if (!aligned16(x)) return QL_ERR_ALIGN;
  int with = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlinear_group_layer& l = layers[i];
    qlinear_status st = check_forward_common(&l.w, m, l.lora_a, l.lora_b, rank, l.y, out_dtype);
    if (st != QL_OK) return st;
    if (l.w.format != QL_NVFP4) return QL_ERR_FORMAT;
    if (l.w.k != layers[0].w.k) return QL_ERR_SHAPE;
    with += (l.lora_a && l.lora_b) ? 1 : 0;
  }
  const bool lora = rank > 0 && lora_scale != 0.0f;
  if (lora && with != 0 && with != count) return QL_ERR_NULL;
  const int32_t r = lora && with == count ? rank : 0;
  const int64_t k = layers[0].w.k;
  int64_t ns[QLINEAR_MAX_GROUP];
  for (int32_t i = 0; i < count; ++i) ns[i] = layers[i].w.n;
  const size_t need = qlinear_forward_group_workspace(m, k, ns, count, r);
  if (need == 0) return QL_ERR_SHAPE;
  if (!ws || ws_bytes < need) return QL_ERR_WORKSPACE;
  if (!aligned16(ws)) return QL_ERR_ALIGN;
  if (!group_fused(count, m, k, r)) {
    for (int32_t i = 0; i < count; ++i) {
      const qlinear_group_layer& l = layers[i];
      const qlinear_status st = ql::forward_impl(&l.w, x, m, r ? l.lora_a : nullptr, r ? l.lora_b : nullptr, r,
                                                 lora_scale, l.y, out_dtype, ws, ws_bytes, stream);
      if (st != QL_OK) return st;
    }
    return QL_OK;
  }
  ql::NvLayer nl[QLINEAR_MAX_GROUP];
  for (int32_t i = 0; i < count; ++i) {
    const qlinear_group_layer& l = layers[i];
    nl[i].codes = (const uint8_t*)l.w.codes;
    nl[i].scales = (const uint8_t*)l.w.scales;
    nl[i].tensor_scale = l.w.tensor_scale;
    nl[i].lora_a = r ? l.lora_a : nullptr;
    nl[i].lora_b = r ? l.lora_b : nullptr;
    nl[i].y = l.y;
    nl[i].n = l.w.n;
  }
  ql::clear_hip_error();
  return hip_status(ql::launch_gemm_nvfp4_f16_layers(x, m, k, nl, count, r, lora_scale, out_dtype == QL_OUT_F32,
                                                     ql::ws_scratch(ws), (hipStream_t)stream));
}

// ------------------------------------------------------------------ backward

static bool backward_shape_ok(int64_t m, int64_t n, int64_t k) {
  return m > 0 && m <= QLINEAR_MAX_M && n % 64 == 0 && k % 128 == 0 && elems_ok(n, k) && elems_ok(m, n) &&
         elems_ok(m, k);
}

size_t qlinear_backward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank) {
  if (format != QL_NVFP4 || !backward_shape_ok(m, n, k) || rank < 0 || rank > QLINEAR_MAX_RANK) return 0;
  return up(ql::backward_scratch_bytes(m, n, k, rank));
}

qlinear_status qlinear_backward(const qlinear_qweight* w, const uint16_t* x, const uint16_t* dy,
                                int64_t m, const uint16_t* lora_a, const uint16_t* lora_b,
                                int32_t rank, float lora_scale, void* dx, int32_t dx_dtype,
                                float* da, float* db, void* ws, size_t ws_bytes, void* stream) {
  qlinear_status st = check_qweight(w);
  if (st != QL_OK) return st;
  if (w->format != QL_NVFP4) return QL_ERR_FORMAT;
  if (!dy || !dx) return QL_ERR_NULL;
  if (!backward_shape_ok(m, w->n, w->k)) return QL_ERR_SHAPE;
  if (rank < 0 || rank > QLINEAR_MAX_RANK) return QL_ERR_ARG;
  if (dx_dtype != QL_OUT_BF16 && dx_dtype != QL_OUT_F32) return QL_ERR_FORMAT;
  const int32_t r = lora_rank(lora_a, lora_b, rank, lora_scale);
  if (r > 0 && (!x || !da || !db)) return QL_ERR_NULL;
  if (!aligned16(dy) || !aligned16(dx) || (x && !aligned16(x)) || (lora_a && !aligned16(lora_a)) ||
      (lora_b && !aligned16(lora_b)) || (da && !aligned16(da)) || (db && !aligned16(db)))
    return QL_ERR_ALIGN;
  const size_t need = up(ql::backward_scratch_bytes(m, w->n, w->k, r));
  if (need > 0 && (!ws || ws_bytes < need)) return QL_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_backward_nvfp4(x, dy, m, w->n, w->k, (const uint8_t*)w->codes,
                                              (const uint8_t*)w->scales, w->tensor_scale, lora_a, lora_b, r,
                                              lora_scale, dx, dx_dtype == QL_OUT_F32, da, db, ws,
                                              (hipStream_t)stream));
}

// ------------------------------------------------------------------- requant

size_t qlinear_requant_workspace(int32_t count) {
  if (count <= 0 || count > QLINEAR_MAX_REQUANT_ITEMS) return 0;
  return ql::requant_workspace(count);
}

static qlinear_status requant_common(const qlinear_requant_item* items, const uint16_t* const* deltas,
                                     int32_t count, int32_t format, void* ws, size_t ws_bytes, void* stream) {
  if (!items) return QL_ERR_NULL;
  if (count <= 0 || count > QLINEAR_MAX_REQUANT_ITEMS) return QL_ERR_ARG;
  if (format != QL_NVFP4 && !is_fp8(format)) return QL_ERR_FORMAT;
  if (!ws || ws_bytes < ql::requant_workspace(count)) return QL_ERR_WORKSPACE;
  if (!aligned16(items) || !aligned16(ws) || (deltas && ((uintptr_t)deltas & 7))) return QL_ERR_ALIGN;
  ql::clear_hip_error();
  return hip_status(ql::launch_requant(items, deltas, count, format, ws, (hipStream_t)stream));
}

qlinear_status qlinear_requantize_all(const qlinear_requant_item* items, int32_t count,
                                      int32_t format, void* ws, size_t ws_bytes, void* stream) {
  return requant_common(items, nullptr, count, format, ws, ws_bytes, stream);
}

qlinear_status qlinear_update_requantize_all(const qlinear_requant_item* items,
                                             const uint16_t* const* deltas, int32_t count,
                                             int32_t format, void* ws, size_t ws_bytes,
                                             void* stream) {
  if (!deltas) return QL_ERR_NULL;
  return requant_common(items, deltas, count, format, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ KV cache

static qlinear_status check_kv(int64_t tokens, int32_t heads, int32_t head_dim, int64_t cache_slots,
                               const int32_t* status_word) {
  if (tokens < 0 || heads <= 0 || cache_slots <= 0) return QL_ERR_SHAPE;
  if (head_dim < 16 || head_dim > 512 || (head_dim & (head_dim - 1))) return QL_ERR_SHAPE;
  const int64_t vec = (int64_t)heads * head_dim;
  if ((tokens > 0 && !elems_ok(tokens, vec)) || !elems_ok(cache_slots, vec)) return QL_ERR_SHAPE;
  if (status_word && ((uintptr_t)status_word & 3)) return QL_ERR_ALIGN;
  return QL_OK;
}

qlinear_status qlinear_kv_store_fp8(const uint16_t* kv, int64_t tokens, int32_t heads, int32_t head_dim,
                                    const int64_t* slots, uint8_t* cache_codes, float* cache_scales,
                                    int64_t cache_slots, int32_t* status_word, void* stream) {
  if (!kv || !slots || !cache_codes || !cache_scales) return QL_ERR_NULL;
  qlinear_status st = check_kv(tokens, heads, head_dim, cache_slots, status_word);
  if (st != QL_OK) return st;
  if (!aligned16(kv) || !aligned16(cache_codes) || !aligned16(cache_scales) || ((uintptr_t)slots & 7))
    return QL_ERR_ALIGN;
  if (tokens == 0) return QL_OK;
  ql::clear_hip_error();
  return hip_status(ql::launch_kv_store(kv, tokens, heads, head_dim, slots, cache_codes, cache_scales, cache_slots,
                                        status_word, (hipStream_t)stream));
}

qlinear_status qlinear_kv_load_fp8(const uint8_t* cache_codes, const float* cache_scales,
                                   int64_t cache_slots, const int64_t* slots, int64_t tokens,
                                   int32_t heads, int32_t head_dim, uint16_t* out,
                                   int32_t* status_word, void* stream) {
  if (!cache_codes || !cache_scales || !slots || !out) return QL_ERR_NULL;
  qlinear_status st = check_kv(tokens, heads, head_dim, cache_slots, status_word);
  if (st != QL_OK) return st;
  if (!aligned16(out) || !aligned16(cache_codes) || !aligned16(cache_scales) || ((uintptr_t)slots & 7))
    return QL_ERR_ALIGN;
  if (tokens == 0) return QL_OK;
  ql::clear_hip_error();
  return hip_status(ql::launch_kv_load(cache_codes, cache_scales, cache_slots, slots, tokens, heads, head_dim, out,
                                       status_word, (hipStream_t)stream));
}

}  // extern "C"
