// C ABI of libqlinear (declared and documented in include/qlinear.h): host-side argument
// checks, workspace carving and dispatch to the gfx950 kernels.  No device memory is
// allocated here; every buffer, workspace and table comes from the caller.
#include "../../include/qlinear.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "launch.hpp"

namespace {

using ql::SkinnyPlan;

constexpr size_t kAlign = 256;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest token counts served by the few-token (streaming) kernels.
constexpr int64_t kG16MaxM = 64;

bool elems_ok(int64_t n, int64_t k) {
  return n > 0 && k > 0 && n <= QLINEAR_MAX_ELEMS / k;
}

qlinear_status check_qweight(const qlinear_qweight* w) {
  if (!w) return QL_ERR_NULL;
  if (w->format != QL_NVFP4 && w->format != QL_FP8_BLOCK128) return QL_ERR_FORMAT;
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

// Workspace of the LoRA down-projection for the GEMM paths (counters, t, partials).
struct LoraWs {
  SkinnyPlan plan;
  size_t bytes = 0;
  size_t total() const { return up(bytes); }
};
LoraWs lora_ws(int64_t m, int64_t k, int32_t rank) {
  LoraWs w;
  if (rank <= 0) return w;
  w.plan = ql::plan_skinny(m, 0, k, rank);
  w.bytes = ql::skinny_workspace(w.plan, m, k);
  return w;
}

size_t fp8_act_bytes(int64_t m, int64_t k) { return up((size_t)m * (size_t)k) + up((size_t)m * (size_t)(k / 128) * 4); }

qlinear_status hip_status(hipError_t e) { return e == hipSuccess ? QL_OK : QL_ERR_HIP; }

// LoRA intermediate t = bf16(s * x A^T) into the workspace (GEMM paths).
qlinear_status run_lora_t(const LoraWs& lw, char* ws, const uint16_t* x, int64_t m, int64_t k,
                          const uint16_t* lora_a, int32_t rank, float scale, uint16_t** t_out,
                          hipStream_t s) {
  if (ql::launch_lora_down(lw.plan, x, m, k, lora_a, rank, scale, ws, s) != hipSuccess) return QL_ERR_HIP;
  *t_out = ql::lora_t_in_workspace(lw.plan, ws);
  return QL_OK;
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
  return hip_status(ql::launch_fp8_weight_quantize(w, n, k, codes, scales, status_word,
                                                   (hipStream_t)stream));
}

qlinear_status qlinear_quantize_act_fp8(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                        float* sx, void* stream) {
  if (!x || !xq || !sx) return QL_ERR_NULL;
  if (!elems_ok(m, k) || k % 128) return QL_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(sx)) return QL_ERR_ALIGN;
  return hip_status(ql::launch_fp8_act_quantize(x, m, k, xq, sx, (hipStream_t)stream));
}

// --------------------------------------------------------------------- forward

size_t qlinear_forward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank) {
  if (m <= 0 || n <= 0 || k <= 0 || rank < 0) return 0;
  if (format == QL_NVFP4) {
    if (m <= kG16MaxM) return up(ql::g16_workspace(ql::plan_g16(m, n, k, rank), m));
    if (k % 64 == 0) return up(ql::gemm_nvfp4_f16_workspace(m, n, k, rank));
    return lora_ws(m, k, rank).total();
  }
  if (format == QL_FP8_BLOCK128) return fp8_act_bytes(m, k) + lora_ws(m, k, rank).total();
  return 0;
}

size_t qlinear_forward_prequant_workspace(int64_t m, int64_t n, int64_t k, int32_t rank) {
  (void)n;
  if (m <= 0 || k <= 0 || rank < 0) return 0;
  return lora_ws(m, k, rank).total();
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

qlinear_status qlinear_forward(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                               const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                               float lora_scale, void* y, int32_t out_dtype, void* ws,
                               size_t ws_bytes, void* stream) {
  qlinear_status st = check_forward_common(w, m, lora_a, lora_b, rank, y, out_dtype);
  if (st != QL_OK) return st;
  if (!x) return QL_ERR_NULL;
  if (!aligned16(x)) return QL_ERR_ALIGN;
  const int32_t r = lora_rank(lora_a, lora_b, rank, lora_scale);
  const size_t need = qlinear_forward_workspace(w->format, m, w->n, w->k, r);
  if (need > 0 && (!ws || ws_bytes < need)) return QL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int out_f32 = out_dtype == QL_OUT_F32;
  char* wsb = (char*)ws;

  if (w->format == QL_NVFP4) {
    const uint8_t* codes = (const uint8_t*)w->codes;
    const uint8_t* scales = (const uint8_t*)w->scales;
    if (m <= kG16MaxM) {
      const ql::G16Plan p = ql::plan_g16(m, w->n, w->k, r);
      return hip_status(ql::launch_g16(p, x, m, w->n, w->k, codes, scales, w->tensor_scale, lora_a,
                                       lora_b, r, lora_scale, y, out_f32, wsb, s));
    }
    if (w->k % 64 == 0)
      return hip_status(ql::launch_gemm_nvfp4_f16(x, m, w->n, w->k, codes, scales, w->tensor_scale,
                                                  lora_a, lora_b, r, lora_scale, y, out_f32, wsb, s));
    const LoraWs lw = lora_ws(m, w->k, r);
    uint16_t* t = nullptr;
    if (r > 0) {
      st = run_lora_t(lw, wsb, x, m, w->k, lora_a, r, lora_scale, &t, s);
      if (st != QL_OK) return st;
    }
    return hip_status(ql::launch_gemm_nvfp4(x, m, w->n, w->k, codes, scales, w->tensor_scale, t,
                                            lora_b, r, y, out_f32, s));
  }

  // FP8: quantize activations per 1x128 segment, then the block-scaled GEMM.
  if (w->format != QL_FP8_BLOCK128) return QL_ERR_FORMAT;
  uint8_t* xq = (uint8_t*)wsb;
  float* sx = (float*)(wsb + up((size_t)m * (size_t)w->k));
  char* rest = wsb + fp8_act_bytes(m, w->k);
  if (ql::launch_fp8_act_quantize(x, m, w->k, xq, sx, s) != hipSuccess) return QL_ERR_HIP;
  const LoraWs lw = lora_ws(m, w->k, r);
  uint16_t* t = nullptr;
  if (r > 0) {
    st = run_lora_t(lw, rest, x, m, w->k, lora_a, r, lora_scale, &t, s);
    if (st != QL_OK) return st;
  }
  return hip_status(ql::launch_gemm_fp8(xq, sx, m, w->n, w->k, (const uint8_t*)w->codes,
                                        (const float*)w->scales, t, lora_b, r, y, out_f32, s));
}

qlinear_status qlinear_forward_fp8_prequant(const qlinear_qweight* w, const uint8_t* xq,
                                            const float* sx, int64_t m, const uint16_t* x,
                                            const uint16_t* lora_a, const uint16_t* lora_b,
                                            int32_t rank, float lora_scale, void* y,
                                            int32_t out_dtype, void* ws, size_t ws_bytes,
                                            void* stream) {
  qlinear_status st = check_forward_common(w, m, lora_a, lora_b, rank, y, out_dtype);
  if (st != QL_OK) return st;
  if (w->format != QL_FP8_BLOCK128) return QL_ERR_FORMAT;
  if (!xq || !sx) return QL_ERR_NULL;
  if (!aligned16(xq) || !aligned16(sx)) return QL_ERR_ALIGN;
  const int32_t r = lora_rank(lora_a, lora_b, rank, lora_scale);
  if (r > 0 && !x) return QL_ERR_NULL;
  if (x && !aligned16(x)) return QL_ERR_ALIGN;
  const size_t need = qlinear_forward_prequant_workspace(m, w->n, w->k, r);
  if (need > 0 && (!ws || ws_bytes < need)) return QL_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return QL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* t = nullptr;
  if (r > 0) {
    st = run_lora_t(lora_ws(m, w->k, r), (char*)ws, x, m, w->k, lora_a, r, lora_scale, &t, s);
    if (st != QL_OK) return st;
  }
  return hip_status(ql::launch_gemm_fp8(xq, sx, m, w->n, w->k, (const uint8_t*)w->codes,
                                        (const float*)w->scales, t, lora_b, r, y,
                                        out_dtype == QL_OUT_F32, s));
}

// ------------------------------------------------------------------- requant

size_t qlinear_requant_table_bytes(int32_t count) {
  if (count <= 0 || count > 65536) return 0;
  return ql::requant_table_bytes(count);
}

qlinear_status qlinear_requant_prepare(const qlinear_requant_item* items, int32_t count,
                                       int32_t format, void* table, size_t table_bytes,
                                       qlinear_requant_plan* plan, void* stream) {
  if (!items || !table || !plan) return QL_ERR_NULL;
  if (count <= 0 || count > 65536) return QL_ERR_ARG;
  if (format != QL_NVFP4 && format != QL_FP8_BLOCK128) return QL_ERR_FORMAT;
  if (table_bytes < ql::requant_table_bytes(count)) return QL_ERR_WORKSPACE;
  if (!aligned16(table)) return QL_ERR_ALIGN;
  std::vector<char> host(ql::requant_table_bytes(count), 0);
  ql::RequantHeader* h = (ql::RequantHeader*)host.data();
  ql::RequantDesc* d = (ql::RequantDesc*)(host.data() + sizeof(ql::RequantHeader));
  int64_t units = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qlinear_requant_item& it = items[i];
    if (it.q.format != format) return QL_ERR_ARG;
    if (!it.w) return QL_ERR_NULL;
    qlinear_status st = check_qweight(&it.q);
    if (st != QL_OK) return st;
    if (!aligned16(it.w)) return QL_ERR_ALIGN;
    d[i].w = it.w;
    d[i].codes = it.q.codes;
    d[i].scales = it.q.scales;
    d[i].tensor_scale = it.q.tensor_scale;
    d[i].n = it.q.n;
    d[i].k = it.q.k;
    d[i].unit_begin = units;
    d[i].unit_count = ql::requant_units(format, it.q.n, it.q.k);
    units += d[i].unit_count;
  }
  h->count = count;
  h->format = format;
  h->total_units = units;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(table, host.data(), host.size(), hipMemcpyHostToDevice, s) != hipSuccess)
    return QL_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return QL_ERR_HIP;
  plan->count = count;
  plan->format = format;
  plan->total_units = units;
  return QL_OK;
}

qlinear_status qlinear_requantize_all(const qlinear_requant_plan* plan, void* table,
                                      int32_t* status_word, void* stream) {
  if (!plan || !table) return QL_ERR_NULL;
  if (plan->count <= 0 || plan->count > 65536 || plan->total_units <= 0) return QL_ERR_ARG;
  if (plan->format != QL_NVFP4 && plan->format != QL_FP8_BLOCK128) return QL_ERR_FORMAT;
  if (!aligned16(table) || (status_word && ((uintptr_t)status_word & 3))) return QL_ERR_ALIGN;
  ql::RequantHeader h;
  std::memset(&h, 0, sizeof(h));
  h.count = plan->count;
  h.format = plan->format;
  h.total_units = plan->total_units;
  return hip_status(ql::launch_requant(table, h, status_word, (hipStream_t)stream));
}

}  // extern "C"
