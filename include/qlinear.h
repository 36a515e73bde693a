/*
 * qlinear.h -- C ABI of the quantized rollout linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer the quantization-enhanced RL methods run during rollout:
 *
 *     y = x . dequant(Wq)^T  +  s . (x . A^T) . B^T
 *
 * with the weight path in a block-scaled low-precision format and a bf16 LoRA
 * adapter (A [r, K], B [N, r]) on the side.  Two formats:
 *
 *   QL_NVFP4          QeRL moves the policy's weight path to NVFP4 and keeps
 *                     LoRA, logits and gradients in higher precision
 *                     (tldrocket.com page "NVIDIA and MIT Collaborate on QeRL",
 *                     "Key Features of QeRL" and the paragraph after it; QeRL
 *                     abstract on the fugumt.com listing of arXiv 2510.11696).
 *                     Public NVFP4 definition: E2M1 codes, 16-element blocks
 *                     along K, one E4M3 scale per block, one FP32 tensor scale.
 *                     Activations stay bf16 (weight-only quantization).
 *   QL_FP8_BLOCK128   The NeMo RL FP8 recipe: E4M3 codes, one scale per 128x128
 *                     weight tile and per 1x128 activation segment (mexc.co page
 *                     "NVIDIA NeMo RL behaalt 48% snelheidswinst met end-to-end
 *                     FP8-precisietraining", section "De technische doorbraak").
 *
 * Conventions for every entry point below:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *     and owns every buffer; the library allocates no device memory and keeps
 *     no state between calls.  Buffers must be 16-byte aligned.
 *   - All tensors are dense row-major.  bf16 tensors are passed as uint16_t bit
 *     patterns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.
 *   - Argument errors are detected on the host, return a status code and
 *     enqueue nothing.  A failed kernel launch returns QL_ERR_HIP.
 *   - Non-finite weight inputs set bit 0 of `*status_word` (if not NULL) from
 *     the device; the codes produced for such a tensor are unspecified.  The
 *     status word is only ever OR-ed into, never cleared, by the library.
 *   - Results are bitwise reproducible from run to run (fixed reduction order,
 *     no floating-point atomics).
 *
 * Quantizer arithmetic (bit-exact contract; all IEEE float32, round to nearest
 * even; E2M1/E4M3 encoders round to nearest, ties to the even code, saturate
 * at 6 / 448):
 *   NVFP4:  S = amax(|W|)/2688;  e_b = E4M3(amax_b / (6 S));
 *           d_b = E4M3value(e_b) * S;  code = sign(w) | E2M1(|w| / d_b)
 *           (magnitude 0 when d_b == 0; e_b = 0 when S == 0).
 *   FP8:    s = amax_block/448;  code = sign(w) | E4M3(|w| / s)  (0 when s == 0).
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_OK = 0,
  QL_ERR_NULL = 1,      /* a required pointer is NULL                              */
  QL_ERR_SHAPE = 2,     /* a size is <= 0, not a multiple of the block, or too big */
  QL_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                         */
  QL_ERR_FORMAT = 4,    /* unknown format or output type                            */
  QL_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the size query returns    */
  QL_ERR_HIP = 6,       /* a HIP launch failed                                      */
  QL_ERR_ARG = 7        /* another invalid argument (rank, count, ...)              */
} qlinear_status;

typedef enum { QL_NVFP4 = 1, QL_FP8_BLOCK128 = 2 } qlinear_format;
typedef enum { QL_OUT_BF16 = 1, QL_OUT_F32 = 2 } qlinear_out;

/* A quantized weight W [n, k] (host struct holding device pointers).
 *   QL_NVFP4:        codes  u8 [n][k/2]   two E2M1 codes per byte, even k in the low nibble
 *                    scales u8 [n][k/16]  E4M3 block scales
 *                    tensor_scale f32[1]  the FP32 tensor scale S
 *                    requires k % 16 == 0
 *   QL_FP8_BLOCK128: codes  u8 [n][k]     E4M3
 *                    scales f32 [n/128][k/128]  dequantization multipliers
 *                    tensor_scale NULL;   requires n % 128 == 0 and k % 128 == 0  */
typedef struct {
  int32_t format;
  int32_t reserved;
  int64_t n, k;
  void* codes;
  void* scales;
  float* tensor_scale;
} qlinear_qweight;

/* One tensor of a whole-policy requantization: bf16 source and its quantized output. */
typedef struct {
  const uint16_t* w;
  qlinear_qweight q;
} qlinear_requant_item;

/* Largest n*k (elements) one tensor may have: 2^40. */
#define QLINEAR_MAX_ELEMS (((int64_t)1) << 40)
/* Largest LoRA rank accepted by qlinear_forward. */
#define QLINEAR_MAX_RANK 128
/* Largest token count accepted by qlinear_forward. */
#define QLINEAR_MAX_M (((int64_t)1) << 24)

/* Human-readable name of a status code (static storage). */
const char* qlinear_status_string(qlinear_status s);

/* ---------------------------------------------------------------- quantizers */

/* NVFP4 weight quantizer.  W bf16 [n][k] -> codes u8 [n][k/2], scales u8 [n][k/16],
 * tensor_scale f32[1].  Needs a workspace of qlinear_quantize_workspace(QL_NVFP4, n, k)
 * bytes (per-workgroup partial maxima; its contents need no initialisation).
 * Two kernels: a tensor-wide |w| maximum, then the block/element encoder.
 * Errors: QL_ERR_NULL (w, codes, scales, tensor_scale, ws), QL_ERR_SHAPE (n<=0, k<=0,
 * k%16, n*k > QLINEAR_MAX_ELEMS), QL_ERR_ALIGN, QL_ERR_WORKSPACE. */
qlinear_status qlinear_quantize_nvfp4(const uint16_t* w, int64_t n, int64_t k,
                                      uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                      int32_t* status_word, void* ws, size_t ws_bytes,
                                      void* stream);

/* Blockwise FP8 weight quantizer.  W bf16 [n][k] -> codes u8 [n][k] (E4M3),
 * scales f32 [n/128][k/128].  One workgroup per 128x128 tile, no workspace.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (n%128, k%128, n*k too big), QL_ERR_ALIGN. */
qlinear_status qlinear_quantize_fp8_block(const uint16_t* w, int64_t n, int64_t k,
                                          uint8_t* codes, float* scales,
                                          int32_t* status_word, void* stream);

/* Dynamic 1x128 FP8 activation quantizer (the step qlinear_forward runs on bf16
 * activations in the FP8 format; exported so callers can quantize one activation
 * tensor once and feed several projections).  x bf16 [m][k] -> xq u8 [m][k],
 * sx f32 [m][k/128].  Errors: QL_ERR_NULL, QL_ERR_SHAPE (k%128), QL_ERR_ALIGN. */
qlinear_status qlinear_quantize_act_fp8(const uint16_t* x, int64_t m, int64_t k,
                                        uint8_t* xq, float* sx, void* stream);

/* Size in bytes of the workspace qlinear_quantize_nvfp4 needs (0 for FP8). */
size_t qlinear_quantize_workspace(int32_t format, int64_t n, int64_t k);

/* ------------------------------------------------------------------- forward */

/* The layer:  y[m][n] = sum_k x[m][k] w_hat[n][k]  +  lora_scale * sum_j t[m][j] B[n][j],
 *             t[m][j] = sum_k x[m][k] A[j][k].
 * w (host struct): a quantized weight from the quantizers above.
 * x bf16 [m][k].  lora_a bf16 [rank][k], lora_b bf16 [n][rank]; rank == 0 or NULL
 * adapters mean no LoRA term.  y: bf16 [m][n] (QL_OUT_BF16, rounded to nearest even
 * from the float32 result) or f32 [m][n] (QL_OUT_F32).  Accumulation is float32.
 * NVFP4: the dequantized weights (E2M1 x E4M3 products, exact in bf16 and in f16)
 * meet the activations in MFMA; S is applied in float32 after the K loop.  For m > 64
 * and k % 64 == 0 the activations are first copied into the workspace as f16, each row
 * scaled by a power of two that puts its largest magnitude in [2^14, 2^15) (exact but
 * for magnitudes below about 2^-29 of the row maximum), and f16 MFMA is used.
 * FP8: x is quantized per 1x128 segment into the workspace, then an FP8 MFMA GEMM
 * rescales each 128-deep partial sum by sx * sw.
 * The LoRA intermediate s*t is rounded to bf16 before the up-projection.
 * Needs a workspace of qlinear_forward_workspace(format, m, n, k, rank) bytes.  The
 * workspace must be zero-filled before its FIRST use: the few-token NVFP4 path (m <= 64)
 * and the LoRA down-projection coordinate their workgroups through integer counters kept
 * in it, and every such call leaves those counters zero again.  Calls with m > 64 and FP8
 * calls use the workspace as scratch and leave it non-zero: a workspace they used must be
 * zero-filled again before a few-token NVFP4 call (m <= 64) uses it.  Calls that share a
 * workspace must not overlap (same stream, or ordered by events).
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (m<=0, m > QLINEAR_MAX_M, sizes vs format),
 * QL_ERR_ARG (rank < 0 or > QLINEAR_MAX_RANK), QL_ERR_FORMAT, QL_ERR_ALIGN,
 * QL_ERR_WORKSPACE. */
qlinear_status qlinear_forward(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                               const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                               float lora_scale, void* y, int32_t out_dtype,
                               void* ws, size_t ws_bytes, void* stream);

/* FP8 layer on activations already quantized by qlinear_quantize_act_fp8:
 * xq u8 [m][k], sx f32 [m][k/128].  x (bf16 [m][k]) is read only for the LoRA
 * term and may be NULL when rank == 0.  Workspace: qlinear_forward_workspace with
 * format QL_FP8_BLOCK128 minus the activation buffers, i.e.
 * qlinear_forward_prequant_workspace(m, n, k, rank).  Errors as qlinear_forward. */
qlinear_status qlinear_forward_fp8_prequant(const qlinear_qweight* w, const uint8_t* xq,
                                            const float* sx, int64_t m, const uint16_t* x,
                                            const uint16_t* lora_a, const uint16_t* lora_b,
                                            int32_t rank, float lora_scale, void* y,
                                            int32_t out_dtype, void* ws, size_t ws_bytes,
                                            void* stream);

size_t qlinear_forward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank);
size_t qlinear_forward_prequant_workspace(int64_t m, int64_t n, int64_t k, int32_t rank);

/* ------------------------------------------------------ whole-policy requant */

/* After every training step the RL recipe recalibrates the quantization of the
 * constantly updated policy weights (mexc.co NeMo RL FP8 page, section
 * "Praktische prestatiewinsten").  Here: re-run the per-tensor quantizer of
 * `format` on every tensor of the policy (new scales AND codes), grouped into
 * three launches (NVFP4: clear maxima, tensor maxima, encode) or one (FP8) over all
 * tensors instead of two launches per tensor.
 *
 * qlinear_requant_prepare (once, whenever the set of tensors changes): checks every
 * item of the host array `items` (count entries) like the per-tensor quantizer would,
 * writes a device table of qlinear_requant_table_bytes(count) bytes into `table`
 * (device memory owned by the caller), fills the host struct *plan, and
 * synchronises `stream` (the host array may be reused on return).
 * qlinear_requantize_all (every step): requantizes every tensor the table names.
 * The table also holds per-tensor scratch (tensor maxima), so two requantize_all
 * calls on one table must not overlap.
 * Errors: QL_ERR_NULL, QL_ERR_ARG (count <= 0 or > 65536, an item's format differs
 * from `format`, plan does not match), QL_ERR_SHAPE, QL_ERR_ALIGN, QL_ERR_FORMAT,
 * QL_ERR_WORKSPACE (table_bytes too small), QL_ERR_HIP (the table copy failed). */
typedef struct {
  int32_t count;
  int32_t format;
  int64_t total_units; /* workgroup-sized work units over all tensors */
} qlinear_requant_plan;

size_t qlinear_requant_table_bytes(int32_t count);
qlinear_status qlinear_requant_prepare(const qlinear_requant_item* items, int32_t count,
                                       int32_t format, void* table, size_t table_bytes,
                                       qlinear_requant_plan* plan, void* stream);
qlinear_status qlinear_requantize_all(const qlinear_requant_plan* plan, void* table,
                                      int32_t* status_word, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
