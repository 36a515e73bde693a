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

typedef enum { QL_NVFP4 = 1, QL_FP8_BLOCK128 = 2, QL_FP8_POW2 = 3 } qlinear_format;
typedef enum { QL_OUT_BF16 = 1, QL_OUT_F32 = 2 } qlinear_out;

/* A quantized weight W [n, k] (host struct holding device pointers).
 *   QL_NVFP4:        codes  u8 [n][k/2]   two E2M1 codes per byte, even k in the low nibble
 *                    scales u8 [n][k/16]  E4M3 block scales
 *                    tensor_scale f32[1]  the FP32 tensor scale S
 *                    requires k % 16 == 0
 *   QL_FP8_BLOCK128: codes  u8 [n][k]     E4M3
 *                    scales f32 [n/128][k/128]  dequantization multipliers amax/448
 *                    tensor_scale NULL;   requires n % 128 == 0 and k % 128 == 0
 *   QL_FP8_POW2:     the FP8 recipe with its power-of-two scale option (mexc.co NeMo RL
 *                    FP8 page, closing section): as QL_FP8_BLOCK128, but
 *                    scales u8 [n/128][k/128]  E8M0 bytes e + 127 of the scale 2^e, e the
 *                    smallest integer with amax <= 448 * 2^e (0 for a zero block),
 *                    clamped to [-127, 127]; activations get the same 1x128 rule.  */
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
/* Most tensors one qlinear_requantize_all call takes. */
#define QLINEAR_MAX_REQUANT_ITEMS 65536

/* Bits the kernels OR into a workspace's status word (never cleared by the library). */
#define QLINEAR_STATUS_NONFINITE 1 /* a weight input held Inf or NaN (requantization)        */
#define QLINEAR_STATUS_TIMEOUT 2   /* a bounded wait for another workgroup gave up; the
                                      outputs that depended on it were stored as NaN        */
#define QLINEAR_STATUS_BAD_ITEM 4  /* a requantization item failed its checks and was skipped */

/* Human-readable name of a status code (static storage). */
const char* qlinear_status_string(qlinear_status s);

/* Device address of the status word of a forward or requantization workspace: its first
 * int32 (host-side pointer arithmetic only; nothing is launched).  Kernels OR the
 * QLINEAR_STATUS_* bits into it; read it after the stream has reached the call. */
int32_t* qlinear_status_word(void* ws);

/* ---------------------------------------------------------------- quantizers */

/* NVFP4 weight quantizer (QeRL's weight format: tldrocket.com QeRL page, "Key Features of
 * QeRL"; public NVFP4 definition: E2M1 elements, 16-element blocks along K, E4M3 block
 * scales, an FP32 tensor scale; arithmetic as in the contract at the top of this file).
 * W bf16 [n][k] -> codes u8 [n][k/2] (even k in the low nibble), scales u8 [n][k/16],
 * tensor_scale f32[1].  Needs a workspace of qlinear_quantize_workspace(QL_NVFP4, n, k)
 * bytes (per-workgroup partial maxima; its contents need no initialisation).
 * Two kernels: a tensor-wide |w| maximum, then the block/element encoder.
 * Errors: QL_ERR_NULL (w, codes, scales, tensor_scale, ws), QL_ERR_SHAPE (n<=0, k<=0,
 * k%16, n*k > QLINEAR_MAX_ELEMS), QL_ERR_ALIGN, QL_ERR_WORKSPACE. */
qlinear_status qlinear_quantize_nvfp4(const uint16_t* w, int64_t n, int64_t k,
                                      uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                      int32_t* status_word, void* ws, size_t ws_bytes,
                                      void* stream);

/* Blockwise FP8 weight quantizer (mexc.co NeMo RL FP8 page, "De technische doorbraak":
 * E4M3, one scale per 128x128 weight tile).  W bf16 [n][k] -> codes u8 [n][k] (E4M3),
 * scales f32 [n/128][k/128] (dequantization multipliers amax/448).  One workgroup per
 * 128x128 tile, no workspace.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (n%128, k%128, n*k too big), QL_ERR_ALIGN. */
qlinear_status qlinear_quantize_fp8_block(const uint16_t* w, int64_t n, int64_t k,
                                          uint8_t* codes, float* scales,
                                          int32_t* status_word, void* stream);

/* Dynamic 1x128 FP8 activation quantizer (same page and section: one scale per 1x128
 * activation segment), the step qlinear_forward runs on bf16 activations in the FP8
 * format; exported so callers can quantize one activation tensor once and feed several
 * projections.  x bf16 [m][k] -> xq u8 [m][k], sx f32 [m][k/128].
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (k%128), QL_ERR_ALIGN. */
qlinear_status qlinear_quantize_act_fp8(const uint16_t* x, int64_t m, int64_t k,
                                        uint8_t* xq, float* sx, void* stream);

/* The power-of-two variants of the two FP8 quantizers above (QL_FP8_POW2): scales are
 * E8M0 bytes, u8 [n/128][k/128] for weights and u8 [m][k/128] for activations; codes are
 * sign | E4M3(fl32(|v| / 2^e)).  Errors as their float-scale counterparts. */
qlinear_status qlinear_quantize_fp8_pow2(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                         uint8_t* scales, int32_t* status_word, void* stream);
qlinear_status qlinear_quantize_act_fp8_pow2(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                             uint8_t* sx, void* stream);

/* Size in bytes of the workspace qlinear_quantize_nvfp4 needs (0 for FP8). */
size_t qlinear_quantize_workspace(int32_t format, int64_t n, int64_t k);

/* ------------------------------------------------------------------- forward */

/* The rollout linear layer (QeRL: NVFP4 weight path plus a LoRA adapter kept in higher
 * precision, tldrocket.com QeRL page, "Key Features of QeRL" and the paragraph after it,
 * which puts the speedup in rollout prefill and decoding; the FP8 format follows the
 * mexc.co NeMo RL FP8 page, "De technische doorbraak"):
 *             y[m][n] = sum_k x[m][k] w_hat[n][k]  +  lora_scale * sum_j t[m][j] B[n][j],
 *             t[m][j] = sum_k x[m][k] A[j][k].
 * w (host struct): a quantized weight from the quantizers above.
 * x bf16 [m][k].  lora_a bf16 [rank][k], lora_b bf16 [n][rank]; rank == 0, NULL adapters
 * or lora_scale == 0 mean no LoRA term.  y: bf16 [m][n] (QL_OUT_BF16, rounded to nearest
 * even from the float32 result) or f32 [m][n] (QL_OUT_F32).  Accumulation is float32.
 * NVFP4: the dequantized weights (E2M1 x E4M3 products, exact in bf16 and in f16)
 * meet the activations in MFMA; S is applied in float32 after the K loop.  For m > 64
 * and k % 64 == 0 the activations are first copied into the workspace as f16, each row
 * scaled by a power of two that puts its largest magnitude in [2^14, 2^15) (exact but
 * for magnitudes below about 2^-29 of the row maximum), and f16 MFMA is used.
 * FP8: x is quantized per 1x128 segment into the workspace, then an FP8 MFMA GEMM
 * rescales each 128-deep partial sum by sx * sw.  QL_FP8_POW2: the same with power-of-two
 * scales, which the scaled MFMA applies itself (E8M0 operand scales), so partial sums
 * accumulate directly.
 * The LoRA intermediate s*t is rounded to bf16 before the up-projection.
 *
 * Workspace: qlinear_forward_workspace(format, m, n, k, rank) bytes, 16-byte aligned,
 * owned by the caller.  Its first QLINEAR_WS_RESERVED_BYTES hold the status word and the
 * integer counters through which the workgroups of one launch coordinate; they must be
 * zero before the first call, and every call returns the counters it used to zero.  No
 * call uses that region as scratch, and everything after it is scratch that a call writes
 * before reading.  So one zero-filled workspace, as large as the largest query, may serve
 * calls of every shape, format and path in any order.  Calls that share a workspace must
 * not overlap (same stream, or ordered by events).  The few-token NVFP4 path (m <= 64)
 * waits for its LoRA intermediate with a bound in time; if the bound is reached (never in
 * a launch whose workgroups all make progress) the affected outputs are NaN and
 * QLINEAR_STATUS_TIMEOUT is set in the status word.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE (m<=0, m > QLINEAR_MAX_M, sizes vs format, or a shape
 * the kernels cannot run: FP8 k >= 2^24, few-token NVFP4 counters or partials beyond the
 * workspace's reach -- the size query returns 0 for those), QL_ERR_ARG (rank < 0 or >
 * QLINEAR_MAX_RANK), QL_ERR_FORMAT, QL_ERR_ALIGN, QL_ERR_WORKSPACE. */
#define QLINEAR_WS_RESERVED_BYTES 131072
qlinear_status qlinear_forward(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                               const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                               float lora_scale, void* y, int32_t out_dtype,
                               void* ws, size_t ws_bytes, void* stream);

/* FP8 layer on activations already quantized by qlinear_quantize_act_fp8 (the FP8 GEMM
 * of the recipe, same page and section, without the activation step): xq u8 [m][k],
 * sx f32 [m][k/128] (QL_FP8_BLOCK128) or E8M0 u8 [m][k/128] from
 * qlinear_quantize_act_fp8_pow2 (QL_FP8_POW2).  x (bf16 [m][k]) is read only for the LoRA
 * term and may be NULL when there is none.  Workspace:
 * qlinear_forward_prequant_workspace(m, n, k, rank) bytes, with the same layout and rules
 * as qlinear_forward's.  Errors as qlinear_forward, plus QL_ERR_FORMAT if w is not FP8. */
qlinear_status qlinear_forward_fp8_prequant(const qlinear_qweight* w, const uint8_t* xq,
                                            const void* sx, int64_t m, const uint16_t* x,
                                            const uint16_t* lora_a, const uint16_t* lora_b,
                                            int32_t rank, float lora_scale, void* y,
                                            int32_t out_dtype, void* ws, size_t ws_bytes,
                                            void* stream);

/* Allocation-free variant of qlinear_forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, checks, kernels and results as qlinear_forward, without
 * ws/ws_bytes: the library's own device array of QLINEAR_NOALLOC_MAX_BYTES per GPU (held
 * until the process ends) serves as the workspace.  Calls whose
 * qlinear_forward_workspace(...) exceeds that size return QL_ERR_WORKSPACE and enqueue
 * nothing (decode-size calls fit; large prefill and FP8 GEMMs do not).  The first call on
 * each device sets the array up synchronously and must not be made under stream capture
 * (QL_ERR_ARG); later calls allocate nothing and may be captured.  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (different streams without
 * ordering, several host threads) race and give wrong results.  The array's status word
 * is not exposed: a timed-out wait shows as NaN outputs. */
#define QLINEAR_NOALLOC_MAX_BYTES (((size_t)32) << 20)
qlinear_status qlinear_forward_noalloc(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                                       const uint16_t* lora_a, const uint16_t* lora_b,
                                       int32_t rank, float lora_scale, void* y,
                                       int32_t out_dtype, void* stream);

/* Workspace sizes (0 for invalid arguments and for shapes the kernels cannot run). */
size_t qlinear_forward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank);

/* One layer of a qlinear_forward_group call (host struct holding device pointers). */
typedef struct {
  qlinear_qweight w;       /* QL_NVFP4, the group's common k                        */
  const uint16_t* lora_a;  /* bf16 [rank][k], or NULL (then every layer's is NULL)  */
  const uint16_t* lora_b;  /* bf16 [n][rank], NULL when lora_a is                   */
  void* y;                 /* [m][n], bf16 or f32 per out_dtype                      */
} qlinear_group_layer;

/* Up to QLINEAR_MAX_GROUP NVFP4 layers that read the same activations -- the q, k and v
 * projections of a decoder layer, or its gate and up projections -- each computing
 * qlinear_forward's y = x . dequant(w)^T + lora_scale (x A^T) B^T into its own output.
 * The whole policy runs every one of them once per decode step (tldrocket.com QeRL page,
 * the paragraph after "Key Features of QeRL": rollout decoding is where the NVFP4 layer
 * pays; the 32B-class layer's projections share their inputs).  For m > 64 and
 * k % 64 == 0, with every adapter's rank a multiple of 32 and count * rank <= 128, the
 * layers run as ONE activation pre-pass (row statistics, and every adapter's x A^T with
 * the A matrices stacked) and ONE GEMM over all their weight rows (each layer's n rounded
 * up to whole 256-row tiles, every tile in one layer, with that layer's tensor scale,
 * adapter and output): the activations are converted once, and the split-K schedule that
 * fills the chip covers the layers together.  Otherwise the layers run one after another
 * exactly as qlinear_forward.  Results match qlinear_forward on each layer within the
 * forward's tolerance (the K split order may differ).
 * layers: host array of `count` entries; all share k (layers[0].w.k) and rank; either
 * every layer has both adapter matrices or (rank 0, lora_scale 0, or all NULL) none.
 * Workspace: qlinear_forward_group_workspace(m, k, n, count, rank) bytes (n: host array
 * of the layers' n), with qlinear_forward's layout and reuse rules.
 * Errors: as qlinear_forward for each layer, plus QL_ERR_ARG (count < 1 or >
 * QLINEAR_MAX_GROUP), QL_ERR_SHAPE (a layer's k differs from the first), QL_ERR_NULL
 * (layers NULL, or adapters on some layers but not all). */
#define QLINEAR_MAX_GROUP 4
qlinear_status qlinear_forward_group(const qlinear_group_layer* layers, int32_t count, const uint16_t* x,
                                     int64_t m, int32_t rank, float lora_scale, int32_t out_dtype,
                                     void* ws, size_t ws_bytes, void* stream);
size_t qlinear_forward_group_workspace(int64_t m, int64_t k, const int64_t* n, int32_t count, int32_t rank);
size_t qlinear_forward_prequant_workspace(int64_t m, int64_t n, int64_t k, int32_t rank);

/* Backward pass of the NVFP4 + LoRA layer for LoRA training on the frozen 4-bit base
 * (tldrocket.com QeRL page, "Key Features of QeRL" and the paragraph after it: backprop
 * stays stable through LoRA, its gradients in higher precision; rapidrecap.app Jet-RL
 * summary, "Key Points": BF16 backward).  Given dy = dL/dy (bf16 [m][n]) of
 * y = x W^T + s (x A^T) B^T with W = dequant(w):
 *   dx [m][k] = dy . W + bf16(du) . A,  du = s . dy . B      (bf16 or float32 per dx_dtype)
 *   da [r][k] = du^T . x                                       (float32)
 *   db [n][r] = dy^T . t,                t = s . x . A^T        (float32)
 * with float32 accumulation; du and t enter da and db with about 16 significant bits (a
 * bf16 pair) and du enters dx rounded to bf16, as the forward rounds t.  w must be QL_NVFP4 with n % 64 == 0 and k % 128 == 0.  Without
 * an adapter (rank 0, a NULL lora pointer or lora_scale 0) only dx is computed and x, da,
 * db may be NULL.  Workspace: qlinear_backward_workspace(format, m, n, k, rank) bytes of
 * scratch (about 2 m n bytes for an f16 copy of dy, plus the adapter's intermediates); no
 * zeroing or reserved region is needed and it may be reused by any call once this one has
 * finished on its stream.
 * All pointers 16-byte aligned; the caller owns every buffer.  Errors: QL_ERR_NULL,
 * QL_ERR_SHAPE (m <= 0, m > QLINEAR_MAX_M, n % 64, k % 128, sizes beyond
 * QLINEAR_MAX_ELEMS), QL_ERR_FORMAT (not NVFP4, or dx_dtype), QL_ERR_ARG (rank < 0 or >
 * QLINEAR_MAX_RANK), QL_ERR_ALIGN, QL_ERR_WORKSPACE. */
qlinear_status qlinear_backward(const qlinear_qweight* w, const uint16_t* x, const uint16_t* dy,
                                int64_t m, const uint16_t* lora_a, const uint16_t* lora_b,
                                int32_t rank, float lora_scale, void* dx, int32_t dx_dtype,
                                float* da, float* db, void* ws, size_t ws_bytes, void* stream);
size_t qlinear_backward_workspace(int32_t format, int64_t m, int64_t n, int64_t k, int32_t rank);

/* ------------------------------------------------------ whole-policy requant */

/* After every training step the RL recipe recalibrates the quantization of the
 * constantly updated policy weights (mexc.co NeMo RL FP8 page, section
 * "Praktische prestatiewinsten").  Here: re-run the per-tensor quantizer of `format` on
 * every tensor of the policy (new scales AND codes), with a few launches over all tensors
 * instead of two per tensor.
 * items: DEVICE array of `count` entries (filled once by the caller; the same array may
 * serve every step).  Every item must have q.format == format and pass the checks of the
 * per-tensor quantizer; an item that does not is skipped and sets QLINEAR_STATUS_BAD_ITEM
 * in the workspace's status word (the host never reads the array).  Non-finite weights
 * set QLINEAR_STATUS_NONFINITE there.  ws: qlinear_requant_workspace(count) bytes,
 * 16-byte aligned, owned by the caller; it holds the status word (zero it before the
 * first call), the descriptor table rebuilt on the device by every call and the
 * per-tensor maxima.  Two calls on one workspace must not overlap.
 * Errors: QL_ERR_NULL, QL_ERR_ARG (count <= 0 or > QLINEAR_MAX_REQUANT_ITEMS),
 * QL_ERR_FORMAT, QL_ERR_WORKSPACE, QL_ERR_ALIGN (items or ws). */
qlinear_status qlinear_requantize_all(const qlinear_requant_item* items, int32_t count,
                                      int32_t format, void* ws, size_t ws_bytes, void* stream);
size_t qlinear_requant_workspace(int32_t count);

/* The training step's update fused with the requantization that follows it (same page and
 * section: the weights change every step, the scales are recalibrated after each).
 * deltas: DEVICE array of `count` pointers to dense bf16 updates, deltas[i] [n_i][k_i]
 * (16-byte aligned).  Each weight is replaced in place, through items[i].w, by
 * bf16_RNE(fl32(W) + fl32(delta)) and requantized in `format` exactly as
 * qlinear_requantize_all would requantize the new weights -- but the update pass also
 * takes the maxima (NVFP4) or does the whole FP8 tile, so only one more pass (the NVFP4
 * encode) reads the new weights.  Workspace, status word and errors as
 * qlinear_requantize_all; an item whose delta is NULL or misaligned is skipped (weight
 * untouched) and sets QLINEAR_STATUS_BAD_ITEM. */
qlinear_status qlinear_update_requantize_all(const qlinear_requant_item* items,
                                             const uint16_t* const* deltas, int32_t count,
                                             int32_t format, void* ws, size_t ws_bytes,
                                             void* stream);

/* ------------------------------------------------------------ FP8 KV cache */

/* FP8 KV-cache codec (mexc.co NeMo RL FP8 page, "Praktische prestatiewinsten": FP8
 * extended to the KV cache).  Each (token, head) vector of head_dim elements gets one
 * float32 scale s = amax/448 and E4M3 codes sign | E4M3(fl32(|v| / s)) -- the recipe's
 * 1 x 128 activation rule applied per vector.
 * Store: kv bf16 [tokens][heads][head_dim] -> cache_codes u8 [cache_slots][heads][head_dim]
 * and cache_scales f32 [cache_slots][heads] at rows slots[t] (int64, device, distinct).
 * Load: rows slots[t] of the cache -> out bf16 [tokens][heads][head_dim], each element
 * bf16_RNE(fl32(E4M3(code) * s)).
 * head_dim must be a power of two in [16, 512].  A slot outside [0, cache_slots) is skipped
 * (a load writes zeros for it) and sets QLINEAR_STATUS_BAD_ITEM in *status_word (if not
 * NULL).  Errors: QL_ERR_NULL, QL_ERR_SHAPE (tokens < 0, heads <= 0, head_dim,
 * cache_slots <= 0, sizes beyond QLINEAR_MAX_ELEMS), QL_ERR_ALIGN.  tokens == 0 launches
 * nothing. */
qlinear_status qlinear_kv_store_fp8(const uint16_t* kv, int64_t tokens, int32_t heads, int32_t head_dim,
                                    const int64_t* slots, uint8_t* cache_codes, float* cache_scales,
                                    int64_t cache_slots, int32_t* status_word, void* stream);
qlinear_status qlinear_kv_load_fp8(const uint8_t* cache_codes, const float* cache_scales,
                                   int64_t cache_slots, const int64_t* slots, int64_t tokens,
                                   int32_t heads, int32_t head_dim, uint16_t* out,
                                   int32_t* status_word, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
