// Host-side launchers of the gfx950 kernels (internal to libqlinear; the C ABI in
// api.cpp validates arguments before calling any of these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qlinear.h"

namespace ql {

// hipGetLastError reports the last failure of any HIP call on the thread, not only of the
// launches just made: every entry point clears it before its first launch, so a launch
// status reflects this library's launches alone.
inline void clear_hip_error() { (void)hipGetLastError(); }

// qlinear_forward's checks and dispatch (api.cpp), shared with the allocation-free variant.
qlinear_status forward_impl(const qlinear_qweight* w, const uint16_t* x, int64_t m,
                            const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                            float lora_scale, void* y, int32_t out_dtype, void* ws, size_t ws_bytes,
                            void* stream);

// ---- forward workspace layout, shared by every path
// [0, kWsReserved): the status word (int32 at offset 0) and, from kWsCounterOff on, the
// integer counters and flags through which the workgroups of one launch coordinate.  They
// must be zero before the first call and every call returns the ones it used to zero, so
// calls of any shape may share one workspace.  No path ever uses this region as scratch.
// [kWsReserved, ...): per-call scratch, always written before it is read within a call.
constexpr size_t kWsReserved = 128 * 1024;
constexpr size_t kWsCounterOff = 256;
constexpr uint32_t kStatusNonFinite = 1u;  // a weight input held Inf or NaN
constexpr uint32_t kStatusTimeout = 2u;    // a bounded wait for another workgroup gave up
constexpr uint32_t kStatusBadItem = 4u;    // a requantization item failed its checks
inline int32_t* ws_status(void* ws) { return (int32_t*)ws; }
inline uint32_t* ws_counters(void* ws) { return (uint32_t*)((char*)ws + kWsCounterOff); }
inline char* ws_scratch(void* ws) { return (char*)ws + kWsReserved; }

// ---- quantizers (quant.hip)
constexpr int kAmaxParts = 1024;  // partial maxima written by the NVFP4 amax pass
hipError_t launch_nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 uint8_t* scales, float* tensor_scale, int32_t* status,
                                 uint32_t* partials, hipStream_t s);
// FP8 scales: float32 amax/448, or with pow2 the E8M0 byte of the power-of-two scale.
hipError_t launch_fp8_weight_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      void* scales, bool pow2, int32_t* status, hipStream_t s);
hipError_t launch_fp8_act_quantize(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                   void* sx, bool pow2, hipStream_t s);

// ---- whole-policy requantization (quant.hip)
// Workspace: status word | header | descriptors[count] | per-tensor maxima[count].  The
// descriptors are rebuilt on the device from the caller's item array by every call.  With
// deltas (a device array of count update pointers) each weight is first updated in place.
size_t requant_workspace(int32_t count);
hipError_t launch_requant(const void* items, const uint16_t* const* deltas, int32_t count,
                          int32_t format, void* ws, hipStream_t s);

// ---- FP8 KV-cache codec (kv.hip); head_dim a power of two in [16, 512]
hipError_t launch_kv_store(const uint16_t* kv, int64_t tokens, int heads, int head_dim, const int64_t* slots,
                           uint8_t* codes, float* scales, int64_t cache_slots, int32_t* status, hipStream_t s);
hipError_t launch_kv_load(const uint8_t* codes, const float* scales, int64_t cache_slots, const int64_t* slots,
                          int64_t tokens, int heads, int head_dim, uint16_t* out, int32_t* status, hipStream_t s);

// ---- backward of the NVFP4 + LoRA layer (backward.hip); n % 64 == 0, k % 128 == 0
size_t backward_scratch_bytes(int64_t m, int64_t n, int64_t k, int32_t rank);
hipError_t launch_backward_nvfp4(const uint16_t* x, const uint16_t* dy, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                 const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank, float lora_scale,
                                 void* dx, int out_f32, float* da, float* db, void* scratch, hipStream_t s);

// ---- NVFP4 layer for up to 64 tokens (gemv16.hip)
struct G16Plan {
  int mt;             // m tiles of 16 (1, 2 or 4)
  int rt;             // row tiles of 16 per workgroup (1 or 2)
  int64_t tiles_w;    // weight tiles of 16 * rt rows (64 rows for 33..64 tokens)
  int64_t kchunks;    // 256-wide K chunks
  int64_t tiles_l;    // LoRA row tiles of 16
  int64_t lgroups;    // LoRA chunk groups
  int lc;             // chunks per LoRA item
  int rank_pad;
  int64_t cps;        // chunks per K split
  int splits;
  int64_t n_pad;
  int xstride;        // LDS row stride of the staged activations
  int64_t kst = 0;    // 128-wide K stages of the 33..64-token stage path (0: not used)
  int64_t sps = 0;    // stages per K split on that path
  int64_t full = 0;   // that path: tiles [0, full) whole, the others split `splits` ways
  size_t lds_bytes;
  int ctr_stride = 0; // words between two counters in the reserved region (0: does not fit)
};
G16Plan plan_g16(int64_t m, int64_t n, int64_t k, int32_t rank);
// false if the launch cannot run this shape (counters do not fit the reserved region,
// partial offsets beyond 32 bits): the C ABI reports QL_ERR_SHAPE before launching.
bool g16_plan_ok(const G16Plan& p, int64_t m);
size_t g16_workspace(const G16Plan& p, int64_t m);  // scratch bytes after the reserved region
hipError_t launch_g16(const G16Plan& p, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                      const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                      const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                      float lora_scale, void* y, int out_f32, void* ws, hipStream_t s);

// ---- LoRA down-projection for the GEMM paths (gemm_nvfp4.hip)
// t = bf16(s x A^T) as [m][rank_pad] (zero past the rank) in `scratch`; two kernels (split-K
// partials, then their fixed-order sum), no inter-workgroup counters.  k % 16 == 0.
size_t lora_down_bytes(int64_t m, int64_t k, int32_t rank);
// The same product s . x . A^T kept in higher precision: bf16 [m][2 rank_pad], row = the
// rounded value hi (columns [0, rank_pad)) and the rounded remainder lo (columns [rank_pad,
// 2 rank_pad)).
size_t lora_down_hilo_bytes(int64_t m, int64_t k, int32_t rank);
hipError_t launch_lora_down_hilo(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a,
                                 int32_t rank, float lora_scale, void* scratch, uint16_t** t_hl_out,
                                 hipStream_t s);
hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a,
                            int32_t rank, float lora_scale, void* scratch, uint16_t** t_out,
                            hipStream_t s);

// ---- large-M GEMMs (gemm_nvfp4.hip, gemm_fp8.hip)
// Generic K (k % 16 == 0): t = bf16(s x A^T) computed beforehand, or null.
hipError_t launch_gemm_nvfp4(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const uint16_t* t, const uint16_t* lora_b, int32_t rank, void* y,
                             int out_f32, hipStream_t s);
// k % 64 == 0 and k < kNvF16MaxK: f16 activations, row factors and the LoRA intermediate
// are formed in `scratch` (gemm_nvfp4_f16_workspace bytes) by a pre-pass.
constexpr int64_t kNvF16MaxK = int64_t(1) << 22;
hipError_t launch_gemm_nvfp4_f16(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scale, const uint16_t* lora_a,
                                 const uint16_t* lora_b, int32_t rank, float lora_scale, void* y,
                                 int out_f32, void* scratch, hipStream_t s);
size_t gemm_nvfp4_f16_workspace(int64_t m, int64_t n, int64_t k, int32_t rank);
// Up to kNvMaxSeg layers that read the same x (a fused projection) as one pre-pass and one
// GEMM over all their n tiles (each layer's n rounded up to whole 256-row tiles); the
// adapters (all of rank `rank`, a multiple of 32 for more than one layer, nl * rank <= 128)
// are stacked for the pre-pass.  nl == 1 is launch_gemm_nvfp4_f16.
constexpr int kNvMaxSeg = 4;
struct NvLayer {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* lora_a;
  const uint16_t* lora_b;
  void* y;
  int64_t n;
};
size_t gemm_nvfp4_f16_layers_workspace(int64_t m, int64_t k, const int64_t* n, int nl, int32_t rank);
hipError_t launch_gemm_nvfp4_f16_layers(const uint16_t* x, int64_t m, int64_t k, const NvLayer* layers, int nl,
                                        int32_t rank, float lora_scale, int out_f32, void* scratch, hipStream_t s);
// x as f16 rows scaled by powers of two (x16 [m][k], rs [m]: x[r] = rs[r] x16[r], exact but
// for values below about 2^-29 of the row maximum) and, with rank > 0, t = s x A^T as hi | lo
// bf16 pairs [m][2 rank_pad] (null without).  k % 64 == 0, k < kNvF16MaxK.
size_t f16_rows_bytes(int64_t m, int64_t k, int32_t rank);
hipError_t launch_f16_rows(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a, int32_t rank,
                           float lora_scale, void* scratch, uint16_t** x16, float** rs, uint16_t** t_hl,
                           hipStream_t s);
// Backward dX [m][k] = S rs[m] (dY16 W)[m][k] + (du A)[m][k] over the n weight rows, with
// A^T [k][rank_pad] and du [m][du_stride] (first rank_pad columns) zero past the rank
// (rank_pad 0: no adapter).  n % 64 == 0, n < kNvF16MaxK, k % 128 == 0, k < kNvDxMaxK (copy
// offsets within a stage are 32-bit); part: nvfp4_dx_part_bytes of split-tile partials.
constexpr int64_t kNvDxMaxK = int64_t(1) << 27;
size_t nvfp4_dx_part_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_nvfp4_dx(const uint16_t* dy16, const float* rs, int64_t m, int64_t n, int64_t k,
                           const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                           const uint16_t* at, const uint16_t* du, int32_t rank_pad, int64_t du_stride, void* dx,
                           int out_f32, float* part, hipStream_t s);
// k % 128 == 0 and k < kFp8MaxK (copy offsets within a 256-row tile are 32-bit).
constexpr int64_t kFp8MaxK = int64_t(1) << 24;
// pow2: sx, sw are E8M0 bytes applied by the scaled MFMA; else float32, folded per K block.
hipError_t launch_gemm_fp8(const uint8_t* xq, const void* sx, int64_t m, int64_t n, int64_t k,
                           const uint8_t* wq, const void* sw, bool pow2, const uint16_t* t,
                           const uint16_t* lora_b, int32_t rank, void* y, int out_f32,
                           hipStream_t s);

}  // namespace ql
