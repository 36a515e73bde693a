// Host-side launchers of the gfx950 kernels (internal to libqlinear; the C ABI in
// api.cpp validates arguments before calling any of these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

// ---- quantizers (quant.hip)
constexpr int kAmaxParts = 1024;  // partial maxima written by the NVFP4 amax pass
hipError_t launch_nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 uint8_t* scales, float* tensor_scale, int32_t* status,
                                 uint32_t* partials, hipStream_t s);
hipError_t launch_fp8_weight_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      float* scales, int32_t* status, hipStream_t s);
hipError_t launch_fp8_act_quantize(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                   float* sx, hipStream_t s);

// ---- whole-policy requantization (requant.hip)
struct RequantDesc {       // one tensor, as stored in the device table
  const uint16_t* w;
  void* codes;
  void* scales;
  float* tensor_scale;
  int64_t n, k;
  int64_t unit_begin;      // first work unit of this tensor in the global unit space
  int64_t unit_count;
};
struct RequantHeader {
  int32_t count;
  int32_t format;
  int64_t total_units;
  int64_t pad[2];
};
// Table layout: header | descs[count] | amax[count] (uint32, per-tensor |w| maximum bits)
size_t requant_table_bytes(int32_t count);
hipError_t launch_requant(void* table, const RequantHeader& h, int32_t* status, hipStream_t s);
int64_t requant_units(int32_t format, int64_t n, int64_t k);

// ---- NVFP4 few-token layer and LoRA down-projection (gemv.hip)
struct SkinnyPlan {
  int mt;                     // m tiles of 16 per workgroup (1, 2, 4)
  int r;                      // row tiles of 16 per wave
  int splits;                 // K splits
  int64_t kchunks_per_split;  // 256-wide K chunks per split
  int m_groups;               // groups of 16 mt tokens
  int64_t rows_w;             // NVFP4 rows (n)
  int64_t rows_w_pad;         // n rounded up to whole row groups
  int64_t rows_l;             // LoRA rows (rank rounded up to 16), 0 if none
  int64_t rows_total;         // row length of the LoRA partials
  int64_t groups_w, groups_l; // row groups of 16 r rows
  int rank_pad;               // row length of t (rank rounded up to 32)
};
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int32_t rank);
size_t skinny_workspace(const SkinnyPlan& p, int64_t m, int64_t k);
// t = bf16(s x A^T) [m][rank_pad] into the workspace (plan from plan_skinny(m, 0, k, rank)).
hipError_t launch_lora_down(const SkinnyPlan& p, const uint16_t* x, int64_t m, int64_t k,
                            const uint16_t* lora_a, int32_t rank, float lora_scale, void* ws,
                            hipStream_t s);
uint16_t* lora_t_in_workspace(const SkinnyPlan& p, void* ws);

// ---- NVFP4 layer for up to 64 tokens (gemv16.hip); workspace zero before first use
struct G16Plan {
  int mt;             // m tiles of 16 (1 or 2)
  int rt;             // row tiles of 16 per workgroup (1 or 2)
  int64_t tiles_w;    // weight tiles of 16 * rt rows
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
  size_t lds_bytes;
};
G16Plan plan_g16(int64_t m, int64_t n, int64_t k, int32_t rank);
size_t g16_workspace(const G16Plan& p, int64_t m);
hipError_t launch_g16(const G16Plan& p, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                      const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                      const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                      float lora_scale, void* y, int out_f32, void* ws, hipStream_t s);

// ---- large-M GEMMs (gemm_nvfp4.hip, gemm_fp8.hip)
// Generic K (k % 16 == 0): t = bf16(s x A^T) computed beforehand, or null.
hipError_t launch_gemm_nvfp4(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const uint16_t* t, const uint16_t* lora_b, int32_t rank, void* y,
                             int out_f32, hipStream_t s);
// k % 64 == 0: f16 activations, row factors and the LoRA intermediate are formed in the
// workspace (gemm_nvfp4_f16_workspace bytes) by a pre-pass.
hipError_t launch_gemm_nvfp4_f16(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scale, const uint16_t* lora_a,
                                 const uint16_t* lora_b, int32_t rank, float lora_scale, void* y,
                                 int out_f32, void* ws, hipStream_t s);
size_t gemm_nvfp4_f16_workspace(int64_t m, int64_t n, int64_t k, int32_t rank);
hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, int64_t m, int64_t n, int64_t k,
                           const uint8_t* wq, const float* sw, const uint16_t* t,
                           const uint16_t* lora_b, int32_t rank, void* y, int out_f32,
                           hipStream_t s);

}  // namespace ql
