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

// ---- NVFP4 / bf16 skinny GEMM for few tokens (gemv.hip)
// partials[split][m][rows_total] float32 with rows_total = n + rank_pad
struct SkinnyPlan {
  int mt;          // m tiles of 16 per workgroup (1..4)
  int splits;      // k splits
  int64_t kchunks_per_split;  // 512-wide k chunks per split
  int m_groups;    // workgroups along m
  int64_t rows_w;      // NVFP4 rows (n)
  int64_t rows_w_pad;  // n rounded up to a whole number of workgroup row tiles
  int64_t rows_l;      // bf16 LoRA rows (rank padded to 16), 0 if none
  int64_t rows_total;
};
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int32_t rank);
size_t skinny_workspace(const SkinnyPlan& p, int64_t m);
hipError_t launch_skinny(const SkinnyPlan& p, const uint16_t* x, int64_t m, int64_t k,
                         const uint8_t* codes, const uint8_t* scales, const uint16_t* lora_a,
                         int32_t rank, float* partials, hipStream_t s);
hipError_t launch_skinny_reduce(const SkinnyPlan& p, int64_t m, int64_t n, const float* partials,
                                const float* tensor_scale, const uint16_t* lora_b, int32_t rank,
                                float lora_scale, void* y, int out_f32, hipStream_t s);
// t[m][j] = bf16(lora_scale * sum over splits of partials[s][m][rows_w + j]) for the GEMM paths
hipError_t launch_lora_t(const SkinnyPlan& p, int64_t m, const float* partials, int32_t rank,
                         float lora_scale, uint16_t* t, hipStream_t s);

// ---- large-M GEMMs (gemm_nvfp4.hip, gemm_fp8.hip)
hipError_t launch_gemm_nvfp4(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const uint16_t* t, const uint16_t* lora_b, int32_t rank, void* y,
                             int out_f32, hipStream_t s);
hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, int64_t m, int64_t n, int64_t k,
                           const uint8_t* wq, const float* sw, const uint16_t* t,
                           const uint16_t* lora_b, int32_t rank, void* y, int out_f32,
                           hipStream_t s);

}  // namespace ql
