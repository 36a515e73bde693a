// Pieces shared by the large-M GEMMs (gemm_fp8.hip, gemm_nvfp4.hip): workgroup tile
// order, direct global-to-LDS copies, the LDS slot swizzle, the LoRA up-projection tile
// and the guarded output store.
#pragma once
#include "common.hpp"

namespace ql {

// Workgroup id -> (tile along m, tile along n): XCD-contiguous, grouped by 8 along m.
__device__ __forceinline__ void gemm_tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                 int64_t& tn) {
  const int64_t nb = (int64_t)gridDim.x;
  int64_t id = blockIdx.x;
  if (nb % 8 == 0) id = (id % 8) * (nb / 8) + id / 8;
  const int64_t group = 8;
  const int64_t per_group = group * tiles_n;
  const int64_t g = id / per_group;
  const int64_t first_m = g * group;
  const int64_t gsize = tiles_m - first_m < group ? tiles_m - first_m : group;
  const int64_t in = id % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// 16-byte slot of logical chunk `chunk` in LDS row `row`.  A fragment read has 16 lanes
// reading one chunk column of 16 consecutive rows; with 128-byte rows, rows r and r + 8
// would share banks under a 64-bank LDS, so bit 3 of the row flips the slot as well.
// Conflict-free for 8-lane / 32-bank and 16-lane / 64-bank service alike.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }

// Store a float4 of outputs for one m and four consecutive n.
__device__ __forceinline__ void store4(void* y, int out_f32, int64_t n_total, int64_t m,
                                       int64_t n, f32x4 v, int64_t n_lim) {
  if (out_f32) {
    float* p = (float*)y + m * n_total + n;
    if (n + 4 <= n_lim && (n_total & 3) == 0) {
      *(f32x4*)p = v;
    } else {
      for (int i = 0; i < 4; ++i)
        if (n + i < n_lim) p[i] = v[i];
    }
  } else {
    uint16_t* p = (uint16_t*)y + m * n_total + n;
    const uint32_t lo = pack_bf16x2_rne(v[0], v[1]), hi = pack_bf16x2_rne(v[2], v[3]);
    if (n + 4 <= n_lim && (n_total & 3) == 0) {
      *(uint2*)p = make_uint2(lo, hi);
    } else {
      const uint32_t b[4] = {lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16};
      for (int i = 0; i < 4; ++i)
        if (n + i < n_lim) p[i] = (uint16_t)b[i];
    }
  }
}

// LoRA up-projection for one 16 (n) x 16 (m) MFMA tile: C[n][m] += sum_j B[n][j] t[m][j],
// with B = lora_b rows (MFMA A operand) and t rows (B operand, rank_pad columns, zero
// padded).  VEC: rank % 8 == 0, so a lane's 8 consecutive rank entries are one aligned
// 16-byte load (lora_b is 16-byte aligned) and are either all in range or all out.
template <bool VEC>
__device__ __forceinline__ f32x4 lora_tile(const uint16_t* __restrict__ lora_b,
                                           const uint16_t* __restrict__ t, int32_t rank,
                                           int32_t rank_pad, int64_t n_lim, int64_t m_lim,
                                           int64_t nrow, int64_t mrow, int g, f32x4 c) {
  const int64_t nr = nrow < n_lim ? nrow : n_lim - 1;
  const int64_t mr = mrow < m_lim ? mrow : m_lim - 1;
  for (int j0 = 0; j0 < rank_pad; j0 += 32) {
    const int j = j0 + 8 * g;
    i32x4 bi, ti;
    if (VEC) {
      const int jc = j < rank ? j : 0;
      bi = *(const i32x4*)(lora_b + nr * rank + jc);
      if (j >= rank) bi = i32x4{0, 0, 0, 0};
      ti = *(const i32x4*)(t + mr * rank_pad + j);
    } else {
      uint32_t bw[4], tw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t b0 = j + e < rank ? lora_b[nr * rank + j + e] : 0u;
        const uint32_t b1 = j + e + 1 < rank ? lora_b[nr * rank + j + e + 1] : 0u;
        bw[e / 2] = b0 | (b1 << 16);
        tw[e / 2] = (uint32_t)t[mr * rank_pad + j + e] | ((uint32_t)t[mr * rank_pad + j + e + 1] << 16);
      }
      bi = i32x4{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
      ti = i32x4{(int)tw[0], (int)tw[1], (int)tw[2], (int)tw[3]};
    }
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bi),
                                                __builtin_bit_cast(bf16x8, ti), c, 0, 0, 0);
  }
  return c;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)p;
}

// 16 bytes per lane from global memory (uniform base + per-lane byte offset) straight
// into LDS at m0 + 16 * lane (m0 uniform).  An LDS-DMA load needs one wait state after
// the write of m0.
__device__ __forceinline__ void lds_copy16(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(lds_base)
               : "memory", "m0");
}

// 4 bytes per lane from global memory straight into LDS at m0 + 4 * lane.
__device__ __forceinline__ void lds_copy4(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base),
               "s"(lds_base)
               : "memory", "m0");
}

}  // namespace ql
