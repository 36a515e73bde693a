// Pieces shared by the large-M GEMMs (gemm_fp8.hip, gemm_nvfp4.hip): workgroup tile
// order, direct global-to-LDS copies, the LDS slot swizzle, the LoRA up-projection tile
// and the guarded output store.
#pragma once
#include "common.hpp"

namespace ql {

// Tile index -> (tile along m, tile along n), in groups of 8 tiles along m.
__device__ __forceinline__ void gemm_group_tile(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                int64_t& tn) {
  const int64_t group = 8;
  const int64_t per_group = group * tiles_n;
  const int64_t g = t / per_group;
  const int64_t first_m = g * group;
  const int64_t gsize = tiles_m - first_m < group ? tiles_m - first_m : group;
  const int64_t in = t % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Within a launch phase of n workgroups, consecutive indices go to one XCD (workgroups
// are dealt to the 8 XCDs round-robin), so that the tiles one L2 serves are neighbours.
__device__ __forceinline__ int64_t gemm_xcd_remap(int64_t b, int64_t n) {
  return n % 8 == 0 ? (b % 8) * (n / 8) + b / 8 : b;
}

// Workgroup id -> (tile along m, tile along n): XCD-contiguous, grouped by 8 along m.
__device__ __forceinline__ void gemm_tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                                 int64_t& tn) {
  gemm_group_tile(gemm_xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
}

// Schedule with a split tail: the first `full` workgroups take whole tiles; the tiles
// left over after the last full round are each split `tail_split` ways along K, so that
// the final round fills the chip.  slot numbers the split workgroups (tile-major).
struct GemmWork {
  int64_t tm, tn;
  int64_t slot;  // -1 for a whole tile
  int split, nsplit;
};
__device__ __forceinline__ GemmWork gemm_schedule(int64_t tiles_m, int64_t tiles_n, int64_t full,
                                                  int tail_split) {
  GemmWork w;
  const int64_t b = blockIdx.x;
  int64_t t;
  if (b < full) {
    t = gemm_xcd_remap(b, full);
    w.slot = -1;
    w.split = 0;
    w.nsplit = 1;
  } else {
    const int64_t id = gemm_xcd_remap(b - full, (int64_t)gridDim.x - full);
    t = full + id / tail_split;
    w.slot = id;
    w.split = (int)(id % tail_split);
    w.nsplit = tail_split;
  }
  gemm_group_tile(t, tiles_m, tiles_n, w.tm, w.tn);
  return w;
}

// 16-byte slot of logical chunk `chunk` in LDS row `row` (128-byte rows, 8 slots).  A
// fragment read has 16 lanes (fixed g) reading chunk 2 g or 2 g + 1 of 16 consecutive
// rows.  With the row's low three bits alone, rows r and r + 8 collide; flipping the
// slot with bit 3 as well makes this pattern conflict-free on gfx950 (measured with
// the LDS bank-conflict counter; other chunk-per-lane patterns, e.g. chunk 4 h + g, do
// conflict under this swizzle).
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

// LoRA up-projection for a wave's NI x NJ grid of 16 (n) x 16 (m) output tiles:
//   acc[i][j][n][m] += sum_q B[n][q] t[m][q],  n = nbase + 16 i + ..., m = mbase + 16 j + ...
// with B = lora_b [n][rank] (MFMA A operand, rows clamped to n_lim) and t [m][rank_pad]
// (B operand, zero padded to rank_pad, rows of t_stride elements -- rank_pad when 0 --
// clamped to m_lim); lane (r, g) supplies ranks q0 + 8 g .. + 7 of row r.  Per 32-rank chunk every fragment is loaded once and
// all NI x NJ MFMAs follow.  With rank % 8 == 0 a lane's 8 ranks are one aligned
// 16-byte load (lora_b is 16-byte aligned) and are either all in range or all out.
// The MFMA operands of ranks q0 .. q0 + 32: rows of B (A operand) and of t (B operand).
template <int NI, int NJ>
__device__ __forceinline__ void lora_frags(const uint16_t* __restrict__ lora_b, const uint16_t* __restrict__ t,
                                           int32_t rank, int64_t n_lim, int64_t m_lim, int64_t nbase,
                                           int64_t mbase, int r, int g, int64_t ts, int q0, i32x4 (&af)[NI],
                                           i32x4 (&bfr)[NJ]) {
  const bool vec = (rank & 7) == 0;
  const int q = q0 + 8 * g;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t nr0 = nbase + 16 * i + r;
    const int64_t nr = nr0 < n_lim ? nr0 : n_lim - 1;
    if (vec) {
      af[i] = *(const i32x4*)(lora_b + nr * rank + (q < rank ? q : 0));
      if (q >= rank) af[i] = i32x4{0, 0, 0, 0};
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t b0 = q + e < rank ? lora_b[nr * rank + q + e] : 0u;
        const uint32_t b1 = q + e + 1 < rank ? lora_b[nr * rank + q + e + 1] : 0u;
        w[e / 2] = b0 | (b1 << 16);
      }
      af[i] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t mr0 = mbase + 16 * j + r;
    const int64_t mr = mr0 < m_lim ? mr0 : m_lim - 1;
    bfr[j] = *(const i32x4*)(t + mr * ts + q);
  }
}
template <int NI, int NJ>
__device__ __forceinline__ void lora_mfma(const i32x4 (&af)[NI], const i32x4 (&bfr)[NJ], f32x4 (&acc)[NI][NJ]) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                          __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
}
// acc += (t B^T) for ranks q_from .. rank_pad, 32 at a time.
template <int NI, int NJ>
__device__ __forceinline__ void lora_wave(const uint16_t* __restrict__ lora_b, const uint16_t* __restrict__ t,
                                          int32_t rank, int32_t rank_pad, int64_t n_lim, int64_t m_lim,
                                          int64_t nbase, int64_t mbase, int r, int g,
                                          f32x4 (&acc)[NI][NJ], int64_t t_stride = 0, int q_from = 0) {
  const int64_t ts = t_stride > 0 ? t_stride : rank_pad;
  for (int q0 = q_from; q0 < rank_pad; q0 += 32) {
    i32x4 af[NI], bfr[NJ];
    lora_frags<NI, NJ>(lora_b, t, rank, n_lim, m_lim, nbase, mbase, r, g, ts, q0, af, bfr);
    lora_mfma<NI, NJ>(af, bfr, acc);
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)p;
}

// 16 bytes per lane from global memory (uniform base + per-lane byte offset) straight
// into LDS at m0 + 16 * lane (m0 uniform).  An LDS-DMA load needs one wait state after
// the write of m0, which is read when the load issues; the asm keeps the compiler's own
// m0 value in a scratch register and puts it back, so m0 is not clobbered.  Issued as
// inline assembly (not the compiler builtin) because the compiler would otherwise take
// these LDS writes to alias every fragment read and wait for them before each one;
// completion is awaited explicitly with vmcnt.
__device__ __forceinline__ void lds_copy16(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(off), "s"(base), "s"(lds_base)
               : "memory");
}

// 16 bytes per lane from a per-lane 64-bit global address into LDS at m0 + 16 * lane.
__device__ __forceinline__ void lds_copy16_va(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(lds_base)
               : "memory");
}

// 4 bytes per lane from global memory straight into LDS at m0 + 4 * lane.
__device__ __forceinline__ void lds_copy4(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(off), "s"(base), "s"(lds_base)
               : "memory");
}

}  // namespace ql
