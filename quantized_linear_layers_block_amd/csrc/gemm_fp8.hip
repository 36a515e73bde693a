// Blockwise-FP8 layer for many tokens on gfx950 (the FP8 recipe of the mexc.co NeMo RL
// page, "De technische doorbraak": E4M3 operands, 128x128 weight blocks, 1x128
// activation blocks; the page puts FP8 linear layers at twice the BF16 peak):
//
//   y[m][n] = sum_kb sx[m][kb] * sw[n/128][kb] * sum_{k in kb} xq[m][k] * wq[n][k]  (+ LoRA)
//
// One K block of 128 is exactly one 16x16x128 FP8 MFMA, so every MFMA starts from zero
// and its result is folded into the float32 accumulator with one FMA by the combined
// scale.  The weights are the MFMA's A operand (rows n) and the activations its B
// operand (columns m): a lane's four accumulators then share one m and one 128-row
// weight block, i.e. one scale per lane per K block.
//
// Tiling: 256 (n) x 256 (m) per workgroup of four waves (2 x 2), 128 x 128 per wave
// (8 x 8 MFMA tiles), K step 128.  Operand tiles (32 KB each) are double-buffered in
// LDS (128 KB) with a 16-byte XOR swizzle so that the 16 lanes reading one column of
// 16 rows hit distinct banks; the next K block is fetched into registers while the
// current one is multiplied.  Workgroup ids are remapped so that the tiles an XCD
// (one L2) runs are neighbours, grouped eight m tiles at a time.
#include "common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kGThreads = 256;
constexpr int kTile = 256;     // rows of n and of m per workgroup
constexpr int kRowBytes = 128; // one K block of fp8 per LDS row

struct Fp8GemmArgs {
  const uint8_t* xq;
  const float* sx;
  const uint8_t* wq;
  const float* sw;
  int64_t m, n, k;
  const uint16_t* t;       // bf16 [m][rank_pad] (lora_scale already applied) or null
  const uint16_t* lora_b;  // bf16 [n][rank]
  int32_t rank;
  int32_t rank_pad;
  void* y;
  int64_t tiles_m, tiles_n;
};

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

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

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
    const uint32_t b0 = f32_to_bf16_rne(v[0]), b1 = f32_to_bf16_rne(v[1]);
    const uint32_t b2 = f32_to_bf16_rne(v[2]), b3 = f32_to_bf16_rne(v[3]);
    if (n + 4 <= n_lim && (n_total & 3) == 0) {
      *(uint2*)p = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else {
      const uint32_t b[4] = {b0, b1, b2, b3};
      for (int i = 0; i < 4; ++i)
        if (n + i < n_lim) p[i] = (uint16_t)b[i];
    }
  }
}

// LoRA up-projection for one 16 (n) x 16 (m) MFMA tile: C[n][m] += sum_j B[n][j] t[m][j].
__device__ __forceinline__ f32x4 lora_tile(const uint16_t* __restrict__ lora_b,
                                           const uint16_t* __restrict__ t, int32_t rank,
                                           int32_t rank_pad, int64_t n_lim, int64_t m_lim,
                                           int64_t nrow, int64_t mrow, int g, f32x4 c) {
  for (int j0 = 0; j0 < rank_pad; j0 += 32) {
    uint32_t bw[4], tw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int j = j0 + 8 * g + e;
      const uint32_t b0 = (nrow < n_lim && j < rank) ? lora_b[nrow * rank + j] : 0u;
      const uint32_t b1 = (nrow < n_lim && j + 1 < rank) ? lora_b[nrow * rank + j + 1] : 0u;
      bw[e / 2] = b0 | (b1 << 16);
      const uint32_t t0 = mrow < m_lim ? t[mrow * rank_pad + j] : 0u;
      const uint32_t t1 = mrow < m_lim ? t[mrow * rank_pad + j + 1] : 0u;
      tw[e / 2] = t0 | (t1 << 16);
    }
    i32x4 bi = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
    i32x4 ti = {(int)tw[0], (int)tw[1], (int)tw[2], (int)tw[3]};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bi),
                                                __builtin_bit_cast(bf16x8, ti), c, 0, 0, 0);
  }
  return c;
}

template <int OUT_F32>
__global__ __launch_bounds__(kGThreads, 1) void gemm_fp8_kernel(Fp8GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* As = smem;                                  // [2][256][128] weights (rows n)
  uint8_t* Bs = smem + 2 * kTile * kRowBytes;          // [2][256][128] activations (rows m)
  float* Ss = (float*)(smem + 4 * kTile * kRowBytes);  // [2][256] sx of the tile's m rows

  int64_t tm, tn;
  gemm_tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int64_t n0 = tn * kTile, m0 = tm * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const int64_t kblocks = a.k / 128;

  // global -> register staging: 8 x 16 B per operand per thread (rows tid/8 + 32 i, chunk tid%8)
  uint4 ga[8], gb[8];
  float gs;
  auto fetch = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tid / 8 + 32 * i;
      const int ch = tid & 7;
      const int64_t nr = n0 + row, mr = m0 + row;
      ga[i] = nr < a.n ? *(const uint4*)(a.wq + nr * a.k + kb * 128 + ch * 16) : make_uint4(0, 0, 0, 0);
      gb[i] = mr < a.m ? *(const uint4*)(a.xq + mr * a.k + kb * 128 + ch * 16) : make_uint4(0, 0, 0, 0);
    }
    const int64_t mr = m0 + tid;
    gs = mr < a.m ? a.sx[mr * kblocks + kb] : 0.0f;
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tid / 8 + 32 * i;
      const int ch = swz(row, tid & 7);
      *(uint4*)(As + (buf * kTile + row) * kRowBytes + ch * 16) = ga[i];
      *(uint4*)(Bs + (buf * kTile + row) * kRowBytes + ch * 16) = gb[i];
    }
    Ss[buf * kTile + tid] = gs;
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  fetch(0);
  stash(0);
  __syncthreads();

  const f32x4 zero = {0, 0, 0, 0};
  const int64_t nblk = (n0 + 128 * wn) / 128;  // this wave's 128-row weight block
  for (int64_t kb = 0; kb < kblocks; ++kb) {
    const int buf = (int)(kb & 1);
    if (kb + 1 < kblocks) fetch(kb + 1);
    const float swv = nblk * 128 < a.n ? a.sw[nblk * kblocks + kb] : 0.0f;
    // B fragments (activations) and combined scales for the wave's 8 m tiles
    i32x8 bf[8];
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 128 * wm + 16 * j + r;
      const uint8_t* p = Bs + (buf * kTile + row) * kRowBytes;
      const uint4 lo = *(const uint4*)(p + swz(row, 2 * g) * 16);
      const uint4 hi = *(const uint4*)(p + swz(row, 2 * g + 1) * 16);
      i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      bf[j] = v;
      sc[j] = Ss[buf * kTile + row] * swv;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 128 * wn + 16 * i + r;
      const uint8_t* p = As + (buf * kTile + row) * kRowBytes;
      const uint4 lo = *(const uint4*)(p + swz(row, 2 * g) * 16);
      const uint4 hi = *(const uint4*)(p + swz(row, 2 * g + 1) * 16);
      i32x8 af = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 127, 0, 127);
        acc[i][j] += sc[j] * pr;
      }
    }
    if (kb + 1 < kblocks) stash(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds m = m0 + 128 wm + 16 j + r, n = n0 + 128 wn + 16 i + 4 g + (0..3).
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t mrow = m0 + 128 * wm + 16 * j + r;
      f32x4 v = acc[i][j];
      if (a.rank_pad > 0) {
        // MFMA tile: A operand rows n (B_lora), B operand columns m (t)
        const int64_t nrow = n0 + 128 * wn + 16 * i + r;
        f32x4 lz = lora_tile(a.lora_b, a.t, a.rank, a.rank_pad, a.n, a.m, nrow, mrow, g, zero);
        v += lz;
      }
      if (mrow < a.m) store4(a.y, OUT_F32, a.n, mrow, n0 + 128 * wn + 16 * i + 4 * g, v, a.n);
    }
  }
}

hipError_t launch_gemm_fp8(const uint8_t* xq, const float* sx, int64_t m, int64_t n, int64_t k,
                           const uint8_t* wq, const float* sw, const uint16_t* t,
                           const uint16_t* lora_b, int32_t rank, void* y, int out_f32,
                           hipStream_t s) {
  Fp8GemmArgs a;
  a.xq = xq;
  a.sx = sx;
  a.wq = wq;
  a.sw = sw;
  a.m = m;
  a.n = n;
  a.k = k;
  a.t = t;
  a.lora_b = lora_b;
  a.rank = t ? rank : 0;
  a.rank_pad = t ? (rank + 31) / 32 * 32 : 0;
  a.y = y;
  a.tiles_m = (m + kTile - 1) / kTile;
  a.tiles_n = (n + kTile - 1) / kTile;
  const size_t lds = 4 * kTile * kRowBytes + 2 * kTile * sizeof(float);
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (out_f32) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_fp8_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_fp8_kernel<1><<<grid, kGThreads, lds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_fp8_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_fp8_kernel<0><<<grid, kGThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ql
