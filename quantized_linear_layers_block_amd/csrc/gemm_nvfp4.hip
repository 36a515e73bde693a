// NVFP4-weight layer for many tokens (rollout prefill) on gfx950:
//
//   y[m][n] = S * sum_k x[m][k] * E2M1(c[n][k]) * E4M3(e[n][k/16])  +  sum_j t[m][j] B[n][j]
//
// QeRL speeds up prefill as well as decoding with the NVFP4 weight path
// (tldrocket.com QeRL page, paragraph after "Key Features of QeRL").  NVFP4's
// E4M3-scaled 16-element blocks have no counterpart in gfx950's block-scaled MFMA
// (power-of-two scales per 32 elements), but every E2M1 x E4M3 product is an exact
// bf16, so weight tiles are dequantized exactly into LDS as bf16 and multiplied with
// the bf16 activations by 16x16x32 bf16 MFMAs; S is applied in float32 after the K
// loop and the LoRA up-projection (t = s.x.A^T rounded to bf16, computed beforehand)
// is one more MFMA K chunk per 32 ranks.
//
// Tiling: 256 (n) x 256 (m) per workgroup of four waves (2 x 2), 128 x 128 per wave,
// K step 64 (two MFMAs per tile and step).  Each thread dequantizes one weight row's
// 64 elements per step (32 bytes of codes, 4 block scales).  Both bf16 tiles (32 KB
// each) are double-buffered in LDS with a 16-byte XOR swizzle.
#include "common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kNThreads = 256;
constexpr int kNTile = 256;
constexpr int kNRowBytes = 128;  // 64 bf16 per LDS row
constexpr int kNK = 64;

struct Nvfp4GemmArgs {
  const uint16_t* x;
  int64_t m, n, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* t;
  const uint16_t* lora_b;
  int32_t rank, rank_pad;
  void* y;
  int64_t tiles_m, tiles_n;
};

__device__ __forceinline__ void nv_tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
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

__device__ __forceinline__ int nswz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ uint4 dequant8_u4(uint32_t c, float sc) {
  const f32x2 p0 = e2m1_unpack2<0>(c), p1 = e2m1_unpack2<1>(c), p2 = e2m1_unpack2<2>(c),
              p3 = e2m1_unpack2<3>(c);
  return make_uint4(pack_exact_bf16(p0.x * sc, p0.y * sc), pack_exact_bf16(p1.x * sc, p1.y * sc),
                    pack_exact_bf16(p2.x * sc, p2.y * sc), pack_exact_bf16(p3.x * sc, p3.y * sc));
}

__device__ __forceinline__ void nv_store4(void* y, int out_f32, int64_t n_total, int64_t m,
                                          int64_t n, f32x4 v) {
  if (out_f32) {
    float* p = (float*)y + m * n_total + n;
    if (n + 4 <= n_total && (n_total & 3) == 0) {
      *(f32x4*)p = v;
    } else {
      for (int i = 0; i < 4; ++i)
        if (n + i < n_total) p[i] = v[i];
    }
  } else {
    uint16_t* p = (uint16_t*)y + m * n_total + n;
    const uint32_t b[4] = {f32_to_bf16_rne(v[0]), f32_to_bf16_rne(v[1]), f32_to_bf16_rne(v[2]),
                           f32_to_bf16_rne(v[3])};
    if (n + 4 <= n_total && (n_total & 3) == 0) {
      *(uint2*)p = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    } else {
      for (int i = 0; i < 4; ++i)
        if (n + i < n_total) p[i] = (uint16_t)b[i];
    }
  }
}

template <int OUT_F32>
__global__ __launch_bounds__(kNThreads, 1) void gemm_nvfp4_kernel(Nvfp4GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* As = smem;                                 // [2][256][128 B] dequantized weights
  uint8_t* Bs = smem + 2 * kNTile * kNRowBytes;       // [2][256][128 B] activations

  int64_t tm, tn;
  nv_tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int64_t n0 = tn * kNTile, m0 = tm * kNTile;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const int64_t ksteps = (a.k + kNK - 1) / kNK;
  const bool aligned = (a.k % kNK) == 0;

  // staging: activations 8 x 16 B (rows tid/8 + 32 i, chunk tid%8); weights: row tid,
  // 32 bytes of codes and 4 scale bytes.
  uint4 gx[8];
  uint4 gc0, gc1;
  uint32_t gsc;
  auto fetch = [&](int64_t ks) {
    const int64_t kk = ks * kNK;
    const bool full = aligned || kk + kNK <= a.k;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tid / 8 + 32 * i;
      const int ch = tid & 7;
      const int64_t mr = m0 + row;
      const bool ok = mr < a.m && (full || kk + 8 * ch < a.k);
      gx[i] = ok ? *(const uint4*)(a.x + mr * a.k + kk + 8 * ch) : make_uint4(0, 0, 0, 0);
    }
    const int64_t nr = n0 + tid;
    if (nr < a.n) {
      const uint8_t* cp = a.codes + nr * (a.k / 2) + kk / 2;
      const uint8_t* sp = a.scales + nr * (a.k / 16) + kk / 16;
      if (full && (a.k % 128) == 0) {
        gc0 = *(const uint4*)cp;
        gc1 = *(const uint4*)(cp + 16);
        gsc = *(const uint32_t*)sp;
      } else {
        uint32_t cw[8], sb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool ok = kk + 16 * b < a.k;
          const uint2 v = ok ? *(const uint2*)(cp + 8 * b) : make_uint2(0, 0);
          cw[2 * b] = v.x;
          cw[2 * b + 1] = v.y;
          sb[b] = ok ? sp[b] : 0u;
        }
        gc0 = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        gc1 = make_uint4(cw[4], cw[5], cw[6], cw[7]);
        gsc = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
      }
    } else {
      gc0 = gc1 = make_uint4(0, 0, 0, 0);
      gsc = 0;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = tid / 8 + 32 * i;
      *(uint4*)(Bs + (buf * kNTile + row) * kNRowBytes + nswz(row, tid & 7) * 16) = gx[i];
    }
    uint8_t* arow = As + (buf * kNTile + tid) * kNRowBytes;
    const uint32_t cw[8] = {gc0.x, gc0.y, gc0.z, gc0.w, gc1.x, gc1.y, gc1.z, gc1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {  // chunk c = elements [8c, 8c+8), block c/2
      const float sc = e4m3_value((gsc >> (8 * (c / 2))) & 0xFFu);
      *(uint4*)(arow + nswz(tid, c) * 16) = dequant8_u4(cw[c], sc);
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  fetch(0);
  stash(0);
  __syncthreads();

  for (int64_t ks = 0; ks < ksteps; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < ksteps) fetch(ks + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // two MFMA k-steps of 32: chunks 4h + g
      bf16x8 bfr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 128 * wm + 16 * j + r;
        const uint4 v = *(const uint4*)(Bs + (buf * kNTile + row) * kNRowBytes + nswz(row, 4 * h + g) * 16);
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 128 * wn + 16 * i + r;
        const uint4 v = *(const uint4*)(As + (buf * kNTile + row) * kNRowBytes + nswz(row, 4 * h + g) * 16);
        const bf16x8 af = __builtin_bit_cast(bf16x8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    if (ks + 1 < ksteps) stash(buf ^ 1);
    __syncthreads();
  }

  const float S = *a.tensor_scale;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t mrow = m0 + 128 * wm + 16 * j + r;
      const int64_t nrow = n0 + 128 * wn + 16 * i + r;
      f32x4 v = S * acc[i][j];
      for (int j0 = 0; j0 < a.rank_pad; j0 += 32) {
        uint32_t bw[4], tw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int jj = j0 + 8 * g + e;
          const uint32_t b0 = (nrow < a.n && jj < a.rank) ? a.lora_b[nrow * a.rank + jj] : 0u;
          const uint32_t b1 = (nrow < a.n && jj + 1 < a.rank) ? a.lora_b[nrow * a.rank + jj + 1] : 0u;
          bw[e / 2] = b0 | (b1 << 16);
          const uint32_t t0 = mrow < a.m ? a.t[mrow * a.rank_pad + jj] : 0u;
          const uint32_t t1 = mrow < a.m ? a.t[mrow * a.rank_pad + jj + 1] : 0u;
          tw[e / 2] = t0 | (t1 << 16);
        }
        i32x4 bi = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
        i32x4 ti = {(int)tw[0], (int)tw[1], (int)tw[2], (int)tw[3]};
        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bi),
                                                    __builtin_bit_cast(bf16x8, ti), v, 0, 0, 0);
      }
      if (mrow < a.m) nv_store4(a.y, OUT_F32, a.n, mrow, n0 + 128 * wn + 16 * i + 4 * g, v);
    }
  }
}

hipError_t launch_gemm_nvfp4(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const uint16_t* t, const uint16_t* lora_b, int32_t rank, void* y,
                             int out_f32, hipStream_t s) {
  Nvfp4GemmArgs a;
  a.x = x;
  a.m = m;
  a.n = n;
  a.k = k;
  a.codes = codes;
  a.scales = scales;
  a.tensor_scale = tensor_scale;
  a.t = t;
  a.lora_b = lora_b;
  a.rank = t ? rank : 0;
  a.rank_pad = t ? (rank + 31) / 32 * 32 : 0;
  a.y = y;
  a.tiles_m = (m + kNTile - 1) / kNTile;
  a.tiles_n = (n + kNTile - 1) / kNTile;
  const size_t lds = 4 * kNTile * kNRowBytes;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (out_f32) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_kernel<1><<<grid, kNThreads, lds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_kernel<0><<<grid, kNThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ql
