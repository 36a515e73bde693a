// Few-token ("decode") NVFP4 layer for gfx950:  y = S . x . (E2M1 * E4M3)^T + s . (x A^T) B^T.
//
// QeRL's speedup is in rollout decoding, where the policy's weight path is NVFP4
// (tldrocket.com QeRL page, paragraph after "Key Features of QeRL"); with a handful of
// tokens the layer streams 0.5625 byte per weight and is bound by HBM, so the kernel
// is organised around streaming the packed codes once with 16-byte loads.
//
// Kernel 1 (skinny_kernel): every wave owns R tiles of 16 weight rows and a set of
// 512-wide K chunks.  Lane l reads row (l % 16) of each tile and the 128 consecutive
// K of lane group g = l / 16 (64 bytes of codes, 8 block scales), dequantizes them in
// registers -- E2M1 -> float by the hardware converter, times the E4M3 block scale in
// float32 (the product is exact and has at most 6 significant bits, so it is an exact
// bf16) -- and feeds 16x16x32 bf16 MFMAs with the activations as the other operand.
// The K order inside an MFMA is a permutation shared by both operands, which lets each
// lane keep 128 contiguous K.  The four waves of a workgroup split the K chunks of one
// split and add their partial tiles through LDS.  The LoRA down-projection x A^T runs
// in the same launch: extra workgroups treat the bf16 rows of A as weight rows.
// Output: float32 partial sums [split][m][row].
//
// Kernel 2 (skinny_reduce_kernel): sums the K splits in a fixed order, multiplies by
// S, rounds s.t to bf16 and adds the LoRA up-projection with one 16x16x32 bf16 MFMA per
// 32 ranks, then writes bf16 (round to nearest even) or float32.
#include "common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kSkThreads = 256;
constexpr int kChunk = 512;  // K per wave iteration: 4 lane groups x 128

struct SkinnyArgs {
  const uint16_t* x;
  int64_t m, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* lora_a;
  int32_t rank;
  int64_t rows_w;        // NVFP4 rows (n)
  int64_t rows_w_pad;    // first LoRA row in the partials (n padded to whole row tiles)
  int64_t rows_total;
  int64_t wg_w;          // workgroups along rows for the NVFP4 rows
  int64_t kchunks;
  int64_t cps;           // chunks per split
  float* partials;
};

// 8 E2M1 codes (one dword) times one block scale -> 8 exact bf16 values.
__device__ __forceinline__ bf16x8 dequant8(uint32_t c, float sc) {
  f32x2 p0 = e2m1_unpack2<0>(c), p1 = e2m1_unpack2<1>(c), p2 = e2m1_unpack2<2>(c),
        p3 = e2m1_unpack2<3>(c);
  uint32_t o0 = pack_exact_bf16(p0.x * sc, p0.y * sc);
  uint32_t o1 = pack_exact_bf16(p1.x * sc, p1.y * sc);
  uint32_t o2 = pack_exact_bf16(p2.x * sc, p2.y * sc);
  uint32_t o3 = pack_exact_bf16(p3.x * sc, p3.y * sc);
  i32x4 o = {(int)o0, (int)o1, (int)o2, (int)o3};
  return __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  i32x4 z = {0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  uint4 v = *(const uint4*)p;
  return __builtin_bit_cast(bf16x8, v);
}

template <int MT, int R, bool LORA, bool FULL>
__device__ __forceinline__ void skinny_chunk(const SkinnyArgs& a, int64_t row0, int64_t row_lim,
                                             int64_t mbase, int64_t kk, f32x4 (&acc)[R][MT]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t kl = kk + 128 * g;                              // first K of this lane
  const int valid = FULL ? 128 : (int)max((int64_t)0, min((int64_t)128, a.k - kl));

  // A operand source for each row tile: NVFP4 codes + scales, or bf16 rows of LoRA A.
  uint4 cw[R][4];
  uint2 sw[R];
  if constexpr (!LORA) {
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int64_t row = row0 + 16 * p + r;
      const bool rv = row < row_lim;
      const uint8_t* cp = a.codes + row * (a.k / 2) + kl / 2;
      const uint8_t* sp = a.scales + row * (a.k / 16) + kl / 16;
      if (FULL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[p][j] = rv ? *(const uint4*)(cp + 16 * j) : make_uint4(0, 0, 0, 0);
        sw[p] = rv ? *(const uint2*)sp : make_uint2(0, 0);
      } else {
        uint32_t cd[16];
        uint32_t sb[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {  // 16-element blocks: 8 code bytes, 1 scale byte
          const bool bv = rv && 16 * b < valid;
          uint2 v = bv ? *(const uint2*)(cp + 8 * b) : make_uint2(0, 0);
          cd[2 * b] = v.x;
          cd[2 * b + 1] = v.y;
          sb[b] = bv ? sp[b] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[p][j] = make_uint4(cd[4 * j], cd[4 * j + 1], cd[4 * j + 2], cd[4 * j + 3]);
        sw[p].x = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
        sw[p].y = sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24);
      }
    }
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {  // 32 K per step of j, 4 MFMA k-steps of 8 per lane
    bf16x8 bx[4][MT];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e0 = 32 * j + 8 * t;                              // element offset in lane range
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mrow = mbase + 16 * q + r;
        const bool ok = mrow < a.m && (FULL || e0 < valid);
        bx[t][q] = ok ? load_bf16x8(a.x + mrow * a.k + kl + e0) : zero_bf16x8();
      }
    }
#pragma unroll
    for (int p = 0; p < R; ++p) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 av;
        if constexpr (LORA) {
          const int64_t row = row0 + 16 * p + r;
          const int e0 = 32 * j + 8 * t;
          const bool ok = row < row_lim && (FULL || e0 < valid);
          av = ok ? load_bf16x8(a.lora_a + row * a.k + kl + e0) : zero_bf16x8();
        } else {
          const uint32_t c = t == 0 ? cw[p][j].x : t == 1 ? cw[p][j].y : t == 2 ? cw[p][j].z : cw[p][j].w;
          const int blk = (32 * j + 8 * t) / 16;                  // block within the lane's 8
          const uint32_t sbyte = ((blk < 4 ? sw[p].x : sw[p].y) >> (8 * (blk & 3))) & 0xFFu;
          av = dequant8(c, e4m3_value(sbyte));
        }
#pragma unroll
        for (int q = 0; q < MT; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[t][q], acc[p][q], 0, 0, 0);
      }
    }
  }
}

template <int MT, int R, bool LORA>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& a, int64_t row0, int64_t row_lim,
                                            int64_t row_out0, f32x4* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t split = blockIdx.y;
  const int64_t mbase = (int64_t)blockIdx.z * 16 * MT;
  const int64_t c0 = split * a.cps;
  const int64_t c1 = min(c0 + a.cps, a.kchunks);

  f32x4 acc[R][MT];
#pragma unroll
  for (int p = 0; p < R; ++p)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[p][q] = f32x4{0, 0, 0, 0};

  for (int64_t c = c0 + wave; c < c1; c += 4) {
    const int64_t kk = c * kChunk;
    // The unguarded path needs whole 512-chunks and 8-byte aligned scale rows (k % 128 == 0).
    if (kk + kChunk <= a.k && (a.k & 127) == 0) skinny_chunk<MT, R, LORA, true>(a, row0, row_lim, mbase, kk, acc);
    else skinny_chunk<MT, R, LORA, false>(a, row0, row_lim, mbase, kk, acc);
  }

  // Add the four waves' tiles (fixed order) and store wave 0's result.
#pragma unroll
  for (int p = 0; p < R; ++p) {
#pragma unroll
    for (int q = 0; q < MT; ++q) red[(wave * MT + q) * kWave + lane] = acc[p][q];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        f32x4 s = red[(0 * MT + q) * kWave + lane];
        s += red[(1 * MT + q) * kWave + lane];
        s += red[(2 * MT + q) * kWave + lane];
        s += red[(3 * MT + q) * kWave + lane];
        const int64_t mrow = mbase + 16 * q + (lane & 15);
        if (mrow < a.m) {
          const int64_t row = row_out0 + 16 * p + 4 * (lane >> 4);
          *(f32x4*)(a.partials + (split * a.m + mrow) * a.rows_total + row) = s;
        }
      }
    }
    __syncthreads();
  }
}

template <int MT, int R>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs a) {
  __shared__ f32x4 red[4 * MT * kWave];
  const int64_t bx = blockIdx.x;
  if (bx < a.wg_w) {
    const int64_t row0 = bx * 16 * R;
    skinny_body<MT, R, false>(a, row0, a.rows_w, row0, red);
  } else {
    const int64_t row0 = (bx - a.wg_w) * 16 * R;
    skinny_body<MT, R, true>(a, row0, a.rank, a.rows_w_pad + row0, red);
  }
}

// ----------------------------------------------------------------- planning

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

static int skinny_r(int mt) { return mt >= 3 ? 4 : (mt == 2 ? 2 : 1); }

SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int32_t rank) {
  SkinnyPlan p;
  p.mt = (int)min((int64_t)4, cdiv(m, 16));
  p.m_groups = (int)cdiv(m, 16 * p.mt);
  const int R = skinny_r(p.mt);
  p.rows_w = n;
  p.rows_w_pad = round_up(n, 16 * R);
  p.rows_l = rank > 0 ? round_up(rank, 16) : 0;
  p.rows_total = p.rows_w_pad + round_up(p.rows_l, 16 * R);
  const int64_t kchunks = cdiv(k, kChunk);
  const int64_t row_wgs = cdiv(n, 16 * R) + cdiv(p.rows_l, 16 * R);
  // Aim for >= ~1024 workgroups (4 per CU) while keeping >= 4 chunks (one per wave) per split.
  int64_t splits = 1;
  while (row_wgs * p.m_groups * splits < 1024 && cdiv(kchunks, splits * 2) >= 4) splits *= 2;
  p.kchunks_per_split = cdiv(kchunks, splits);
  p.splits = (int)cdiv(kchunks, p.kchunks_per_split);
  return p;
}

size_t skinny_workspace(const SkinnyPlan& p, int64_t m) {
  return (size_t)p.splits * (size_t)m * (size_t)p.rows_total * sizeof(float);
}

template <int MT, int R>
static hipError_t launch_skinny_t(const SkinnyPlan& p, const SkinnyArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.wg_w + cdiv(p.rows_l, 16 * R)), (unsigned)p.splits, (unsigned)p.m_groups);
  skinny_kernel<MT, R><<<grid, kSkThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_skinny(const SkinnyPlan& p, const uint16_t* x, int64_t m, int64_t k,
                         const uint8_t* codes, const uint8_t* scales, const uint16_t* lora_a,
                         int32_t rank, float* partials, hipStream_t s) {
  SkinnyArgs a;
  a.x = x;
  a.m = m;
  a.k = k;
  a.codes = codes;
  a.scales = scales;
  a.lora_a = lora_a;
  a.rank = p.rows_l > 0 ? rank : 0;
  a.rows_w = p.rows_w;
  a.rows_w_pad = p.rows_w_pad;
  a.rows_total = p.rows_total;
  const int R = skinny_r(p.mt);
  a.wg_w = cdiv(p.rows_w, 16 * R);
  a.kchunks = cdiv(k, kChunk);
  a.cps = p.kchunks_per_split;
  a.partials = partials;
  switch (p.mt) {
    case 1: return launch_skinny_t<1, 1>(p, a, s);
    case 2: return launch_skinny_t<2, 2>(p, a, s);
    case 3: return launch_skinny_t<3, 4>(p, a, s);
    default: return launch_skinny_t<4, 4>(p, a, s);
  }
}

// ------------------------------------------------------------------- reduce

struct ReduceArgs {
  int64_t m, n;
  int splits;
  int64_t rows_total, rows_w_pad;
  const float* partials;
  const float* tensor_scale;
  const uint16_t* lora_b;
  int32_t rank;
  float lora_scale;
  void* y;
  int out_f32;
};

// bf16(lora_scale * t[m][j]) from the partials, 0 outside [0, rank) or for m >= M.
__device__ __forceinline__ uint32_t lora_t_bf16(const ReduceArgs& a, int64_t m, int j) {
  if (m >= a.m || j >= a.rank) return 0;
  float t = 0.0f;
  for (int s = 0; s < a.splits; ++s)
    t += a.partials[((int64_t)s * a.m + m) * a.rows_total + a.rows_w_pad + j];
  return f32_to_bf16_rne(a.lora_scale * t);
}

// One wave per 16 (n) x 16 (m) output tile; a workgroup holds four tiles along m.
__global__ __launch_bounds__(kSkThreads) void skinny_reduce_kernel(ReduceArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = ((int64_t)blockIdx.y * 4 + wave) * 16;
  if (m0 >= a.m) return;
  const int r = lane & 15;
  const int g = lane >> 4;
  f32x4 lo = {0, 0, 0, 0};
  if (a.rank > 0) {
    for (int j0 = 0; j0 < a.rank; j0 += 32) {
      // A operand: B_lora rows n0 + r, ranks j0 + 8g .. +8 (bf16); B operand: s.t for m0 + r.
      uint32_t bw[4] = {0, 0, 0, 0}, tw[4] = {0, 0, 0, 0};
      const int64_t nrow = n0 + r;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int j = j0 + 8 * g + e;
        uint32_t b0 = (nrow < a.n && j < a.rank) ? a.lora_b[nrow * a.rank + j] : 0u;
        uint32_t b1 = (nrow < a.n && j + 1 < a.rank) ? a.lora_b[nrow * a.rank + j + 1] : 0u;
        bw[e / 2] = b0 | (b1 << 16);
        tw[e / 2] = lora_t_bf16(a, m0 + r, j) | (lora_t_bf16(a, m0 + r, j + 1) << 16);
      }
      i32x4 bi = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
      i32x4 ti = {(int)tw[0], (int)tw[1], (int)tw[2], (int)tw[3]};
      lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bi),
                                                   __builtin_bit_cast(bf16x8, ti), lo, 0, 0, 0);
    }
  }
  // lane holds m = m0 + r, n = n0 + 4g + i
  const int64_t m = m0 + r;
  if (m >= a.m) return;
  const float S = *a.tensor_scale;
  const int64_t nb = n0 + 4 * g;
  f32x4 acc = {0, 0, 0, 0};
  for (int s = 0; s < a.splits; ++s)
    acc += *(const f32x4*)(a.partials + ((int64_t)s * a.m + m) * a.rows_total + nb);
  float out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = S * acc[i] + lo[i];
  if (a.out_f32) {
    float* y = (float*)a.y + m * a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nb + i < a.n) y[nb + i] = out[i];
  } else {
    uint16_t* y = (uint16_t*)a.y + m * a.n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nb + i < a.n) y[nb + i] = (uint16_t)f32_to_bf16_rne(out[i]);
  }
}

hipError_t launch_skinny_reduce(const SkinnyPlan& p, int64_t m, int64_t n, const float* partials,
                                const float* tensor_scale, const uint16_t* lora_b, int32_t rank,
                                float lora_scale, void* y, int out_f32, hipStream_t s) {
  ReduceArgs a;
  a.m = m;
  a.n = n;
  a.splits = p.splits;
  a.rows_total = p.rows_total;
  a.rows_w_pad = p.rows_w_pad;
  a.partials = partials;
  a.tensor_scale = tensor_scale;
  a.lora_b = lora_b;
  a.rank = p.rows_l > 0 ? rank : 0;
  a.lora_scale = lora_scale;
  a.y = y;
  a.out_f32 = out_f32;
  dim3 grid((unsigned)cdiv(n, 16), (unsigned)cdiv(m, 64));
  skinny_reduce_kernel<<<grid, kSkThreads, 0, s>>>(a);
  return hipGetLastError();
}

// ------------------------------------------- LoRA intermediate for the GEMM paths

__global__ __launch_bounds__(kSkThreads) void lora_t_kernel(const float* __restrict__ partials,
                                                            int64_t m, int splits,
                                                            int64_t rows_total, int64_t row0,
                                                            int32_t rank, int32_t rank_pad,
                                                            float lora_scale, uint16_t* __restrict__ t) {
  const int64_t total = m * rank_pad;
  for (int64_t i = (int64_t)blockIdx.x * kSkThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kSkThreads) {
    const int64_t mm = i / rank_pad;
    const int j = (int)(i % rank_pad);
    float v = 0.0f;
    if (j < rank)
      for (int s = 0; s < splits; ++s) v += partials[((int64_t)s * m + mm) * rows_total + row0 + j];
    t[i] = (uint16_t)f32_to_bf16_rne(lora_scale * v);
  }
}

hipError_t launch_lora_t(const SkinnyPlan& p, int64_t m, const float* partials, int32_t rank,
                         float lora_scale, uint16_t* t, hipStream_t s) {
  const int32_t rank_pad = (int32_t)round_up(rank, 32);
  const int64_t total = m * rank_pad;
  const int grid = (int)min((int64_t)4096, cdiv(total, kSkThreads));
  lora_t_kernel<<<grid, kSkThreads, 0, s>>>(partials, m, p.splits, p.rows_total,
                                            p.rows_w_pad, rank, rank_pad, lora_scale, t);
  return hipGetLastError();
}

}  // namespace ql
