// Few-token NVFP4 layer for up to 32 tokens on gfx950, one launch per call:
//
//   y = S . x . (E2M1 * E4M3)^T  +  bf16(s . x A^T) . B^T
//
// This is the decoding case of QeRL's NVFP4 weight path (tldrocket.com QeRL page,
// paragraph after "Key Features of QeRL"): 0.5625 byte per weight streamed once, so the
// design minimises the latency chain of every workgroup.
//
// * A workgroup owns 16 weight rows; its four waves take interleaved 256-wide K chunks,
//   each lane reading row (l % 16) and the 64 consecutive K of lane group g = l / 16
//   (32 bytes of codes, 4 block scales) -- four chunks per wave are loaded before any
//   is used, and the next four while these are multiplied.
// * The activations of the workgroup's whole K range (at most 32 KB) are copied into LDS
//   once, while the first codes are in flight; they are the B operand of 16x16x32 bf16
//   MFMAs whose A operand is the codes dequantized in registers (E2M1 -> float by the
//   hardware converter, times the E4M3 block scale in float32: exact, at most 6
//   significant bits, hence an exact bf16).  The K order inside an MFMA is a permutation
//   shared by both operands.
// * The four waves' tiles are added in LDS.  K is split over several workgroups only when
//   there are too few row tiles to fill the chip; the partial tiles then go to the
//   workspace with device-scope stores, and the last arrival on the row tile's counter
//   loads all of them at once and adds them in split order.
// * LoRA: items that multiply 16 rows of A by up to eight K chunks are dispatched before
//   all weight items; each stores its partial of x A^T (device scope) and bumps a counter.
//   A row tile's finishing workgroup (its B rows were fetched at the start) waits for the
//   counter (bounded; the LoRA items were dispatched first, so they are running or done),
//   loads every partial at once, forms t = bf16(s . x A^T) in LDS in a fixed order, adds
//   t B^T with one MFMA per 32 ranks, applies S and stores y.  Counters are returned to
//   zero by the call that used them.
#include "../../include/qlinear.h"
#include "common.hpp"
#include "gemv_common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kG16Threads = 256;
constexpr int kG16Chunk = 256;
constexpr int kG16Batch = 4;          // chunks per wave loaded ahead
constexpr int kG16MaxSplits = 16;
constexpr int kG16XBytes = 32768;     // LDS for staged activations (5 workgroups per CU)

struct G16Args {
  const uint16_t* x;
  int64_t m, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* lora_a;
  const uint16_t* lora_b;
  int32_t rank;
  float lora_scale;
  int64_t n;
  void* y;
  int out_f32;
  int splits;
  int64_t cps;        // chunks per split
  int64_t kchunks;
  int64_t tiles_w;    // weight row tiles (16 rows)
  int64_t tiles_l;    // LoRA row tiles (16 rows of A)
  int64_t lgroups;    // LoRA chunk groups
  int lc;             // chunks per LoRA item (at most 8: two per wave)
  int rank_pad;       // t row length (multiple of 32)
  int64_t n_pad;      // row length of the weight partials
  int xstride;        // LDS row stride of the activations (elements)
  uint32_t* cnt_w;    // [tiles_w]
  uint32_t* cnt_l;    // [1]
  uint32_t* t_ready;  // [1]
  uint32_t* fin;      // [1]
  uint16_t* t;        // [m][rank_pad]
  float* part_w;      // [splits][m][n_pad]
  float* part_l;      // [lgroups][m][tiles_l * 16]
};

struct G16Chunk {
  uint4 c0, c1;
  uint32_t s;
};

template <bool ALIGNED>
__device__ __forceinline__ G16Chunk g16_load(const G16Args& a, int64_t row, bool ok, int64_t kl) {
  G16Chunk cr;
  const uint8_t* cp = a.codes + row * (a.k / 2) + kl / 2;
  const uint8_t* sp = a.scales + row * (a.k / 16) + kl / 16;
  if (ALIGNED) {  // K % 256 == 0: whole chunks, naturally aligned 16- and 4-byte loads
    cr.c0 = ok ? *(const uint4*)cp : make_uint4(0, 0, 0, 0);
    cr.c1 = ok ? *(const uint4*)(cp + 16) : make_uint4(0, 0, 0, 0);
    cr.s = ok ? *(const uint32_t*)sp : 0u;
  } else {        // K % 16 == 0: whole 16-element blocks, 8-byte code loads, byte scales
    uint32_t cw[8], sb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool bok = ok && kl + 16 * b < a.k;
      const uint2 v = bok ? *(const uint2*)(cp + 8 * b) : make_uint2(0, 0);
      cw[2 * b] = v.x;
      cw[2 * b + 1] = v.y;
      sb[b] = bok ? sp[b] : 0u;
    }
    cr.c0 = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    cr.c1 = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    cr.s = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
  }
  return cr;
}

// Copy x[0 .. mrows) x [c0*256, c1*256) into LDS (row stride xstride), zero past K.
__device__ __forceinline__ void g16_stage_x(const G16Args& a, uint16_t* xs, int mrows, int64_t c0,
                                            int64_t c1) {
  const int per_row = (int)(c1 - c0) * (kG16Chunk / 8);  // 16-byte units per row
  const int units = mrows * per_row;
  for (int u = threadIdx.x; u < units; u += kG16Threads) {
    const int i = u / per_row;
    const int col = (u - i * per_row) * 8;
    const int64_t k = c0 * kG16Chunk + col;
    // K % 16 == 0 and k % 8 == 0: a unit lies entirely inside or entirely past K
    const uint4 v = k < a.k ? *(const uint4*)(a.x + (int64_t)i * a.k + k) : make_uint4(0, 0, 0, 0);
    *(uint4*)(xs + i * a.xstride + col) = v;
  }
}

// B operand: 8 activations of token 16 q + r at LDS column `col`.
__device__ __forceinline__ bf16x8 g16_xfrag(const G16Args& a, const uint16_t* xs, int mrows, int q,
                                            int col) {
  const int r = threadIdx.x & 15;
  const int mi = 16 * q + r;
  if (mi >= mrows) return gv_zero8();
  return __builtin_bit_cast(bf16x8, *(const uint4*)(xs + mi * a.xstride + col));
}

template <int MT>
__device__ __forceinline__ void g16_mul_chunk(const G16Args& a, const uint16_t* xs, int mrows,
                                              int col0, const G16Chunk& cr, f32x4 (&acc)[MT]) {
  const int g = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t c = t == 0 ? cr.c0.x : t == 1 ? cr.c0.y : t == 2 ? cr.c0.z : t == 3 ? cr.c0.w :
                       t == 4 ? cr.c1.x : t == 5 ? cr.c1.y : t == 6 ? cr.c1.z : cr.c1.w;
    const bf16x8 av = gv_dequant8(c, e4m3_value((cr.s >> (8 * (t >> 1))) & 0xFFu));
#pragma unroll
    for (int q = 0; q < MT; ++q)
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, g16_xfrag(a, xs, mrows, q, col0 + 64 * g + 8 * t),
                                                       acc[q], 0, 0, 0);
  }
}

// Sum the four waves' tiles (fixed order) into wave 0.
template <int MT>
__device__ __forceinline__ void g16_reduce(f32x4 (&acc)[MT], f32x4* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < MT; ++q) red[((wave - 1) * MT + q) * kWave + lane] = acc[q];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < MT; ++q) {
      acc[q] += red[(0 * MT + q) * kWave + lane];
      acc[q] += red[(1 * MT + q) * kWave + lane];
      acc[q] += red[(2 * MT + q) * kWave + lane];
    }
  }
}

__device__ __forceinline__ bool g16_arrive(uint32_t* cnt, uint32_t total, int* flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == total - 1;
  }
  __syncthreads();
  return *flag != 0;
}

template <int MT, bool ALIGNED, bool MULTI>
__global__ __launch_bounds__(kG16Threads) void g16_kernel(G16Args a) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ f32x4 red[3 * MT * kWave];
  __shared__ int flag;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int mrows = (int)min((int64_t)16 * MT, a.m);
  const int64_t items_l = a.tiles_l * a.lgroups;
  int64_t id = blockIdx.x;
  f32x4 acc[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) acc[q] = f32x4{0, 0, 0, 0};

  if (id < items_l) {
    // ------------------------------------- LoRA item: 16 rows of A, lc chunks (2 per wave)
    const int64_t tile = id % a.tiles_l;
    const int64_t cg = id / a.tiles_l;
    const int64_t c0 = cg * a.lc, c1 = min(c0 + a.lc, a.kchunks);
    const int64_t row = tile * 16 + r;
    uint4 av[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t c = c0 + wave + 4 * i;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int64_t k = c * kG16Chunk + 64 * g + 8 * t;
        av[i][t] = (row < a.rank && c < c1 && k < a.k) ? *(const uint4*)(a.lora_a + row * a.k + k)
                                                      : make_uint4(0, 0, 0, 0);
      }
    }
    g16_stage_x(a, xs, mrows, c0, c1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t c = c0 + wave + 4 * i;
      if (c < c1) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int q = 0; q < MT; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av[i][t]),
                g16_xfrag(a, xs, mrows, q, (int)(c - c0) * kG16Chunk + 64 * g + 8 * t), acc[q], 0, 0, 0);
      }
    }
    g16_reduce<MT>(acc, red);
    const int64_t lrow = a.tiles_l * 16;
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mi = 16 * q + r;
        if (mi < a.m) st_dev4(a.part_l + (cg * a.m + mi) * lrow + tile * 16 + 4 * g, acc[q]);
      }
    }
    // announce the partial; the weight tiles add all partials themselves
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.cnt_l, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // -------------------------------------------------------------------- weight item
  id -= items_l;
  const int64_t tile = id % a.tiles_w;
  const int64_t split = id / a.tiles_w;
  const int64_t c0 = split * a.cps, c1 = min(c0 + a.cps, a.kchunks);
  const int64_t row = tile * 16 + r;
  const bool rv = row < a.n;

  // B rows of the LoRA up-projection do not depend on anything: fetch them first
  // (lane: row tile*16 + r, ranks 32 c + 8 g .. +8, the A-operand layout of the MFMA)
  constexpr int kMaxRankChunks = QLINEAR_MAX_RANK / 32;
  i32x4 bw[kMaxRankChunks];
  if (a.rank > 0) {
    const int rc = a.rank_pad / 32;
    const bool vec = (a.rank & 7) == 0;
#pragma unroll
    for (int c = 0; c < kMaxRankChunks; ++c) {
      uint32_t w4[4] = {0, 0, 0, 0};
      const int j0 = 32 * c + 8 * g;
      if (c < rc && rv) {
        if (vec) {
          if (j0 < a.rank) {
            const uint4 v = *(const uint4*)(a.lora_b + row * a.rank + j0);
            w4[0] = v.x; w4[1] = v.y; w4[2] = v.z; w4[3] = v.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t b0 = j0 + e < a.rank ? a.lora_b[row * a.rank + j0 + e] : 0u;
            const uint32_t b1 = j0 + e + 1 < a.rank ? a.lora_b[row * a.rank + j0 + e + 1] : 0u;
            w4[e / 2] = b0 | (b1 << 16);
          }
        }
      }
      bw[c] = i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
    }
  }

  G16Chunk ca[kG16Batch];
#pragma unroll
  for (int i = 0; i < kG16Batch; ++i) {
    const int64_t c = c0 + wave + 4 * i;
    ca[i] = g16_load<ALIGNED>(a, row, rv && c < c1, c * kG16Chunk + 64 * g);
  }
  g16_stage_x(a, xs, mrows, c0, c1);
  __syncthreads();
  if constexpr (!MULTI) {  // every wave has at most kG16Batch chunks
#pragma unroll
    for (int i = 0; i < kG16Batch; ++i) {
      const int64_t c = c0 + wave + 4 * i;
      if (c < c1) g16_mul_chunk<MT>(a, xs, mrows, (int)(c - c0) * kG16Chunk, ca[i], acc);
    }
  } else {
    G16Chunk cb[kG16Batch];
    for (int64_t b0 = c0 + wave;;) {
      // current batch in ca (chunks b0 + 4 i); prefetch the next into cb
      const int64_t b1 = b0 + 4 * kG16Batch;
      if (b1 < c1) {
#pragma unroll
        for (int i = 0; i < kG16Batch; ++i) {
          const int64_t c = b1 + 4 * i;
          cb[i] = g16_load<ALIGNED>(a, row, rv && c < c1, c * kG16Chunk + 64 * g);
        }
      }
#pragma unroll
      for (int i = 0; i < kG16Batch; ++i) {
        const int64_t c = b0 + 4 * i;
        if (c < c1) g16_mul_chunk<MT>(a, xs, mrows, (int)(c - c0) * kG16Chunk, ca[i], acc);
      }
      if (b1 >= c1) break;
      const int64_t b2 = b1 + 4 * kG16Batch;
      if (b2 < c1) {
#pragma unroll
        for (int i = 0; i < kG16Batch; ++i) {
          const int64_t c = b2 + 4 * i;
          ca[i] = g16_load<ALIGNED>(a, row, rv && c < c1, c * kG16Chunk + 64 * g);
        }
      }
#pragma unroll
      for (int i = 0; i < kG16Batch; ++i) {
        const int64_t c = b1 + 4 * i;
        if (c < c1) g16_mul_chunk<MT>(a, xs, mrows, (int)(c - c0) * kG16Chunk, cb[i], acc);
      }
      if (b2 >= c1) break;
      b0 = b2;
    }
  }
  g16_reduce<MT>(acc, red);

  if (a.splits > 1) {
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mi = 16 * q + r;
        if (mi < a.m) st_dev4(a.part_w + (split * a.m + mi) * a.n_pad + tile * 16 + 4 * g, acc[q]);
      }
    }
    if (!g16_arrive(a.cnt_w + tile, (uint32_t)a.splits, &flag)) return;
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mi = 16 * q + r;
        f32x4 part[kG16MaxSplits];
#pragma unroll
        for (int sp = 0; sp < kG16MaxSplits; ++sp)
          part[sp] = (sp < a.splits && mi < a.m)
                         ? ld_dev4(a.part_w + ((int64_t)sp * a.m + mi) * a.n_pad + tile * 16 + 4 * g)
                         : f32x4{0, 0, 0, 0};
        f32x4 s = part[0];
#pragma unroll
        for (int sp = 1; sp < kG16MaxSplits; ++sp) s += part[sp];
        acc[q] = s;
      }
      if (lane == 0) st_dev_u32(a.cnt_w + tile, 0u);
    }
  }
  // t = bf16(s . x A^T) from the LoRA partials, computed by the whole workgroup into LDS
  uint16_t* tl = xs;  // the staged activations are no longer needed
  if (a.rank > 0) {
    if (threadIdx.x == 0) {  // bounded wait until every LoRA item has announced its partial
      int it = 0;
      while (ld_dev_u32(a.cnt_l) < (uint32_t)items_l && ++it < kGvSpinLimit) __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
    const int64_t lrow = a.tiles_l * 16;
    const int E = mrows * a.rank_pad;
    for (int e = threadIdx.x; e < E; e += kG16Threads) {
      const int mi = e / a.rank_pad;
      const int j = e - mi * a.rank_pad;
      float v = 0.0f;
      if (j < a.rank) {
        const float* pp = a.part_l + (int64_t)mi * lrow + j;
        const int64_t stride = a.m * lrow;
        for (int64_t g0 = 0; g0 < a.lgroups; g0 += 16) {  // 16 loads in flight, summed in order
          float part[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) part[u] = g0 + u < a.lgroups ? ld_dev(pp + (g0 + u) * stride) : 0.0f;
#pragma unroll
          for (int u = 0; u < 16; ++u) v += part[u];
        }
      }
      tl[e] = (uint16_t)f32_to_bf16_rne(a.lora_scale * v);
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // wave 0 finishes the tile: acc[q] is C[n][m] with m = 16 q + r, n = tile*16 + 4 g + i
  const float S = *a.tensor_scale;
#pragma unroll
  for (int q = 0; q < MT; ++q) acc[q] *= S;
  if (a.rank > 0) {
    const int rc = a.rank_pad / 32;
#pragma unroll
    for (int c = 0; c < kMaxRankChunks; ++c) {
      if (c >= rc) break;
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int mi = 16 * q + r;
        const bf16x8 tv = mi < mrows ? __builtin_bit_cast(bf16x8, *(const uint4*)(tl + mi * a.rank_pad + 32 * c + 8 * g))
                                     : gv_zero8();
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw[c]), tv, acc[q], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    const int64_t mi = 16 * q + r;
    const int64_t nb = tile * 16 + 4 * g;
    if (mi >= a.m || nb >= a.n) continue;
    const f32x4 v = acc[q];
    if (a.out_f32) {
      float* y = (float*)a.y + mi * a.n;
      if (nb + 4 <= a.n && (a.n & 3) == 0) {
        *(f32x4*)(y + nb) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (nb + i < a.n) y[nb + i] = v[i];
      }
    } else {
      uint16_t* y = (uint16_t*)a.y + mi * a.n;
      const uint32_t b0 = f32_to_bf16_rne(v[0]), b1 = f32_to_bf16_rne(v[1]);
      const uint32_t b2 = f32_to_bf16_rne(v[2]), b3 = f32_to_bf16_rne(v[3]);
      if (nb + 4 <= a.n && (a.n & 3) == 0) {
        *(uint2*)(y + nb) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      } else {
        if (nb + 0 < a.n) y[nb + 0] = (uint16_t)b0;
        if (nb + 1 < a.n) y[nb + 1] = (uint16_t)b1;
        if (nb + 2 < a.n) y[nb + 2] = (uint16_t)b2;
        if (nb + 3 < a.n) y[nb + 3] = (uint16_t)b3;
      }
    }
  }
  if (a.rank > 0 && lane == 0) {  // this tile is done with the LoRA partials
    const uint32_t done = __hip_atomic_fetch_add(a.fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)a.tiles_w - 1) {  // every tile has read the LoRA partials
      st_dev_u32(a.cnt_l, 0u);
      st_dev_u32(a.fin, 0u);
    }
  }
}

// ------------------------------------------------------------------ planning

static int64_t g16_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t g16_align(size_t b) { return (b + 255) & ~(size_t)255; }

G16Plan plan_g16(int64_t m, int64_t n, int64_t k, int32_t rank) {
  G16Plan p;
  p.mt = m <= 16 ? 1 : 2;
  p.tiles_w = g16_cdiv(n, 16);
  p.kchunks = g16_cdiv(k, kG16Chunk);
  p.tiles_l = rank > 0 ? g16_cdiv(rank, 16) : 0;
  int64_t lc = ((int64_t)kG16XBytes / 2 / m - 8) / kG16Chunk;
  lc = lc < 1 ? 1 : (lc > 8 ? 8 : lc);
  p.lc = (int)lc;
  p.lgroups = rank > 0 ? g16_cdiv(p.kchunks, lc) : 0;
  p.rank_pad = rank > 0 ? (int)(g16_cdiv(rank, 32) * 32) : 0;
  const int64_t mrows = m;
  // largest K range whose activations fit the LDS budget
  int64_t cps_max = ((int64_t)kG16XBytes / 2 / mrows - 8) / kG16Chunk;
  if (cps_max < 1) cps_max = 1;
  int64_t splits = g16_cdiv(p.kchunks, cps_max);
  // fill the chip: with few row tiles, split K (at most 16 ways)
  while (p.tiles_w * splits < 512 && splits < kG16MaxSplits && splits < p.kchunks) ++splits;
  p.cps = g16_cdiv(p.kchunks, splits);
  p.splits = (int)g16_cdiv(p.kchunks, p.cps);
  p.n_pad = g16_cdiv(n, 16) * 16;
  const int64_t xcols = (p.cps > p.lc ? p.cps : p.lc) * kG16Chunk;
  p.xstride = (int)(xcols + 8);
  p.lds_bytes = (size_t)mrows * (size_t)p.xstride * 2;
  const size_t t_bytes = (size_t)m * (size_t)p.rank_pad * 2;   // t is formed in the same LDS
  if (p.lds_bytes < t_bytes) p.lds_bytes = t_bytes;
  return p;
}

size_t g16_workspace(const G16Plan& p, int64_t m) {
  const size_t counters = g16_align((size_t)(p.tiles_w + 3) * 4);
  const size_t t = g16_align((size_t)m * (size_t)p.rank_pad * 2);
  const size_t pw = p.splits > 1 ? g16_align((size_t)p.splits * (size_t)m * (size_t)p.n_pad * 4) : 0;
  const size_t pl = g16_align((size_t)p.lgroups * (size_t)m * (size_t)(p.tiles_l * 16) * 4);
  return counters + t + pw + pl;
}

hipError_t launch_g16(const G16Plan& p, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                      const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                      const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank,
                      float lora_scale, void* y, int out_f32, void* ws, hipStream_t s) {
  G16Args a = {};
  a.x = x;
  a.m = m;
  a.k = k;
  a.codes = codes;
  a.scales = scales;
  a.tensor_scale = tensor_scale;
  a.lora_a = lora_a;
  a.lora_b = lora_b;
  a.rank = p.tiles_l > 0 ? rank : 0;
  a.lora_scale = lora_scale;
  a.n = n;
  a.y = y;
  a.out_f32 = out_f32;
  a.splits = p.splits;
  a.cps = p.cps;
  a.kchunks = p.kchunks;
  a.tiles_w = p.tiles_w;
  a.tiles_l = p.tiles_l;
  a.lgroups = p.lgroups;
  a.lc = p.lc;
  a.rank_pad = p.rank_pad;
  a.n_pad = p.n_pad;
  a.xstride = p.xstride;
  char* w = (char*)ws;
  uint32_t* cnt = (uint32_t*)w;
  a.cnt_w = cnt;
  a.cnt_l = cnt + p.tiles_w;
  a.t_ready = a.cnt_l + 1;
  a.fin = a.t_ready + 1;
  size_t off = g16_align((size_t)(p.tiles_w + 3) * 4);
  a.t = (uint16_t*)(w + off);
  off += g16_align((size_t)m * (size_t)p.rank_pad * 2);
  a.part_w = (float*)(w + off);
  off += p.splits > 1 ? g16_align((size_t)p.splits * (size_t)m * (size_t)p.n_pad * 4) : 0;
  a.part_l = (float*)(w + off);
  const unsigned items = (unsigned)(p.tiles_l * p.lgroups + p.tiles_w * p.splits);
  const bool aligned = (k % kG16Chunk) == 0;
  hipError_t e;
  const bool multi = p.cps > 4 * kG16Batch;
#define QL_G16_LAUNCH(MT, AL, MU)                                                              \
  e = hipFuncSetAttribute((const void*)g16_kernel<MT, AL, MU>,                                 \
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds_bytes);       \
  if (e != hipSuccess) return e;                                                               \
  g16_kernel<MT, AL, MU><<<items, kG16Threads, p.lds_bytes, s>>>(a);
#define QL_G16_LAUNCH_M(MT, AL) if (multi) { QL_G16_LAUNCH(MT, AL, true) } else { QL_G16_LAUNCH(MT, AL, false) }
  if (p.mt == 1) {
    if (aligned) { QL_G16_LAUNCH_M(1, true) } else { QL_G16_LAUNCH_M(1, false) }
  } else {
    if (aligned) { QL_G16_LAUNCH_M(2, true) } else { QL_G16_LAUNCH_M(2, false) }
  }
#undef QL_G16_LAUNCH_M
#undef QL_G16_LAUNCH
  return hipGetLastError();
}

}  // namespace ql
