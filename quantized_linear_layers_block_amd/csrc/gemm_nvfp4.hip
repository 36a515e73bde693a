// NVFP4-weight layer for many tokens (rollout prefill) on gfx950:
//
//   y[m][n] = S * sum_k x[m][k] * E2M1(c[n][k]) * E4M3(e[n][k/16])  +  sum_j t[m][j] B[n][j]
//
// QeRL speeds up prefill as well as decoding with the NVFP4 weight path
// (tldrocket.com QeRL page, paragraph after "Key Features of QeRL").  NVFP4's
// E4M3-scaled 16-element blocks have no counterpart in gfx950's block-scaled MFMA
// (power-of-two scales per 32 elements), so weights are dequantized in registers and
// multiplied by 16x16x32 f16 MFMAs; S is applied in float32 after the K loop and the
// LoRA up-projection (t = s.x.A^T rounded to bf16, computed beforehand) is one more
// bf16 MFMA K chunk per 32 ranks.
//
// Exact f16 dequantization: every E2M1 x E4M3 product is an f16 (at most 5 significant
// bits, magnitude in [2^-10, 2688]).  The scaled fp4 conversion multiplies by the
// exponent of its float scale only, so the codes are converted with scale 2^8 and then
// multiplied (packed f16) by the E4M3 byte shifted left by 7, whose f16 reading is
// exactly scale * 2^-8.  Activations are brought to f16 by a pre-pass that scales each
// row by a power of two putting its largest magnitude in [2^14, 2^15): bf16's 8-bit
// significands fit, so the conversion is exact except for values below about 2^-29 of
// the row maximum, and the row factor is undone in float32 in the epilogue.
//
// Tiling (K % 64 == 0): 256 (n) x 256 (m) per workgroup of eight waves (4 along n x 2
// along m), 64 x 128 per wave (4 x 8 MFMA tiles), K stage 64.  Each stage (activations
// 32 KB, codes 8 KB, scales 1 KB) is copied straight into LDS: activations three stages
// deep, codes and scales six (they stream from HBM).  Other K take the generic kernel at
// the end of this file, which dequantizes into LDS as bf16.
#include "common.hpp"
#include "gemm_common.hpp"
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
__global__ __launch_bounds__(kNThreads, 1) void gemm_nvfp4_generic_kernel(Nvfp4GemmArgs a) {
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

// ------------------------------------------------------------ f16 path (K % 64 == 0)

constexpr int kQThreads = 512;
constexpr int kQTile = 256;
constexpr int kQK = 64;
constexpr int kQXSlots = 3;                  // activation ring: copies run 2 stages ahead
constexpr int kQCSlots = 6;                  // code/scale ring: copies run 5 stages ahead
constexpr int kQXBytes = kQTile * 128;       // activations: 256 rows x 64 f16
constexpr int kQCBytes = kQTile * 32;        // codes: 256 rows x 32 bytes
constexpr int kQSBytes = (kQTile + 32) * 4;  // scales: 256 rows x 4 bytes (+32 rows of overrun)
constexpr int kQCSBytes = kQCBytes + kQSBytes;
constexpr int kQRingBytes = kQXSlots * kQXBytes + kQCSlots * kQCSBytes;
constexpr int kQPitch = 144;                 // output staging row: 64 bf16 + 16 bytes
constexpr int kQStagePerWave = 128 * kQPitch;
constexpr size_t kQLds = kQRingBytes > 8 * kQStagePerWave ? kQRingBytes : 8 * kQStagePerWave;

// Up to kNvMaxSeg layers of one fused projection, as the GEMM and its tail see them.
struct NvSegs {
  int32_t nseg;                        // 1: a single layer
  int64_t tile[kNvMaxSeg + 1];         // first n tile of each layer; tile[nseg] = all n tiles
  const uint8_t* codes[kNvMaxSeg];
  const uint8_t* scales[kNvMaxSeg];
  const float* tensor_scale[kNvMaxSeg];
  const uint16_t* lora_b[kNvMaxSeg];
  void* y[kNvMaxSeg];
  int64_t n[kNvMaxSeg];
};

// Layer of n tile tn (the segments are few and their bounds uniform).
__device__ __forceinline__ int nv_seg_of(const NvSegs& sg, int64_t tn) {
  int s = 0;
  for (int i = 1; i < sg.nseg; ++i)
    if (tn >= sg.tile[i]) s = i;
  return s;
}

struct Nvfp4F16Args {
  const uint16_t* x16;  // f16 [m][k], row r scaled by 1 / rs[r]
  const float* rs;      // [m] row factors (powers of two)
  int64_t m, n, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* t;
  const uint16_t* lora_b;
  int32_t rank, rank_pad;
  void* y;
  int64_t tiles_m, tiles_n;
  int64_t full_tiles;  // workgroups that take whole tiles
  int32_t tail_split;  // K splits of each remaining tile
  float* part;         // [split workgroup][256 m][256 n] float32 partial tiles
  // Layers that share x (a fused projection): n tiles [seg.tile[s], seg.tile[s + 1]) are
  // those of layer s, with its own codes, scales, tensor scale, B, output and n (the
  // fields above are unused then), and its t columns at s * rank of rows t_stride long.
  NvSegs seg;
  int32_t t_stride;
};

// Activation pre-pass, in two kernels.
//
// nv_stats_kernel: workgroup (split, tile) covers rows 64 tile .. +64 (16 per wave) and
// k in [kchunk split, kchunk (split + 1)).  It streams the rows in MFMA operand layout
// (lane (r, g) holds row r, 8 consecutive k at 8 g of each 32-wide step), records each
// row's largest bf16 magnitude (bit pattern) in amax_part[split][row] and, with RT > 0,
// accumulates x A^T over RT 16-row tiles of A with bf16 MFMAs (A rows past the rank
// read as zero) into t_part[split][row][16 RT].  Workgroups of one split are adjacent
// so that they share the same range of A in L2.  k % 16 == 0; split boundaries are
// multiples of 32, and a last step that runs past k reads zeros for the 8-element units
// beyond it.
// The A matrices of up to kNvMaxSeg adapters stacked into one: stacked row j is row
// j - s seg_rank of adapter s, s = j / seg_rank (one adapter: seg_rank = its rank).
struct NvLoraA {
  const uint16_t* a[kNvMaxSeg];
  int32_t seg_rank;
};
__device__ __forceinline__ const uint16_t* nv_a_row(const NvLoraA& A, int j, int64_t k) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kNvMaxSeg; ++i)
    if (j >= i * A.seg_rank) s = i;
  const uint16_t* p = s == 0 ? A.a[0] : s == 1 ? A.a[1] : s == 2 ? A.a[2] : A.a[3];
  return p + (int64_t)(j - s * A.seg_rank) * k;
}

template <int RT, int MF>
__global__ __launch_bounds__(256) void nv_stats_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t k,
                                                       NvLoraA lora_a, int32_t rank,
                                                       int64_t tiles, int64_t kchunk,
                                                       uint32_t* __restrict__ amax_part,
                                                       float* __restrict__ t_part) {
  constexpr int RA = RT > 0 ? RT : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t split = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int64_t k0 = split * kchunk;
  const int64_t k1 = k0 + kchunk < k ? k0 + kchunk : k;
  int64_t row[MF];
  const uint16_t* xr[MF];
#pragma unroll
  for (int h = 0; h < MF; ++h) {
    row[h] = tile * (64 * MF) + 16 * (MF * wave + h) + r;
    xr[h] = x + (row[h] < m ? row[h] : m - 1) * k + 8 * g;
  }
  const uint16_t* ar[RA];
  bool aok[RA];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int j = 16 * i + r;
    aok[i] = j < rank;
    ar[i] = nv_a_row(lora_a, aok[i] ? j : 0, k) + 8 * g;
  }
  f32x4 acc[MF][RA];
  uint32_t mx[MF];
#pragma unroll
  for (int h = 0; h < MF; ++h) {
    mx[h] = 0;
#pragma unroll
    for (int i = 0; i < RT; ++i) acc[h][i] = f32x4{0, 0, 0, 0};
  }
  // one 32-wide step: each A fragment serves the MF row fragments of the wave
  auto use = [&](const i32x4 (&xv)[MF], const i32x4 (&av)[RA]) {
#pragma unroll
    for (int h = 0; h < MF; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = (uint32_t)xv[h][e];
        const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
        mx[h] = mx[h] > lo ? mx[h] : lo;
        mx[h] = mx[h] > hi ? mx[h] : hi;
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const i32x4 a = aok[i] ? av[i] : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < MF; ++h)
        acc[h][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, xv[h]), acc[h][i], 0, 0, 0);
    }
  };
  // four 32-wide steps per batch, all of their loads issued before any is used (used one by
  // one they would cost a memory round trip each)
  int64_t kk = k0;
  for (; kk + 128 <= k1; kk += 128) {
    i32x4 xq[4][MF], aq[4][RA];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int h = 0; h < MF; ++h) xq[u][h] = *(const i32x4*)(xr[h] + kk + 32 * u);
#pragma unroll
      for (int i = 0; i < RT; ++i) aq[u][i] = *(const i32x4*)(ar[i] + kk + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) use(xq[u], aq[u]);
  }
  for (; kk < k1; kk += 32) {
    const bool in = kk + 8 * g < k1;  // this lane's unit of 8 lies inside or past k1
    i32x4 xq[MF], aq[RA];
#pragma unroll
    for (int h = 0; h < MF; ++h) xq[h] = in ? *(const i32x4*)(xr[h] + kk) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < RT; ++i) aq[i] = in ? *(const i32x4*)(ar[i] + kk) : i32x4{0, 0, 0, 0};
    use(xq, aq);
  }
#pragma unroll
  for (int h = 0; h < MF; ++h) {
    uint32_t v = mx[h];
    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    if (row[h] < m) {
      if (g == 0) amax_part[split * m + row[h]] = v;
      // lane (r, g) of tile i holds rank 16 i + 4 g + (0..3) of row r
#pragma unroll
      for (int i = 0; i < RT; ++i)
        *(f32x4*)(t_part + (split * m + row[h]) * (16 * RT) + 16 * i + 4 * g) = acc[h][i];
    }
  }
}

// nv_stats_lds_kernel: nv_stats_kernel's outputs for m >= kNvStatsWideRows and an adapter
// (128 rows per workgroup, two row fragments per wave), with the operands staged through
// LDS.  Loaded straight into the MFMA operand layout, every instruction of nv_stats_kernel
// fetches 16 rows x 64 bytes -- half of each 128-byte line -- and every wave fetches the A
// slice on its own (at rank 64 twice the x bytes; 104 us for a 4096 x 27648 x).  Here
// (87 us there; without an adapter it gains nothing, so nv_stats_kernel stays for rank 0)
// each 128-column stage of the x tile (128 rows x 256
// B) and of A (16 RT rows) is copied into LDS by whole lines (one copy: 4 rows x 256 B),
// once per workgroup, and the fragments are read from LDS (16-byte unit u of row j at slot
// u ^ (j % 16): conflict-free).  Same split boundaries, same k order inside each 32-wide
// step, same fixed order of MFMA steps: amax_part and t_part equal nv_stats_kernel's (a
// zero sum may come out +0 where it gave -0: steps past the split add zero products).
// Columns past the split (the last stage may run past it) are zeroed in the fragments;
// rows past m and A rows past the rank read a valid row and are masked as in
// nv_stats_kernel.
template <int RT>
struct NvStatsLds {
  static constexpr int kRows = 128, kARows = 16 * RT;
  static constexpr int kStage = (kRows + kARows) * 256;
  static constexpr int kSlots = 3 * kStage <= 160 * 1024 ? 3 : 2;
  static constexpr int kXI = kRows / 16, kAI = kARows / 16;  // copies per wave per stage
  static constexpr size_t kLds = (size_t)kSlots * kStage;
};

template <int RT>
__global__ __launch_bounds__(256) void nv_stats_lds_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t k,
                                                           NvLoraA lora_a, int32_t rank,
                                                           int64_t tiles, int64_t kchunk,
                                                           uint32_t* __restrict__ amax_part,
                                                           float* __restrict__ t_part) {
  using P = NvStatsLds<RT>;
  constexpr int MF = 2, RA = RT > 0 ? RT : 1;
  constexpr int L = P::kSlots - 1;  // stages of copy lead
  constexpr int D = P::kXI + P::kAI;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int r = lane & 15, g = lane >> 4;
  const int64_t split = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int64_t k0 = split * kchunk;
  const int64_t k1 = k0 + kchunk < k ? k0 + kchunk : k;
  const int64_t nst = k1 > k0 ? (k1 - k0 + 127) / 128 : 0;
  const int64_t row0 = tile * P::kRows;
  // copy sources: x copy v of wave w covers tile rows 4 (w kXI + v) + lane / 16, A copy v
  // A rows 4 (w kAI + v) + lane / 16; physical unit lane % 16 holds logical unit
  // (lane % 16) ^ (row % 16)
  const uint16_t* xs[P::kXI];
  int xu[P::kXI];
#pragma unroll
  for (int v = 0; v < P::kXI; ++v) {
    const int row = 4 * (wave * P::kXI + v) + (lane >> 4);
    const int64_t gr = row0 + row < m ? row0 + row : m - 1;
    xs[v] = x + gr * k;
    xu[v] = (lane & 15) ^ (row & 15);
  }
  const uint16_t* as[P::kAI > 0 ? P::kAI : 1];
  int au[P::kAI > 0 ? P::kAI : 1];
#pragma unroll
  for (int v = 0; v < P::kAI; ++v) {
    const int row = 4 * (wave * P::kAI + v) + (lane >> 4);
    as[v] = nv_a_row(lora_a, row < rank ? row : 0, k);
    au[v] = (lane & 15) ^ (row & 15);
  }
  auto dma = [&](int64_t st, int slot) {
    const int64_t kb = k0 + st * 128;
    const uint32_t lb = lds_addr(smem) + slot * P::kStage;
#pragma unroll
    for (int v = 0; v < P::kXI; ++v) {
      const int64_t col = kb + 8 * xu[v] <= k - 8 ? kb + 8 * xu[v] : k - 8;
      lds_copy16_va(xs[v] + col, lb + 1024 * (wave * P::kXI + v));
    }
#pragma unroll
    for (int v = 0; v < P::kAI; ++v) {
      const int64_t col = kb + 8 * au[v] <= k - 8 ? kb + 8 * au[v] : k - 8;
      lds_copy16_va(as[v] + col, lb + P::kRows * 256 + 1024 * (wave * P::kAI + v));
    }
  };
  auto clamp_st = [&](int64_t st) { return st < nst ? st : nst - 1; };

  bool aok[RA];
#pragma unroll
  for (int i = 0; i < RA; ++i) aok[i] = 16 * i + r < rank;
  f32x4 acc[MF][RA];
  uint32_t mx[MF];
#pragma unroll
  for (int h = 0; h < MF; ++h) {
    mx[h] = 0;
#pragma unroll
    for (int i = 0; i < RT; ++i) acc[h][i] = f32x4{0, 0, 0, 0};
  }
  if (nst > 0) {
#pragma unroll
    for (int v = 0; v < L; ++v) dma(clamp_st(v), v);
  }
  for (int64_t st = 0; st < nst; ++st) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((L - 1) * D) : "memory");  // stage st has landed
    __syncthreads();  // ... for every wave, and every wave is done with stage st - 1's slot
    dma(clamp_st(st + L), (int)((st + L) % P::kSlots));
    const uint8_t* X = smem + (st % P::kSlots) * P::kStage;
    const uint8_t* A = X + P::kRows * 256;
    const int64_t kb = k0 + st * 128;
    const bool tail = kb + 128 > k1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int u = 4 * ks + g;
      const bool in = !tail || kb + 8 * u < k1;
      i32x4 xv[MF], av[RA];
#pragma unroll
      for (int h = 0; h < MF; ++h) {
        const int row = 16 * (MF * wave + h) + r;
        xv[h] = *(const i32x4*)(X + row * 256 + 16 * (u ^ (row & 15)));
        if (!in) xv[h] = i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int row = 16 * i + r;
        av[i] = *(const i32x4*)(A + row * 256 + 16 * (u ^ (row & 15)));
      }
#pragma unroll
      for (int h = 0; h < MF; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = (uint32_t)xv[h][e];
          const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
          mx[h] = mx[h] > lo ? mx[h] : lo;
          mx[h] = mx[h] > hi ? mx[h] : hi;
        }
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const i32x4 a = aok[i] ? av[i] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < MF; ++h)
          acc[h][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, xv[h]), acc[h][i], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped copies past the range too
#pragma unroll
  for (int h = 0; h < MF; ++h) {
    const int64_t row = row0 + 16 * (MF * wave + h) + r;
    uint32_t v = mx[h];
    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    if (row < m) {
      if (g == 0) amax_part[split * m + row] = v;
      // lane (r, g) of tile i holds rank 16 i + 4 g + (0..3) of row r
#pragma unroll
      for (int i = 0; i < RT; ++i)
        *(f32x4*)(t_part + (split * m + row) * (16 * RT) + 16 * i + 4 * g) = acc[h][i];
    }
  }
}

// nv_finish_kernel: one (row, chunk) unit per wave, chunk c covering the row's 16-byte
// units 256 c .. +256 (four per lane, so a K = 5120 row takes three waves).  Row maximum
// over the splits -> e putting it in [2^14, 2^15) (zero, Inf and NaN rows keep e = 0),
// the chunk as f16 scaled by 2^e; chunk 0 also writes rs[row] = 2^-e and t[row] =
// bf16(lora_scale * sum over splits of t_part) for ranks below `rank`, zero up to
// rank_pad.  The split maxima and the chunk are loaded together: one round trip to
// memory before the conversion instead of one per step of a whole row.
constexpr int64_t kNvChunk8 = 256;  // 16-byte units per wave

// bf16(s * sum over the K splits of t_part[split][row][j]) for j < rank, 0 up to rank_pad.
// Fixed order: eight interleaved partial sums (split sp goes to sum sp % 8), then those
// eight in order; the loads of one round are independent so they overlap.
__device__ __forceinline__ float lora_t_sum(const float* __restrict__ t_part, int64_t m, int64_t splits,
                                            int32_t rank_pad, int64_t row, int j) {
  float acc8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc8[u] += t_part[((sp + u) * m + row) * rank_pad + j];
  }
  for (int u = 0; sp < splits; ++sp, ++u) acc8[u] += t_part[(sp * m + row) * rank_pad + j];
  float sum = acc8[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) sum += acc8[u];
  return sum;
}
__device__ __forceinline__ uint16_t lora_t_value(const float* __restrict__ t_part, int64_t m, int64_t splits,
                                                 int32_t rank, int32_t rank_pad, float lora_scale, int64_t row,
                                                 int j) {
  return (uint16_t)(j < rank ? f32_to_bf16_rne(lora_scale * lora_t_sum(t_part, m, splits, rank_pad, row, j)) : 0u);
}
__global__ __launch_bounds__(256) void nv_finish_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t k,
                                                        int64_t splits, const uint32_t* __restrict__ amax_part,
                                                        const float* __restrict__ t_part, int32_t rank,
                                                        int32_t rank_pad, float lora_scale,
                                                        uint16_t* __restrict__ x16, float* __restrict__ rs,
                                                        uint16_t* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const int64_t n8 = k / 8;  // k % 64 == 0: a multiple of 8
  const int64_t chunks = (n8 + kNvChunk8 - 1) / kNvChunk8;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = unit / chunks, chunk = unit % chunks;
  if (row >= m) return;
  const uint4* src = (const uint4*)(x + row * k);
  uint4* dst = (uint4*)(x16 + row * k);
  const int64_t c0 = chunk * kNvChunk8 + lane;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t c = c0 + 64 * u;
    v[u] = c < n8 ? src[c] : make_uint4(0, 0, 0, 0);
  }
  uint32_t mx = 0;
  for (int64_t sp = lane; sp < splits; sp += 64) mx = max(mx, amax_part[sp * m + row]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  const int be = (int)(mx >> 7);  // bf16 biased exponent of the row maximum
  int e = (mx == 0 || be == 0xFF) ? 0 : 141 - (be > 0 ? be : 1);
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  const float up = __uint_as_float((uint32_t)(e + 127) << 23);
  auto conv = [&](const uint4 w4) {
    const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
    uint32_t o[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float a0 = __uint_as_float(w[e2] << 16) * up, a1 = __uint_as_float(w[e2] & 0xFFFF0000u) * up;
      o[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a0, a1}, f16x2));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t c = c0 + 64 * u;
    if (c < n8) dst[c] = conv(v[u]);
  }
  if (chunk != 0) return;
  if (lane == 0) rs[row] = __uint_as_float((uint32_t)(127 - e) << 23);
  for (int j = lane; j < rank_pad; j += 64) t[row * rank_pad + j] = lora_t_value(t_part, m, splits, rank, rank_pad, lora_scale, row, j);
}

// t[row][j] alone (the GEMM paths that take bf16 activations): one row per wave.
__global__ __launch_bounds__(256) void lora_t_finish_kernel(int64_t m, int64_t splits,
                                                            const float* __restrict__ t_part, int32_t rank,
                                                            int32_t rank_pad, float lora_scale,
                                                            uint16_t* __restrict__ t) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  for (int j = threadIdx.x & 63; j < rank_pad; j += 64)
    t[row * rank_pad + j] = lora_t_value(t_part, m, splits, rank, rank_pad, lora_scale, row, j);
}

// v = s * (fixed-order sum of the partials) as a bf16 pair hi = bf16(v), lo = bf16(v - hi)
// (v - hi is exact in float32): t_hl[row][j] = hi, t_hl[row][rank_pad + j] = lo, zero
// past rank.  hi + lo carries about 16 significant bits of v.
__global__ __launch_bounds__(256) void lora_t_hilo_kernel(int64_t m, int64_t splits,
                                                          const float* __restrict__ t_part, int32_t rank,
                                                          int32_t rank_pad, float lora_scale,
                                                          uint16_t* __restrict__ t_hl) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  for (int j = threadIdx.x & 63; j < rank_pad; j += 64) {
    uint32_t hi = 0, lo = 0;
    if (j < rank) {
      const float v = lora_scale * lora_t_sum(t_part, m, splits, rank_pad, row, j);
      hi = f32_to_bf16_rne(v);
      lo = f32_to_bf16_rne(v - __uint_as_float(hi << 16));
    }
    t_hl[row * 2 * rank_pad + j] = (uint16_t)hi;
    t_hl[row * 2 * rank_pad + rank_pad + j] = (uint16_t)lo;
  }
}

template <int OUT_F32>
__global__ __launch_bounds__(kQThreads) void gemm_nvfp4_f16_kernel(Nvfp4F16Args a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GemmWork work = gemm_schedule(a.tiles_m, a.tiles_n, a.full_tiles, a.tail_split);
  // the layer this n tile belongs to, and the tile's place in it
  const int sg = nv_seg_of(a.seg, work.tn);
  const int64_t N = a.seg.n[sg];
  const uint8_t* const codes = a.seg.codes[sg];
  const uint8_t* const scales = a.seg.scales[sg];
  const uint16_t* const lora_b = a.seg.lora_b[sg];
  void* const yout = a.seg.y[sg];
  const int64_t n0 = (work.tn - a.seg.tile[sg]) * kQTile, m0 = work.tm * kQTile;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int wn = wave & 3, wm = wave >> 2;  // wave tile: n 64 wn .. +64, m 128 wm .. +128
  const int r = lane & 15, g = lane >> 4;
  // K stages [st0, st1) of this workgroup (all of K for a whole tile)
  const int64_t kst_all = a.k / kQK;
  const int64_t kper = (kst_all + work.nsplit - 1) / work.nsplit;
  const int64_t st0 = work.split * kper;
  const int64_t st1 = st0 + kper < kst_all ? st0 + kper : kst_all;
  const int64_t n_last = N - 1 - n0, m_last = a.m - 1 - m0;

  // Copies of one stage, per wave: 4 x activations (8 rows of 128 bytes each, swizzled
  // 16-byte slots), 1 x codes (32 rows of 32 bytes), 1 x scales (64 rows of 4 bytes from
  // row 32 wave: neighbouring waves overlap by 32 rows with identical data, and the last
  // one runs 32 rows into the padding).
  // Rows past the matrix edge copy the last row; their outputs are never stored.
  uint32_t xo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (wave + 8 * q) + (lane >> 3);
    xo[q] = (uint32_t)((row < m_last ? row : m_last) * a.k * 2 + swz(row, lane & 7) * 16);
  }
  uint32_t co, so;
  {
    const int row = 32 * wave + (lane >> 1);
    co = (uint32_t)((row < n_last ? row : n_last) * (a.k / 2) + (lane & 1) * 16);
    const int srow = 32 * wave + lane;
    so = (uint32_t)((srow < n_last ? srow : n_last) * (a.k / 16));
  }
  const uint8_t* xb = (const uint8_t*)(a.x16 + m0 * a.k);
  const uint8_t* cb = codes + n0 * (a.k / 2);
  const uint8_t* sb = scales + n0 * (a.k / 16);
  // Copies of stage st into activation slot xb / code slot cb.  Activations are shared by
  // every workgroup of an m tile (mostly L2 hits); codes stream from HBM once per m tile,
  // so their ring is deeper.
  auto dma_x = [&](int64_t st, int slot) {
    const int64_t kk = st * kQK;
    const uint32_t lb = lds_addr(smem) + slot * kQXBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_copy16(xb + kk * 2, xo[q], lb + 8 * (wave + 8 * q) * 128);
  };
  auto dma_c = [&](int64_t st, int slot) {
    const int64_t kk = st * kQK;
    const uint32_t lb = lds_addr(smem) + kQXSlots * kQXBytes + slot * kQCSBytes;
    lds_copy16(cb + kk / 2, co, lb + wave * 1024);
    lds_copy4(sb + kk / 16, so, lb + kQCBytes + wave * 128);
  };
  auto clamp_st = [&](int64_t st) { return st < st1 ? st : st1 - 1; };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  // K assignment inside a stage: MFMA step h, lane group g takes the 8 k of chunk 2 g + h
  // (any assignment works as long as both operands use it).  A lane then reads activation
  // chunks 2 g and 2 g + 1 of its rows (the conflict-free fragment pattern), both steps'
  // codes as one 8-byte word at byte 8 g of the 32-byte code row, and one block scale
  // (block g) for both steps.
  //
  // Software pipeline.  The eight (step h, A fragment i) groups of a stage run their
  // eight MFMAs each while the weights of the next group are dequantized; the B fragments
  // of the second step are read during group 3.  The stage barrier sits before group 7:
  // by then every wave has read all it needs from the stage's buffer, so the buffer takes
  // the copies of stage st + 3 (two stages of lead), and group 7 overlaps the reads of
  // stage st + 1's codes, scales and first-step B fragments and the dequantization of its
  // first group.  Stage s lives in buffer (s - st0) % 3.
  uint32_t sbyte[4];
  uint2 cw[4];
  f16x8 bq[2][8];
  f16x8 af;
  auto read_stage_head = [&](int cslot) {
    const uint8_t* cs = smem + kQXSlots * kQXBytes + cslot * kQCSBytes;
    const uint8_t* ss = cs + kQCBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wn + 16 * i + r;
      sbyte[i] = (*(const uint32_t*)(ss + row * 4) >> (8 * g)) & 0xFFu;
      cw[i] = *(const uint2*)(cs + row * 32 + 8 * g);
    }
  };
  // Issue order: codes of stages 0..2, then per stage s (virtually from s = -3) the
  // activations of s + 3 and the codes of s + 6.  When stage st + 1 is needed (before
  // group 7 of stage st) the only copies issued after its activations are the codes of
  // st + 4 and the 6 copies of the last batch: vmcnt(8) leaves exactly those in flight.
  if (st1 > st0) {
    dma_c(st0, 0);
    dma_c(clamp_st(st0 + 1), 1);
    dma_c(clamp_st(st0 + 2), 2);
#pragma unroll
    for (int v = 0; v < 3; ++v) {
      dma_x(clamp_st(st0 + v), v);
      dma_c(clamp_st(st0 + 3 + v), 3 + v);
    }
    asm volatile("s_waitcnt vmcnt(14)" ::: "memory");  // stage st0 has landed
    __syncthreads();
    read_stage_head(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 128 * wm + 16 * j + r;
      bq[0][j] = *(const f16x8*)(smem + row * 128 + swz(row, 2 * g) * 16);
    }
    af = dequant8_f16(cw[0].x, sbyte[0]);
  }
  int xslot = 0, cslot = 0;
  for (int64_t st = st0; st < st1; ++st) {
    const int xn_slot = xslot == kQXSlots - 1 ? 0 : xslot + 1;  // slots of stage st + 1
    const int cn_slot = cslot == kQCSlots - 1 ? 0 : cslot + 1;
    const uint8_t* xs = smem + xslot * kQXBytes;
    const uint8_t* xn = smem + xn_slot * kQXBytes;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int h = q >> 2, i = q & 3;
      if (q == 7) {
        // stage st + 1 has landed; after the barrier no wave reads stage st's slots
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        __syncthreads();
        dma_x(clamp_st(st + 3), xslot);
        dma_c(clamp_st(st + 6), cslot);
        read_stage_head(cn_slot);
      }
      f16x8 an = af;
      if (q < 7) {
        const int h1 = (q + 1) >> 2, i1 = (q + 1) & 3;
        an = dequant8_f16(h1 ? cw[i1].y : cw[i1].x, sbyte[i1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bq[h][j], acc[i][j], 0, 0, 0);
        if (q == 3 || q == 7) {  // last use of fragment j of this step: fetch the next one
          __builtin_amdgcn_sched_barrier(0);
          const int row = 128 * wm + 16 * j + r;
          if (q == 3)
            bq[1][j] = *(const f16x8*)(xs + row * 128 + swz(row, 2 * g + 1) * 16);
          else
            bq[0][j] = *(const f16x8*)(xn + row * 128 + swz(row, 2 * g) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two vector ALU
        if (q == 3 || q == 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      if (q == 7) an = dequant8_f16(cw[0].x, sbyte[0]);  // next stage, group 0 (codes read at the barrier)
      __builtin_amdgcn_sched_barrier(0);
      af = an;
    }
    xslot = xn_slot;
    cslot = cn_slot;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: lane holds n = n0 + 64 wn + 16 i + 4 g + (0..3), m = m0 + 128 wm + 16 j + r.
  // The first 32 ranks' LoRA operands are loaded together with S and the row factors, so
  // that the epilogue waits for one memory round trip instead of two.
  const bool lora = a.rank_pad > 0 && work.split == 0;
  const uint16_t* const tl = a.t + (int64_t)sg * a.rank;
  const int64_t tstride = a.t_stride > 0 ? a.t_stride : a.rank_pad;
  i32x4 laf[4], lbf[8];
  if (lora) lora_frags<4, 8>(lora_b, tl, a.rank, N, a.m, n0 + 64 * wn, m0 + 128 * wm, r, g, tstride, 0, laf, lbf);
  const float S = *a.seg.tensor_scale[sg];
  float fac[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t mr = m0 + 128 * wm + 16 * j + r;
    fac[j] = S * a.rs[mr < a.m ? mr : a.m - 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] *= fac[j];
  if (lora) {
    lora_mfma<4, 8>(laf, lbf, acc);
    lora_wave<4, 8>(lora_b, tl, a.rank, a.rank_pad, N, a.m, n0 + 64 * wn, m0 + 128 * wm, r, g, acc, a.t_stride, 32);
  }
  if (work.slot >= 0) {
    // split tile: scaled float32 partial (LoRA in split 0), summed by nv_tail_reduce_kernel
    float* pt = a.part + work.slot * (kQTile * kQTile);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *(f32x4*)(pt + (128 * wm + 16 * j + r) * kQTile + 64 * wn + 16 * i + 4 * g) = acc[i][j];
    return;
  }
  if (!OUT_F32 && m0 + kQTile <= a.m && n0 + kQTile <= N && (N & 7) == 0) {
    // Interior bf16 tile: the wave's 128 (m) x 64 (n) block is transposed through LDS (row
    // pitch 144 bytes keeps the 8-byte writes conflict-free) and leaves as whole 128-byte
    // rows, eight rows per store instruction.
    __syncthreads();  // every wave is done with the operand buffers
    uint8_t* stage = smem + wave * kQStagePerWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = acc[i][j];
        *(uint2*)(stage + (16 * j + r) * kQPitch + (16 * i + 4 * g) * 2) =
            make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
    }
    uint16_t* ybase = (uint16_t*)yout + (m0 + 128 * wm) * N + n0 + 64 * wn + (lane & 7) * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * q + (lane >> 3);
      *(i32x4*)(ybase + row * N) = *(const i32x4*)(stage + row * kQPitch + (lane & 7) * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t mrow = m0 + 128 * wm + 16 * j + r;
        if (mrow < a.m) store4(yout, OUT_F32, N, mrow, n0 + 64 * wn + 16 * i + 4 * g, acc[i][j], N);
      }
    }
  }
}

// Sum of the split partials of the tail tiles (fixed order), stored like the GEMM's
// epilogue.  Workgroup: 4 rows of one tail tile, 4 consecutive n per thread.
__global__ __launch_bounds__(256) void nv_tail_reduce_kernel(const float* __restrict__ part, int64_t tiles_m,
                                                             int64_t tiles_n, int64_t full, int32_t splits,
                                                             int64_t m, NvSegs seg, int out_f32) {
  const int64_t tail = blockIdx.x / 64;
  const int row = (int)(blockIdx.x % 64) * 4 + (int)(threadIdx.x >> 6);
  const int col = (int)(threadIdx.x & 63) * 4;
  int64_t tm, tn;
  gemm_group_tile(full + tail, tiles_m, tiles_n, tm, tn);
  const int64_t mr = tm * kQTile + row;
  if (mr >= m) return;
  const int sg = nv_seg_of(seg, tn);
  const int64_t n = seg.n[sg], c = (tn - seg.tile[sg]) * kQTile + col;
  const float* p = part + tail * splits * (kQTile * kQTile) + row * kQTile + col;
  f32x4 v = *(const f32x4*)p;
  for (int sp = 1; sp < splits; ++sp) v += *(const f32x4*)(p + sp * (kQTile * kQTile));
  if (c < n) store4(seg.y[sg], out_f32, n, mr, c, v, n);
}

// ------------------------------------------------------------ transposed product (backward)
//
//   dX[m][k] = S rs[m] sum_n dY16[m][n] E2M1(c[n][k]) E4M3(e[n][k/16])  +  sum_q du[m][q] A[q][k]
//
// The gradient of the activations reduces over the weight rows n, so the weights enter
// transposed: an MFMA A fragment needs 8 consecutive n at one k, across 8 rows of the
// packed codes.  Each stage's codes and scales (64 rows of n x 256 columns of k) are copied
// into LDS, dequantized to f16 exactly as in the forward (dequant8_f16) and written back to
// LDS in their own row-major layout, 16 bytes per write; the fragments are then read with
// gfx950's transposing LDS read ds_read_b64_tr_b16.  Within each 16-lane group that read
// takes 4 consecutive 16-bit elements from the address of every lane and hands element c
// of lane 4 e + b to lane 4 b + c, as element e (lane layout checked on the device); so
// lanes 4 e + b naming k 4 b .. 4 b + 3 of W row n0 + e leave lane j holding W[n0 .. n0 + 3]
// at column j.  dY, the B operand, comes as f16 rows scaled by powers of two (rs, the
// forward's activation pre-pass, exact but for values below about 2^-29 of the row
// maximum) and is copied into LDS exactly like the forward's activations.  S rs[m] is
// applied in float32 after the n loop; du . A (bf16(du), A^T zero-padded to rank_pad) is
// one more bf16 MFMA chunk per 32 ranks.
//
// Tiling: 256 (k) x 256 (m) per workgroup of eight waves (4 along k x 2 along m), 64 x 128
// per wave, stages of 64 n.  LDS: dY two stages (copies one stage ahead), dequantized W
// two stages (the next stage's is written while this one's is multiplied), codes and
// scales three stages (copies two stages ahead).  Tiles and the split tail are those of
// the forward (nv_tile_plan over (m, k) with stages along n, nv_tail_reduce_kernel).
constexpr int kDThreads = 512;
constexpr int kDN = 64;                         // n per stage
constexpr int kDXBytes = kQTile * 128;          // dY16: 256 rows (m) x 64 f16
constexpr int kDWBytes = kDN * 512;             // W: 64 rows (n) x 256 f16 (k)
constexpr int kDCBytes = kDN * 128;             // codes: 64 rows x 128 bytes
constexpr int kDCSBytes = kDCBytes + kDN * 16;  // + scales: 64 rows x 16 bytes
constexpr int kDXSlots = 2, kDCSlots = 3;
constexpr int kDWOff = kDXSlots * kDXBytes;
constexpr int kDCOff = kDWOff + 2 * kDWBytes;
constexpr size_t kDLds = (size_t)kDCOff + kDCSlots * kDCSBytes;
static_assert(kDLds >= 8 * kQStagePerWave, "the output staging fits in the operand buffers");

// 16-byte slot of logical slot s (k 8 s .. 8 s + 7) in W row n (32 slots of 512 bytes).
// A transposing fragment read (fixed s pair, 2 lanes per slot) covers rows 16 g + 8 h + 4 q
// + (0..3): over a half wave the slots' bits 1..3 take (n & 3) | (bit 4 of n) << 2, eight
// distinct values.  A dequantized write (16 lanes: rows 2 p, 2 p + 1 x units u = 0..7 at
// slot 4 u + v) differs in bit 0 between u < 4 and u >= 4 (from slot bit 4) and in bit 1
// between the two rows.  So both touch 16 distinct bank groups per 256 bytes.
__device__ __forceinline__ int wslot(int n, int s) { return s ^ ((s >> 4) & 1) ^ (2 * ((n & 3) | ((n >> 2) & 4))); }


struct Nvfp4DxArgs {
  const uint16_t* dy16;  // f16 [m][n], row r scaled by 1 / rs[r]
  const float* rs;       // [m] row factors (powers of two)
  int64_t m, n, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* at;    // A^T [k][rank_pad] bf16, zero past the rank
  const uint16_t* du;    // [m][du_stride] bf16: bf16(du) in columns [0, rank_pad), zero past the rank
  int32_t rank_pad;      // 0: no adapter
  int64_t du_stride;
  void* dx;
  int64_t tiles_m, tiles_n;
  int64_t full_tiles;
  int32_t tail_split;
  float* part;           // [split workgroup][256 m][256 k] float32 partial tiles
};

template <int OUT_F32>
__global__ __launch_bounds__(kDThreads) void gemm_nvfp4_dx_kernel(Nvfp4DxArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const GemmWork work = gemm_schedule(a.tiles_m, a.tiles_n, a.full_tiles, a.tail_split);
  const int64_t k0 = work.tn * kQTile, m0 = work.tm * kQTile;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int wk = wave & 3, wm = wave >> 2;  // wave tile: k 64 wk .. +64, m 128 wm .. +128
  const int r = lane & 15, g = lane >> 4;
  // n stages [st0, st1) of this workgroup (all of n for a whole tile)
  const int64_t nst_all = a.n / kDN;
  const int64_t per = (nst_all + work.nsplit - 1) / work.nsplit;
  const int64_t st0 = work.split * per;
  const int64_t st1 = st0 + per < nst_all ? st0 + per : nst_all;
  const int64_t m_last = a.m - 1 - m0;
  const int64_t k_room = a.k - k0;  // at least 128 (k % 128 == 0)

  // Copies of one stage, per wave: 4 x dY16 (8 rows of 128 bytes each, swizzled 16-byte
  // slots; rows past the edge copy the last row), 1 x codes (rows 8 wave .. +8 of the stage,
  // 16 bytes = 32 k per lane), 1 x scales (rows 16 (wave % 4) .. +16, 4 bytes = 64 k per
  // lane; waves 4..7 repeat the copies of 0..3, so that every wave issues the same number
  // of copies).  Columns past k re-read the last full unit; their outputs are never stored.
  uint32_t xo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (wave + 8 * q) + (lane >> 3);
    xo[q] = (uint32_t)((row < m_last ? row : m_last) * a.n * 2 + swz(row, lane & 7) * 16);
  }
  uint32_t co, so;
  {
    const int64_t kc = 32 * (lane & 7) < k_room - 32 ? 32 * (lane & 7) : k_room - 32;
    co = (uint32_t)((8 * wave + (lane >> 3)) * (a.k / 2) + kc / 2);
    const int64_t ks = 64 * (lane & 3) < k_room - 64 ? 64 * (lane & 3) : k_room - 64;
    so = (uint32_t)((16 * (wave & 3) + (lane >> 2)) * (a.k / 16) + ks / 16);
  }
  const uint8_t* xb = (const uint8_t*)(a.dy16 + m0 * a.n);
  const uint8_t* cb = a.codes + k0 / 2;
  const uint8_t* sb = a.scales + k0 / 16;
  auto dma_x = [&](int64_t st, int slot) {
    const uint32_t lb = lds_addr(smem) + slot * kDXBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_copy16(xb + st * (kDN * 2), xo[q], lb + 8 * (wave + 8 * q) * 128);
  };
  auto dma_c = [&](int64_t st, int slot) {
    const uint32_t lb = lds_addr(smem) + kDCOff + slot * kDCSBytes;
    lds_copy16(cb + st * kDN * (a.k / 2), co, lb + wave * 1024);
    lds_copy4(sb + st * kDN * (a.k / 16), so, lb + kDCBytes + (wave & 3) * 256);
  };
  auto clamp_st = [&](int64_t st) { return st < st1 ? st : st1 - 1; };

  // Dequantization: thread (wave, lane) takes W row 8 wave + lane / 8 of the stage, k 32 u
  // .. +32 (u = lane % 8): the 16 code bytes its own lane copied and the two block scales.
  const int wr = 8 * wave + (lane >> 3), wu = lane & 7;
  auto dequant = [&](int cslot, int wbuf) {
    const uint8_t* cs = smem + kDCOff + cslot * kDCSBytes;
    const uint4 c = *(const uint4*)(cs + wr * 128 + 16 * wu);
    const uint32_t sc = *(const uint16_t*)(cs + kDCBytes + wr * 16 + 2 * wu);
    uint8_t* row = smem + kDWOff + wbuf * kDWBytes + wr * 512;
    *(f16x8*)(row + wslot(wr, 4 * wu + 0) * 16) = dequant8_f16(c.x, sc & 0xFFu);
    *(f16x8*)(row + wslot(wr, 4 * wu + 1) * 16) = dequant8_f16(c.y, sc & 0xFFu);
    *(f16x8*)(row + wslot(wr, 4 * wu + 2) * 16) = dequant8_f16(c.z, sc >> 8);
    *(f16x8*)(row + wslot(wr, 4 * wu + 3) * 16) = dequant8_f16(c.w, sc >> 8);
  };

  // Fragments of MFMA step h (n 16 g + 8 h .. +8 for lane group g, on both operands):
  // A (tile i: k 64 wk + 16 i + r) from two transposing reads of W rows 16 g + 8 h + 4 q +
  // r / 4 at k 64 wk + 16 i + 4 (r % 4); B (tile j: m 128 wm + 16 j + r) as in the forward.
  const int tre = r >> 2, trb = r & 3;
  auto read_a = [&](int wbuf, int h, int i) {
    const uint8_t* wb = smem + kDWOff + wbuf * kDWBytes;
    const int s = 8 * wk + 2 * i + (trb >> 1);
    i16x4 p[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = 16 * g + 8 * h + 4 * q + tre;
      p[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(wb + n * 512 + wslot(n, s) * 16 + (trb & 1) * 8));
    }
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_b = [&](int xslot, int h, int j) {
    const int row = 128 * wm + 16 * j + r;
    return *(const f16x8*)(smem + xslot * kDXBytes + row * 128 + swz(row, 2 * g + h) * 16);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  // Stage s (relative to st0) uses dY slot s % 2, W buffer s % 2 and, for the next stage's
  // dequantization, code slot (s + 1) % 3.  Issue order: codes 0, 1, dY 0, codes 2; then
  // (after W 0 is written) dY 1, codes 3; and after the barrier inside stage s, dY s + 2
  // and codes s + 4.  At that barrier vmcnt(2) leaves only codes s + 3 in flight: dY s + 1
  // and codes s + 2 have landed.
  //
  // Software pipeline.  A stage is two MFMA steps of four groups (one A fragment i x the
  // eight B fragments).  Each A fragment is refetched for the next step right after its
  // group, each B fragment after its last use in group 3, so the reads overlap the MFMAs
  // of the following groups.  Step 0 also reads the next stage's codes and writes its
  // dequantized weights.  The barrier sits between the steps: every wave has then read
  // all of stage s, so its dY slot and code slot take new copies, and the next stage's W
  // is complete, so step 1's refetches read stage s + 1's step 0.
  f16x8 af[4], bq[8];
  if (st1 > st0) {
    dma_c(st0, 0);
    dma_c(clamp_st(st0 + 1), 1);
    dma_x(st0, 0);
    dma_c(clamp_st(st0 + 2), 2);
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    __syncthreads();
    dequant(0, 0);
    __syncthreads();  // W 0 complete; code slot 0 free
    dma_x(clamp_st(st0 + 1), 1);
    dma_c(clamp_st(st0 + 3), 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = read_a(0, 0, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = read_b(0, 0, j);
  }
  for (int64_t st = st0; st < st1; ++st) {
    const int ls = (int)(st - st0);
    const int cur = ls & 1, nxt = cur ^ 1;
    const int cn = (ls + 1) % kDCSlots;
    // step 0, with the next stage's dequantization (its codes and scales read first)
    const uint8_t* cs = smem + kDCOff + cn * kDCSBytes;
    const uint4 cw = *(const uint4*)(cs + wr * 128 + 16 * wu);
    const uint32_t sc = *(const uint16_t*)(cs + kDCBytes + wr * 16 + 2 * wu);
    uint8_t* wrow = smem + kDWOff + nxt * kDWBytes + wr * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bq[j], acc[i][j], 0, 0, 0);
        if (i == 3) {
          __builtin_amdgcn_sched_barrier(0);
          bq[j] = read_b(cur, 1, j);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      af[i] = read_a(cur, 1, i);
      if (i == 1) {
        *(f16x8*)(wrow + wslot(wr, 4 * wu + 0) * 16) = dequant8_f16(cw.x, sc & 0xFFu);
        *(f16x8*)(wrow + wslot(wr, 4 * wu + 1) * 16) = dequant8_f16(cw.y, sc & 0xFFu);
      } else if (i == 2) {
        *(f16x8*)(wrow + wslot(wr, 4 * wu + 2) * 16) = dequant8_f16(cw.z, sc >> 8);
        *(f16x8*)(wrow + wslot(wr, 4 * wu + 3) * 16) = dequant8_f16(cw.w, sc >> 8);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    __syncthreads();
    dma_x(clamp_st(st + 2), cur);
    dma_c(clamp_st(st + 4), cn);
    __builtin_amdgcn_sched_barrier(0);
    // step 1, refetching step 0 of the next stage (unused after the last stage)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bq[j], acc[i][j], 0, 0, 0);
        if (i == 3) {
          __builtin_amdgcn_sched_barrier(0);
          bq[j] = read_b(nxt, 0, j);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      af[i] = read_a(nxt, 0, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: lane holds k = k0 + 64 wk + 16 i + 4 g + (0..3), m = m0 + 128 wm + 16 j + r.
  const float S = *a.tensor_scale;
  float fac[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t mr = m0 + 128 * wm + 16 * j + r;
    fac[j] = S * a.rs[mr < a.m ? mr : a.m - 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] *= fac[j];
  if (a.rank_pad > 0 && work.split == 0)
    lora_wave<4, 8>(a.at, a.du, a.rank_pad, a.rank_pad, a.k, a.m, k0 + 64 * wk, m0 + 128 * wm, r, g, acc,
                    a.du_stride);
  if (work.slot >= 0) {
    float* pt = a.part + work.slot * (kQTile * kQTile);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *(f32x4*)(pt + (128 * wm + 16 * j + r) * kQTile + 64 * wk + 16 * i + 4 * g) = acc[i][j];
    return;
  }
  if (!OUT_F32 && m0 + kQTile <= a.m && k0 + kQTile <= a.k) {
    // Interior bf16 tile, staged through LDS as in the forward: whole 128-byte rows out.
    __syncthreads();
    uint8_t* stage = smem + wave * kQStagePerWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = acc[i][j];
        *(uint2*)(stage + (16 * j + r) * kQPitch + (16 * i + 4 * g) * 2) =
            make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
    }
    uint16_t* ybase = (uint16_t*)a.dx + (m0 + 128 * wm) * a.k + k0 + 64 * wk + (lane & 7) * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * q + (lane >> 3);
      *(i32x4*)(ybase + row * a.k) = *(const i32x4*)(stage + row * kQPitch + (lane & 7) * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t mrow = m0 + 128 * wm + 16 * j + r;
        const int64_t kk = k0 + 64 * wk + 16 * i + 4 * g;
        if (mrow < a.m && kk < a.k) store4(a.dx, OUT_F32, a.k, mrow, kk, acc[i][j], a.k);
      }
    }
  }
}

namespace {
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
int32_t nv_rank_pad(int32_t rank) { return rank > 0 ? (rank + 31) / 32 * 32 : 0; }

// Pre-pass splits along K: about four (tile, split) workgroups per compute unit, so that
// enough loads are in flight, with at least 256 k per split.
constexpr int64_t kNvStatsWideRows = 1024;  // from this many rows on, two row fragments per wave
int64_t nv_prep_splits(int64_t m, int64_t k) {
  const int64_t tiles = (m + 63) / 64;
  int64_t sp = (1024 + tiles - 1) / tiles;
  // Splits of at least 256 columns; with at most four row tiles (up to 256 tokens) and
  // K <= 5120, of 128: at 256 tokens the 256-column floor left 80 workgroups for K = 5120
  // (the stacked q/k/v adapters' pass 14.4 -> 9.1 us, gate/up 8.0 -> 5.6 at 128).  Larger K
  // keeps 256: nv_finish_kernel adds every split's partials (K = 27648 at 216 splits: 13.0
  // -> 17.4 us), and at K = 8192, 40 uneven splits were slower than 32 even ones.
  const int64_t s128 = tiles <= 4 && k / 128 <= 40 ? k / 128 : 0;
  const int64_t smax = k / 256 > s128 ? k / 256 : (s128 > 0 ? s128 : 1);
  return sp < 1 ? 1 : (sp > smax ? smax : sp);
}

// Whole-tile rounds on kQPlanCUs compute units, then the leftover tiles split along K
// so that the last round fills the chip (only when at most half a round is left).
constexpr int64_t kQPlanCUs = 256;
struct NvTilePlan {
  int64_t tiles_m, tiles_n, full;
  int32_t split;
  int64_t tail() const { return tiles_m * tiles_n - full; }
};
NvTilePlan nv_tile_plan(int64_t m, int64_t n, int64_t k) {
  NvTilePlan p;
  p.tiles_m = (m + kQTile - 1) / kQTile;
  p.tiles_n = (n + kQTile - 1) / kQTile;
  const int64_t tiles = p.tiles_m * p.tiles_n;
  const int64_t rem = tiles % kQPlanCUs;
  int64_t sp = rem > 0 && rem <= kQPlanCUs / 2 ? kQPlanCUs / rem : 1;
  const int64_t kst = k / kQK;
  if (sp > 16) sp = 16;
  if (sp > kst) sp = kst;
  p.split = (int32_t)(sp > 1 ? sp : 1);
  p.full = p.split > 1 ? tiles - rem : tiles;
  return p;
}

struct NvPrepWs {
  uint16_t* x16;
  float* rs;
  uint16_t* t;
  uint32_t* amax_part;
  float* t_part;
  float* tile_part;
  size_t bytes;
};

// Row statistics and LoRA partials (nv_stats_kernel) over nv_prep_splits(m, k) K splits;
// rank: rows of the stacked A.
hipError_t launch_nv_stats(const uint16_t* x, int64_t m, int64_t k, const NvLoraA& lora_a, int32_t rank,
                           uint32_t* amax_part, float* t_part, hipStream_t s) {
  const int32_t rank_pad = nv_rank_pad(rank);
  // Large m: 128 rows per workgroup, so each load of A serves two row fragments (the split
  // count, and with it the workspace, is that of 64-row tiles either way).
  const int mf = m >= kNvStatsWideRows ? 2 : 1;
  const int64_t tiles = (m + 64 * mf - 1) / (64 * mf), sp = nv_prep_splits(m, k);
  const int64_t kchunk = ((k + sp - 1) / sp + 31) / 32 * 32;
  const unsigned sgrid = (unsigned)(tiles * sp);
#define QL_NV_STATS(RT_)                                                                               \
  case RT_ / 16:                                                                                      \
    if (mf == 2 && RT_ > 0) {                                                                         \
      const size_t lds = NvStatsLds<RT_ / 16>::kLds;                                                  \
      hipError_t e = hipFuncSetAttribute((const void*)nv_stats_lds_kernel<RT_ / 16>,                 \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);      \
      if (e != hipSuccess) return e;                                                                  \
      nv_stats_lds_kernel<RT_ / 16><<<sgrid, 256, lds, s>>>(x, m, k, lora_a, rank, tiles, kchunk, amax_part, t_part); \
    } else if (mf == 2) {                                                                             \
      nv_stats_kernel<RT_ / 16, 2><<<sgrid, 256, 0, s>>>(x, m, k, lora_a, rank, tiles, kchunk, amax_part, t_part); \
    } else {                                                                                          \
      nv_stats_kernel<RT_ / 16, 1><<<sgrid, 256, 0, s>>>(x, m, k, lora_a, rank, tiles, kchunk, amax_part, t_part); \
    }                                                                                                 \
    break;
  switch (rank_pad / 16) {
    QL_NV_STATS(0)
    QL_NV_STATS(32)
    QL_NV_STATS(64)
    QL_NV_STATS(96)
    QL_NV_STATS(128)
#undef QL_NV_STATS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_nv_stats(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a, int32_t rank,
                           uint32_t* amax_part, float* t_part, hipStream_t s) {
  NvLoraA A = {};
  A.a[0] = lora_a;
  A.seg_rank = rank > 0 ? rank : 1;
  return launch_nv_stats(x, m, k, A, rank, amax_part, t_part, s);
}

NvPrepWs nv_prep_ws(void* ws, int64_t m, int64_t n, int64_t k, int32_t rank) {
  const int64_t sp = nv_prep_splits(m, k);
  const size_t rp = (size_t)nv_rank_pad(rank);
  const NvTilePlan tp = nv_tile_plan(m, n, k);
  NvPrepWs w;
  char* p = (char*)ws;
  size_t off = 0;
  w.x16 = (uint16_t*)(p + off);
  off += up256((size_t)m * (size_t)k * 2);
  w.rs = (float*)(p + off);
  off += up256((size_t)m * 4);
  w.t = (uint16_t*)(p + off);
  off += up256((size_t)m * rp * 2);
  w.amax_part = (uint32_t*)(p + off);
  off += up256((size_t)sp * (size_t)m * 4);
  w.t_part = (float*)(p + off);
  off += up256((size_t)sp * (size_t)m * rp * 4);
  w.tile_part = (float*)(p + off);
  if (tp.split > 1) off += (size_t)tp.tail() * (size_t)tp.split * kQTile * kQTile * 4;
  w.bytes = off;
  return w;
}

// LoRA down-projection scratch: split maxima (unused here), split partials, t.
struct LoraDownWs {
  uint32_t* amax_part;
  float* t_part;
  uint16_t* t;
  size_t bytes;
};
LoraDownWs lora_down_ws(void* scratch, int64_t m, int64_t k, int32_t rank) {
  const int64_t sp = nv_prep_splits(m, k);
  const size_t rp = (size_t)nv_rank_pad(rank);
  char* p = (char*)scratch;
  LoraDownWs w;
  size_t off = 0;
  w.t = (uint16_t*)(p + off);
  off += up256((size_t)m * rp * 2);
  w.amax_part = (uint32_t*)(p + off);
  off += up256((size_t)sp * (size_t)m * 4);
  w.t_part = (float*)(p + off);
  off += up256((size_t)sp * (size_t)m * rp * 4);
  w.bytes = off;
  return w;
}
}  // namespace

size_t lora_down_bytes(int64_t m, int64_t k, int32_t rank) {
  if (m <= 0 || k <= 0 || rank <= 0) return 0;
  return lora_down_ws(nullptr, m, k, rank).bytes;
}

hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a,
                            int32_t rank, float lora_scale, void* scratch, uint16_t** t_out,
                            hipStream_t s) {
  if (m <= 0 || k <= 0 || k % 16 != 0 || rank <= 0 || rank > 128 || !scratch) return hipErrorInvalidValue;
  const LoraDownWs w = lora_down_ws(scratch, m, k, rank);
  hipError_t e = launch_nv_stats(x, m, k, lora_a, rank, w.amax_part, w.t_part, s);
  if (e != hipSuccess) return e;
  lora_t_finish_kernel<<<(unsigned)((m + 3) / 4), 256, 0, s>>>(m, nv_prep_splits(m, k), w.t_part, rank,
                                                               nv_rank_pad(rank), lora_scale, w.t);
  *t_out = w.t;
  return hipGetLastError();
}

size_t lora_down_hilo_bytes(int64_t m, int64_t k, int32_t rank) {
  if (m <= 0 || k <= 0 || rank <= 0) return 0;
  return lora_down_ws(nullptr, m, k, rank).bytes + up256((size_t)m * (size_t)nv_rank_pad(rank) * 4);
}

hipError_t launch_lora_down_hilo(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a,
                                 int32_t rank, float lora_scale, void* scratch, uint16_t** t_hl_out,
                                 hipStream_t s) {
  if (m <= 0 || k <= 0 || k % 16 != 0 || rank <= 0 || rank > 128 || !scratch) return hipErrorInvalidValue;
  const LoraDownWs w = lora_down_ws(scratch, m, k, rank);
  uint16_t* t_hl = (uint16_t*)((char*)scratch + w.bytes);
  hipError_t e = launch_nv_stats(x, m, k, lora_a, rank, w.amax_part, w.t_part, s);
  if (e != hipSuccess) return e;
  lora_t_hilo_kernel<<<(unsigned)((m + 3) / 4), 256, 0, s>>>(m, nv_prep_splits(m, k), w.t_part, rank,
                                                             nv_rank_pad(rank), lora_scale, t_hl);
  *t_hl_out = t_hl;
  return hipGetLastError();
}

size_t gemm_nvfp4_f16_workspace(int64_t m, int64_t n, int64_t k, int32_t rank) {
  if (m <= 0 || n <= 0 || k <= 0 || k % kQK != 0) return 0;
  return nv_prep_ws(nullptr, m, n, k, rank).bytes;
}

// n of the tile plan of layers sharing x: each layer's n rounded up to whole tiles.
static int64_t nv_layers_n(const int64_t* n, int nl) {
  int64_t t = 0;
  for (int i = 0; i < nl; ++i) t += (n[i] + kQTile - 1) / kQTile;
  return t * kQTile;
}

size_t gemm_nvfp4_f16_layers_workspace(int64_t m, int64_t k, const int64_t* n, int nl, int32_t rank) {
  if (nl < 1 || nl > kNvMaxSeg) return 0;
  return gemm_nvfp4_f16_workspace(m, nv_layers_n(n, nl), k, nl * rank);
}

hipError_t launch_gemm_nvfp4_f16_layers(const uint16_t* x, int64_t m, int64_t k, const NvLayer* layers, int nl,
                                        int32_t rank, float lora_scale, int out_f32, void* ws, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  // Copy offsets are 32-bit within a 256-row tile.  Several layers stack their adapters'
  // ranks (each a multiple of 32, so every layer's t columns start on a 64-byte boundary).
  if (k % kQK != 0 || k >= kNvF16MaxK || !ws || rank < 0 || nl < 1 || nl > kNvMaxSeg ||
      nl * rank > 128 || (nl > 1 && rank % 32 != 0))
    return hipErrorInvalidValue;
  int64_t ns[kNvMaxSeg];
  for (int i = 0; i < nl; ++i) {
    if (layers[i].n <= 0) return hipErrorInvalidValue;
    ns[i] = layers[i].n;
  }
  const int32_t rank_all = nl * rank;
  const int32_t rank_pad = nv_rank_pad(rank_all);
  const int64_t n_all = nv_layers_n(ns, nl);
  const NvPrepWs w = nv_prep_ws(ws, m, n_all, k, rank_all);
  const int64_t sp = nv_prep_splits(m, k);
  NvLoraA A = {};
  for (int i = 0; i < nl; ++i) A.a[i] = layers[i].lora_a;
  A.seg_rank = rank > 0 ? rank : 1;
  hipError_t e0 = launch_nv_stats(x, m, k, A, rank_all, w.amax_part, w.t_part, s);
  if (e0 != hipSuccess) return e0;
  const int64_t fin_units = m * ((k / 8 + kNvChunk8 - 1) / kNvChunk8);
  nv_finish_kernel<<<(unsigned)((fin_units + 3) / 4), 256, 0, s>>>(x, m, k, sp, w.amax_part, w.t_part, rank_all,
                                                                    rank_pad, lora_scale, w.x16, w.rs, w.t);
  Nvfp4F16Args a = {};
  a.x16 = w.x16;
  a.rs = w.rs;
  a.m = m;
  a.n = n_all;
  a.k = k;
  a.t = rank > 0 ? w.t : nullptr;
  a.rank = rank;
  // one layer: its t rows are rank_pad long; several: layer i's ranks at i * rank
  a.rank_pad = rank > 0 ? (nl > 1 ? rank : rank_pad) : 0;
  a.t_stride = rank_pad;
  a.seg.nseg = nl;
  int64_t tile = 0;
  for (int i = 0; i < nl; ++i) {
    a.seg.tile[i] = tile;
    tile += (layers[i].n + kQTile - 1) / kQTile;
    a.seg.codes[i] = layers[i].codes;
    a.seg.scales[i] = layers[i].scales;
    a.seg.tensor_scale[i] = layers[i].tensor_scale;
    a.seg.lora_b[i] = layers[i].lora_b;
    a.seg.y[i] = layers[i].y;
    a.seg.n[i] = layers[i].n;
  }
  a.seg.tile[nl] = tile;
  const NvTilePlan tp = nv_tile_plan(m, n_all, k);
  a.tiles_m = tp.tiles_m;
  a.tiles_n = tp.tiles_n;
  a.full_tiles = tp.full;
  a.tail_split = tp.split;
  a.part = w.tile_part;
  const unsigned grid = (unsigned)(tp.full + (tp.split > 1 ? tp.tail() * tp.split : 0));
  if (out_f32) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_f16_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQLds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_f16_kernel<1><<<grid, kQThreads, kQLds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_f16_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQLds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_f16_kernel<0><<<grid, kQThreads, kQLds, s>>>(a);
  }
  if (tp.split > 1)
    nv_tail_reduce_kernel<<<(unsigned)(tp.tail() * 64), 256, 0, s>>>(w.tile_part, tp.tiles_m, tp.tiles_n, tp.full,
                                                                    tp.split, m, a.seg, out_f32);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4_f16(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales,
                                 const float* tensor_scale, const uint16_t* lora_a,
                                 const uint16_t* lora_b, int32_t rank, float lora_scale, void* y,
                                 int out_f32, void* ws, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  if (rank > 128) return hipErrorInvalidValue;
  NvLayer l;
  l.codes = codes;
  l.scales = scales;
  l.tensor_scale = tensor_scale;
  l.lora_a = lora_a;
  l.lora_b = lora_b;
  l.y = y;
  l.n = n;
  return launch_gemm_nvfp4_f16_layers(x, m, k, &l, 1, rank, lora_scale, out_f32, ws, s);
}

hipError_t launch_gemm_nvfp4(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const uint16_t* t, const uint16_t* lora_b, int32_t rank, void* y,
                             int out_f32, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  const int32_t rk = t ? rank : 0;
  const int32_t rk_pad = t ? (rank + 31) / 32 * 32 : 0;
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
  a.rank = rk;
  a.rank_pad = rk_pad;
  a.y = y;
  a.tiles_m = (m + kNTile - 1) / kNTile;
  a.tiles_n = (n + kNTile - 1) / kNTile;
  const size_t lds = 4 * kNTile * kNRowBytes;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (out_f32) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_generic_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_generic_kernel<1><<<grid, kNThreads, lds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_generic_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_generic_kernel<0><<<grid, kNThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

// ---- f16 rows with the adapter's down-projection as hi | lo pairs (backward pre-pass)
namespace {
struct F16RowsWs {
  uint16_t* x16;
  float* rs;
  uint16_t* t_hl;
  uint32_t* amax_part;
  float* t_part;
  size_t bytes;
};
F16RowsWs f16_rows_ws(void* scratch, int64_t m, int64_t k, int32_t rank) {
  const int64_t sp = nv_prep_splits(m, k);
  const size_t rp = (size_t)nv_rank_pad(rank);
  char* p = (char*)scratch;
  F16RowsWs w;
  size_t off = 0;
  w.x16 = (uint16_t*)(p + off);
  off += up256((size_t)m * (size_t)k * 2);
  w.rs = (float*)(p + off);
  off += up256((size_t)m * 4);
  w.t_hl = (uint16_t*)(p + off);
  off += up256((size_t)m * rp * 4);
  w.amax_part = (uint32_t*)(p + off);
  off += up256((size_t)sp * (size_t)m * 4);
  w.t_part = (float*)(p + off);
  off += up256((size_t)sp * (size_t)m * rp * 4);
  w.bytes = off;
  return w;
}
}  // namespace

size_t f16_rows_bytes(int64_t m, int64_t k, int32_t rank) { return f16_rows_ws(nullptr, m, k, rank).bytes; }

hipError_t launch_f16_rows(const uint16_t* x, int64_t m, int64_t k, const uint16_t* lora_a, int32_t rank,
                           float lora_scale, void* scratch, uint16_t** x16, float** rs, uint16_t** t_hl,
                           hipStream_t s) {
  if (m <= 0 || k % kQK != 0 || k >= kNvF16MaxK || rank < 0 || rank > 128 || !scratch) return hipErrorInvalidValue;
  const F16RowsWs w = f16_rows_ws(scratch, m, k, rank);
  const int64_t sp = nv_prep_splits(m, k);
  hipError_t e = launch_nv_stats(x, m, k, rank > 0 ? lora_a : nullptr, rank, w.amax_part, w.t_part, s);
  if (e != hipSuccess) return e;
  if (rank > 0)
    lora_t_hilo_kernel<<<(unsigned)((m + 3) / 4), 256, 0, s>>>(m, sp, w.t_part, rank, nv_rank_pad(rank), lora_scale,
                                                               w.t_hl);
  const int64_t fin_units = m * ((k / 8 + kNvChunk8 - 1) / kNvChunk8);
  nv_finish_kernel<<<(unsigned)((fin_units + 3) / 4), 256, 0, s>>>(x, m, k, sp, w.amax_part, w.t_part, 0, 0, 0.0f,
                                                                    w.x16, w.rs, nullptr);
  *x16 = w.x16;
  *rs = w.rs;
  *t_hl = rank > 0 ? w.t_hl : nullptr;
  return hipGetLastError();
}

// ---- dX = S rs dY16 W (+ bf16(du) A) of the backward
size_t nvfp4_dx_part_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0) return 0;
  const NvTilePlan tp = nv_tile_plan(m, k, n);
  return tp.split > 1 ? (size_t)tp.tail() * (size_t)tp.split * kQTile * kQTile * 4 : 0;
}

hipError_t launch_nvfp4_dx(const uint16_t* dy16, const float* rs, int64_t m, int64_t n, int64_t k,
                           const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                           const uint16_t* at, const uint16_t* du, int32_t rank_pad, int64_t du_stride, void* dx,
                           int out_f32, float* part, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  if (n % kDN != 0 || n >= kNvF16MaxK || k % 128 != 0 || k >= kNvDxMaxK || rank_pad < 0 || rank_pad % 32 != 0)
    return hipErrorInvalidValue;
  Nvfp4DxArgs a;
  a.dy16 = dy16;
  a.rs = rs;
  a.m = m;
  a.n = n;
  a.k = k;
  a.codes = codes;
  a.scales = scales;
  a.tensor_scale = tensor_scale;
  a.at = at;
  a.du = du;
  a.rank_pad = rank_pad;
  a.du_stride = du_stride;
  a.dx = dx;
  const NvTilePlan tp = nv_tile_plan(m, k, n);
  a.tiles_m = tp.tiles_m;
  a.tiles_n = tp.tiles_n;
  a.full_tiles = tp.full;
  a.tail_split = tp.split;
  a.part = part;
  const unsigned grid = (unsigned)(tp.full + (tp.split > 1 ? tp.tail() * tp.split : 0));
  if (out_f32) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_dx_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDLds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_dx_kernel<1><<<grid, kDThreads, kDLds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_nvfp4_dx_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDLds);
    if (e != hipSuccess) return e;
    gemm_nvfp4_dx_kernel<0><<<grid, kDThreads, kDLds, s>>>(a);
  }
  if (tp.split > 1) {
    NvSegs one = {};
    one.nseg = 1;
    one.tile[1] = tp.tiles_n;
    one.y[0] = dx;
    one.n[0] = k;
    nv_tail_reduce_kernel<<<(unsigned)(tp.tail() * 64), 256, 0, s>>>(part, tp.tiles_m, tp.tiles_n, tp.full, tp.split,
                                                                    m, one, out_f32);
  }
  return hipGetLastError();
}

}  // namespace ql
