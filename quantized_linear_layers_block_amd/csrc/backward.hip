// Backward pass of the NVFP4 + LoRA layer on gfx950, for LoRA training on top of the frozen
// 4-bit base (QeRL keeps backprop stable through LoRA with its gradients in higher
// precision: tldrocket.com QeRL page, "Key Features of QeRL" and the paragraph after it;
// Jet-RL keeps the backward in BF16: rapidrecap.app Jet-RL summary, "Key Points"):
//
//   dX = S . dY . (E2M1 * E4M3)  +  du . A        du = s . dY . B          [M, K]
//   dA = du^T . x                                                          [r, K] float32
//   dB = dY^T . t                                 t  = s . x . A^T         [N, r] float32
//
// du and t come from the forward's LoRA down-projection (du from a transposed copy of B) in
// float32, each carried as a pair of bf16 values hi = bf16(v), lo = bf16(v - hi) (about 16
// significant bits).  The adapter gradients use both (their sums over tokens keep the
// precision the pages ask for); dX, an activation gradient like the forward's output, uses
// du rounded to bf16 as the forward uses t.
//
// dX normally takes the transposed f16 product of gemm_nvfp4.hip (dY as row-scaled f16,
// the weights dequantized into LDS and read with the transposing LDS read), its pre-pass
// also forming du.  Kernels here:
//
// * bwd_dx_kernel: the generic transposed product, for weights too wide for that path's
//   32-bit copy offsets.  Each stage's code tile (64 rows of N x 128 columns of K) is
//   dequantized in registers -- E2M1 by the hardware converter, times the E4M3 block
//   scale, an exact bf16 -- and written to LDS transposed (K-major), where it is the A
//   operand of 16x16x32 bf16 MFMAs; the dY tile (128 tokens x 64) is the B operand.
//   Workgroup tile 128 (K) x 128 (M), four waves of 64 x 64, stages of 64 along N with the
//   next stage's loads in flight during the MFMAs.  S is applied in float32, then
//   bf16(du) . A is added as r_pad / 32 more MFMA steps.
// * bwd_tn_kernel: G[c][j] = sum over a range of tokens of P[m][c] Q[m][j] (P = dY, Q = the
//   hi | lo columns of t for dB; P = x, Q = those of du for dA): P's token-major tiles are
//   copied into LDS and read as MFMA fragments with the transposing LDS read, Q^T (small)
//   is transposed once (bwd_transpose2d_kernel); bf16 MFMAs into float32, the token range
//   split over workgroups, and bwd_reduce_kernel adds, in a fixed order, the split
//   partials of the hi columns, those of the lo columns, and the two sums.
// * bwd_transpose_kernel: B [N, r] -> B^T [r, N] for the down-projection of dY.
#include "../../include/qlinear.h"
#include "common.hpp"
#include "gemm_common.hpp"
#include "launch.hpp"

namespace ql {

// ------------------------------------------------------------------ dX
constexpr int kBxTK = 128, kBxTM = 128, kBxTN = 64;

struct BwdDxArgs {
  const uint16_t* dy;  // [m][n] bf16
  int64_t m, n, k;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  const uint16_t* du;      // [m][2 rank_pad] bf16, hi columns first (zero past rank), or null
  const uint16_t* lora_a;  // [rank][k] bf16
  int32_t rank, rank_pad;
  void* dx;
  int out_f32;
};

// LDS tiles, 128-byte rows of 64 bf16 in 16-byte slots swizzled by swz(): dY [128 m][64 n]
// and the dequantized weights transposed, W^T [128 k][64 n].  A fragment read has 16 lanes
// reading slot 2 g + h of 16 consecutive rows (conflict-free with this swizzle).
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdDxArgs a) {
  __shared__ __align__(16) uint16_t ys[kBxTM * kBxTN];
  __shared__ __align__(16) uint16_t wt[kBxTK * kBxTN];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int wk = wave & 1, wm = wave >> 1;  // wave tile: k 64 wk .. +64, m 64 wm .. +64
  const int64_t k0 = (int64_t)blockIdx.x * kBxTK, m0 = (int64_t)blockIdx.y * kBxTM;

  // Loads of one stage.  dY: units u = tid + 256 j, token row u / 8, 8-column slot u % 8
  // (rows past M read zero).  Codes: rows 2 p and 2 p + 1 of the stage (p = tid / 8), 16
  // columns of K from 16 (tid % 8) (8 bytes each), and the one block scale of each.
  uint4 yv[4];
  uint2 c0, c1;
  uint32_t s0, s1;
  const int pr = tid >> 3, kq = tid & 7;
  auto issue = [&](int64_t n0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = tid + 256 * j;
      const int64_t mr = m0 + (u >> 3);
      const bool ok = mr < a.m;
      const uint4 v = *(const uint4*)(a.dy + (ok ? mr : 0) * a.n + n0 + 8 * (u & 7));
      const uint32_t mk = ok ? 0xFFFFFFFFu : 0u;
      yv[j] = make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
    }
    const int64_t n_a = n0 + 2 * pr;
    c0 = *(const uint2*)(a.codes + n_a * (a.k / 2) + k0 / 2 + 8 * kq);
    c1 = *(const uint2*)(a.codes + (n_a + 1) * (a.k / 2) + k0 / 2 + 8 * kq);
    s0 = a.scales[n_a * (a.k / 16) + k0 / 16 + kq];
    s1 = a.scales[(n_a + 1) * (a.k / 16) + k0 / 16 + kq];
  };
  // Stage to LDS: dY as loaded; the weights dequantized (exact bf16: at most 6 significant
  // bits) and stored as pairs (n = 2 p, 2 p + 1) at W^T[16 kq + e][2 p .. 2 p + 1].
  auto store = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = tid + 256 * j;
      const int row = u >> 3;
      *(uint4*)(ys + row * kBxTN + swz(row, u & 7) * 8) = yv[j];
    }
    const float sc0 = e4m3_value(s0), sc1 = e4m3_value(s1);
    const uint32_t w0[2] = {c0.x, c0.y}, w1[2] = {c1.x, c1.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 u0[4] = {e2m1_unpack2<0>(w0[h]), e2m1_unpack2<1>(w0[h]), e2m1_unpack2<2>(w0[h]),
                           e2m1_unpack2<3>(w0[h])};
      const f32x2 u1[4] = {e2m1_unpack2<0>(w1[h]), e2m1_unpack2<1>(w1[h]), e2m1_unpack2<2>(w1[h]),
                           e2m1_unpack2<3>(w1[h])};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x2 v0 = u0[b], v1 = u1[b];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kl = 16 * kq + 8 * h + 2 * b + e;
          const uint32_t lo = __float_as_uint(v0[e] * sc0) >> 16, hi = __float_as_uint(v1[e] * sc1) & 0xFFFF0000u;
          *(uint32_t*)(wt + kl * kBxTN + swz(kl, pr >> 2) * 8 + 2 * (pr & 3)) = lo | hi;
        }
      }
    }
  };

  f32x4 acc[4][4];  // [k tile i][m tile j]: lane (r, g) holds k = 16 i + 4 g + e, m = 16 j + r
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  issue(0);
  for (int64_t n0 = 0; n0 < a.n; n0 += kBxTN) {
    __syncthreads();  // every wave is done reading the previous stage
    store();
    __syncthreads();
    if (n0 + kBxTN < a.n) issue(n0 + kBxTN);  // in flight during the MFMAs
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 af[4], bq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = 64 * wk + 16 * i + r;
        af[i] = *(const bf16x8*)(wt + kl * kBxTN + swz(kl, 2 * g + h) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = 64 * wm + 16 * j + r;
        bq[j] = *(const bf16x8*)(ys + ml * kBxTN + swz(ml, 2 * g + h) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bq[j], acc[i][j], 0, 0, 0);
    }
  }

  const float S = *a.tensor_scale;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] *= S;
  // du . A: A operand A^T[k][q] (rows q past the rank read zero), B operand du[m][q]
  for (int q0 = 0; q0 < a.rank_pad; q0 += 32) {
    const int q = q0 + 8 * g;
    bf16x8 af[4], bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kk = k0 + 64 * wk + 16 * i + r;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t lo = q + e < a.rank ? a.lora_a[(int64_t)(q + e) * a.k + kk] : 0u;
        const uint32_t hi = q + e + 1 < a.rank ? a.lora_a[(int64_t)(q + e + 1) * a.k + kk] : 0u;
        w[e / 2] = lo | (hi << 16);
      }
      af[i] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t mr = m0 + 64 * wm + 16 * j + r;
      const uint4 v = *(const uint4*)(a.du + (mr < a.m ? mr : 0) * 2 * a.rank_pad + q);
      bq[j] = __builtin_bit_cast(bf16x8, mr < a.m ? v : make_uint4(0, 0, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bq[j], acc[i][j], 0, 0, 0);
  }
  // store: four consecutive k of one token per lane and tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t mr = m0 + 64 * wm + 16 * j + r;
    if (mr >= a.m) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kk = k0 + 64 * wk + 16 * i + 4 * g;
      const f32x4 v = acc[i][j];
      if (a.out_f32) {
        *(f32x4*)((float*)a.dx + mr * a.k + kk) = v;
      } else {
        *(uint2*)((uint16_t*)a.dx + mr * a.k + kk) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
    }
  }
}

// ------------------------------------------------------------------ adapter gradients
// The token reductions G[c][j] = sum_m P[m][c] Q[m][j] (dB: P = dY, Q = t; dA: P = x,
// Q = du, each Q as its hi | lo columns) have the reduction index in the rows of both
// operands.  P, large, is read in its own token-major layout: each stage's tile (32 tokens
// x 256 columns) is copied into LDS and the MFMA A fragments (16 columns x 8 tokens per
// lane group) are taken with the transposing LDS read, as in the dX product.  Q, small,
// is transposed once into the workspace (bwd_transpose2d_kernel: Q^T [qcp][ld], the token
// count padded to ld, a multiple of 32, with zeros) and its stage tile copied into LDS
// beside P's; the B fragments are then plain 16-byte LDS reads.
constexpr int kTr = 64;

// dst[c][r] = src[r][c] for r < rows, c < cols; zero for rows <= r < rows_pad or
// cols <= c < cols_pad.  64 x 64 tiles through LDS; cols and src_ld multiples of 8.
__global__ __launch_bounds__(256) void bwd_transpose2d_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                              int64_t cols, int64_t src_ld, int64_t rows_pad,
                                                              int64_t cols_pad, uint16_t* __restrict__ dst) {
  __shared__ uint32_t tile[kTr][kTr / 2 + 1];  // row r: elements 2 i, 2 i + 1 in word i
  const int64_t c0 = (int64_t)blockIdx.x * kTr, r0 = (int64_t)blockIdx.y * kTr;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = tid + 256 * j;
    const int rl = u >> 3, cq = u & 7;
    const int64_t rr = r0 + rl, cc = c0 + 8 * cq;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < rows && cc < cols) v = *(const uint4*)(src + rr * src_ld + cc);
    tile[rl][4 * cq] = v.x;
    tile[rl][4 * cq + 1] = v.y;
    tile[rl][4 * cq + 2] = v.z;
    tile[rl][4 * cq + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = tid + 256 * j;
    const int cl = u >> 3, rq = u & 7;
    const int64_t cc = c0 + cl, rr = r0 + 8 * rq;
    if (cc >= cols_pad || rr >= rows_pad) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (tile[8 * rq + 2 * e][cl >> 1] >> (16 * (cl & 1))) & 0xFFFFu;
      const uint32_t hi = (tile[8 * rq + 2 * e + 1][cl >> 1] >> (16 * (cl & 1))) & 0xFFFFu;
      w[e] = lo | (hi << 16);
    }
    *(uint4*)(dst + cc * rows_pad + rr) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

constexpr int kTnM = 32;                               // tokens per stage
constexpr int kTnC = 256;                              // columns c per workgroup (4 waves x 64)
constexpr int kTnJ = 64;                               // columns j per workgroup
constexpr int kTnPBytes = kTnM * kTnC * 2;             // P: 32 rows (tokens) of 512 bytes
constexpr int kTnQBytes = kTnJ * kTnM * 2;             // Q^T: 64 rows (j) of 64 bytes
constexpr int kTnStage = kTnPBytes + kTnQBytes;
constexpr int kTnSlots = 4;                            // copies run three stages ahead
constexpr size_t kTnLds = (size_t)kTnSlots * kTnStage;

// 16-byte slot of logical slot s (c 8 s .. 8 s + 7) in token row m of a P tile (32 slots): a
// fragment read takes one slot pair of rows 8 g + 4 q + (0..3); over a half wave (g = 0, 1)
// the slots' bits 1..3 take (m & 3) | (bit 3 of m) << 2, eight distinct values.
__device__ __forceinline__ int tn_pslot(int m, int s) { return s ^ (2 * ((m & 3) | ((m >> 1) & 4))); }
// 16-byte slot of logical slot s (tokens 8 s .. 8 s + 7) in row j of a Q^T tile (4 slots):
// the 16 lanes of a B fragment read take rows 16 jt + (0..15), slot g.
__device__ __forceinline__ int tn_qslot(int j, int s) { return s ^ ((j >> 2) & 3); }


struct BwdTnArgs {
  const uint16_t* p;   // [m][p_ld] bf16
  int64_t p_ld;
  const uint16_t* qt;  // [qcp][ld] bf16: Q^T, zero past m
  int64_t m, ld, c_total, m_per_split;
  int32_t qcp;         // a multiple of 64
  float* part;         // [split][c_total][qcp]
};

// Workgroup (x, y, split): columns c = 256 x .. +256 (wave w: 64 w .. +64, four 16-column
// tiles), j = 64 y .. +64 (four tiles), the split's tokens in stages of 32.  Token rows past
// m copy row m - 1 and are zeroed in the fragments; columns past c_total copy the last
// in-range unit and their outputs are not stored.
__global__ __launch_bounds__(256) void bwd_tn_kernel(BwdTnArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int r = lane & 15, g = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kTnC, jb = (int64_t)blockIdx.y * kTnJ, split = blockIdx.z;
  const int64_t m_lo = split * a.m_per_split;
  const int64_t m_hi = a.ld < m_lo + a.m_per_split ? a.ld : m_lo + a.m_per_split;
  const int64_t nst = m_hi > m_lo ? (m_hi - m_lo) / kTnM : 0;
  // Copies of one stage, per wave: 4 x P (token rows 8 wave + 2 v + lane / 32, 16 bytes at
  // physical slot lane % 32) and 1 x Q^T (rows 16 wave + lane / 4, physical slot lane % 4).
  int prow[4];
  const uint16_t* pcol[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    prow[v] = 8 * wave + 2 * v + (lane >> 5);
    const int64_t c = c0 + 8 * tn_pslot(prow[v], lane & 31);
    pcol[v] = a.p + (c < a.c_total ? c : a.c_total - 8);
  }
  const int qrow = 16 * wave + (lane >> 2);
  const uint16_t* qsrc = a.qt + (jb + qrow) * a.ld + 8 * tn_qslot(qrow, lane & 3);
  auto dma = [&](int64_t st, int slot) {
    const int64_t mb = m_lo + st * kTnM;
    const uint32_t lb = lds_addr(smem) + slot * kTnStage;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mr = mb + prow[v] < a.m ? mb + prow[v] : a.m - 1;
      lds_copy16_va(pcol[v] + mr * a.p_ld, lb + 1024 * (4 * wave + v));
    }
    lds_copy16_va(qsrc + mb, lb + kTnPBytes + 1024 * wave);
  };
  auto clamp_st = [&](int64_t st) { return st < nst ? st : nst - 1; };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  if (nst > 0) {
    dma(0, 0);
    dma(clamp_st(1), 1);
    dma(clamp_st(2), 2);
  }
  const int tre = r >> 2, trb = r & 3;
  for (int64_t st = 0; st < nst; ++st) {
    const int slot = (int)(st & 3);
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");  // stage st has landed; st + 1, st + 2 in flight
    __syncthreads();  // ... for every wave, and every wave is done with stage st - 1's slot
    dma(clamp_st(st + 3), (int)((st + 3) & 3));
    const uint8_t* pb = smem + slot * kTnStage;
    const uint8_t* qb = pb + kTnPBytes;
    // A (tile i: c 64 wave + 16 i + r): two transposing reads of token rows 8 g + 4 q + r / 4
    // at c 64 wave + 16 i + 4 (r % 4); element e of the fragment is token 8 g + e.
    bf16x8 af[4], bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = 8 * wave + 2 * i + (trb >> 1);
      i16x4 pr[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int mrow = 8 * g + 4 * q + tre;
        pr[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(pb + mrow * 512 + tn_pslot(mrow, sl) * 16 + (trb & 1) * 8));
      }
      af[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int64_t mb = m_lo + st * kTnM;
    if (mb + kTnM > a.m) {
      // the stage runs past the last token: zero the copied duplicates of row m - 1
      const int64_t room = a.m - mb - 8 * g;  // elements e < room are real tokens
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= room) af[i][e] = (__bf16)0.0f;
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + r;
      bq[jt] = *(const bf16x8*)(qb + j * 64 + tn_qslot(j, g) * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[i][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bq[jt], acc[i][jt], 0, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lane (r, g) of tile (i, jt): c = c0 + 64 wave + 16 i + 4 g + e, column jb + 16 jt + r
  float* out = a.part + split * a.c_total * a.qcp;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t c = c0 + 64 * wave + 16 * i + 4 * g + e;
      if (c >= a.c_total) continue;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) out[c * a.qcp + jb + 16 * jt + r] = acc[i][jt][e];
    }
  }
}

// out[c * stride_c + j * stride_j] = (sum over splits of part[split][c][j]) + (sum over
// splits of part[split][c][rp + j]), each in split order, for j < rank (hi, then lo
// columns; partial rows of qcp floats).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part, int64_t splits,
                                                         int64_t c_total, int32_t qcp, int32_t rp, int32_t rank,
                                                         float* __restrict__ out, int64_t stride_c,
                                                         int64_t stride_j) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= c_total * rank) return;
  const int64_t c = i / rank;
  const int j = (int)(i - c * rank);
  float hi = 0.0f, lo = 0.0f;
  for (int64_t sp = 0; sp < splits; ++sp) {
    hi += part[(sp * c_total + c) * qcp + j];
    lo += part[(sp * c_total + c) * qcp + rp + j];
  }
  out[c * stride_c + j * stride_j] = hi + lo;
}

__global__ __launch_bounds__(256) void bwd_transpose_kernel(const uint16_t* __restrict__ b, int64_t n, int32_t rank,
                                                            uint16_t* __restrict__ bt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * rank) return;
  const int64_t row = i / rank;
  const int j = (int)(i - row * rank);
  bt[(int64_t)j * n + row] = b[i];
}

// ------------------------------------------------------------------ host side
namespace {
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
int32_t rank_pad32(int32_t r) { return (r + 31) / 32 * 32; }
int64_t ld32(int64_t m) { return (m + 31) / 32 * 32; }
int32_t qc_pad(int32_t rank) { return 2 * rank_pad32(rank); }  // hi | lo columns, a multiple of 64
// Token splits of the adapter-gradient products: about 1024 workgroups (two per compute
// unit fit in LDS), at least 128 tokens per split, at most 32 splits.
int64_t tn_splits(int64_t m, int64_t c_total, int32_t qcp) {
  const int64_t wgs = (c_total + kTnC - 1) / kTnC * (qcp / kTnJ);
  int64_t sp = (1024 + wgs - 1) / wgs;
  const int64_t smax = (m + 127) / 128;
  if (sp > smax) sp = smax;
  if (sp > 32) sp = 32;
  return sp < 1 ? 1 : sp;
}
// dX takes the transposed f16 product (gemm_nvfp4.hip) unless n or k exceed its 32-bit copy
// offsets; then bwd_dx_kernel.
bool dx_f16_path(int64_t n, int64_t k) { return n < kNvF16MaxK && k < kNvDxMaxK; }
struct BwdWs {
  uint16_t* bt;      // [rank][n]
  char* rows;        // f16 path: dY as f16 rows, du (hi | lo)
  uint16_t* at;      // f16 path: A^T [k][rank_pad]
  float* dx_part;    // f16 path: split-tile partials of dX
  char* down_u;      // other path: lora_down scratch of dY B (hi | lo)
  char* down_t;      // lora_down scratch of x A^T (hi | lo)
  uint16_t* tt;      // [qcp][ld]
  uint16_t* ut;      // [qcp][ld]
  float* part_b;     // [splits][n][qcp]
  float* part_a;     // [splits][k][qcp]
  size_t bytes;
};
BwdWs bwd_ws(void* scratch, int64_t m, int64_t n, int64_t k, int32_t rank) {
  BwdWs w{};
  char* p = (char*)scratch;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p + off;
    off += up256(bytes);
    return q;
  };
  const bool f16 = dx_f16_path(n, k);
  if (rank > 0) w.bt = (uint16_t*)take((size_t)rank * (size_t)n * 2);
  if (f16) {
    w.rows = take(f16_rows_bytes(m, n, rank));
    if (rank > 0) w.at = (uint16_t*)take((size_t)k * (size_t)rank_pad32(rank) * 2);
    w.dx_part = (float*)take(nvfp4_dx_part_bytes(m, n, k));
  } else if (rank > 0) {
    w.down_u = take(lora_down_hilo_bytes(m, n, rank));
  }
  if (rank > 0) {
    const size_t ld = (size_t)ld32(m), qcp = (size_t)qc_pad(rank);
    w.down_t = take(lora_down_hilo_bytes(m, k, rank));
    w.tt = (uint16_t*)take(qcp * ld * 2);
    w.ut = (uint16_t*)take(qcp * ld * 2);
    w.part_b = (float*)take((size_t)tn_splits(m, n, (int32_t)qcp) * (size_t)n * qcp * 4);
    w.part_a = (float*)take((size_t)tn_splits(m, k, (int32_t)qcp) * (size_t)k * qcp * 4);
  }
  w.bytes = off;
  return w;
}
void transpose2d(const uint16_t* src, int64_t rows, int64_t cols, int64_t src_ld, int64_t rows_pad,
                 int64_t cols_pad, uint16_t* dst, hipStream_t s) {
  bwd_transpose2d_kernel<<<dim3((unsigned)((cols_pad + kTr - 1) / kTr), (unsigned)((rows_pad + kTr - 1) / kTr)), 256, 0,
                           s>>>(src, rows, cols, src_ld, rows_pad, cols_pad, dst);
}
}  // namespace

size_t backward_scratch_bytes(int64_t m, int64_t n, int64_t k, int32_t rank) {
  return bwd_ws(nullptr, m, n, k, rank).bytes;
}

hipError_t launch_backward_nvfp4(const uint16_t* x, const uint16_t* dy, int64_t m, int64_t n, int64_t k,
                                 const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                 const uint16_t* lora_a, const uint16_t* lora_b, int32_t rank, float lora_scale,
                                 void* dx, int out_f32, float* da, float* db, void* scratch, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  if (n % kBxTN != 0 || k % kBxTK != 0 || rank < 0 || rank > 128) return hipErrorInvalidValue;
  const BwdWs w = bwd_ws(scratch, m, n, k, rank);
  const int32_t rp = rank > 0 ? rank_pad32(rank) : 0;
  uint16_t* t = nullptr;
  uint16_t* du = nullptr;
  hipError_t e = hipSuccess;
  if (rank > 0) bwd_transpose_kernel<<<(unsigned)((n * rank + 255) / 256), 256, 0, s>>>(lora_b, n, rank, w.bt);
  if (dx_f16_path(n, k)) {
    uint16_t* dy16 = nullptr;
    float* rs = nullptr;
    e = launch_f16_rows(dy, m, n, w.bt, rank, lora_scale, w.rows, &dy16, &rs, &du, s);
    if (e != hipSuccess) return e;
    if (rank > 0) transpose2d(lora_a, rank, k, k, rp, k, w.at, s);
    e = launch_nvfp4_dx(dy16, rs, m, n, k, codes, scales, tensor_scale, w.at, du, rp, 2 * rp, dx, out_f32, w.dx_part,
                        s);
    if (e != hipSuccess) return e;
  } else {
    if (rank > 0) {
      e = launch_lora_down_hilo(dy, m, n, w.bt, rank, lora_scale, w.down_u, &du, s);
      if (e != hipSuccess) return e;
    }
    BwdDxArgs a;
    a.dy = dy;
    a.m = m;
    a.n = n;
    a.k = k;
    a.codes = codes;
    a.scales = scales;
    a.tensor_scale = tensor_scale;
    a.du = du;
    a.lora_a = lora_a;
    a.rank = rank;
    a.rank_pad = rp;
    a.dx = dx;
    a.out_f32 = out_f32;
    bwd_dx_kernel<<<dim3((unsigned)(k / kBxTK), (unsigned)((m + kBxTM - 1) / kBxTM)), 256, 0, s>>>(a);
  }
  if (rank > 0) {
    e = launch_lora_down_hilo(x, m, k, lora_a, rank, lora_scale, w.down_t, &t, s);
    if (e != hipSuccess) return e;
  }
  if (rank > 0) {
    // dB[n][j] = sum_m dY[m][n] t[m][j];  dA[j][k] = sum_m du[m][j] x[m][k]  (hi and lo columns)
    const int64_t ld = ld32(m);
    const int32_t qcp = qc_pad(rank);
    transpose2d(t, m, 2 * rp, 2 * rp, ld, qcp, w.tt, s);
    transpose2d(du, m, 2 * rp, 2 * rp, ld, qcp, w.ut, s);
    e = hipFuncSetAttribute((const void*)bwd_tn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTnLds);
    if (e != hipSuccess) return e;
    const struct { const uint16_t* p; int64_t p_ld; const uint16_t* qt; int64_t c; float* part; float* out; int64_t sc, sj; }
        jobs[2] = {{dy, n, w.tt, n, w.part_b, db, rank, 1}, {x, k, w.ut, k, w.part_a, da, 1, k}};
    for (const auto& jb : jobs) {
      const int64_t sp = tn_splits(m, jb.c, qcp);
      BwdTnArgs g;
      g.p = jb.p;
      g.p_ld = jb.p_ld;
      g.qt = jb.qt;
      g.m = m;
      g.ld = ld;
      g.c_total = jb.c;
      g.m_per_split = ((ld + sp - 1) / sp + kTnM - 1) / kTnM * kTnM;
      g.qcp = qcp;
      g.part = jb.part;
      const int64_t used = (ld + g.m_per_split - 1) / g.m_per_split;
      bwd_tn_kernel<<<dim3((unsigned)((jb.c + kTnC - 1) / kTnC), (unsigned)(qcp / kTnJ), (unsigned)used), 256, kTnLds,
                      s>>>(g);
      bwd_reduce_kernel<<<(unsigned)((jb.c * rank + 255) / 256), 256, 0, s>>>(jb.part, used, jb.c, qcp, rp, rank,
                                                                            jb.out, jb.sc, jb.sj);
    }
  }
  return hipGetLastError();
}

}  // namespace ql
