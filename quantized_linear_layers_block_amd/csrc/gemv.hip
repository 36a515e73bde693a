// Few-token ("decode") NVFP4 layer for gfx950, one launch per call:
//
//   y = S . x . (E2M1 * E4M3)^T  +  bf16(s . x A^T) . B^T
//
// QeRL's rollout speedup comes from decoding with the policy's weight path in NVFP4
// (tldrocket.com QeRL page, paragraph after "Key Features of QeRL").  With a handful of
// tokens the layer streams 0.5625 byte per weight and is bound by HBM, so everything is
// organised around reading the packed codes once, as early as possible.
//
// Work items (one workgroup of four waves each, 1-D grid):
//   * LoRA items come first in dispatch order: 64 R bf16 rows of A (16 R per wave)
//     against the activations over ONE 256-wide K chunk; float32 partials of x A^T.
//   * weight items: 64 R NVFP4 rows (16 R per wave) over one K split of several chunks.
// Within a chunk, lane l reads row (l % 16) of each of its wave's row tiles and the 64
// consecutive K of lane group g = l / 16 (32 bytes of codes, 4 block scales).  Chunks
// are processed in batches of CB: the codes of the next batch are loaded into registers
// and its activations x[m][k] staged into LDS (double buffer) while the current batch is
// multiplied.  Codes are dequantized in registers -- E2M1 -> float by the hardware
// converter, times the E4M3 block scale in float32 (exact, at most 6 significant bits,
// hence an exact bf16) -- and fed to 16x16x32 bf16 MFMAs whose B operand (activations)
// comes from LDS.  The K order inside an MFMA is a permutation shared by both operands.
//
// Completion without a second launch: when K is split over several items, each stores its
// partial tile with device-scope (write-through) stores and increments an integer counter;
// the last arrival reads the partials back with device-scope loads and adds them in split
// order.  The last LoRA item of an m group
// writes t = bf16(s . sum) and raises a flag; a weight row group's last arrival waits for
// that flag (LoRA items are dispatched before every weight item, so they are running or
// done; the wait is bounded), adds t B^T with one MFMA per 32 ranks, applies S and stores
// y.  Every counter and flag is returned to zero by the call that used it, so the
// workspace only has to be zero before its first use.
#include "common.hpp"
#include "gemv_common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kGvThreads = 256;
constexpr int kGvChunk = 256;  // K per chunk: 4 lane groups x 64

struct GvArgs {
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
  int produce_y;          // 0: LoRA-only launch that just leaves t in the workspace
  // plan
  int splits;
  int64_t cps;            // chunks per split
  int64_t kchunks;
  int64_t groups_w;       // weight row groups (64 R rows each)
  int64_t groups_l;       // LoRA row groups
  int m_groups;           // m groups (16 MT rows each); weight items only use m group 0
  int64_t rows_w_pad;     // row length of the weight partials
  int64_t rows_l_pad;     // row length of the LoRA partials
  int rank_pad;           // row length of t (multiple of 32)
  int xstride;            // LDS row stride of staged activations (elements)
  int xbuf;               // elements per LDS activation buffer (two buffers)
  // workspace
  uint32_t* cnt_w;        // [groups_w]
  uint32_t* cnt_l;        // [m_groups]
  uint32_t* t_ready;      // [m_groups]
  uint32_t* fin;          // [1]
  uint16_t* t;            // [m][rank_pad] bf16
  float* part_w;          // [splits][m][rows_w_pad]
  float* part_l;          // [kchunks][m][rows_l_pad]
};

// Register image of one chunk for one row tile: 32 bytes of codes and 4 scale bytes.
struct ChunkRegs {
  uint4 c0, c1;
  uint32_t s;
};

template <bool ALIGNED>
__device__ __forceinline__ ChunkRegs load_chunk(const GvArgs& a, int64_t row, bool rv, int64_t kl) {
  ChunkRegs cr;
  const uint8_t* cp = a.codes + row * (a.k / 2) + kl / 2;
  const uint8_t* sp = a.scales + row * (a.k / 16) + kl / 16;
  if (ALIGNED) {  // K % 256 == 0: whole chunks, naturally aligned 16- and 4-byte loads
    cr.c0 = rv ? *(const uint4*)cp : make_uint4(0, 0, 0, 0);
    cr.c1 = rv ? *(const uint4*)(cp + 16) : make_uint4(0, 0, 0, 0);
    cr.s = rv ? *(const uint32_t*)sp : 0u;
  } else {        // K % 16 == 0: 16-element blocks, 8-byte code loads, byte scale loads
    uint32_t cw[8], sb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool ok = rv && kl + 16 * b < a.k;
      const uint2 v = ok ? *(const uint2*)(cp + 8 * b) : make_uint2(0, 0);
      cw[2 * b] = v.x;
      cw[2 * b + 1] = v.y;
      sb[b] = ok ? sp[b] : 0u;
    }
    cr.c0 = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    cr.c1 = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    cr.s = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
  }
  return cr;
}

// Stage x[mbase .. mbase+mrows) x [c_begin*256, c_end*256) into one LDS buffer (zero past K).
__device__ __forceinline__ void stage_x(const GvArgs& a, uint16_t* xs, int64_t mbase, int mrows,
                                        int64_t cbeg, int64_t cend) {
  const int per_row = (int)(cend - cbeg) * (kGvChunk / 8);  // 16-byte units per row
  const int units = mrows * per_row;
  for (int u = threadIdx.x; u < units; u += kGvThreads) {
    const int i = u / per_row;
    const int col = (u - i * per_row) * 8;
    const int64_t k = cbeg * kGvChunk + col;
    // K % 16 == 0 and k % 8 == 0: a unit is entirely inside or entirely past K
    const uint4 v = k < a.k ? *(const uint4*)(a.x + (mbase + i) * a.k + k) : make_uint4(0, 0, 0, 0);
    *(uint4*)(xs + i * a.xstride + col) = v;
  }
}

// B fragment of m tile q, chunk slot ci, k-step t (8 bf16 of row 16q + r).
template <int MT>
__device__ __forceinline__ bf16x8 x_frag(const GvArgs& a, const uint16_t* xs, int mrows, int q,
                                         int ci, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  const int mi = 16 * q + r;
  if (mi >= mrows) return gv_zero8();
  return __builtin_bit_cast(bf16x8, *(const uint4*)(xs + mi * a.xstride + ci * kGvChunk + 64 * g + 8 * t));
}

// Multiply a batch of weight chunks held in registers against staged activations.
template <int MT, int R, int CB>
__device__ __forceinline__ void mul_batch(const GvArgs& a, const uint16_t* xs, int mrows, int nch,
                                          const ChunkRegs (&cr)[CB][R], f32x4 (&acc)[R][MT]) {
#pragma unroll
  for (int ci = 0; ci < CB; ++ci) {
    if (ci >= nch) break;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8 bx[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) bx[q] = x_frag<MT>(a, xs, mrows, q, ci, t);
#pragma unroll
      for (int p = 0; p < R; ++p) {
        const uint32_t c = t == 0 ? cr[ci][p].c0.x : t == 1 ? cr[ci][p].c0.y : t == 2 ? cr[ci][p].c0.z :
                           t == 3 ? cr[ci][p].c0.w : t == 4 ? cr[ci][p].c1.x : t == 5 ? cr[ci][p].c1.y :
                           t == 6 ? cr[ci][p].c1.z : cr[ci][p].c1.w;
        const bf16x8 av = gv_dequant8(c, e4m3_value((cr[ci][p].s >> (8 * (t >> 1))) & 0xFFu));
#pragma unroll
        for (int q = 0; q < MT; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[q], acc[p][q], 0, 0, 0);
      }
    }
  }
}

template <int R, int CB, bool ALIGNED>
__device__ __forceinline__ void load_batch(const GvArgs& a, int64_t wrow0, int64_t cbeg, int64_t cend,
                                           ChunkRegs (&cr)[CB][R]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ci = 0; ci < CB; ++ci) {
    const int64_t c = cbeg + ci;
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int64_t row = wrow0 + 16 * p + r;
      cr[ci][p] = load_chunk<ALIGNED>(a, row, row < a.n && c < cend, c * kGvChunk + 64 * g);
    }
  }
}

// Counter arrival; true in every thread of the last-arriving workgroup.
__device__ __forceinline__ bool arrive(uint32_t* cnt, uint32_t total, int* flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == total - 1;
  }
  __syncthreads();
  return *flag != 0;
}

// Bounded wait for a flag raised by another workgroup (device-scope polls).
__device__ __forceinline__ void wait_flag(const uint32_t* f) {
  if (threadIdx.x == 0) {
    int it = 0;
    while (ld_dev_u32(f) == 0u && ++it < kGvSpinLimit) __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
}

template <int MT, int R, int CB, bool ALIGNED>
__global__ __launch_bounds__(kGvThreads) void gv_kernel(GvArgs a) {
  extern __shared__ __align__(16) uint16_t gv_smem[];
  __shared__ int flag;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int64_t items_l = a.groups_l * a.kchunks * a.m_groups;
  const int xbuf = a.xbuf;
  int64_t id = blockIdx.x;

  f32x4 acc[R][MT];
#pragma unroll
  for (int p = 0; p < R; ++p)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[p][q] = f32x4{0, 0, 0, 0};

  if (id < items_l) {
    // ------------------------------------------------- LoRA item: one chunk of A rows
    const int64_t grp = id % a.groups_l;
    const int64_t c = (id / a.groups_l) % a.kchunks;
    const int mg = (int)(id / (a.groups_l * a.kchunks));
    const int64_t mbase = (int64_t)mg * 16 * MT;
    const int mrows = (int)min((int64_t)16 * MT, a.m - mbase);
    const int64_t wrow0 = grp * 64 * R + wave * 16 * R;
    uint4 av[R][8];
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int64_t row = wrow0 + 16 * p + r;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int64_t k = c * kGvChunk + 64 * g + 8 * t;
        av[p][t] = (row < a.rank && k < a.k) ? *(const uint4*)(a.lora_a + row * a.k + k) : make_uint4(0, 0, 0, 0);
      }
    }
    stage_x(a, gv_smem, mbase, mrows, c, c + 1);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8 bx[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) bx[q] = x_frag<MT>(a, gv_smem, mrows, q, 0, t);
#pragma unroll
      for (int p = 0; p < R; ++p)
#pragma unroll
        for (int q = 0; q < MT; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[p][t]), bx[q], acc[p][q], 0, 0, 0);
    }
    // partials [chunk][m][rows_l_pad]; lane holds m = mbase + 16 q + r, rows wrow0 + 16 p + 4 g + i
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mrow = mbase + 16 * q + r;
        if (mrow < a.m) st_dev4(a.part_l + (c * a.m + mrow) * a.rows_l_pad + wrow0 + 16 * p + 4 * g, acc[p][q]);
      }
    if (!arrive(a.cnt_l + mg, (uint32_t)(a.groups_l * a.kchunks), &flag)) return;
    // last LoRA item of this m group: t = bf16(s . sum over chunks), then raise the flag
    for (int64_t i = threadIdx.x; i < (int64_t)mrows * a.rank_pad; i += kGvThreads) {
      const int64_t mm = mbase + i / a.rank_pad;
      const int j = (int)(i % a.rank_pad);
      float v = 0.0f;
      if (j < a.rank)
        for (int64_t cc = 0; cc < a.kchunks; ++cc) v += ld_dev(a.part_l + (cc * a.m + mm) * a.rows_l_pad + j);
      a.t[mm * a.rank_pad + j] = (uint16_t)f32_to_bf16_rne(a.lora_scale * v);
    }
    // t is read by weight items of this launch (device-scope, see below) or by the next
    // launch on the stream; make it visible before the flag goes up.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
      st_dev_u32(a.cnt_l + mg, 0u);
      if (a.produce_y) st_dev_u32(a.t_ready + mg, 1u);
    }
    return;
  }

  // ------------------------------------------------------------------ weight item
  id -= items_l;
  const int64_t grp = id % a.groups_w;
  const int64_t split = id / a.groups_w;
  const int64_t wrow0 = grp * 64 * R + wave * 16 * R;   // this wave's first row
  const int64_t c0 = split * a.cps, c1 = min(c0 + a.cps, a.kchunks);
  const int mrows = (int)min((int64_t)16 * MT, a.m);

  ChunkRegs ca[CB][R], cb_[CB][R];
  int64_t cb = c0;
  load_batch<R, CB, ALIGNED>(a, wrow0, cb, c1, ca);
  stage_x(a, gv_smem, 0, mrows, cb, min(cb + CB, c1));
  __syncthreads();
  int buf = 0;
  while (true) {
    // batch in ca / LDS buffer `buf`; prefetch the next into cb_ / buf ^ 1
    int64_t nb = cb + CB;
    if (nb < c1) {
      load_batch<R, CB, ALIGNED>(a, wrow0, nb, c1, cb_);
      stage_x(a, gv_smem + (buf ^ 1) * xbuf, 0, mrows, nb, min(nb + CB, c1));
    }
    mul_batch<MT, R, CB>(a, gv_smem + buf * xbuf, mrows, (int)(min(cb + CB, c1) - cb), ca, acc);
    __syncthreads();
    if (nb >= c1) break;
    buf ^= 1;
    cb = nb;
    nb = cb + CB;
    if (nb < c1) {
      load_batch<R, CB, ALIGNED>(a, wrow0, nb, c1, ca);
      stage_x(a, gv_smem + (buf ^ 1) * xbuf, 0, mrows, nb, min(nb + CB, c1));
    }
    mul_batch<MT, R, CB>(a, gv_smem + buf * xbuf, mrows, (int)(min(cb + CB, c1) - cb), cb_, acc);
    __syncthreads();
    if (nb >= c1) break;
    buf ^= 1;
    cb = nb;
  }

  if (a.splits > 1) {
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mrow = 16 * q + r;
        if (mrow < a.m) st_dev4(a.part_w + (split * a.m + mrow) * a.rows_w_pad + wrow0 + 16 * p + 4 * g, acc[p][q]);
      }
    if (!arrive(a.cnt_w + grp, (uint32_t)a.splits, &flag)) return;
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mrow = 16 * q + r;
        f32x4 s = {0, 0, 0, 0};
        if (mrow < a.m)
          for (int sp = 0; sp < a.splits; ++sp)
            s += ld_dev4(a.part_w + ((int64_t)sp * a.m + mrow) * a.rows_w_pad + wrow0 + 16 * p + 4 * g);
        acc[p][q] = s;
      }
    if (threadIdx.x == 0) st_dev_u32(a.cnt_w + grp, 0u);
  }
  // The last arrival finishes the row group: lane holds C[n][m], m = 16 q + r, n = wrow0 + 16 p + 4 g + i
  const float S = *a.tensor_scale;
#pragma unroll
  for (int p = 0; p < R; ++p)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[p][q] *= S;
  if (a.rank > 0) {  // wait (bounded) for t from the LoRA items
    wait_flag(a.t_ready);
    for (int j0 = 0; j0 < a.rank_pad; j0 += 32) {
      bf16x8 tb[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mrow = 16 * q + r;
        if (mrow < a.m) {
          const uint32_t* tp = (const uint32_t*)(a.t + mrow * a.rank_pad + j0 + 8 * g);
          i32x4 tv = {(int)ld_dev_u32(tp), (int)ld_dev_u32(tp + 1), (int)ld_dev_u32(tp + 2), (int)ld_dev_u32(tp + 3)};
          tb[q] = __builtin_bit_cast(bf16x8, tv);
        } else {
          tb[q] = gv_zero8();
        }
      }
#pragma unroll
      for (int p = 0; p < R; ++p) {
        const int64_t nrow = wrow0 + 16 * p + r;
        uint32_t bw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int j = j0 + 8 * g + e;
          const uint32_t b0 = (nrow < a.n && j < a.rank) ? a.lora_b[nrow * a.rank + j] : 0u;
          const uint32_t b1 = (nrow < a.n && j + 1 < a.rank) ? a.lora_b[nrow * a.rank + j + 1] : 0u;
          bw[e / 2] = b0 | (b1 << 16);
        }
        i32x4 bi = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bi);
#pragma unroll
        for (int q = 0; q < MT; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, tb[q], acc[p][q], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < R; ++p)
#pragma unroll
    for (int q = 0; q < MT; ++q) {
      const int64_t mrow = 16 * q + r;
      const int64_t nb = wrow0 + 16 * p + 4 * g;
      if (mrow >= a.m || nb >= a.n) continue;
      const f32x4 v = acc[p][q];
      if (a.out_f32) {
        float* y = (float*)a.y + mrow * a.n;
        if (nb + 4 <= a.n && (a.n & 3) == 0) {
          *(f32x4*)(y + nb) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < a.n) y[nb + i] = v[i];
        }
      } else {
        uint16_t* y = (uint16_t*)a.y + mrow * a.n;
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
  if (a.rank > 0) {
    __syncthreads();  // every wave has read t
    if (threadIdx.x == 0) {  // t was read (values in registers) before this point
      const uint32_t done = __hip_atomic_fetch_add(a.fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)a.groups_w - 1) {  // every row group has read t: lower the flag
        st_dev_u32(a.t_ready, 0u);
        st_dev_u32(a.fin, 0u);
      }
    }
  }
}

// ----------------------------------------------------------------- planning

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static int batch_chunks(int mt) { return mt == 1 ? 4 : (mt == 2 ? 2 : 1); }

// m <= 64 with weight rows (n > 0), or any m for a LoRA-only launch (n == 0, m groups of 64).
SkinnyPlan plan_skinny(int64_t m, int64_t n, int64_t k, int32_t rank) {
  SkinnyPlan p;
  const int64_t mt_rows = n > 0 ? m : 64;
  p.mt = mt_rows <= 16 ? 1 : (mt_rows <= 32 ? 2 : 4);
  p.r = p.mt;
  p.m_groups = (int)cdiv(m, 16 * p.mt);
  p.rows_w = n;
  p.rows_w_pad = round_up(n, 64 * p.r);
  p.rows_l = rank > 0 ? round_up(rank, 16) : 0;
  p.rows_total = round_up(p.rows_l, 64 * p.r);  // LoRA partial row length
  p.groups_w = n > 0 ? cdiv(n, 64 * p.r) : 0;
  p.groups_l = p.rows_l > 0 ? cdiv(p.rows_l, 64 * p.r) : 0;
  p.rank_pad = (int)round_up(p.rows_l, 32);
  const int64_t kchunks = cdiv(k, kGvChunk);
  const int cb = batch_chunks(p.mt);
  // At least ~4 workgroups per CU (2 for the wider tiles), splits of >= CB chunks while
  // there are already more workgroups than CUs.
  const int64_t target = p.mt == 1 ? 1024 : 512;
  int64_t splits = 1;
  if (p.groups_w > 0) {
    while (p.groups_w * splits < target && splits < kchunks) {
      const int64_t next = splits * 2;
      if (cdiv(kchunks, next) < cb && p.groups_w * splits >= 256) break;
      splits = next;
    }
  }
  p.kchunks_per_split = cdiv(kchunks, splits);
  p.splits = (int)cdiv(kchunks, p.kchunks_per_split);
  return p;
}

// Workspace: counters (zero before first use, zero after every call) | t | partials.
static size_t counter_words(const SkinnyPlan& p) { return (size_t)(p.groups_w + 2 * p.m_groups + 1); }

static size_t part_w_bytes(const SkinnyPlan& p, int64_t m) {
  return p.splits > 1 ? (size_t)p.splits * (size_t)m * (size_t)p.rows_w_pad * 4 : 0;
}
static size_t part_l_bytes(const SkinnyPlan& p, int64_t m, int64_t k) {
  return p.rows_l > 0 ? (size_t)cdiv(k, kGvChunk) * (size_t)m * (size_t)p.rows_total * 4 : 0;
}

size_t skinny_workspace(const SkinnyPlan& p, int64_t m, int64_t k) {
  return align256(counter_words(p) * 4) + align256((size_t)m * (size_t)p.rank_pad * 2) +
         align256(part_w_bytes(p, m)) + align256(part_l_bytes(p, m, k));
}

template <int MT, int R, int CB>
static hipError_t launch_gv(const GvArgs& a, int64_t items, int mrows_lds, hipStream_t s) {
  const size_t lds = 2 * (size_t)mrows_lds * (size_t)a.xstride * 2;
  if (a.k % kGvChunk == 0) {
    hipError_t e = hipFuncSetAttribute((const void*)gv_kernel<MT, R, CB, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gv_kernel<MT, R, CB, true><<<(unsigned)items, kGvThreads, lds, s>>>(a);
  } else {
    hipError_t e = hipFuncSetAttribute((const void*)gv_kernel<MT, R, CB, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    gv_kernel<MT, R, CB, false><<<(unsigned)items, kGvThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

static hipError_t launch_gv_plan(const SkinnyPlan& p, GvArgs& a, char* ws, int64_t m, hipStream_t s) {
  const int cb = batch_chunks(p.mt);
  a.splits = p.splits;
  a.cps = p.kchunks_per_split;
  a.kchunks = cdiv(a.k, kGvChunk);
  a.groups_w = p.groups_w;
  a.groups_l = p.groups_l;
  a.m_groups = p.m_groups;
  a.rows_w_pad = p.rows_w_pad;
  a.rows_l_pad = p.rows_total;
  a.rank_pad = p.rank_pad;
  a.xstride = cb * kGvChunk + 8;
  uint32_t* cnt = (uint32_t*)ws;
  a.cnt_w = cnt;
  a.cnt_l = cnt + p.groups_w;
  a.t_ready = a.cnt_l + p.m_groups;
  a.fin = a.t_ready + p.m_groups;
  size_t off = align256(counter_words(p) * 4);
  a.t = (uint16_t*)(ws + off);
  off += align256((size_t)m * (size_t)p.rank_pad * 2);
  a.part_w = (float*)(ws + off);
  off += align256(part_w_bytes(p, m));
  a.part_l = (float*)(ws + off);
  const int64_t items = a.groups_l * a.kchunks * a.m_groups + (a.produce_y ? a.groups_w * a.splits : 0);
  if (items <= 0) return hipSuccess;
  // LDS rows: the weight items stage min(m, 16 MT) rows; LoRA items 16 MT rows at most
  const int mrows_lds = (int)min((int64_t)16 * p.mt, m);
  a.xbuf = mrows_lds * a.xstride;
  if (p.mt == 1) return launch_gv<1, 1, 4>(a, items, mrows_lds, s);
  if (p.mt == 2) return launch_gv<2, 2, 2>(a, items, mrows_lds, s);
  return launch_gv<4, 4, 1>(a, items, mrows_lds, s);
}

hipError_t launch_lora_down(const SkinnyPlan& p, const uint16_t* x, int64_t m, int64_t k,
                            const uint16_t* lora_a, int32_t rank, float lora_scale, void* ws,
                            hipStream_t s) {
  GvArgs a = {};
  a.x = x;
  a.m = m;
  a.k = k;
  a.lora_a = lora_a;
  a.rank = rank;
  a.lora_scale = lora_scale;
  a.n = 0;
  a.produce_y = 0;
  return launch_gv_plan(p, a, (char*)ws, m, s);
}

uint16_t* lora_t_in_workspace(const SkinnyPlan& p, void* ws) {
  return (uint16_t*)((char*)ws + align256(counter_words(p) * 4));
}

}  // namespace ql
