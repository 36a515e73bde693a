// Few-token NVFP4 layer for up to 64 tokens on gfx950, one launch per call:
//
//   y = S . x . (E2M1 * E4M3)^T  +  bf16(s . x A^T) . B^T
//
// This is the decoding case of QeRL's NVFP4 weight path (tldrocket.com QeRL page,
// paragraph after "Key Features of QeRL"): 0.5625 byte per weight is streamed once, so the
// design is about keeping HBM busy from the first cycle and hiding every other latency
// behind that stream.
//
// * Up to 32 tokens: a workgroup owns RT tiles of 16 weight rows (RT = 1 or 2) and a range
//   of 256-wide K chunks; its four waves take the chunks in turn.  For each chunk a lane reads row
//   (l % 16) of every row tile, K columns 64 (l / 16) .. +64 (32 bytes of codes and 4 block
//   scales).  A wave issues up to four such (chunk, row tile) loads before using any.
// * The activations of the workgroup's K range (at most 30 KB) are fetched into registers
//   first, then the LoRA B rows, then the codes; the activations are written to LDS and the
//   workgroup synchronises while the codes are still in flight, so each chunk is multiplied
//   as soon as it arrives.  They are the B operand of 16x16x32 bf16 MFMAs whose A operand is
//   the codes dequantized in registers (E2M1 -> float by the hardware converter, times the
//   E4M3 block scale in float32: exact, at most 6 significant bits, hence an exact bf16).
//   The K order inside an MFMA is a permutation shared by both operands.
// * 33 to 64 tokens (g16_stream_item): 64-row workgroups walk their K chunks with the
//   activations double-buffered in LDS and the next chunk prefetched in registers.
// * The four waves' tiles are added in LDS in a fixed order.  When the K range is split
//   over several workgroups, the partial tiles go to the workspace with device-scope stores
//   and the last arrival on the row tile's counter adds all of them in split order.
// * LoRA: items that multiply 16 rows of A by up to four K chunks are dispatched before all
//   weight items; each stores its partial of x A^T (device scope) and counts itself on a
//   counter.  The last one adds the partials in a fixed order, publishes t = bf16(s . x A^T)
//   once and raises a flag.  A row tile's finishing waves (their B rows were fetched at the
//   start) wait for the flag (bounded in time; LoRA items are dispatched first, so they are
//   running or done), add t B^T with one MFMA per 32 ranks, apply S and store y.  A wait
//   that gives up stores NaN for its tile and sets the timeout bit of the workspace's
//   status word.
// * Counters live in the workspace's reserved region, at a spacing that depends on the
//   plan, and every call returns the ones it used to zero: the split counters by their
//   tile's last arrival, and the LoRA counter and the t flag by the last of all LoRA items
//   and finishing tiles (counted on a two-level "done" counter), after which no workgroup
//   of the launch touches them.  A late flag can therefore never reach the next call.
#include "../../include/qlinear.h"
#include "common.hpp"
#include "gemm_common.hpp"
#include "gemv_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace ql {

constexpr int kG16Threads = 256;
constexpr int kG16Waves = kG16Threads / kWave;
constexpr int kG16Chunk = 256;
constexpr int kG16Pairs = 4;           // (chunk, row tile) code loads in flight per wave
constexpr int kG16XBytes = 30720;      // LDS for staged activations (5 workgroups per CU)
constexpr int kG16XUnits = 8;          // 16-byte activation units per thread (8 * 256 * 16 >= 30720)
constexpr int kG16XUnits1 = 2;         // the same for one token: 16 chunks of 32 units
constexpr int kG16EarlyRank = 64;      // B rows of ranks up to 64 are fetched at the start (64 tokens)
constexpr int kG16EarlyRankFew = 32;   // the same for up to 32 tokens (one fragment: fewer registers)
constexpr int kG16LoraGroupsFew = 32;  // K groups of the LoRA partials (at most about), <= 32 tokens
constexpr int kG16LoraGroups64 = 16;   // the same for 33..64 tokens
constexpr int kG16CUs = 256;           // workgroups that run at once: 5 per CU for one token tile, 4 for two

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
  int64_t tiles_w;    // weight tiles of 16 * RT rows
  int64_t tiles_l;    // LoRA row tiles (16 rows of A)
  int64_t lgroups;    // LoRA chunk groups
  int lc;             // chunks per LoRA item (a multiple of four: the waves take them in turn)
  int rank_pad;       // t row length (multiple of 32)
  int64_t n_pad;      // row length of the weight partials (the split tiles' rows)
  int xstride;        // LDS row stride of the activations (elements)
  int64_t kst;        // 128-wide K stages (33..64 tokens with K % 128 == 0), else 0
  int64_t sps;        // stages per K split
  int64_t full;       // stage path: tiles [0, full) run whole, the rest split `splits` ways
  uint32_t* ctr;      // counters and flags in the reserved region (g16_line_*)
  int ctr_stride;     // words between two of them
  int32_t* status;    // the workspace's status word
  uint32_t* t;        // [m][rank_pad / 2] bf16 pairs
  float* part_w;      // [splits][m][n_pad]: rows from 64 full on (only split tiles write partials)
  float* part_l;      // [lgroups][m][tiles_l * 16]
};

struct G16Chunk {
  uint4 c0, c1;
  uint32_t s;
};

// Counters and flags, one per line of ctr_stride words (128 bytes when the region has room:
// atomics on one line serialise and delay every other access to it): [0, tiles_w) split
// arrivals per row tile, the LoRA counter, the t flag, 32 "done" groups, the done top counter.
constexpr int kG16DoneGroups = 32;
constexpr int64_t kG16ExtraLines = 3 + kG16DoneGroups;
__device__ __forceinline__ uint32_t* g16_ctr(const G16Args& a, int64_t line) { return a.ctr + line * a.ctr_stride; }
__device__ __forceinline__ int64_t g16_line_l(const G16Args& a) { return a.tiles_w; }
__device__ __forceinline__ int64_t g16_line_t(const G16Args& a) { return a.tiles_w + 1; }
__device__ __forceinline__ int64_t g16_line_dg(const G16Args& a, int j) { return a.tiles_w + 2 + j; }
__device__ __forceinline__ int64_t g16_line_dt(const G16Args& a) { return a.tiles_w + 2 + kG16DoneGroups; }

// Thread 0 only, with LoRA.  Counts one of the launch's LoRA items (idx < items) or finishing
// row tiles (idx = items + tile) as done with the LoRA counter, the t flag and t, on a
// two-level counter (arrival idx counts in group idx % 32).  Every group's last arrival
// returns its counter to zero; the last arrival overall also returns the LoRA counter and
// the t flag to zero: every other user of them has finished with them by then.
__device__ __forceinline__ void g16_done(const G16Args& a, int64_t idx) {
  const int64_t total = a.tiles_l * a.lgroups + a.tiles_w;
  const int j = (int)(idx % kG16DoneGroups);
  const int64_t gsize = (total - j + kG16DoneGroups - 1) / kG16DoneGroups;
  const int ngroups = total < kG16DoneGroups ? (int)total : kG16DoneGroups;
  uint32_t* cg = g16_ctr(a, g16_line_dg(a, j));
  if (__hip_atomic_fetch_add(cg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)gsize - 1) return;
  st_dev_u32(cg, 0u);
  uint32_t* ct = g16_ctr(a, g16_line_dt(a));
  if (__hip_atomic_fetch_add(ct, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)ngroups - 1) return;
  st_dev_u32(ct, 0u);
  st_dev_u32(g16_ctr(a, g16_line_l(a)), 0u);
  st_dev_u32(g16_ctr(a, g16_line_t(a)), 0u);
}

// Memory operations complete in order, and the compiler can only count the ones still in
// flight (and wait for exactly the ones a value needs) across straight-line code.  So every
// load below is issued unconditionally, from a clamped in-bounds address when the lane has
// nothing to load, and its value is then masked to zero.  The mask goes through an empty asm
// statement: otherwise the compiler turns "ok ? load : 0" back into a branch around the load.
__device__ __forceinline__ uint32_t opaque_mask(bool ok) {
  uint32_t m = ok ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}
__device__ __forceinline__ uint4 mask4(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}
__device__ __forceinline__ uint4 ld16_or0(const void* p, bool ok, const void* dummy) {
  const uint4 v = *(const uint4*)(ok ? p : dummy);
  return mask4(v, opaque_mask(ok));
}

// One chunk (16 rows from `row0`, 256 K columns from `kl`) of a row tile.  The loads read
// whole 64-byte runs per group of four lanes (lane l: row l / 4, chunk bytes 16 (l % 4) and
// 64 + 16 (l % 4), scale bytes 4 (l % 4)), which streams markedly faster than lanes of one
// quad reading four different rows; g16_transpose then moves the data into the MFMA operand
// layout.  Rows past N and chunks past the range load from row 0 / column 0; for K not a
// multiple of 256 those loads and the blocks past K are masked to zero.
template <bool ALIGNED>
__device__ __forceinline__ G16Chunk g16_issue(const G16Args& a, int64_t row0, bool ok, int64_t kl) {
  const int lane = threadIdx.x & (kWave - 1);
  const int q = lane & 3;
  const int64_t row = row0 + (lane >> 2);
  ok = ok && row < a.n;
  const int64_t rr = ok ? row : 0, kc = ok ? kl : 0;
  const uint8_t* cp = a.codes + rr * (a.k / 2) + kc / 2 + 16 * q;
  const uint8_t* sp = a.scales + rr * (a.k / 16) + kc / 16 + 4 * q;
  G16Chunk cr;
  if (ALIGNED) {  // K % 256 == 0: whole chunks, naturally aligned 16- and 4-byte loads
    // Nothing to mask: a chunk past the range is never multiplied, and a row past N only
    // feeds outputs that are never stored (it reads row 0).
    cr.c0 = *(const uint4*)cp;
    cr.c1 = *(const uint4*)(cp + 64);
    cr.s = *(const uint32_t*)sp;
  } else {        // K % 16 == 0: whole 16-element blocks, 8-byte code loads, byte scales
    // chunk byte 64 j + 16 q + 8 h holds block 8 j + 2 q + h; scale byte b is block 4 q + b
    uint32_t cw[8], sb[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool bok = ok && kl + 16 * (8 * j + 2 * q + h) < a.k;
        const uint2 v = *(const uint2*)(cp + (bok ? 64 * j + 8 * h : 0));
        const uint32_t m = opaque_mask(bok);
        cw[4 * j + 2 * h] = v.x & m;
        cw[4 * j + 2 * h + 1] = v.y & m;
      }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool bok = ok && kl + 16 * (4 * q + b) < a.k;
      sb[b] = (uint32_t)sp[bok ? b : 0] & opaque_mask(bok);
    }
    cr.c0 = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    cr.c1 = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    cr.s = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
  }
  return cr;
}

// Loaded chunk -> MFMA layout.  Lane (r, g) takes from lane 4 r + g (row r, bytes 16 g and
// 64 + 16 g): for K step t it then holds the 8 codes of row r at chunk columns
// 128 (t / 4) + 32 g + 8 (t % 4) (g16_kcol), and in byte t / 2 of `s` their block scale
// (blocks 2 g, 2 g + 1, 8 + 2 g, 9 + 2 g, from lanes 4 r + g / 2 and 4 r + 2 + g / 2).
__device__ __forceinline__ int g16_kcol(int g, int t) { return 128 * (t >> 2) + 32 * g + 8 * (t & 3); }
__device__ __forceinline__ G16Chunk g16_transpose(const G16Chunk& cr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  const int src = 4 * (4 * r + g);
  auto bp = [](int addr, uint32_t v) { return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v); };
  G16Chunk c;
  c.c0 = make_uint4(bp(src, cr.c0.x), bp(src, cr.c0.y), bp(src, cr.c0.z), bp(src, cr.c0.w));
  c.c1 = make_uint4(bp(src, cr.c1.x), bp(src, cr.c1.y), bp(src, cr.c1.z), bp(src, cr.c1.w));
  const int sh = 16 * (g & 1);
  const uint32_t lo = bp(4 * (4 * r + (g >> 1)), cr.s) >> sh;
  const uint32_t hi = bp(4 * (4 * r + 2 + (g >> 1)), cr.s) >> sh;
  c.s = (lo & 0xFFFFu) | (hi << 16);
  return c;
}

// Activations x[0 .. mrows) x [c0*256, c1*256) in 16-byte units: thread i takes units
// i + 256 j (j < XU).  They are issued into registers first, so that the code loads issued
// after them do not delay the copy to LDS (memory operations complete in order).  Row i of
// the copy starts at element i * xstride (g16_x_off gives a unit's byte offset, or -1 for a
// unit past the range).  With TAIL (K not a multiple of 256) units past K are zeroed;
// K % 16 == 0 and units are 8-element aligned, so a unit lies entirely inside or entirely
// past K.
// Row of unit u: u / per_row through a float reciprocal taken once, not an integer division
// per unit (about 45 instructions each, ahead of the first code load).  Exact: u < 2^11 and
// per_row = 32 x (chunks per split) <= 2^9, so (u + 1/2) / per_row lies at least 2^-10 from
// an integer, far beyond the error of the rounded reciprocal and product (below 2^-16 here).
__device__ __forceinline__ float g16_row_inv(int per_row) { return 1.0f / (float)per_row; }
__device__ __forceinline__ int g16_row_of(int u, float inv) { return (int)(((float)u + 0.5f) * inv); }

template <int XU, bool TAIL>
__device__ __forceinline__ void g16_x_issue(const G16Args& a, int mrows, int64_t c0, int64_t c1,
                                            i32x4 (&xv)[XU]) {
  const int per_row = (int)(c1 - c0) * (kG16Chunk / 8);
  const int units = mrows * per_row;
  const float inv = g16_row_inv(per_row);
#pragma unroll
  for (int j = 0; j < XU; ++j) {
    const int u = threadIdx.x + kG16Threads * j;
    const int i = g16_row_of(u, inv);
    const int64_t kk = c0 * kG16Chunk + (int64_t)(u - i * per_row) * 8;
    const bool ok = TAIL ? (u < units && kk < a.k) : u < units;
    const i32x4 v = *(const i32x4*)(ok ? a.x + (int64_t)i * a.k + kk : a.x);
    if (TAIL) {
      const int m = (int)opaque_mask(ok);
      xv[j] = i32x4{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
    } else {
      xv[j] = v;
    }
  }
}
// LDS byte offset of unit u (row u / per_row, column 8 (u % per_row)), or -1 past the range.
__device__ __forceinline__ int g16_x_off(const G16Args& a, int u, int per_row, int units, float inv) {
  const int i = g16_row_of(u, inv);
  return u < units ? (i * a.xstride + (u - i * per_row) * 8) * 2 : -1;
}

template <int XU>
__device__ __forceinline__ void g16_x_store(const G16Args& a, uint16_t* xs, int per_row, int units,
                                            const i32x4 (&xv)[XU]) {
  const float inv = g16_row_inv(per_row);
#pragma unroll
  for (int j = 0; j < XU; ++j) {
    const int xo = g16_x_off(a, threadIdx.x + kG16Threads * j, per_row, units, inv);
    if (xo >= 0) *(i32x4*)((char*)xs + xo) = xv[j];
  }
}

// LDS elements after the staged activation rows that read as zero: the B fragments of
// tokens past M come from there (offsets up to 128 + 24 + 8 elements), so that every
// fragment read is one unconditional LDS load at an immediate offset from a per-chunk base.
constexpr int kG16ZeroElems = 160;

// One 256-wide chunk of RT row tiles: 8 K steps of 32, each MFMA'd against MT token tiles.
template <int MT, int RT>
__device__ __forceinline__ void g16_mul_chunk(const G16Args& a, const uint16_t* xs, int mrows,
                                              int col0, const G16Chunk (&cr)[RT], f32x4 (&acc)[RT][MT]) {
  const int r = threadIdx.x & 15;
  const int g = (threadIdx.x & (kWave - 1)) >> 4;
  G16Chunk ct[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) ct[rt] = g16_transpose(cr[rt]);
  // B fragment of token 16 q + r at K step t: 8 elements at column col0 + g16_kcol(g, t)
  const uint16_t* xb[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    const int mi = 16 * q + r;
    xb[q] = mi < mrows ? xs + mi * a.xstride + col0 + 32 * g : xs + mrows * a.xstride;
  }
  // block scales of K steps 2 b and 2 b + 1: byte b of s
  float sc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    sc[rt][0] = __builtin_amdgcn_cvt_f32_fp8((int)ct[rt].s, 0);
    sc[rt][1] = __builtin_amdgcn_cvt_f32_fp8((int)ct[rt].s, 1);
    sc[rt][2] = __builtin_amdgcn_cvt_f32_fp8((int)ct[rt].s, 2);
    sc[rt][3] = __builtin_amdgcn_cvt_f32_fp8((int)ct[rt].s, 3);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    bf16x8 xf[MT];
#pragma unroll
    for (int q = 0; q < MT; ++q)
      xf[q] = __builtin_bit_cast(bf16x8, *(const uint4*)(xb[q] + 128 * (t >> 2) + 8 * (t & 3)));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const G16Chunk& c = ct[rt];
      const uint32_t w = t == 0 ? c.c0.x : t == 1 ? c.c0.y : t == 2 ? c.c0.z : t == 3 ? c.c0.w :
                         t == 4 ? c.c1.x : t == 5 ? c.c1.y : t == 6 ? c.c1.z : c.c1.w;
      const bf16x8 av = gv_dequant8(w, sc[rt][t >> 1]);
#pragma unroll
      for (int q = 0; q < MT; ++q)
        acc[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xf[q], acc[rt][q], 0, 0, 0);
    }
  }
}

// Sum the four waves' tiles in a fixed order; wave w < RT*MT receives tile (w / MT, w % MT).
// The LDS of the staged activations is reused, so every wave must be done reading it.
template <int RT, int MT>
__device__ __forceinline__ f32x4 g16_reduce(const f32x4 (&acc)[RT][MT], uint16_t* xs) {
  f32x4* red = (f32x4*)xs;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < MT; ++q) red[(wave * RT * MT + rt * MT + q) * kWave + lane] = acc[rt][q];
  __syncthreads();
  f32x4 v = {0, 0, 0, 0};
  if (wave < RT * MT) {
#pragma unroll
    for (int w = 0; w < kG16Waves; ++w) v += red[(w * RT * MT + wave) * kWave + lane];
  }
  return v;
}

// All threads: count this workgroup on `cnt` once its device-scope stores have completed;
// true in every thread of the workgroup that arrived last.
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

// LoRA up-projection A operand: row `row` of B, ranks 32 c + 8 g .. +8 (zero past the rank).
// Ranks that are a multiple of 8: one 16-byte load (straight-line).
__device__ __forceinline__ i32x4 g16_b_frag_vec(const G16Args& a, int64_t row, bool ok, int c) {
  const int g = (threadIdx.x & (kWave - 1)) >> 4;
  const int j0 = 32 * c + 8 * g;
  ok = ok && j0 < a.rank;
  return __builtin_bit_cast(i32x4, ld16_or0(a.lora_b + row * a.rank + j0, ok, a.x));
}
// Any rank: element loads.
__device__ __forceinline__ i32x4 g16_b_frag_any(const G16Args& a, int64_t row, bool ok, int c) {
  const int g = (threadIdx.x & (kWave - 1)) >> 4;
  uint32_t w4[4] = {0, 0, 0, 0};
  const int j0 = 32 * c + 8 * g;
  if (ok) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t b0 = j0 + e < a.rank ? a.lora_b[row * a.rank + j0 + e] : 0u;
      const uint32_t b1 = j0 + e + 1 < a.rank ? a.lora_b[row * a.rank + j0 + e + 1] : 0u;
      w4[e / 2] = b0 | (b1 << 16);
    }
  }
  return i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
}

// y[mi][nb .. nb+4) = v (bf16, round to nearest even, or float32), within N.
__device__ __forceinline__ void g16_store(const G16Args& a, int64_t mi, int64_t nb, const f32x4& v) {
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

// ------------------------------------------------------------------ LoRA item
// 16 rows of A times chunks [c0, c1) of x: wave w takes chunks c0 + w, c0 + w + 4, ... and
// loads both MFMA operands straight from memory (each wave reads its own columns of x, so
// staging them in LDS would save nothing).  The waves' tiles are added in LDS, the item's
// partial is stored, and the last item to finish adds all partials in group order and
// publishes t.
template <int MT, bool TAIL>
__device__ __forceinline__ void g16_lora_item(const G16Args& a, uint16_t* xs, int* flag, int64_t id) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int64_t tile = id % a.tiles_l;
  const int64_t cg = id / a.tiles_l;
  const int64_t c0 = cg * a.lc, c1 = min(c0 + a.lc, a.kchunks);
  const int64_t row = tile * 16 + r;

  f32x4 acc[1][MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) acc[0][q] = f32x4{0, 0, 0, 0};
  // rows past the rank or past the tokens read row 0 and are masked to zero
  const uint16_t* abase = a.lora_a + (row < a.rank ? row : 0) * a.k + 64 * g;
  const uint32_t amask = opaque_mask(row < a.rank);
  const uint16_t* xbase[MT];
  uint32_t xmask[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    const int64_t mi = 16 * q + r;
    xbase[q] = a.x + (mi < a.m ? mi : 0) * a.k + 64 * g;
    xmask[q] = opaque_mask(mi < a.m);
  }
  for (int64_t c = c0 + wave; c < c1; c += kG16Waves) {
    uint4 av[8], xv[8][MT];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t kk = c * kG16Chunk + 8 * t;  // column of lane group 0
      if (TAIL) {  // K % 16 == 0: an 8-column unit is inside or past K
        const bool kin = kk + 64 * g < a.k;
        av[t] = ld16_or0(abase + kk, kin && row < a.rank, a.x);
#pragma unroll
        for (int q = 0; q < MT; ++q) xv[t][q] = ld16_or0(xbase[q] + kk, kin && 16 * q + r < a.m, a.x);
      } else {
        av[t] = mask4(*(const uint4*)(abase + kk), amask);
#pragma unroll
        for (int q = 0; q < MT; ++q) xv[t][q] = mask4(*(const uint4*)(xbase[q] + kk), xmask[q]);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q = 0; q < MT; ++q)
        acc[0][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[t]),
                                                            __builtin_bit_cast(bf16x8, xv[t][q]), acc[0][q], 0, 0, 0);
  }
  const f32x4 v = g16_reduce<1, MT>(acc, xs);
  const int64_t lrow = a.tiles_l * 16;
  if (wave < MT) {
    const int64_t mi = 16 * wave + r;
    if (mi < a.m) st_dev4v(dev_rsrc(a.part_l), (uint32_t)(((cg * a.m + mi) * lrow + tile * 16 + 4 * g) * 4), v);
  }
  if (!g16_arrive(g16_ctr(a, g16_line_l(a)), (uint32_t)(a.tiles_l * a.lgroups), flag)) {
    if (threadIdx.x == 0) g16_done(a, id);  // its arrival has returned: done with the counter
    return;
  }

  // last LoRA item: t = bf16(s . (partials added in group order)), published once.  A unit
  // is four ranks of one token; all of its partials are loaded before any is added.
  constexpr int kB = MT == 4 ? 16 : 8;  // partials in flight per unit
  const int rp4 = a.rank_pad / 4;
  const auto rs = dev_rsrc(a.part_l);
  for (int u = threadIdx.x; u < (int)a.m * rp4; u += kG16Threads) {
    const int mi = u / rp4;
    const int j = 4 * (u - mi * rp4);
    const bool in = j < lrow;
    f32x4 sum = {0, 0, 0, 0};
    for (int64_t g0 = 0; g0 < a.lgroups; g0 += kB) {
      f32x4 pv[kB];
#pragma unroll
      for (int e = 0; e < kB; ++e) {
        const int64_t gi = g0 + e < a.lgroups ? g0 + e : 0;
        pv[e] = ld_dev4v(rs, (uint32_t)(((gi * a.m + mi) * lrow + (in ? j : 0)) * 4));
      }
#pragma unroll
      for (int e = 0; e < kB; ++e)
        if (in && g0 + e < a.lgroups) sum += pv[e];
    }
    sum *= a.lora_scale;
    uint32_t* tp = a.t + (mi * a.rank_pad + j) / 2;
    st_dev_u32(tp, f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16));
    st_dev_u32(tp + 1, f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16));
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    st_dev_u32(g16_ctr(a, g16_line_t(a)), 1u);
    wait_stores();  // the flag has reached L2 before this item counts as done
    g16_done(a, id);
  }
}


// Finishing a 64-row streaming tile (wave w: rows row0 .. +16 RT, all four token tiles)
// whose K range is split `nsplit` ways: split partials (device scope) and the last
// arrival's fixed-order sum, S, the LoRA term once t is published, and the store.
template <int RT>
__device__ __forceinline__ void g16_stream_finish(const G16Args& a, int* flag, int64_t tile, int64_t split,
                                                  int nsplit, int64_t row0, f32x4 (&acc)[RT][4], const i32x4 (&bw)[RT][2],
                                                  bool early_b, float ts) {
  constexpr int MT = 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, g = lane >> 4;
  // tiles (rt, q): acc[rt][q] is C[n][m] with m = 16 q + r, n = row0 + 16 rt + 4 g + i
  if (nsplit > 1) {
    const int64_t prow = row0 - 64 * a.full;  // partial rows start at the first split tile
    const auto ws_rs = dev_rsrc(a.part_w);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mi = 16 * q + r;
        if (mi < a.m)
          st_dev4v(ws_rs, (uint32_t)(((split * a.m + mi) * a.n_pad + prow + 16 * rt + 4 * g) * 4), acc[rt][q]);
      }
    if (!g16_arrive(g16_ctr(a, tile), (uint32_t)nsplit, flag)) return;
    // the partials of all MT token tiles in flight together (up to kSB splits each at a time:
    // a device-scope round trip costs microseconds), added in split order
    constexpr int kSB = 8;
    const auto rs = dev_rsrc(a.part_w);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sum[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) sum[q] = f32x4{0, 0, 0, 0};
      for (int sp0 = 0; sp0 < nsplit; sp0 += kSB) {
        f32x4 part[kSB][MT];
#pragma unroll
        for (int u = 0; u < kSB; ++u)
#pragma unroll
          for (int q = 0; q < MT; ++q) {
            const int sp = sp0 + u < nsplit ? sp0 + u : 0;
            const int64_t mi = min((int64_t)(16 * q + r), a.m - 1);
            part[u][q] = ld_dev4v(rs, (uint32_t)((((int64_t)sp * a.m + mi) * a.n_pad + prow + 16 * rt + 4 * g) * 4));
          }
#pragma unroll
        for (int u = 0; u < kSB; ++u)
#pragma unroll
          for (int q = 0; q < MT; ++q)
            if (sp0 + u < nsplit) sum[q] += sp0 + u == split ? acc[rt][q] : part[u][q];
      }
#pragma unroll
      for (int q = 0; q < MT; ++q) acc[rt][q] = sum[q];
    }
    if (threadIdx.x == 0) st_dev_u32(g16_ctr(a, tile), 0u);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[rt][q] *= ts;
  if (a.rank > 0) {
    // bounded wait for t (one poller per workgroup; flag[1] is not the arrival flag, which
    // other waves may still be reading)
    const bool have_t = wait_flag_bounded(g16_ctr(a, g16_line_t(a)), flag + 1);
    if (!have_t) {  // t never came: NaN outputs for this tile, reported in the status word
      if (threadIdx.x == 0) __hip_atomic_fetch_or(a.status, (int32_t)kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int q = 0; q < MT; ++q) acc[rt][q] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    const int rc = have_t ? a.rank_pad / 32 : 0;
#pragma unroll
    for (int c = 0; c < QLINEAR_MAX_RANK / 32; ++c) {
      if (c >= rc) break;
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int64_t mi = 16 * q + r;
        i32x4 tv = {0, 0, 0, 0};
        if (mi < a.m) {
          const uint32_t* tp = a.t + (mi * a.rank_pad + 32 * c + 8 * g) / 2;
          tv = i32x4{(int)ld_dev_u32(tp), (int)ld_dev_u32(tp + 1), (int)ld_dev_u32(tp + 2), (int)ld_dev_u32(tp + 3)};
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int64_t brow = row0 + 16 * rt + r;
          const i32x4 b = early_b ? (c == 0 ? bw[rt][0] : bw[rt][1]) : g16_b_frag_any(a, brow, brow < a.n, c);
          acc[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                               __builtin_bit_cast(bf16x8, tv), acc[rt][q], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave of this workgroup has read t
    if (threadIdx.x == 0) g16_done(a, a.tiles_l * a.lgroups + tile);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < MT; ++q) {
      const int64_t mi = 16 * q + r;
      const int64_t nb = row0 + 16 * rt + 4 * g;
      if (mi < a.m && nb < a.n) g16_store(a, mi, nb, acc[rt][q]);
    }
}

// ------------------------------------------------------------------ many-token weight item
// 33 to 64 tokens: the activations of a whole K range no longer fit in LDS, so the
// workgroup (64 RT rows: wave w owns rows 16 RT w .. +16 RT, all four 16-token tiles) runs
// over its K chunks with the activations of two chunks in LDS (the one being multiplied and
// the next) and those of the chunk after in registers, and the codes of each wave two
// chunks ahead.  Every load is issued unconditionally (clamped past the range) so the
// compiler waits for exactly the data each step needs.
template <int RT, bool ALIGNED>
__device__ __forceinline__ void g16_stream_item(const G16Args& a, uint16_t* xs, int* flag, int64_t id) {
  constexpr int MT = 4;
  constexpr int XU = kG16Chunk / 8 * 16 * MT / kG16Threads;  // 8 activation units per thread
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int64_t tile = id % a.tiles_w;
  const int64_t split = id / a.tiles_w;
  const int64_t c0 = split * a.cps, c1 = min(c0 + a.cps, a.kchunks);
  const int64_t row0 = tile * 64 * RT + 16 * RT * wave;  // this wave's first row
  const int xbuf = 16 * MT * a.xstride;                   // elements per LDS buffer

  // x chunk c -> registers (units u = tid + 256 j: token u / 32, 8 columns at (u % 32) * 8)
  auto x_issue = [&](int64_t c, i32x4 (&xr)[XU]) {
    const int64_t cc = c < c1 ? c : c0;
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      const int u = threadIdx.x + kG16Threads * j;
      const int i = u >> 5;
      const int64_t kk = cc * kG16Chunk + (u & 31) * 8;
      const bool ok = i < a.m && kk < a.k;
      const i32x4 v = *(const i32x4*)(ok ? a.x + (int64_t)i * a.k + kk : a.x);
      if (!ALIGNED || 16 * MT > a.m) {  // zero tokens past m and columns past K
        const int mk = (int)opaque_mask(ok);
        xr[j] = i32x4{v[0] & mk, v[1] & mk, v[2] & mk, v[3] & mk};
      } else {
        xr[j] = v;
      }
    }
  };
  auto x_store = [&](int buf, const i32x4 (&xr)[XU]) {
#pragma unroll
    for (int j = 0; j < XU; ++j) {
      const int u = threadIdx.x + kG16Threads * j;
      *(i32x4*)(xs + buf * xbuf + (u >> 5) * a.xstride + (u & 31) * 8) = xr[j];
    }
  };
  auto c_issue = [&](int64_t c, G16Chunk (&cr)[RT]) {
    const int64_t cc = c < c1 ? c : c0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      cr[rt] = g16_issue<ALIGNED>(a, row0 + 16 * rt, true, cc * kG16Chunk);
    }
  };
  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[rt][q] = f32x4{0, 0, 0, 0};
  auto compute = [&](int buf, const G16Chunk (&cr)[RT]) {
    const uint16_t* xb = xs + buf * xbuf + r * a.xstride;
    G16Chunk ct[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ct[rt] = g16_transpose(cr[rt]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bf16x8 xf[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        xf[q] = gv_zero8();
        if (16 * q + r < a.m) xf[q] = __builtin_bit_cast(bf16x8, *(const uint4*)(xb + 16 * q * a.xstride + g16_kcol(g, t)));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const G16Chunk& c = ct[rt];
        const uint32_t w = t == 0 ? c.c0.x : t == 1 ? c.c0.y : t == 2 ? c.c0.z : t == 3 ? c.c0.w :
                           t == 4 ? c.c1.x : t == 5 ? c.c1.y : t == 6 ? c.c1.z : c.c1.w;
        const bf16x8 av = gv_dequant8(w, e4m3_value((c.s >> (8 * (t >> 1))) & 0xFFu));
#pragma unroll
        for (int q = 0; q < MT; ++q)
          acc[rt][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xf[q], acc[rt][q], 0, 0, 0);
      }
    }
  };

  // LoRA B rows and S first, then the pipeline prologue
  constexpr int kMaxB = 2;
  const bool early_b = a.rank > 0 && a.rank <= kG16EarlyRank && (a.rank & 7) == 0;
  i32x4 bw[RT][kMaxB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t brow = row0 + 16 * rt + r;
#pragma unroll
    for (int c = 0; c < kMaxB; ++c) bw[rt][c] = g16_b_frag_vec(a, brow, early_b && brow < a.n, c);
  }
  const float ts = __hip_atomic_load(a.tensor_scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  i32x4 xr0[XU], xr1[XU];
  G16Chunk cs0[RT], cs1[RT];
  x_issue(c0, xr0);
  x_issue(c0 + 1, xr1);
  c_issue(c0, cs0);
  c_issue(c0 + 1, cs1);
  x_store(0, xr0);
  __syncthreads();
  for (int64_t c = c0; c < c1; c += 2) {
    // chunk c: LDS buffer 0, codes cs0; x(c+1) in flight in xr1
    x_issue(c + 2, xr0);
    compute(0, cs0);
    c_issue(c + 2, cs0);
    if (c + 1 < c1) x_store(1, xr1);
    __syncthreads();
    if (c + 1 >= c1) break;
    // chunk c+1: LDS buffer 1, codes cs1; x(c+2) in flight in xr0
    x_issue(c + 3, xr1);
    compute(1, cs1);
    c_issue(c + 3, cs1);
    if (c + 2 < c1) x_store(0, xr0);
    __syncthreads();
  }

  g16_stream_finish<RT>(a, flag, tile, split, a.splits, row0, acc, bw, early_b, ts);
}

// ------------------------------------------------------------------ 128-wide stage item
// 33 to 64 tokens, K % 128 == 0.  A workgroup owns 64 weight rows and all (up to) 64 tokens
// over its K range, walked in stages of 128 columns.  Each stage's activations (16 KB),
// codes (4 KB) and block scales are copied straight from global memory into LDS
// (global_load_lds, issued as inline assembly), activations three stages deep and codes
// and scales six, so the codes stream five stages ahead of the multiply and no register
// holds data in flight.  Wave w
// takes MFMA K step w (32 columns) of every stage for all 64 rows and all 64 tokens: each
// activation byte is then read from LDS by one wave only, and the four waves' tiles are
// added in LDS in a fixed order at the end (wave w keeps rows 16 w .. +16).
//
// LDS (bytes): activations [0, 49152) as 3 slots of 64 token rows x 256 B, the 16-byte unit
// u of token t at slot u ^ (t % 16); codes [49152, 73728) as 6 slots of 64 rows x 4 parts
// of 16 B (part p = columns 32 p .. +32), part p of row j at position (p + j / 4) % 4 of the
// row's four; scales [73728, 79872) as 6 slots of 64 rows x 8 B (waves 2 and 3 copy a
// second, unread image).  Both placements make every fragment read conflict-free.

constexpr int kS128X = 16384, kS128C = 4096, kS128S = 1024;
constexpr int kS128XSlots = 3, kS128CSlots = 6;
constexpr int kS128COff = kS128XSlots * kS128X;
constexpr int kS128SOff = kS128COff + kS128CSlots * kS128C;
constexpr int kS128Lds = kS128SOff + kS128CSlots * kS128S;  // 79872: two workgroups per CU

__device__ __forceinline__ void g16_stream128_item(const G16Args& a, uint16_t* xs16, int* flag, int64_t id) {
  constexpr int MT = 4;
  uint8_t* smem = (uint8_t*)xs16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int r = lane & 15, g = lane >> 4;
  // the first `full` items take whole tiles (all of K); the remaining tiles are split along K
  int64_t tile, split, s0, s1;
  int nsplit;
  if (id < a.full) {
    tile = id;
    split = 0;
    nsplit = 1;
    s0 = 0;
    s1 = a.kst;
  } else {
    const int64_t tail = a.tiles_w - a.full, j = id - a.full;
    tile = a.full + j % tail;
    split = j / tail;
    nsplit = a.splits;
    s0 = split * a.sps;
    s1 = min(s0 + a.sps, a.kst);
  }
  const int64_t rbase = tile * 64;
  const int64_t row_f = rbase + 16 * wave;
  // No copy of this item is in flight yet: a wait the compiler can see clears what it
  // believes of loads on the kernel's other paths.  Without it, and with copies it could
  // track, it put vmcnt(0) into every stage -- each stage then waited out a whole memory
  // round trip and the copy leads below did nothing (18944 -> 3584 at 64 tokens: 37.9 ->
  // 33.5 us once fixed; deeper rings then gain nothing more).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // per-lane global byte offsets (stage 0) of this wave's copies
  uint32_t xo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 16 * wave + 4 * j + (lane >> 4);
    const int64_t tc = t < a.m ? t : a.m - 1;
    const int u = (lane & 15) ^ (t & 15);
    xo[j] = (uint32_t)((tc * a.k + 8 * u) * 2);
  }
  uint32_t co, so;
  {
    const int rho = 16 * wave + (lane >> 2);
    const int64_t gr = rbase + rho < a.n ? rbase + rho : a.n - 1;
    const int part = ((lane & 3) - ((rho >> 2) & 3)) & 3;
    co = (uint32_t)(gr * (a.k / 2) + 16 * part);
    const int srow = 32 * (wave & 1) + (lane >> 1);
    const int64_t gs = rbase + srow < a.n ? rbase + srow : a.n - 1;
    so = (uint32_t)(gs * (a.k / 16) + 4 * (lane & 1));
  }
  // Copies as inline assembly (lds_copy16/lds_copy4), awaited only by the explicit vmcnt
  // below: through the compiler's builtin, with slot indices known only at run time, the
  // compiler waited for every copy in flight before the stage's LDS reads.
  const uint32_t lb = lds_addr(smem);
  auto dma_x = [&](int64_t st, int slot) {
    const uint8_t* base = (const uint8_t*)a.x + st * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(base, xo[j], lb + slot * kS128X + (4 * wave + j) * 1024);
  };
  auto dma_c = [&](int64_t st, int slot) {
    lds_copy16(a.codes + st * 64, co, lb + kS128COff + slot * kS128C + wave * 1024);
    lds_copy4(a.scales + st * 8, so, lb + kS128SOff + slot * kS128S + wave * 256);
  };
  auto cl = [&](int64_t st) { return st < s1 ? st : s1 - 1; };

  f32x4 acc[4][MT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[i][q] = f32x4{0, 0, 0, 0};

  // issue order: C(s0) X(s0) C(s0+1) X(s0+1) C(s0+2) C(s0+3) C(s0+4), then per stage st the
  // batch X(st+2) C(st+5) (six copies per wave).  Copies complete in issue order, so when
  // stage st is needed the wait leaves in flight the C(st+3) issued after X(st) and the
  // last batch (eight copies; more only in the prologue, where vmcnt(8) merely waits a
  // little longer): codes keep their lead over the activations.
  dma_c(s0, 0);
  dma_x(s0, 0);
  dma_c(cl(s0 + 1), 1);
  dma_x(cl(s0 + 1), 1);
  dma_c(cl(s0 + 2), 2);
  dma_c(cl(s0 + 3), 3);
  dma_c(cl(s0 + 4), 4);
  // Codes and scales of a wave's K step: the four row tiles' 8-element words and their
  // block scales.
  auto read_codes = [&](int slot, uint32_t (&cw)[4], uint32_t (&sb)[4]) {
    const uint8_t* C = smem + kS128COff + slot * kS128C;
    const uint8_t* Sc = smem + kS128SOff + slot * kS128S;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rho = 16 * i + r;
      cw[i] = *(const uint32_t*)(C + (4 * rho + ((wave + (r >> 2)) & 3)) * 16 + 4 * g);
      sb[i] = Sc[rho * 8 + 2 * wave + (g >> 1)];
    }
  };
  // Software pipeline: stage st + 1's weights are dequantized under stage st's MFMAs.  Its
  // codes and scales were issued before X(st), so they have landed for every wave once the
  // stage-st barrier is passed (the copies of C(st + 1) precede X(st) in issue order).  Per
  // MFMA about five VALU instructions of the next stage's dequantization are interleaved.
  // The dequantized weights alternate between two register sets (the loop is unrolled by
  // two stages): a set is rewritten one stage after the MFMAs that read it were issued,
  // instead of right behind them, where each write would wait for the queued MFMAs.
  bf16x8 av[2][4];
  int xsl = 0, csl = 0;
  auto stage = [&](int64_t st, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();  // stage st landed for every wave; nobody reads stage st - 1 any more
    const int xsl2 = xsl + 2 >= kS128XSlots ? xsl + 2 - kS128XSlots : xsl + 2;
    const int csl5 = csl + 5 >= kS128CSlots ? csl + 5 - kS128CSlots : csl + 5;
    const int csl1 = csl + 1 == kS128CSlots ? 0 : csl + 1;
    dma_x(cl(st + 2), xsl2);
    dma_c(cl(st + 5), csl5);
    const uint8_t* X = smem + xsl * kS128X;
    bf16x8 bv[MT];
#pragma unroll
    for (int q = 0; q < MT; ++q)
      bv[q] = *(const bf16x8*)(X + (16 * q + r) * 256 + 16 * ((4 * wave + g) ^ r));
    // the next stage's codes (past the last stage: a clamped copy, dequantized and unused)
    uint32_t cwn[4], sbn[4];
    read_codes(csl1, cwn, sbn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < MT; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cur][i], bv[q], acc[i][q], 0, 0, 0);
      av[nxt][i] = gv_dequant8(cwn[i], e4m3_value(sbn[i]));
    }
#pragma unroll
    for (int u = 0; u < 4 * MT; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five vector ALU
    }
    xsl = xsl + 1 == kS128XSlots ? 0 : xsl + 1;
    csl = csl1;
  };
  {  // the first stage's weights, before the loop (its codes came in the first copies)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();
    uint32_t cw[4], sb[4];
    read_codes(0, cw, sb);
#pragma unroll
    for (int i = 0; i < 4; ++i) av[0][i] = gv_dequant8(cw[i], e4m3_value(sb[i]));
  }
  int64_t st = s0;
  for (; st + 1 < s1; st += 2) {
    stage(st, std::integral_constant<int, 0>{});
    stage(st + 1, std::integral_constant<int, 1>{});
  }
  if (st < s1) stage(st, std::integral_constant<int, 0>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the clamped copies past the range too
  __syncthreads();

  // LoRA B rows of this wave's finishing rows (16 w .. +16) and S: loads the compiler
  // tracks stay out of the copy loop (see the wait at the top)
  const bool early_b = a.rank > 0 && a.rank <= kG16EarlyRank && (a.rank & 7) == 0;
  i32x4 bw[1][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) bw[0][c] = g16_b_frag_vec(a, row_f + r, early_b && row_f + r < a.n, c);
  const float ts = __hip_atomic_load(a.tensor_scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // the four waves' K steps added in wave order; wave w keeps row tile w
  f32x4* red = (f32x4*)smem;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < MT; ++q) red[((wave * 4 + i) * MT + q) * kWave + lane] = acc[i][q];
  __syncthreads();
  f32x4 v[1][MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    f32x4 sum = red[((0 * 4 + wave) * MT + q) * kWave + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += red[((w * 4 + wave) * MT + q) * kWave + lane];
    v[0][q] = sum;
  }
  g16_stream_finish<1>(a, flag, tile, split, nsplit, row_f, v, bw, early_b, ts);
}

// ------------------------------------------------------------------ kernel

template <int MT, int RT, bool ALIGNED, int XU>
__global__ __launch_bounds__(kG16Threads) __attribute__((amdgpu_waves_per_eu(ALIGNED ? (MT == 1 ? 5 : MT == 2 ? 4 : 2) : 1))) void g16_kernel(G16Args a) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ int flag[2];  // [0]: arrival results, [1]: bounded-wait results
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int mrows = (int)min((int64_t)16 * MT, a.m);
  const int64_t items_l = a.tiles_l * a.lgroups;
  int64_t id = blockIdx.x;
  if (id < items_l) {
    g16_lora_item<MT, !ALIGNED>(a, xs, flag, id);
    return;
  }

  // -------------------------------------------------------------------- weight item
  if constexpr (MT == 4) {
    if (a.kst > 0)
      g16_stream128_item(a, xs, flag, id - items_l);
    else
      g16_stream_item<RT, ALIGNED>(a, xs, flag, id - items_l);
  } else {
  id -= items_l;
  const int64_t tile = id % a.tiles_w;
  const int64_t split = id / a.tiles_w;
  const int64_t c0 = split * a.cps, c1 = min(c0 + a.cps, a.kchunks);
  const int64_t row0 = tile * 16 * RT;
  constexpr int kCB = kG16Pairs / RT;  // chunks per wave batch

  i32x4 xv[XU];
  g16_x_issue<XU, !ALIGNED>(a, mrows, c0, c1, xv);
  __builtin_amdgcn_sched_barrier(0);

  // waves w < RT*MT finish output tile (w / MT, w % MT); their B rows do not depend on
  // anything, so small ranks fetch them now
  const bool tile_wave = wave < RT * MT;
  const int rt_e = tile_wave ? wave / MT : 0, q_e = tile_wave ? wave % MT : 0;
  const int64_t brow = row0 + 16 * rt_e + r;
  const bool early_b = a.rank > 0 && a.rank <= kG16EarlyRankFew && (a.rank & 7) == 0;
  const i32x4 bw0 = g16_b_frag_vec(a, brow, early_b && tile_wave && brow < a.n, 0);
  const float ts = __hip_atomic_load(a.tensor_scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_sched_barrier(0);

  // every code load is issued before the activations are copied to LDS: that copy waits
  // for the activations only (issued first), and the codes arrive while it runs
  constexpr int kEarly = XU > 4 ? (RT == 1 ? 2 : 1) : kG16Pairs;
  G16Chunk ca[kCB][RT];
#pragma unroll
  for (int p = 0; p < kEarly; ++p) {
    const int i = p / RT, rt = p % RT;
    const int64_t c = c0 + wave + kG16Waves * i;
    ca[i][rt] = g16_issue<ALIGNED>(a, row0 + 16 * rt, c < c1, c * kG16Chunk);
  }
  const int per_row = (int)(c1 - c0) * (kG16Chunk / 8);
  g16_x_store<XU>(a, xs, per_row, mrows * per_row, xv);
  if (threadIdx.x < kG16ZeroElems / 8)  // the zero fragments of tokens past M
    *(uint4*)(xs + mrows * a.xstride + 8 * threadIdx.x) = make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = kEarly; p < kG16Pairs; ++p) {
    const int i = p / RT, rt = p % RT;
    const int64_t c = c0 + wave + kG16Waves * i;
    ca[i][rt] = g16_issue<ALIGNED>(a, row0 + 16 * rt, c < c1, c * kG16Chunk);
  }
  __syncthreads();

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < MT; ++q) acc[rt][q] = f32x4{0, 0, 0, 0};
  // the plan gives every wave at most kCB chunks
#pragma unroll
  for (int i = 0; i < kCB; ++i) {
    const int64_t c = c0 + wave + kG16Waves * i;
    if (c < c1) g16_mul_chunk<MT, RT>(a, xs, mrows, (int)(c - c0) * kG16Chunk, ca[i], acc);
  }
  f32x4 v = g16_reduce<RT, MT>(acc, xs);

  // v is C[n][m] of tile (rt_e, q_e): m = 16 q_e + r, n = nb + i; undo the row factor
  const int64_t mi = 16 * q_e + r;
  const int64_t nb = row0 + 16 * rt_e + 4 * g;
  if (a.splits > 1) {
    if (tile_wave && mi < a.m) st_dev4v(dev_rsrc(a.part_w), (uint32_t)(((split * a.m + mi) * a.n_pad + nb) * 4), v);
    if (!g16_arrive(g16_ctr(a, tile), (uint32_t)a.splits, flag)) return;
    if (tile_wave) {
      const auto rs = dev_rsrc(a.part_w);
      const int64_t mc = mi < a.m ? mi : a.m - 1;
      f32x4 s = {0, 0, 0, 0};
      for (int sp0 = 0; sp0 < a.splits; sp0 += 8) {  // 8 partials in flight, added in order
        f32x4 part[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = sp0 + u < a.splits ? sp0 + u : 0;
          part[u] = ld_dev4v(rs, (uint32_t)((((int64_t)sp * a.m + mc) * a.n_pad + nb) * 4));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (sp0 + u < a.splits) s += sp0 + u == split ? v : part[u];
      }
      v = s;
    }
    if (threadIdx.x == 0) st_dev_u32(g16_ctr(a, tile), 0u);
  }

  v *= ts;
  if (a.rank > 0) {  // every wave passes the two barriers
    // bounded wait for t, one poller per workgroup (see g16_stream_finish)
    const bool have_t = wait_flag_bounded(g16_ctr(a, g16_line_t(a)), flag + 1);
    if (!have_t) {
      if (threadIdx.x == 0) __hip_atomic_fetch_or(a.status, (int32_t)kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    if (tile_wave && have_t) {
      const int rc = a.rank_pad / 32;
#pragma unroll
      for (int c = 0; c < QLINEAR_MAX_RANK / 32; ++c) {
        if (c >= rc) break;
        const i32x4 b = early_b ? bw0 : g16_b_frag_any(a, brow, brow < a.n, c);
        i32x4 tv = {0, 0, 0, 0};
        if (mi < a.m) {
          const uint32_t* tp = a.t + (mi * a.rank_pad + 32 * c + 8 * g) / 2;
          tv = i32x4{(int)ld_dev_u32(tp), (int)ld_dev_u32(tp + 1), (int)ld_dev_u32(tp + 2), (int)ld_dev_u32(tp + 3)};
        }
        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, tv),
                                                    v, 0, 0, 0);
      }
    }
    __syncthreads();  // every tile wave of this workgroup has read t
    if (threadIdx.x == 0) g16_done(a, a.tiles_l * a.lgroups + tile);
  }
  if (!tile_wave) return;
  if (mi >= a.m || nb >= a.n) return;
  g16_store(a, mi, nb, v);
  }
}

// ------------------------------------------------------------------ planning

static int64_t g16_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static size_t g16_align(size_t b) { return (b + 255) & ~(size_t)255; }

// Counter spacing in the reserved region: a 128-byte line per counter when they fit, else
// the widest power-of-two spacing that fits (0: they do not fit even one word apart).
static int g16_ctr_stride(int64_t tiles_w) {
  const int64_t lines = tiles_w + kG16ExtraLines;
  const int64_t words = (int64_t)((kWsReserved - kWsCounterOff) / 4);
  for (int st = 32; st >= 1; st /= 2)
    if (lines * st <= words) return st;
  return 0;
}

G16Plan plan_g16(int64_t m, int64_t n, int64_t k, int32_t rank) {
  G16Plan p;
  p.kchunks = g16_cdiv(k, kG16Chunk);
  p.tiles_l = rank > 0 ? g16_cdiv(rank, 16) : 0;
  p.rank_pad = rank > 0 ? (int)(g16_cdiv(rank, 32) * 32) : 0;
  // LoRA items: four chunks per wave pass, as many passes as keep the partials to about
  // 32 K groups (16 for more than 32 tokens, whose items cost more per chunk).  The item
  // chain ends in t, which every finishing row tile waits for: at K = 18944 and one token,
  // 32 groups take the call from 18.1 to 16.3 us against 8 groups; at 64 tokens 32 groups
  // cost more than they save.
  const int lgroups_max = m <= 32 ? kG16LoraGroupsFew : kG16LoraGroups64;
  p.lc = kG16Waves * (int)g16_cdiv(p.kchunks, (int64_t)kG16Waves * lgroups_max);
  p.lgroups = rank > 0 ? g16_cdiv(p.kchunks, p.lc) : 0;
  if (m > 32) {
    p.mt = 4;
    p.rt = 1;
    p.tiles_w = g16_cdiv(n, 64);
    p.n_pad = p.tiles_w * 64;
    if (k % 128 == 0 && 64.0 * (double)k * 2.0 < 2147483648.0 && (double)n * (double)(k / 2) < 2147483648.0) {
      // 33..64 tokens, 128-wide stages (g16_stream128_item).  K is split into as many parts
      // as keep every workgroup on a CU of its own (two on one CU run markedly slower than
      // one), at most eight and of at least four stages each: split partials cost 4 M N
      // bytes each way.  More tiles than CUs: whole-tile rounds, then the leftover tiles
      // (when at most half a round) split the same way, so that the last round fills the
      // chip instead of leaving most CUs idle while a few run a second whole tile.
      p.kst = k / 128;
      const int64_t rem = p.tiles_w > kG16CUs ? p.tiles_w % kG16CUs : 0;
      p.full = rem > 0 && rem <= kG16CUs / 2 ? p.tiles_w - rem : 0;
      const int64_t tail = p.tiles_w - p.full;
      int64_t splits = p.tiles_w > kG16CUs && p.full == 0 ? 1 : kG16CUs / tail;
      if (splits > 8) splits = 8;
      if (splits > p.kst / 4) splits = p.kst / 4;
      if (splits < 1) splits = 1;
      p.sps = g16_cdiv(p.kst, splits);
      p.splits = (int)g16_cdiv(p.kst, p.sps);
      if (p.splits == 1) p.full = 0;  // nothing split: every tile whole either way
      p.n_pad = (p.tiles_w - p.full) * 64;  // partials of the split tiles only
      p.cps = 0;
      p.xstride = 0;
      p.lds_bytes = (size_t)kS128Lds;
      p.ctr_stride = g16_ctr_stride(p.tiles_w);
      return p;
    }
    // other K: 64-row workgroups running over 256-wide K chunks.  K is split only when
    // there are too few row tiles to fill the chip (two workgroups on a CU slow each other
    // down more than a longer K loop costs), and into at most eight parts: the last arrival
    // reads the partials in one batch of loads.
    int64_t splits = g16_cdiv(224, p.tiles_w);
    if (splits > 8) splits = 8;
    if (splits > p.kchunks) splits = p.kchunks;
    if (splits < 1) splits = 1;
    p.cps = g16_cdiv(p.kchunks, splits);
    p.splits = (int)g16_cdiv(p.kchunks, p.cps);
    p.xstride = kG16Chunk + 8;
    p.lds_bytes = (size_t)2 * 64 * (size_t)p.xstride * 2;  // two chunks of 64 tokens
    p.ctr_stride = g16_ctr_stride(p.tiles_w);
    return p;
  }
  p.mt = m <= 16 ? 1 : 2;
  // K chunks whose activations fit the LDS budget (at least one for m <= 32)
  int64_t cps_lds = ((int64_t)kG16XBytes / 2 / m - 8) / kG16Chunk;
  if (cps_lds < 1) cps_lds = 1;
  const int64_t items_l = p.tiles_l * p.lgroups;
  // Smallest K split with one batch of loads per wave; one row tile per workgroup if the
  // grid then runs in one round, else two (halves the workgroups of a split).
  for (int rt = 1; rt <= 2; ++rt) {
    const int64_t batch_chunks = (int64_t)kG16Waves * (kG16Pairs / rt);
    int64_t cps = cps_lds < batch_chunks ? cps_lds : batch_chunks;
    int64_t splits = g16_cdiv(p.kchunks, cps);
    cps = g16_cdiv(p.kchunks, splits);
    splits = g16_cdiv(p.kchunks, cps);
    p.rt = rt;
    p.tiles_w = g16_cdiv(n, 16 * rt);
    p.cps = cps;
    p.splits = (int)splits;
    if (items_l + p.tiles_w * splits <= (int64_t)kG16CUs * (p.mt == 1 ? 5 : 4)) break;
  }
  p.n_pad = p.tiles_w * 16 * p.rt;
  const int64_t xcols = p.cps * kG16Chunk;
  p.xstride = (int)(xcols + 8);
  p.lds_bytes = (size_t)m * (size_t)p.xstride * 2 + kG16ZeroElems * 2;
  const size_t red_bytes = (size_t)kG16Waves * p.rt * p.mt * kWave * 16;  // the wave reduction reuses it
  if (p.lds_bytes < red_bytes) p.lds_bytes = red_bytes;
  p.ctr_stride = g16_ctr_stride(p.tiles_w);
  return p;
}

bool g16_plan_ok(const G16Plan& p, int64_t m) {
  if (p.ctr_stride <= 0) return false;
  if (p.mt < 4 && p.cps > (int64_t)kG16Waves * (kG16Pairs / p.rt)) return false;  // one batch per wave
  // partials are read through buffer descriptors with 32-bit byte offsets
  return (double)p.splits * (double)m * (double)p.n_pad * 4.0 < 2147483648.0 &&
         (double)p.lgroups * (double)m * (double)(p.tiles_l * 16) * 4.0 < 2147483648.0;
}

size_t g16_workspace(const G16Plan& p, int64_t m) {
  const size_t t = g16_align((size_t)m * (size_t)p.rank_pad * 2);
  const size_t pw = p.splits > 1 ? g16_align((size_t)p.splits * (size_t)m * (size_t)p.n_pad * 4) : 0;
  const size_t pl = g16_align((size_t)p.lgroups * (size_t)m * (size_t)(p.tiles_l * 16) * 4);
  return t + pw + pl;
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
  a.kst = p.kst;
  a.sps = p.sps;
  a.full = p.full;
  a.ctr = ws_counters(ws);
  a.ctr_stride = p.ctr_stride;
  a.status = ws_status(ws);
  char* w = ws_scratch(ws);
  size_t off = 0;
  a.t = (uint32_t*)(w + off);
  off += g16_align((size_t)m * (size_t)p.rank_pad * 2);
  a.part_w = (float*)(w + off);
  off += p.splits > 1 ? g16_align((size_t)p.splits * (size_t)m * (size_t)p.n_pad * 4) : 0;
  a.part_l = (float*)(w + off);
  const unsigned items = (unsigned)(p.tiles_l * p.lgroups + p.full + (p.tiles_w - p.full) * p.splits);
  const bool aligned = (k % kG16Chunk) == 0;
  if (!g16_plan_ok(p, m)) return hipErrorInvalidValue;  // the C ABI checks this first
  hipError_t e;
#define QL_G16_LAUNCH(MT, RT, AL, XU)                                                          \
  e = hipFuncSetAttribute((const void*)g16_kernel<MT, RT, AL, XU>,                             \
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds_bytes);       \
  if (e != hipSuccess) return e;                                                               \
  g16_kernel<MT, RT, AL, XU><<<items, kG16Threads, p.lds_bytes, s>>>(a);
#define QL_G16_LAUNCH_X(MT, RT, AL) \
  if (m == 1) { QL_G16_LAUNCH(MT, RT, AL, kG16XUnits1) } else { QL_G16_LAUNCH(MT, RT, AL, kG16XUnits) }
#define QL_G16_LAUNCH_A(MT, RT) if (aligned) { QL_G16_LAUNCH_X(MT, RT, true) } else { QL_G16_LAUNCH_X(MT, RT, false) }
  if (p.mt == 1) {
    if (p.rt == 1) { QL_G16_LAUNCH_A(1, 1) } else { QL_G16_LAUNCH_A(1, 2) }
  } else if (p.mt == 2) {
    if (p.rt == 1) {
      if (aligned) { QL_G16_LAUNCH(2, 1, true, kG16XUnits) } else { QL_G16_LAUNCH(2, 1, false, kG16XUnits) }
    } else {
      if (aligned) { QL_G16_LAUNCH(2, 2, true, kG16XUnits) } else { QL_G16_LAUNCH(2, 2, false, kG16XUnits) }
    }
  } else {
    if (aligned) { QL_G16_LAUNCH(4, 1, true, kG16XUnits) } else { QL_G16_LAUNCH(4, 1, false, kG16XUnits) }
  }
#undef QL_G16_LAUNCH_A
#undef QL_G16_LAUNCH_X
#undef QL_G16_LAUNCH
  return hipGetLastError();
}

}  // namespace ql
