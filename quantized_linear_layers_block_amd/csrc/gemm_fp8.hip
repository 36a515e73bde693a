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
// With the page's power-of-two option (closing section) the block scales are E8M0 bytes,
// which is the operand-scale format of gfx950's scaled FP8 MFMA: each lane hands the MFMA
// the scale of the 32 K values it supplies (its weight block's, its token's), the MFMA
// applies both, and accumulates straight into the float32 accumulator -- no fold, no
// per-block vector work (gemm_fp8_pow2_kernel, below, with its own tiling).
//
// Tiling (float32 scales): 256 (n) x 256 (m) per workgroup of eight waves (2 along n x 4
// along m), 128 x 64 per wave (8 x 4 MFMA tiles, 128 float32 accumulators per lane), K step 128.  Operand tiles (32 KB each) are double-buffered in
// LDS (128 KB) with a 16-byte XOR swizzle so that the 16 lanes reading one column of
// 16 rows hit distinct banks; the next K block is fetched into registers while the
// current one is multiplied.  Workgroup ids are remapped so that the tiles an XCD
// (one L2) runs are neighbours, grouped eight m tiles at a time.
#include "common.hpp"
#include "gemm_common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kGThreads = 512;
constexpr int kTile = 256;     // rows of n and of m per workgroup
constexpr int kRowBytes = 128; // one K block of fp8 per LDS row
constexpr int kStagePitch = 272;                 // output staging: bytes per 128-column bf16 row
constexpr int kStagePerWave = 64 * kStagePitch;  // 64 rows per wave
// float32-scale kernel with SW4: a two-slot ring of scale units after the two operand stages
// (per slot 256 activation rows x 16 bytes, then 64 x 16 bytes of weight-block units)
constexpr int kF32ScSlot = 256 * 16 + 64 * 16;
constexpr size_t kFp8Lds = 8 * kStagePerWave > 4 * kTile * kRowBytes + 2 * kF32ScSlot
                               ? 8 * kStagePerWave : 4 * kTile * kRowBytes + 2 * kF32ScSlot;

struct Fp8GemmArgs {
  const uint8_t* xq;
  const void* sx;          // float32 [m][k/128], or E8M0 bytes (power-of-two scales)
  const uint8_t* wq;
  const void* sw;          // float32 [n/128][k/128], or E8M0 bytes (power-of-two scales)
  int64_t m, n, k;
  const uint16_t* t;       // bf16 [m][rank_pad] (lora_scale already applied) or null
  const uint16_t* lora_b;  // bf16 [n][rank]
  int32_t rank;
  int32_t rank_pad;
  void* y;
  int64_t tiles_m, tiles_n;
};

__device__ __forceinline__ i32x8 frag_fp8(const uint8_t* tile, int row, int g) {
  const uint8_t* p = tile + row * kRowBytes;
  const i32x4 lo = *(const i32x4*)(p + swz(row, 2 * g) * 16);
  const i32x4 hi = *(const i32x4*)(p + swz(row, 2 * g + 1) * 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int OUT_F32, bool SW4>
__global__ __launch_bounds__(kGThreads) void gemm_fp8_kernel(Fp8GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];  // [2][A 256x128 | B 256x128]
  constexpr int kStage = 2 * kTile * kRowBytes;

  int64_t tm, tn;
  gemm_tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int64_t n0 = tn * kTile, m0 = tm * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave & 1, wm = wave >> 1;  // wave tile: n 128 wn .. +128, m 64 wm .. +64
  const int r = lane & 15, g = lane >> 4;
  const int64_t kblocks = a.k / 128;

  // Direct global -> LDS copies: one instruction of a wave fills 8 LDS rows (1 KB) with
  // lane l writing row 8 (wave + 8 i) + l / 8, 16-byte slot l % 8.  The slot holds the
  // row's logical chunk swz(row, l % 8) (the swizzle is an XOR, its own inverse), which the
  // fragment reads undo.  Rows past the matrix edge copy the last row; their outputs are never stored.
  // Offsets are relative to the tile's first row, so they fit 32 bits for k < 2^24.
  uint32_t oa[4], ob[4];
  const int64_t n_last = a.n - 1 - n0, m_last = a.m - 1 - m0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * wave + 64 * i + (lane >> 3);
    const uint32_t lc = (uint32_t)swz(row, lane & 7);
    oa[i] = (uint32_t)(row < n_last ? row : n_last) * (uint32_t)a.k + lc * 16;
    ob[i] = (uint32_t)(row < m_last ? row : m_last) * (uint32_t)a.k + lc * 16;
  }
  const uint8_t* wbase = a.wq + n0 * a.k;
  const uint8_t* xbase = a.xq + m0 * a.k;
  // Issued as inline assembly: the compiler would otherwise assume these LDS writes may
  // alias the fragment reads of the other buffer and wait for them before every read.
  // Completion is awaited explicitly (vmcnt 0) before the barrier that ends a K block.
  // Copy q (0..7) of a K block: q < 4 weight rows 64 q.., q >= 4 activation rows.
  auto dma = [&](int64_t kb, int buf, int q) {
    const uint32_t lb = lds_addr(smem + buf * kStage) + 8 * wave * kRowBytes;
    if (q < 4)
      lds_copy16(wbase + kb * 128, oa[q], lb + 64 * q * kRowBytes);
    else
      lds_copy16(xbase + kb * 128, ob[q - 4], lb + (kTile + 64 * (q - 4)) * kRowBytes);
  };
  // Activation scales of the lane's four m rows and the wave's weight-block scale, one K
  // block ahead.
  uint32_t osx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = 64 * wm + 16 * j + r;
    osx[j] = (uint32_t)((row < m_last ? row : m_last) * kblocks);
  }
  const int64_t nblk = (n0 + 128 * wn) / 128;  // the wave's 128-row weight block
  const bool nblk_ok = nblk * 128 < a.n;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  const float* sxbase = (const float*)a.sx + m0 * kblocks;
  const float* swp = (const float*)a.sw + (nblk_ok ? nblk : 0) * kblocks;
  const float swmask = nblk_ok ? 1.0f : 0.0f;
  // SW4 (K a multiple of 512, 16-byte aligned scale arrays): the float scales of four
  // consecutive blocks of a row form one aligned 16-byte unit, copied global -> LDS with
  // the operand copies once per four blocks (waves 0-3: 64 activation rows each, wave 4:
  // the tile's weight blocks n0/128 + lane, clamped) and read from LDS: five 4-byte global
  // loads per lane per block otherwise made the compiler wait at the top of every block.
  constexpr int kScRing = 4 * kTile * kRowBytes;
  const int arow = 64 * (wave & 3) + lane;
  const uint32_t oxu = (uint32_t)((arow < m_last ? arow : m_last) * kblocks * 4);
  const int64_t nb_last = (a.n - 1) / 128 - n0 / 128;
  const uint32_t owu = (uint32_t)((lane < nb_last ? lane : nb_last) * kblocks * 4);
  const uint8_t* sxt = (const uint8_t*)sxbase;
  const uint8_t* swt = (const uint8_t*)((const float*)a.sw + (n0 / 128) * kblocks);
  auto dma_sc = [&](int64_t grp) {  // the units of blocks 4 grp .. 4 grp + 3
    const uint32_t lb = lds_addr(smem + kScRing) + (uint32_t)(grp & 1) * kF32ScSlot;
    if (wave < 4) lds_copy16(sxt + 16 * grp, oxu, lb + wave * 1024);
    else if (wave == 4) lds_copy16(swt + 16 * grp, owu, lb + 4096);
  };
  auto read_sc = [&](int64_t kbk, float (&sx_)[4], float& sw_) {  // block kbk's scales
    const uint8_t* sl = smem + kScRing + (int)((kbk >> 2) & 1) * kF32ScSlot + 4 * (int)(kbk & 3);
    sw_ = *(const float*)(sl + 4096 + 16 * wn);
#pragma unroll
    for (int j = 0; j < 4; ++j) sx_[j] = *(const float*)(sl + 16 * (64 * wm + 16 * j + r));
  };

  float sxn[4] = {0, 0, 0, 0}, swn = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) dma(0, 0, q);
  if (SW4) {
    dma_sc(0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) sxn[j] = sxbase[osx[j]];
    swn = swp[0];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (SW4) read_sc(0, sxn, swn);

  // Software pipeline.  The MFMAs of a K block run fragment by fragment (8 A fragments x
  // 4 B fragments); each MFMA is issued right after the four FMAs that fold the product
  // the same registers held one fragment earlier into its accumulators.  One MFMA and
  // four FMAs per step lets the vector ALU work of one wave proceed while the other
  // wave's MFMA runs (back-to-back MFMAs would hold the issue port instead).  Step 0 of
  // fragment i reads fragment i + 1 from LDS; the next block's copies go out during
  // fragments 0-3.  The block barrier sits before fragment 7, whose steps also load the
  // next block's B fragments, so the next block starts without an LDS wait.  Products of
  // fragment 7 are folded by fragment 0 of the next block with that block's scales
  // (zero products before the first block).
  const f32x4 zero = {0, 0, 0, 0};
  f32x4 p[4] = {zero, zero, zero, zero};
  float sc[4] = {0, 0, 0, 0}, sc_prev[4];
  i32x8 bf[4], af, afn;
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[j] = frag_fp8(smem + kTile * kRowBytes, 64 * wm + 16 * j + r, g);
  af = frag_fp8(smem, 128 * wn + r, g);
  for (int64_t kb = 0; kb < kblocks; ++kb) {
    const int buf = (int)(kb & 1);
    // The last block re-copies itself into the idle buffer, which nothing reads: the
    // copies stay unconditional and the unrolled schedule below stays one basic block.
    const int64_t kn = kb + 1 < kblocks ? kb + 1 : kb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc_prev[j] = sc[j];
      sc[j] = sxn[j] * swn * swmask;
    }
    if (SW4) {
      // kn's group landed at least one block barrier ago: each group's copy goes out two
      // blocks before its first block (its slot was last read a whole group earlier)
      if (((kb + 2) & 3) == 0 && kb + 2 < kblocks) dma_sc((kb + 2) >> 2);
      read_sc(kn, sxn, swn);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) sxn[j] = sxbase[osx[j] + kn];
      swn = swp[kn];
    }
    const uint8_t* As = smem + buf * kStage;
    const uint8_t* An = smem + (buf ^ 1) * kStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i == 7) {
        // this block's LDS reads are done and the next block's copies have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[7][j][e] += sc_prev[j] * p[j][e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i - 1][j][e] += sc[j] * p[j][e];
        }
        p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 127, 0, 127);
        if (j == 0) afn = i < 7 ? frag_fp8(As, 128 * wn + 16 * (i + 1) + r, g) : frag_fp8(An, 128 * wn + r, g);
        if (i < 4 && (j == 1 || j == 2)) dma(kn, buf ^ 1, 2 * i + (j - 1));
        if (i == 7) bf[j] = frag_fp8(An + kTile * kRowBytes, 64 * wm + 16 * j + r, g);
        __builtin_amdgcn_sched_barrier(0);
      }
      af = afn;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[7][j] += sc[j] * p[j];

  // Epilogue: lane holds m = m0 + 64 wm + 16 j + r, n = n0 + 128 wn + 16 i + 4 g + (0..3).
  if (a.rank_pad > 0)
    lora_wave<8, 4>(a.lora_b, a.t, a.rank, a.rank_pad, a.n, a.m, n0 + 128 * wn, m0 + 64 * wm, r, g, acc);
  if (!OUT_F32 && m0 + kTile <= a.m && n0 + kTile <= a.n && (a.n & 7) == 0) {
    // Interior bf16 tile: the wave's 64 (m) x 128 (n) block is transposed through LDS (row
    // pitch 272 bytes keeps the 8-byte writes conflict-free) and leaves as whole 256-byte
    // rows, four rows per store instruction.
    __syncthreads();  // every wave is done with the operand buffers
    uint8_t* stage = smem + wave * kStagePerWave;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = acc[i][j];
        *(uint2*)(stage + (16 * j + r) * kStagePitch + (16 * i + 4 * g) * 2) =
            make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    uint16_t* ybase = (uint16_t*)a.y + (m0 + 64 * wm) * a.n + n0 + 128 * wn + (lane & 15) * 8;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 4 * q + (lane >> 4);
      *(i32x4*)(ybase + row * a.n) = *(const i32x4*)(stage + row * kStagePitch + (lane & 15) * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t mrow = m0 + 64 * wm + 16 * j + r;
        if (mrow < a.m) store4(a.y, OUT_F32, a.n, mrow, n0 + 128 * wn + 16 * i + 4 * g, acc[i][j], a.n);
      }
    }
  }
}

// ------------------------------------------------------------------ power-of-two scales
// With E8M0 scales the MFMAs accumulate in place, so the accumulators need no vector work
// until the epilogue and can live in the accumulation registers: four waves per workgroup,
// each owning 128 (n) x 128 (m) of the 256 x 256 tile (8 x 8 MFMA tiles, 256 accumulators
// per lane).  Per K block a wave then reads 16 operand fragments from LDS for 64 MFMAs
// (512 bytes per MFMA) instead of 12 for 32 (768 bytes): the LDS reads, which otherwise
// take about as long as the MFMAs, drop by a third.  Operand stages, swizzle and copies
// are those of gemm_fp8_kernel (each wave copies 64 rows of each operand); the copies of
// the next block go out during fragments 0-3 and the block barrier sits before fragment 7.
// SW4 (K a multiple of 512 and 4-byte aligned scale arrays): the E8M0 bytes of four
// consecutive K blocks of a row form one aligned word, copied global -> LDS with the
// operand copies once per four blocks (each wave 64 activation rows, wave 0 also the
// tile's two weight blocks) into a two-slot ring after the operand stages; each lane then
// reads its nine scale bytes from LDS.  Nine single-byte global loads per lane per block
// cost about 15% of the kernel's time (measured by leaving them out): the compiler,
// which counts them but not the assembly copies, waited on them at the top of every
// block.  The bytes, and hence the results, are the same either way.
constexpr int kP2Threads = 256;
constexpr int kP2StagePerWave = 128 * kStagePitch;  // 128 rows of 128 bf16 columns per wave
constexpr size_t kP2Lds = 4 * kP2StagePerWave;      // >= the two operand stages (128 KB)
static_assert(kP2Lds >= 4 * kTile * kRowBytes + 2 * 1280, "the scale ring follows the two operand stages");

template <int OUT_F32, bool SW4>
__global__ __launch_bounds__(kP2Threads) void gemm_fp8_pow2_kernel(Fp8GemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];  // [2][A 256x128 | B 256x128]
  constexpr int kStage = 2 * kTile * kRowBytes;

  int64_t tm, tn;
  gemm_tile_coords(a.tiles_m, a.tiles_n, tm, tn);
  const int64_t n0 = tn * kTile, m0 = tm * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave & 1, wm = wave >> 1;  // wave tile: n 128 wn .. +128, m 128 wm .. +128
  const int r = lane & 15, g = lane >> 4;
  const int64_t kblocks = a.k / 128;

  // Copy q (0..15) of a K block: q < 8 weight rows 64 wave + 8 q + lane / 8, q >= 8 the same
  // activation rows; lane l fills 16-byte slot l % 8 with logical chunk swz(row, l % 8).
  uint32_t oa[8], ob[8];
  const int64_t n_last = a.n - 1 - n0, m_last = a.m - 1 - m0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * wave + 8 * i + (lane >> 3);
    const uint32_t lc = (uint32_t)swz(row, lane & 7);
    oa[i] = (uint32_t)(row < n_last ? row : n_last) * (uint32_t)a.k + lc * 16;
    ob[i] = (uint32_t)(row < m_last ? row : m_last) * (uint32_t)a.k + lc * 16;
  }
  const uint8_t* wbase = a.wq + n0 * a.k;
  const uint8_t* xbase = a.xq + m0 * a.k;
  auto dma = [&](int64_t kb, int buf, int q) {
    const uint32_t lb = lds_addr(smem + buf * kStage) + 64 * wave * kRowBytes;
    if (q < 8)
      lds_copy16(wbase + kb * 128, oa[q], lb + 8 * q * kRowBytes);
    else
      lds_copy16(xbase + kb * 128, ob[q - 8], lb + (kTile + 8 * (q - 8)) * kRowBytes);
  };
  // E8M0 scale bytes of the next block, loaded during this one: the wave's 128-row weight
  // block (the A operand's, the same for every lane) and the lane's eight m rows.
  uint32_t osx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = 128 * wm + 16 * j + r;
    osx[j] = (uint32_t)((row < m_last ? row : m_last) * kblocks);
  }
  const int64_t nblk = (n0 + 128 * wn) / 128;
  const bool nblk_ok = nblk * 128 < a.n;
  const uint8_t* sxb = (const uint8_t*)a.sx + m0 * kblocks;
  const uint8_t* swb = (const uint8_t*)a.sw + (nblk_ok ? nblk : 0) * kblocks;
  // SW4 scale ring: slot (group & 1) holds the words of the tile's 256 activation rows
  // (bytes 0..1023) and of its weight blocks n0/128 + 0..63 (clamped; 1024..1279)
  constexpr int kScRing = 2 * kStage, kScSlot = 1280;
  const int arow = 64 * wave + lane;
  const uint32_t oxw = (uint32_t)((arow < m_last ? arow : m_last) * kblocks);
  const int64_t nb_last = (a.n - 1) / 128 - n0 / 128;
  const uint32_t oww = (uint32_t)((lane < nb_last ? lane : nb_last) * kblocks);
  const uint8_t* swt = (const uint8_t*)a.sw + (n0 / 128) * kblocks;
  auto dma_sc = [&](int64_t grp) {  // the words of blocks 4 grp .. 4 grp + 3
    const uint32_t lb = lds_addr(smem + kScRing) + (uint32_t)(grp & 1) * kScSlot;
    lds_copy4(sxb + 4 * grp, oxw, lb + wave * 256);
    if (wave == 0) lds_copy4(swt + 4 * grp, oww, lb + 1024);
  };
  auto read_sc = [&](int64_t kbk, int& sa_, int (&sb_)[8]) {  // block kbk's bytes, from its group's slot
    const uint8_t* sl = smem + kScRing + (int)((kbk >> 2) & 1) * kScSlot + (int)(kbk & 3);
    sa_ = sl[1024 + 4 * wn];
#pragma unroll
    for (int j = 0; j < 8; ++j) sb_[j] = sl[4 * (128 * wm + 16 * j + r)];
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

#pragma unroll
  for (int q = 0; q < 16; ++q) dma(0, 0, q);
  int sa = 0, sb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (SW4) {
    dma_sc(0);
  } else {
    sa = swb[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) sb[j] = sxb[osx[j]];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (SW4) read_sc(0, sa, sb);
  i32x8 bf[8], af, afn;
#pragma unroll
  for (int j = 0; j < 8; ++j) bf[j] = frag_fp8(smem + kTile * kRowBytes, 128 * wm + 16 * j + r, g);
  af = frag_fp8(smem, 128 * wn + r, g);
  for (int64_t kb = 0; kb < kblocks; ++kb) {
    const int buf = (int)(kb & 1);
    const int64_t kn = kb + 1 < kblocks ? kb + 1 : kb;  // the last block re-copies itself into the idle buffer
    // the next block's scales: bytes, or (SW4) from the ring, where kn's group landed at
    // least one block barrier ago: each group's copy goes out two blocks before its first
    // block (its slot was last read a whole group earlier)
    int san = 0, sbn[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (SW4) {
      if (((kb + 2) & 3) == 0 && kb + 2 < kblocks) dma_sc((kb + 2) >> 2);
      read_sc(kn, san, sbn);
    } else {
      san = swb[kn];
#pragma unroll
      for (int j = 0; j < 8; ++j) sbn[j] = sxb[osx[j] + kn];
    }
    const uint8_t* As = smem + buf * kStage;
    const uint8_t* An = smem + (buf ^ 1) * kStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i == 7) {
        // this block's LDS reads are done and the next block's copies have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, sa, 0, sb[j]);
        if (j == 0) afn = i < 7 ? frag_fp8(As, 128 * wn + 16 * (i + 1) + r, g) : frag_fp8(An, 128 * wn + r, g);
        if (i < 4 && (j & 1)) dma(kn, buf ^ 1, 4 * i + (j >> 1));
        if (i == 7) bf[j] = frag_fp8(An + kTile * kRowBytes, 128 * wm + 16 * j + r, g);
        __builtin_amdgcn_sched_barrier(0);
      }
      af = afn;
    }
    sa = san;
#pragma unroll
    for (int j = 0; j < 8; ++j) sb[j] = sbn[j];
  }

  // Epilogue: lane holds m = m0 + 128 wm + 16 j + r, n = n0 + 128 wn + 16 i + 4 g + (0..3).
  if (a.rank_pad > 0)
    lora_wave<8, 8>(a.lora_b, a.t, a.rank, a.rank_pad, a.n, a.m, n0 + 128 * wn, m0 + 128 * wm, r, g, acc);
  if (!OUT_F32 && m0 + kTile <= a.m && n0 + kTile <= a.n && (a.n & 7) == 0) {
    // Interior bf16 tile: the wave's 128 (m) x 128 (n) block goes through LDS (272-byte
    // rows) and leaves as whole 256-byte rows, four rows per store instruction.
    __syncthreads();  // every wave is done with the operand buffers
    uint8_t* stage = smem + wave * kP2StagePerWave;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = acc[i][j];
        *(uint2*)(stage + (16 * j + r) * kStagePitch + (16 * i + 4 * g) * 2) =
            make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    uint16_t* ybase = (uint16_t*)a.y + (m0 + 128 * wm) * a.n + n0 + 128 * wn + (lane & 15) * 8;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int row = 4 * q + (lane >> 4);
      *(i32x4*)(ybase + row * a.n) = *(const i32x4*)(stage + row * kStagePitch + (lane & 15) * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t mrow = m0 + 128 * wm + 16 * j + r;
        if (mrow < a.m) store4(a.y, OUT_F32, a.n, mrow, n0 + 128 * wn + 16 * i + 4 * g, acc[i][j], a.n);
      }
    }
  }
}

hipError_t launch_gemm_fp8(const uint8_t* xq, const void* sx, int64_t m, int64_t n, int64_t k,
                           const uint8_t* wq, const void* sw, bool pow2, const uint16_t* t,
                           const uint16_t* lora_b, int32_t rank, void* y, int out_f32,
                           hipStream_t s) {
  // Copy offsets are 32-bit within a 256-row tile; k is a multiple of the 128 block.
  if (k % 128 != 0 || k >= (int64_t(1) << 24)) return hipErrorInvalidValue;
  if (m <= 0 || n <= 0) return hipSuccess;
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
  const size_t lds = kFp8Lds;
  static_assert(kFp8Lds >= 4 * kTile * kRowBytes, "staging must cover the operand buffers");
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
#define QL_FP8_LAUNCH_W(OF, W)                                                                            \
  {                                                                                                       \
    hipError_t e = hipFuncSetAttribute((const void*)gemm_fp8_kernel<OF, W>,                                \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);             \
    if (e != hipSuccess) return e;                                                                        \
    gemm_fp8_kernel<OF, W><<<grid, kGThreads, lds, s>>>(a);                                                \
  }
  // float32 scale units of four blocks: every row's scales start on a 16-byte boundary
  const bool f4 = (k / 128) % 4 == 0 && ((uintptr_t)sx & 15) == 0 && ((uintptr_t)sw & 15) == 0;
#define QL_FP8_LAUNCH(OF) \
  if (f4) QL_FP8_LAUNCH_W(OF, true) else QL_FP8_LAUNCH_W(OF, false)
#define QL_FP8_P2_LAUNCH_W(OF, W)                                                                         \
  {                                                                                                       \
    hipError_t e = hipFuncSetAttribute((const void*)gemm_fp8_pow2_kernel<OF, W>,                          \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kP2Lds);          \
    if (e != hipSuccess) return e;                                                                        \
    gemm_fp8_pow2_kernel<OF, W><<<grid, kP2Threads, kP2Lds, s>>>(a);                                       \
  }
  // scale words of four blocks: every row's bytes start on a 4-byte boundary
  const bool sw4 = (k / 128) % 4 == 0 && ((uintptr_t)sx & 3) == 0 && ((uintptr_t)sw & 3) == 0;
#define QL_FP8_P2_LAUNCH(OF) \
  if (sw4) QL_FP8_P2_LAUNCH_W(OF, true) else QL_FP8_P2_LAUNCH_W(OF, false)
  if (out_f32) {
    if (pow2) QL_FP8_P2_LAUNCH(1) else QL_FP8_LAUNCH(1)
  } else {
    if (pow2) QL_FP8_P2_LAUNCH(0) else QL_FP8_LAUNCH(0)
  }
#undef QL_FP8_LAUNCH
#undef QL_FP8_P2_LAUNCH
#undef QL_FP8_P2_LAUNCH_W
#undef QL_FP8_LAUNCH_W
  return hipGetLastError();
}

}  // namespace ql
