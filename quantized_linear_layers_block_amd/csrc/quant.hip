// Weight and activation quantizers for gfx950.
//
// NVFP4 (public format definition; QeRL puts the policy's weight path in it,
// tldrocket.com QeRL page, "Key Features of QeRL"): a tensor-wide |w| maximum gives
// the FP32 tensor scale S = amax/2688; every 16-element block along K gets the E4M3
// scale e_b = E4M3(amax_b / (6 S)); elements become E2M1(w / (E4M3(e_b) * S)).
// Because S is global, NVFP4 takes two passes over the bf16 tensor: a maximum pass
// that leaves per-workgroup partial maxima, and an encode pass in which every
// workgroup first reduces those partials (no atomics, no zeroed scratch).
//
// FP8 (mexc.co NeMo RL FP8 page, "De technische doorbraak"): E4M3 with one float32
// scale amax/448 per 128x128 weight tile (one workgroup per tile, one pass) and per
// 1x128 activation segment (16 lanes per segment).
//
// Memory layout and access: bf16 inputs are streamed with 16-byte loads, each wave
// load instruction covering 1 KB of contiguous memory; a 16-element NVFP4 block is
// held by a lane pair (8 elements each) and its maximum is exchanged with one DPP
// move.  Maxima are taken on the integer |bf16| bit patterns, which order like the
// values and are exact.  Element quotients w/d are formed exactly (see
// exact_quotient) and converted by the hardware E2M1/E4M3 encoders.
#include "../../include/qlinear.h"
#include "common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kQThreads = 256;
constexpr int kQUnroll = 4;                                   // 16-byte loads in flight per lane
constexpr int64_t kChunkVec = (int64_t)kQThreads * kQUnroll;  // uint4 (8 bf16) per chunk

// --------------------------------------------------------- NVFP4 building blocks

// Max of |bf16| bits over elements [c*kChunkElems, ...) of a tensor of `nvec` uint4.
__device__ __forceinline__ u16x2 nvfp4_chunk_max(const uint4* __restrict__ w, int64_t nvec,
                                                 int64_t chunk, u16x2 m) {
  const int64_t base = chunk * kChunkVec + threadIdx.x;
  uint4 v[kQUnroll];
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kQThreads;
    v[j] = i < nvec ? w[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    m = max_u16x2(m, abs_bits2(v[j].x));
    m = max_u16x2(m, abs_bits2(v[j].y));
    m = max_u16x2(m, abs_bits2(v[j].z));
    m = max_u16x2(m, abs_bits2(v[j].w));
  }
  return m;
}

struct Nvfp4TensorScale {
  float S;
  float six_S;
  double r6;  // 1 / (double)six_S (0 when S is 0): amax_b / six_S as an exact quotient
};

__device__ __forceinline__ Nvfp4TensorScale nvfp4_tensor_scale(uint32_t amax_bits) {
  Nvfp4TensorScale t;
  const float amax = __uint_as_float(amax_bits << 16);
  t.S = amax / 2688.0f;
  t.six_S = 6.0f * t.S;
  t.r6 = t.six_S > 0.0f ? 1.0 / (double)t.six_S : 0.0;
  return t;
}

// Reciprocals of every block divisor a tensor can use: rtab[e] = 1 / (double)(E4M3(e) * S)
// for the 256 scale codes (0 where the divisor is not positive), so that the encoder looks
// them up instead of dividing once per block.  All threads of the workgroup call this, and
// a barrier must separate it from the table's readers (and from earlier readers).
__device__ __forceinline__ void nvfp4_fill_rtab(double* rtab, float S) {
  for (int e = threadIdx.x; e < 256; e += kQThreads) {
    const float d = e4m3_value((uint32_t)e) * S;
    rtab[e] = d > 0.0f ? 1.0 / (double)d : 0.0;
  }
}

// Encode one chunk: lanes (2i, 2i+1) hold the two halves of one 16-element block.
__device__ __forceinline__ void nvfp4_encode_chunk(const uint4* __restrict__ w, int64_t nvec,
                                                   int64_t chunk, Nvfp4TensorScale ts, const double* rtab,
                                                   uint32_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const int64_t base = chunk * kChunkVec + threadIdx.x;
  uint4 v[kQUnroll];
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kQThreads;
    v[j] = i < nvec ? w[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kQThreads;
    u16x2 m = abs_bits2(v[j].x);
    m = max_u16x2(m, abs_bits2(v[j].y));
    m = max_u16x2(m, abs_bits2(v[j].z));
    m = max_u16x2(m, abs_bits2(v[j].w));
    const uint32_t blk_bits = max_pair(hmax_u16x2(m));
    uint32_t e = 0;  // fl32(amax_b / (6 S)) -> E4M3; the quotient is exact_quotient's
    if (ts.S != 0.0f) e = e4m3_encode(exact_quotient(__uint_as_float(blk_bits << 16), ts.r6));
    const double r = rtab[e];  // 1 / (double)(E4M3(e) * S)
    float q[8];
    q[0] = exact_quotient(bf16_lo(v[j].x), r);
    q[1] = exact_quotient(bf16_hi(v[j].x), r);
    q[2] = exact_quotient(bf16_lo(v[j].y), r);
    q[3] = exact_quotient(bf16_hi(v[j].y), r);
    q[4] = exact_quotient(bf16_lo(v[j].z), r);
    q[5] = exact_quotient(bf16_hi(v[j].z), r);
    q[6] = exact_quotient(bf16_lo(v[j].w), r);
    q[7] = exact_quotient(bf16_hi(v[j].w), r);
    const uint32_t c = e2m1_pack8(q);
    if (i < nvec) {
      codes[i] = c;
      if ((threadIdx.x & 1) == 0) scales[i >> 1] = (uint8_t)e;
    }
  }
}

// ------------------------------------------------------- NVFP4 single-tensor path

__global__ __launch_bounds__(kQThreads) void nvfp4_amax_kernel(const uint4* __restrict__ w,
                                                               int64_t nvec, int64_t nchunks,
                                                               uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[kQThreads / kWave];
  u16x2 m = {0, 0};
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) m = nvfp4_chunk_max(w, nvec, c, m);
  const uint32_t v = max_block<kQThreads>(hmax_u16x2(m), red);
  if (threadIdx.x == 0) partials[blockIdx.x] = v;
}

__global__ __launch_bounds__(kQThreads) void nvfp4_encode_kernel(
    const uint4* __restrict__ w, int64_t nvec, int64_t nchunks,
    const uint32_t* __restrict__ partials, int nparts, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale, int32_t* status) {
  __shared__ uint32_t red[kQThreads / kWave];
  __shared__ double rtab[256];
  uint32_t v = 0;
  for (int i = threadIdx.x; i < nparts; i += kQThreads) v = umax(v, partials[i]);
  const uint32_t amax_bits = max_block<kQThreads>(v, red);
  const Nvfp4TensorScale ts = nvfp4_tensor_scale(amax_bits);
  nvfp4_fill_rtab(rtab, ts.S);
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *tensor_scale = ts.S;
    if (amax_bits >= kBf16InfBits && status != nullptr) atomicOr(status, (int32_t)kStatusNonFinite);
  }
  // Back to front: the tail of the tensor, read last by the maximum pass, is the part
  // most likely still held in the memory-side cache.
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x)
    nvfp4_encode_chunk(w, nvec, nchunks - 1 - c, ts, rtab, codes, scales);
}

static int stream_grid(int64_t nchunks, int cap) {
  return (int)(nchunks < cap ? (nchunks > 0 ? nchunks : 1) : cap);
}

hipError_t launch_nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                 uint8_t* scales, float* tensor_scale, int32_t* status,
                                 uint32_t* partials, hipStream_t s) {
  const int64_t nvec = n * k / 8;
  const int64_t nchunks = (nvec + kChunkVec - 1) / kChunkVec;
  const int gp = stream_grid(nchunks, kAmaxParts);
  nvfp4_amax_kernel<<<gp, kQThreads, 0, s>>>((const uint4*)w, nvec, nchunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ge = stream_grid(nchunks, 4096);
  nvfp4_encode_kernel<<<ge, kQThreads, 0, s>>>((const uint4*)w, nvec, nchunks, partials, gp,
                                               (uint32_t*)codes, scales, tensor_scale, status);
  return hipGetLastError();
}

// ------------------------------------------------------------- FP8 block scale

// Block scale from the block's |bf16| maximum (bit pattern): the float32 multiplier
// amax/448 of the recipe (POW2 false), or the power-of-two option (the mexc.co page's
// closing section): 2^e with e the smallest integer such that amax <= 448 * 2^e, clamped
// to [-127, 127], 0 for an all-zero block (POW2 true).  With amax = (1 + M/128) 2^(E-127)
// (bf16 exponent field E > 0, mantissa M) and 448 = 1.75 * 2^8, e = E - 135 when
// 1 + M/128 <= 1.75 (M <= 96) and E - 134 otherwise; every bf16 subnormal gives e below
// -127.  r is the exact double reciprocal the element quotients use; `stored` is what the
// scale array holds (float32 bits, or the E8M0 byte e + 127).
struct Fp8Scale {
  double r;
  uint32_t stored;
};
template <bool POW2>
__device__ __forceinline__ Fp8Scale fp8_block_scale(uint32_t amax_bits) {
  Fp8Scale o;
  if (!POW2) {
    const float sc = __uint_as_float(amax_bits << 16) / 448.0f;
    o.r = sc > 0.0f ? 1.0 / (double)sc : 0.0;
    o.stored = __float_as_uint(sc);
  } else {
    const int E = (int)(amax_bits >> 7) & 0xFF, M = (int)(amax_bits & 0x7F);
    int e = amax_bits == 0 ? 0 : (E == 0 ? -127 : (M <= 96 ? E - 135 : E - 134));
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    o.r = __longlong_as_double((long long)(1023 - e) << 52);  // 2^-e
    o.stored = (uint32_t)(e + 127);
  }
  return o;
}

// Eight bf16 values (one 16-byte unit) -> eight E4M3 codes (sign | E4M3(fl32(|v| / s))).
__device__ __forceinline__ uint2 fp8_encode8(const uint4& v, double r) {
  float q[8];
  q[0] = exact_quotient(bf16_lo(v.x), r);
  q[1] = exact_quotient(bf16_hi(v.x), r);
  q[2] = exact_quotient(bf16_lo(v.y), r);
  q[3] = exact_quotient(bf16_hi(v.y), r);
  q[4] = exact_quotient(bf16_lo(v.z), r);
  q[5] = exact_quotient(bf16_hi(v.z), r);
  q[6] = exact_quotient(bf16_lo(v.w), r);
  q[7] = exact_quotient(bf16_hi(v.w), r);
#pragma unroll
  for (int t = 0; t < 8; ++t) q[t] = __builtin_amdgcn_fmed3f(q[t], -448.0f, 448.0f);
  uint2 c;
  c.x = e4m3_pack4(q[0], q[1], q[2], q[3]);
  c.y = e4m3_pack4(q[4], q[5], q[6], q[7]);
  return c;
}

// A training step's update applied to eight bf16 weights: bf16_RNE(fl32(w) + fl32(d)).
__device__ __forceinline__ uint4 bf16_add8(const uint4& w, const uint4& d) {
  auto add2 = [](uint32_t a, uint32_t b) { return pack_bf16x2_rne(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b)); };
  return make_uint4(add2(w.x, d.x), add2(w.y, d.y), add2(w.z, d.z), add2(w.w, d.w));
}

// ---------------------------------------------------------------- FP8 weights

// One 128x128 tile per workgroup.  Wave v, lane l holds rows 32v + 4j + l/16 (j = 0..7),
// elements [8 (l%16), 8 (l%16) + 8) of the tile's 128 columns.  With UPDATE the tile is
// first updated (W <- W + delta, written back) and the new values are quantized.
template <bool POW2, bool UPDATE>
__device__ __forceinline__ void fp8_tile(const uint16_t* __restrict__ w, const uint16_t* __restrict__ delta,
                                         int64_t k, int64_t tr, int64_t tc, uint8_t* __restrict__ codes,
                                         void* __restrict__ scales, int32_t* status, uint32_t* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int piece = lane & 15;
  uint4 v[8];
  int64_t off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = tr * 128 + wave * 32 + j * 4 + (lane >> 4);
    off[j] = row * k + tc * 128 + piece * 8;
    v[j] = *(const uint4*)(w + off[j]);
  }
  if (UPDATE) {
    uint4 d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = *(const uint4*)(delta + off[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = bf16_add8(v[j], d[j]);
      *(uint4*)(const_cast<uint16_t*>(w) + off[j]) = v[j];
    }
  }
  u16x2 m = {0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m = max_u16x2(m, abs_bits2(v[j].x));
    m = max_u16x2(m, abs_bits2(v[j].y));
    m = max_u16x2(m, abs_bits2(v[j].z));
    m = max_u16x2(m, abs_bits2(v[j].w));
  }
  const uint32_t amax_bits = max_block<kQThreads>(hmax_u16x2(m), red);
  const Fp8Scale sc = fp8_block_scale<POW2>(amax_bits);
  if (threadIdx.x == 0) {
    if (POW2)
      ((uint8_t*)scales)[tr * (k / 128) + tc] = (uint8_t)sc.stored;
    else
      ((uint32_t*)scales)[tr * (k / 128) + tc] = sc.stored;
    if (amax_bits >= kBf16InfBits && status != nullptr) atomicOr(status, (int32_t)kStatusNonFinite);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) *(uint2*)(codes + off[j]) = fp8_encode8(v[j], sc.r);
}

template <bool POW2>
__global__ __launch_bounds__(kQThreads) void fp8_weight_kernel(const uint16_t* __restrict__ w,
                                                               int64_t k,
                                                               uint8_t* __restrict__ codes,
                                                               void* __restrict__ scales,
                                                               int32_t* status) {
  __shared__ uint32_t red[kQThreads / kWave];
  fp8_tile<POW2, false>(w, nullptr, k, blockIdx.y, blockIdx.x, codes, scales, status, red);
}

hipError_t launch_fp8_weight_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes,
                                      void* scales, bool pow2, int32_t* status, hipStream_t s) {
  dim3 grid((unsigned)(k / 128), (unsigned)(n / 128));
  if (pow2)
    fp8_weight_kernel<true><<<grid, kQThreads, 0, s>>>(w, k, codes, scales, status);
  else
    fp8_weight_kernel<false><<<grid, kQThreads, 0, s>>>(w, k, codes, scales, status);
  return hipGetLastError();
}

// ------------------------------------------------------------ FP8 activations

constexpr int kActSegPerIter = 2;  // segments per 16-lane group per iteration

// Segment = 1x128 of a token row.  16 lanes per segment (8 elements each); a DPP row
// is exactly one segment, so the segment maximum is four DPP moves.
template <bool POW2>
__global__ __launch_bounds__(kQThreads) void fp8_act_kernel(const uint16_t* __restrict__ x,
                                                            int64_t nseg,
                                                            uint8_t* __restrict__ xq,
                                                            void* __restrict__ sx) {
  const int piece = threadIdx.x & 15;
  const int64_t groups = (nseg + (kQThreads / 16) * kActSegPerIter - 1) /
                         ((kQThreads / 16) * kActSegPerIter);
  for (int64_t g = blockIdx.x; g < groups; g += gridDim.x) {
    uint4 v[kActSegPerIter];
    int64_t seg[kActSegPerIter];
#pragma unroll
    for (int j = 0; j < kActSegPerIter; ++j) {
      seg[j] = (g * kActSegPerIter + j) * (kQThreads / 16) + threadIdx.x / 16;
      v[j] = seg[j] < nseg ? *(const uint4*)(x + seg[j] * 128 + piece * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kActSegPerIter; ++j) {
      u16x2 m = abs_bits2(v[j].x);
      m = max_u16x2(m, abs_bits2(v[j].y));
      m = max_u16x2(m, abs_bits2(v[j].z));
      m = max_u16x2(m, abs_bits2(v[j].w));
      const uint32_t amax_bits = max_row16(hmax_u16x2(m));
      const Fp8Scale sc = fp8_block_scale<POW2>(amax_bits);
      const uint2 c = fp8_encode8(v[j], sc.r);
      if (seg[j] < nseg) {
        *(uint2*)(xq + seg[j] * 128 + piece * 8) = c;
        if (piece == 0) {
          if (POW2)
            ((uint8_t*)sx)[seg[j]] = (uint8_t)sc.stored;
          else
            ((uint32_t*)sx)[seg[j]] = sc.stored;
        }
      }
    }
  }
}

hipError_t launch_fp8_act_quantize(const uint16_t* x, int64_t m, int64_t k, uint8_t* xq,
                                   void* sx, bool pow2, hipStream_t s) {
  const int64_t nseg = m * (k / 128);
  const int64_t per_block = (kQThreads / 16) * kActSegPerIter;
  const int64_t groups = (nseg + per_block - 1) / per_block;
  if (pow2)
    fp8_act_kernel<true><<<stream_grid(groups, 4096), kQThreads, 0, s>>>(x, nseg, xq, sx);
  else
    fp8_act_kernel<false><<<stream_grid(groups, 4096), kQThreads, 0, s>>>(x, nseg, xq, sx);
  return hipGetLastError();
}

// ------------------------------------------------ whole-policy requantization
//
// Recalibration after every training step (mexc.co NeMo RL FP8 page, "Praktische
// prestatiewinsten"): the per-tensor quantizer applied to every tensor of the policy,
// grouped into a few launches over all tensors.  The caller's item array lives in device
// memory; a one-workgroup prepare kernel checks every item, numbers the work units of all
// tensors (NVFP4: 8192-element chunks, FP8: 128x128 tiles) and writes the descriptor table
// into the workspace, so nothing crosses from the host per step.
//
// With a device array of dense bf16 updates (one per tensor), the step's update is fused
// in: W <- bf16(fl32(W) + fl32(delta)) is applied, written back and its maximum taken in
// the same pass (NVFP4: the maximum pass; FP8: the one pass over each tile), so the
// requantization itself adds only the encode pass over the new weights.

struct RequantDesc {       // one tensor, as the passes read it
  const uint16_t* w;
  const uint16_t* delta;   // the step's update (fused variant), else null
  void* codes;
  void* scales;
  float* tensor_scale;
  int64_t n, k;
  int64_t unit_begin;      // first work unit of this tensor in the global unit space
  int64_t unit_count;      // 0 for an item that failed its checks
};
struct RequantHeader {
  int32_t count;
  int32_t format;
  int64_t total_units;
};
// Workspace: status word at 0 | header at 16 | descriptors from 64 | maxima[count] (u32)
constexpr size_t kRqHeaderOff = 16, kRqDescOff = 64;

size_t requant_workspace(int32_t count) {
  size_t b = kRqDescOff + (size_t)count * sizeof(RequantDesc) + (size_t)count * 4;
  return (b + 255) & ~(size_t)255;
}

__device__ __forceinline__ int64_t requant_units_dev(int32_t format, int64_t n, int64_t k) {
  if (format == QL_NVFP4) return (n * k / 8 + kChunkVec - 1) / kChunkVec;  // NVFP4 chunks
  return (n / 128) * (k / 128);                                           // FP8 tiles (both kinds)
}

// The checks the host applies to a quantized weight (include/qlinear.h), on the device.
__device__ __forceinline__ bool requant_item_ok(const qlinear_requant_item& it, int32_t format,
                                                const uint16_t* const* deltas, int i) {
  const qlinear_qweight& q = it.q;
  auto al = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  if (deltas && (!deltas[i] || !al(deltas[i]))) return false;
  if (q.format != format || !it.w || !q.codes || !q.scales) return false;
  if (q.n <= 0 || q.k <= 0 || q.n > QLINEAR_MAX_ELEMS / q.k) return false;
  if (!al(it.w) || !al(q.codes) || !al(q.scales)) return false;
  if (format == QL_NVFP4) return q.tensor_scale && al(q.tensor_scale) && q.k % 16 == 0;
  return q.n % 128 == 0 && q.k % 128 == 0;  // both FP8 kinds
}

constexpr int kRqPrepThreads = 1024;
__global__ __launch_bounds__(kRqPrepThreads) void requant_prepare_kernel(const qlinear_requant_item* __restrict__ items,
                                                                         const uint16_t* const* __restrict__ deltas,
                                                                         int32_t count, int32_t format, char* ws) {
  __shared__ int64_t wsum[kRqPrepThreads / kWave];
  RequantHeader* h = (RequantHeader*)(ws + kRqHeaderOff);
  RequantDesc* d = (RequantDesc*)(ws + kRqDescOff);
  int32_t* status = (int32_t*)ws;
  // thread i numbers items [i * per, (i + 1) * per): local sum, block-wide exclusive scan
  const int per = (count + kRqPrepThreads - 1) / kRqPrepThreads;
  const int i0 = threadIdx.x * per, i1 = min(i0 + per, count);
  int64_t local = 0;
  bool bad = false;
  for (int i = i0; i < i1; ++i) {
    const qlinear_requant_item it = items[i];
    const bool ok = requant_item_ok(it, format, deltas, i);
    bad |= !ok;
    local += ok ? requant_units_dev(format, it.q.n, it.q.k) : 0;
  }
  if (bad) atomicOr(status, (int32_t)kStatusBadItem);
  // inclusive scan within the wave, then over the waves' totals
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int64_t v = local;
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  int64_t before = 0, total = 0;
  for (int w = 0; w < kRqPrepThreads / kWave; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int64_t u = before + v - local;
  for (int i = i0; i < i1; ++i) {
    const qlinear_requant_item it = items[i];
    const bool ok = requant_item_ok(it, format, deltas, i);
    RequantDesc r;
    r.w = it.w;
    r.delta = deltas ? deltas[i] : nullptr;
    r.codes = it.q.codes;
    r.scales = it.q.scales;
    r.tensor_scale = it.q.tensor_scale;
    r.n = it.q.n;
    r.k = it.q.k;
    r.unit_begin = u;
    r.unit_count = ok ? requant_units_dev(format, it.q.n, it.q.k) : 0;
    d[i] = r;
    u += r.unit_count;
  }
  if (threadIdx.x == 0) {
    h->count = count;
    h->format = format;
    h->total_units = total;
  }
}

__device__ __forceinline__ int find_tensor(const RequantDesc* __restrict__ d, int count,
                                           int64_t unit) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {  // last tensor whose unit_begin <= unit (the one holding it)
    const int mid = (lo + hi + 1) >> 1;
    if (d[mid].unit_begin <= unit) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kQThreads) void requant_zero_kernel(uint32_t* amax, int count) {
  for (int i = blockIdx.x * kQThreads + threadIdx.x; i < count; i += gridDim.x * kQThreads)
    amax[i] = 0;
}

// UPDATE: one chunk of W <- W + delta written back, and the maximum of the new values.
__device__ __forceinline__ u16x2 nvfp4_chunk_update_max(uint4* __restrict__ w, const uint4* __restrict__ d,
                                                        int64_t nvec, int64_t chunk, u16x2 m) {
  const int64_t base = chunk * kChunkVec + threadIdx.x;
  uint4 v[kQUnroll], dv[kQUnroll];
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kQThreads;
    v[j] = i < nvec ? w[i] : make_uint4(0, 0, 0, 0);
    dv[j] = i < nvec ? d[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kQUnroll; ++j) {
    const int64_t i = base + (int64_t)j * kQThreads;
    v[j] = bf16_add8(v[j], dv[j]);
    if (i < nvec) w[i] = v[j];
    m = max_u16x2(m, abs_bits2(v[j].x));
    m = max_u16x2(m, abs_bits2(v[j].y));
    m = max_u16x2(m, abs_bits2(v[j].z));
    m = max_u16x2(m, abs_bits2(v[j].w));
  }
  return m;
}

// Each workgroup takes a contiguous range of units (so that most of its units belong
// to one tensor) and publishes one integer atomicMax per tensor it touched.
template <bool UPDATE>
__global__ __launch_bounds__(kQThreads) void requant_amax_kernel(const RequantHeader* __restrict__ h,
                                                                 const RequantDesc* __restrict__ d,
                                                                 uint32_t* __restrict__ amax) {
  __shared__ uint32_t red[kQThreads / kWave];
  const int64_t total = h->total_units;
  const int count = h->count;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t u0 = (int64_t)blockIdx.x * per;
  const int64_t u1 = u0 + per < total ? u0 + per : total;
  int64_t u = u0;
  while (u < u1) {
    const int t = find_tensor(d, count, u);
    const int64_t tend = d[t].unit_begin + d[t].unit_count;
    const int64_t stop = tend < u1 ? tend : u1;
    const int64_t nvec = d[t].n * d[t].k / 8;
    u16x2 m = {0, 0};
    if (UPDATE)
      for (; u < stop; ++u)
        m = nvfp4_chunk_update_max((uint4*)const_cast<uint16_t*>(d[t].w), (const uint4*)d[t].delta, nvec,
                                   u - d[t].unit_begin, m);
    else
      for (; u < stop; ++u) m = nvfp4_chunk_max((const uint4*)d[t].w, nvec, u - d[t].unit_begin, m);
    const uint32_t v = max_block<kQThreads>(hmax_u16x2(m), red);
    if (threadIdx.x == 0) atomicMax(amax + t, v);
  }
}

__global__ __launch_bounds__(kQThreads) void requant_encode_kernel(const RequantHeader* __restrict__ h,
                                                                   const RequantDesc* __restrict__ d,
                                                                   const uint32_t* __restrict__ amax,
                                                                   int32_t* status) {
  __shared__ double rtab[256];
  const int64_t total = h->total_units;
  const int count = h->count;
  int t_tab = -1;  // tensor whose divisors rtab holds (uniform over the workgroup)
  // Back to front over the whole table: the most recently read tensors go first.
  for (int64_t i = blockIdx.x; i < total; i += gridDim.x) {
    const int64_t u = total - 1 - i;
    const int t = find_tensor(d, count, u);
    const uint32_t amax_bits = amax[t];
    const Nvfp4TensorScale ts = nvfp4_tensor_scale(amax_bits);
    if (t != t_tab) {
      __syncthreads();  // the previous tensor's table is no longer read
      nvfp4_fill_rtab(rtab, ts.S);
      __syncthreads();
      t_tab = t;
    }
    const int64_t chunk = u - d[t].unit_begin;
    if (chunk == 0 && threadIdx.x == 0) {
      *d[t].tensor_scale = ts.S;
      if (amax_bits >= kBf16InfBits) atomicOr(status, (int32_t)kStatusNonFinite);
    }
    nvfp4_encode_chunk((const uint4*)d[t].w, d[t].n * d[t].k / 8, chunk, ts, rtab,
                       (uint32_t*)d[t].codes, (uint8_t*)d[t].scales);
  }
}

template <bool POW2, bool UPDATE>
__global__ __launch_bounds__(kQThreads) void requant_fp8_kernel(const RequantHeader* __restrict__ h,
                                                                const RequantDesc* __restrict__ d,
                                                                int32_t* status) {
  __shared__ uint32_t red[kQThreads / kWave];
  const int64_t total = h->total_units;
  const int count = h->count;
  for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int t = find_tensor(d, count, u);
    const int64_t tile = u - d[t].unit_begin;
    const int64_t tiles_k = d[t].k / 128;
    fp8_tile<POW2, UPDATE>(d[t].w, d[t].delta, d[t].k, tile / tiles_k, tile % tiles_k, (uint8_t*)d[t].codes,
                           d[t].scales, status, red);
  }
}

// Grids are fixed (the unit count is only known on the device); every kernel loops over
// the units the header announces.
constexpr int kRqAmaxGrid = 4096, kRqEncodeGrid = 4096, kRqFp8Grid = 8192;

hipError_t launch_requant(const void* items, const uint16_t* const* deltas, int32_t count, int32_t format,
                          void* ws, hipStream_t s) {
  char* w = (char*)ws;
  const RequantHeader* dh = (const RequantHeader*)(w + kRqHeaderOff);
  const RequantDesc* dd = (const RequantDesc*)(w + kRqDescOff);
  uint32_t* amax = (uint32_t*)(w + kRqDescOff + (size_t)count * sizeof(RequantDesc));
  int32_t* status = (int32_t*)w;
  requant_prepare_kernel<<<1, kRqPrepThreads, 0, s>>>((const qlinear_requant_item*)items, deltas, count, format, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (format == QL_NVFP4) {
    requant_zero_kernel<<<(count + kQThreads - 1) / kQThreads, kQThreads, 0, s>>>(amax, count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (deltas)
      requant_amax_kernel<true><<<kRqAmaxGrid, kQThreads, 0, s>>>(dh, dd, amax);
    else
      requant_amax_kernel<false><<<kRqAmaxGrid, kQThreads, 0, s>>>(dh, dd, amax);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    requant_encode_kernel<<<kRqEncodeGrid, kQThreads, 0, s>>>(dh, dd, amax, status);
    return hipGetLastError();
  }
  const bool pow2 = format == QL_FP8_POW2;
  if (pow2 && deltas)
    requant_fp8_kernel<true, true><<<kRqFp8Grid, kQThreads, 0, s>>>(dh, dd, status);
  else if (pow2)
    requant_fp8_kernel<true, false><<<kRqFp8Grid, kQThreads, 0, s>>>(dh, dd, status);
  else if (deltas)
    requant_fp8_kernel<false, true><<<kRqFp8Grid, kQThreads, 0, s>>>(dh, dd, status);
  else
    requant_fp8_kernel<false, false><<<kRqFp8Grid, kQThreads, 0, s>>>(dh, dd, status);
  return hipGetLastError();
}

}  // namespace ql
