// Measured compute ceilings of one gfx950 GPU, for scale beside the GEMM measurements
// (measurement infrastructure, not part of the layer's C ABI; loaded by the benchmark only).
//
// qlc_mfma_loop runs `blocks` workgroups of 256 threads; every wave issues `iters` rounds of
// eight independent MFMA chains (no memory traffic, no LDS), so the MFMA pipes are the only
// limit.  kind 0: v_mfma_f32_16x16x32_bf16 (16384 flop each); kind 1: the block-scaled
// v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands and unit E8M0 scales (65536 flop);
// kind 2: v_mfma_f32_16x16x32_f16 (16384); kind 3: v_mfma_f32_32x32x16_bf16 (32768);
// kind 4: v_mfma_f32_32x32x16_f16 (32768); kind 5: v_mfma_scale_f32_32x32x64_f8f6f4
// (131072).
// Thread 0 of every workgroup records, at the start and the end of its loop, the 64-bit
// shader-clock counter (s_memtime) and the constant 100 MHz reference counter
// (s_memrealtime) in times[4 b .. 4 b + 3]; their ratio over the loop is the shader clock
// the workgroup ran at.  The accumulators feed a store that never happens at run time (the
// sum is compared with a value it cannot take) so that no MFMA is dropped.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* sink, uint64_t* times) {
  constexpr bool kWide = KIND >= 3;  // 32x32 output tiles
  typedef typename std::conditional<kWide, f32x16, f32x4>::type acc_t;
  const int lane = threadIdx.x & 63;
  acc_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = acc_t{};
  // small operand values (about 1/64 .. 1/32 as bf16 or f16, 1/16 or so as E4M3) keep the
  // sums finite
  const int wa = (KIND == 2 || KIND == 4) ? 0x24002400 + lane : 0x3C803C80 + lane;
  const int wb = (KIND == 2 || KIND == 4) ? 0x24802480 - lane : 0x3C903C90 - lane;
  const i32x4 a4 = {wa, wa ^ 1, wa ^ 2, wa ^ 3}, b4 = {wb, wb ^ 1, wb ^ 2, wb ^ 3};
  const i32x8 a8 = {0x28282828, 0x28282828 + lane, 0x28282828, 0x28282828, 0x28282828, 0x28282828, 0x28282828, 0x28282828};
  const i32x8 b8 = {0x30303030, 0x30303030, 0x30303030 - lane, 0x30303030, 0x30303030, 0x30303030, 0x30303030, 0x30303030};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (KIND == 0)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                         acc[c], 0, 0, 0);
      else if constexpr (KIND == 1)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127, 0, 127);
      else if constexpr (KIND == 2)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a4), __builtin_bit_cast(f16x8, b4),
                                                        acc[c], 0, 0, 0);
      else if constexpr (KIND == 3)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                         acc[c], 0, 0, 0);
      else if constexpr (KIND == 4)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a4), __builtin_bit_cast(f16x8, b4),
                                                        acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1.0f) sink[blockIdx.x * 256 + threadIdx.x] = s;  // sums of positive products are never -1
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const uint64_t t1 = __builtin_readcyclecounter();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* o = times + 4 * (int64_t)blockIdx.x;
    o[0] = t0;
    o[1] = t1;
    o[2] = r0;
    o[3] = r1;
  }
}

}  // namespace

// sink: float[blocks * 256] (never written in practice), times: uint64[blocks * 4].
// Returns 0 on success, a HIP error code otherwise, -1 for bad arguments.
extern "C" int qlc_mfma_loop(int32_t kind, int64_t blocks, int64_t iters, void* sink, void* times, void* stream) {
  if (kind < 0 || kind > 5 || blocks <= 0 || blocks > (1 << 20) || iters <= 0 || !sink || !times) return -1;
  hipStream_t s = (hipStream_t)stream;
  float* sk = (float*)sink;
  uint64_t* tm = (uint64_t*)times;
  switch (kind) {
    case 0: mfma_loop_kernel<0><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
    case 1: mfma_loop_kernel<1><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
    case 2: mfma_loop_kernel<2><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
    case 3: mfma_loop_kernel<3><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
    case 4: mfma_loop_kernel<4><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
    default: mfma_loop_kernel<5><<<(unsigned)blocks, 256, 0, s>>>(iters, sk, tm); break;
  }
  return (int)hipGetLastError();
}

// flop of one MFMA of the given kind
extern "C" int64_t qlc_mfma_flop(int32_t kind) {
  static const int64_t f[6] = {16384, 65536, 16384, 32768, 32768, 131072};
  return kind >= 0 && kind < 6 ? f[kind] : 0;
}
extern "C" int32_t qlc_chains(void) { return kChains; }
