// FP8 KV-cache codec for gfx950: the keys and values a rollout engine's attention caches,
// stored as E4M3 codes with one float32 scale per cached (token, head) vector.
//
// The mexc.co NeMo RL FP8 page ("Praktische prestatiewinsten") extends FP8 from the linear
// layers to the KV cache and attention.  Each vector is coded like one of the recipe's
// 1x128 activation segments (head_dim = 128 in the 32B-class geometry): s = amax/448,
// codes sign | E4M3(fl32(|v| / s)).  A store scatters the vectors of `tokens` new tokens
// to cache slots slots[t]; a load gathers slots back to bf16 as bf16(fl32(E4M3(c) * s)).
//
// One lane holds 8 elements (16 bytes of bf16, 8 bytes of codes); the head_dim / 8 lanes of
// a vector form an aligned group inside a wave, so the vector's maximum is a few xor
// shuffles.  Both kernels are streaming copies with one pass over the data.  A slot outside
// [0, cache_slots) is skipped (its load row is zero) and reported in the status word.
#include "../../include/qlinear.h"
#include "common.hpp"
#include "launch.hpp"

namespace ql {

constexpr int kKvThreads = 256;

__device__ __forceinline__ uint32_t group_max(uint32_t v, int lanes) {
  for (int o = lanes >> 1; o >= 1; o >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Token and head of vector v (t = v / heads): a 32-bit division when every vector index
// fits in 32 bits (the host passes `narrow`), else the 64-bit one.
__device__ __forceinline__ void kv_token_head(int64_t v, int heads, bool narrow, int64_t& t, int& h) {
  if (narrow) {
    const uint32_t q = (uint32_t)v / (uint32_t)heads;
    t = q;
    h = (int)((uint32_t)v - q * (uint32_t)heads);
  } else {
    t = v / heads;
    h = (int)(v - t * heads);
  }
}

__global__ __launch_bounds__(kKvThreads) void kv_store_kernel(const uint16_t* __restrict__ kv, int64_t vectors,
                                                              int heads, int head_dim, const int64_t* __restrict__ slots,
                                                              uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                              int64_t cache_slots, int32_t* status, bool narrow) {
  const int lsh = __builtin_ctz((unsigned)head_dim) - 3;  // lanes per vector: head_dim / 8, a power of two
  const int lanes = 1 << lsh;
  const int64_t per_block = kKvThreads >> lsh;
  const int part = (int)(threadIdx.x & (lanes - 1));
  for (int64_t v0 = (int64_t)blockIdx.x * per_block; v0 < vectors; v0 += (int64_t)gridDim.x * per_block) {
    const int64_t v = v0 + (threadIdx.x >> lsh);
    const bool in = v < vectors;
    // every load issued at once, from a clamped vector past the end
    int64_t t;
    int h;
    kv_token_head(in ? v : vectors - 1, heads, narrow, t, h);
    const int64_t slot = slots[t];
    const uint4 x = *(const uint4*)(kv + (in ? v : vectors - 1) * head_dim + part * 8);
    u16x2 m = abs_bits2(x.x);
    m = max_u16x2(m, abs_bits2(x.y));
    m = max_u16x2(m, abs_bits2(x.z));
    m = max_u16x2(m, abs_bits2(x.w));
    const uint32_t amax_bits = group_max(hmax_u16x2(m), lanes);  // every lane of the group
    if (!in) continue;
    if (slot < 0 || slot >= cache_slots) {
      if (part == 0 && status) atomicOr(status, (int32_t)kStatusBadItem);
      continue;
    }
    const float sc = __uint_as_float(amax_bits << 16) / 448.0f;
    const double r = sc > 0.0f ? 1.0 / (double)sc : 0.0;
    float q[8];
    q[0] = exact_quotient(bf16_lo(x.x), r);
    q[1] = exact_quotient(bf16_hi(x.x), r);
    q[2] = exact_quotient(bf16_lo(x.y), r);
    q[3] = exact_quotient(bf16_hi(x.y), r);
    q[4] = exact_quotient(bf16_lo(x.z), r);
    q[5] = exact_quotient(bf16_hi(x.z), r);
    q[6] = exact_quotient(bf16_lo(x.w), r);
    q[7] = exact_quotient(bf16_hi(x.w), r);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i], -448.0f, 448.0f);
    const int64_t dst = (slot * heads + h) * head_dim + part * 8;
    *(uint2*)(codes + dst) = make_uint2(e4m3_pack4(q[0], q[1], q[2], q[3]), e4m3_pack4(q[4], q[5], q[6], q[7]));
    if (part == 0) scales[slot * heads + h] = sc;
  }
}

__global__ __launch_bounds__(kKvThreads) void kv_load_kernel(const uint8_t* __restrict__ codes,
                                                             const float* __restrict__ scales, int64_t cache_slots,
                                                             const int64_t* __restrict__ slots, int64_t vectors,
                                                             int heads, int head_dim, uint16_t* __restrict__ out,
                                                             int32_t* status, bool narrow) {
  const int lsh = __builtin_ctz((unsigned)head_dim) - 3;
  const int lanes = 1 << lsh;
  const int64_t per_block = kKvThreads >> lsh;
  const int part = (int)(threadIdx.x & (lanes - 1));
  for (int64_t v0 = (int64_t)blockIdx.x * per_block; v0 < vectors; v0 += (int64_t)gridDim.x * per_block) {
    const int64_t v = v0 + (threadIdx.x >> lsh);
    if (v >= vectors) continue;
    int64_t t;
    int h;
    kv_token_head(v, heads, narrow, t, h);
    const int64_t slot = slots[t];
    const bool ok = slot >= 0 && slot < cache_slots;
    // the codes and the scale of a slot outside the cache are read from slot 0 and dropped
    const int64_t sv = (ok ? slot : 0) * heads + h;
    const uint2 c = *(const uint2*)(codes + sv * head_dim + part * 8);
    const float sc = scales[sv];
    uint4 o = make_uint4(0, 0, 0, 0);
    if (ok) {
      auto dec2 = [&](uint32_t w, int b) {  // bytes b, b + 1 of w
        return pack_bf16x2_rne(e4m3_value((w >> (8 * b)) & 0xFFu) * sc, e4m3_value((w >> (8 * b + 8)) & 0xFFu) * sc);
      };
      o = make_uint4(dec2(c.x, 0), dec2(c.x, 2), dec2(c.y, 0), dec2(c.y, 2));
    } else if (part == 0 && status) {
      atomicOr(status, (int32_t)kStatusBadItem);
    }
    *(uint4*)(out + v * head_dim + part * 8) = o;
  }
}

static unsigned kv_grid(int64_t vectors, int head_dim) {
  const int64_t per_block = kKvThreads / (head_dim / 8);
  const int64_t blocks = (vectors + per_block - 1) / per_block;
  return (unsigned)(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

hipError_t launch_kv_store(const uint16_t* kv, int64_t tokens, int heads, int head_dim, const int64_t* slots,
                           uint8_t* codes, float* scales, int64_t cache_slots, int32_t* status, hipStream_t s) {
  const int64_t vectors = tokens * heads;
  kv_store_kernel<<<kv_grid(vectors, head_dim), kKvThreads, 0, s>>>(kv, vectors, heads, head_dim, slots, codes,
                                                                     scales, cache_slots, status,
                                                                     vectors <= (int64_t)UINT32_MAX);
  return hipGetLastError();
}

hipError_t launch_kv_load(const uint8_t* codes, const float* scales, int64_t cache_slots, const int64_t* slots,
                          int64_t tokens, int heads, int head_dim, uint16_t* out, int32_t* status, hipStream_t s) {
  const int64_t vectors = tokens * heads;
  kv_load_kernel<<<kv_grid(vectors, head_dim), kKvThreads, 0, s>>>(codes, scales, cache_slots, slots, vectors,
                                                                    heads, head_dim, out, status,
                                                                    vectors <= (int64_t)UINT32_MAX);
  return hipGetLastError();
}

}  // namespace ql
