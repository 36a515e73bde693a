// Device helpers shared by the gfx950 kernels: vector types, bf16 views, the
// E2M1 / E4M3 conversions (hardware instructions whose rounding was checked
// against the format definitions: round to nearest even, ties to the even code;
// the FP4 encoder saturates at 6, the FP8 encoder does not saturate by itself and
// is fed values clamped to +-448), DPP/shuffle reductions and launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;  // LDS operand of ds_read_b64_tr_b16

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16 views

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two floats whose values are exact bf16 numbers -> one packed bf16 pair (a low, b high).
// Truncation is exact here because the low 16 bits are zero.
__device__ __forceinline__ uint32_t pack_exact_bf16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Eight E2M1 weights (one codes dword, low nibble first) times their E4M3 block scale, as
// f16, exactly: the converter gives code * 256 (the power-of-two scale argument is applied
// exactly), and (byte << 7) & 0x3F80 read as f16 is the E4M3 value times 2^-8 (same
// mantissa, exponent rebased; E4M3 subnormals land on f16 subnormals).  The product has
// at most 2 + 4 significant bits and lies in [2^-10, 2688], so the f16 multiply is exact.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t codes, uint32_t scale_byte) {
  const uint32_t s = (scale_byte << 7) & 0x3F80u;
  const f16x2 sp = __builtin_bit_cast(f16x2, s | (s << 16));
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * sp;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * sp;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * sp;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * sp;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (low half = a), round to nearest even, with gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

// |bf16| bit patterns of a packed pair, as two 16-bit unsigned lanes.
__device__ __forceinline__ u16x2 abs_bits2(uint32_t v) {
  uint32_t a = v & 0x7FFF7FFFu;
  return __builtin_bit_cast(u16x2, a);
}
__device__ __forceinline__ u16x2 max_u16x2(u16x2 a, u16x2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ uint32_t hmax_u16x2(u16x2 a) { return a.x > a.y ? a.x : a.y; }

// ----------------------------------------------------------------- codecs

// OCP E4M3FN code -> float (all 256 codes; NaN for 0x7F/0xFF).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// float -> E4M3 code (sign kept), RNE, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  v = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}

// Four floats -> four E4M3 codes in one dword (a lowest byte).  Inputs must be in [-448, 448].
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Eight floats -> eight E2M1 codes in one dword (element 0 in the low nibble), RNE,
// saturating at 6, sign kept (also for -0).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* q) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[0], q[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[2], q[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[4], q[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[6], q[7], 1.0f, 3);
  return r;
}

// Byte `sel` of an E2M1-packed dword -> two floats (low nibble first), exact.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_unpack2(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
}

// fl32(w / d) for a bf16-valued w and a float32 d > 0, given r = 1.0 / (double)d.
// The double product has relative error below 2^-51, while w/d (w with at most 8
// significant bits, d with at most 24) is never closer than ~2^-49 (relative) to a
// float32 rounding midpoint, so rounding the double product to float32 gives the
// correctly rounded float32 quotient.  With r = 0 (d == 0) the result is +-0.
__device__ __forceinline__ float exact_quotient(float w, double r) {
  return (float)((double)w * r);
}

// ------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over lane pairs (l, l^1)
__device__ __forceinline__ uint32_t max_pair(uint32_t v) { return umax(v, dpp_u32<0xB1>(v)); }
// max over each 16-lane DPP row, result in every lane of the row
__device__ __forceinline__ uint32_t max_row16(uint32_t v) {
  v = umax(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = umax(v, dpp_u32<0x140>(v));  // row_mirror
  return v;
}
// max over the whole wave, result in every lane
__device__ __forceinline__ uint32_t max_wave(uint32_t v) {
  v = max_row16(v);
  v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
  v = umax(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// Block-wide max of one value per thread (blockDim.x == NT, a multiple of 64).
template <int NT>
__device__ __forceinline__ uint32_t max_block(uint32_t v, uint32_t* lds /* NT/64 words */) {
  v = max_wave(v);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) lds[wave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = umax(r, lds[i]);
  __syncthreads();
  return r;
}

// Non-finite bf16 magnitude bits: exponent all ones.
constexpr uint32_t kBf16InfBits = 0x7F80u;

}  // namespace ql
