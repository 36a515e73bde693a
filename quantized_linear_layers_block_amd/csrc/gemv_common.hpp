// Device helpers shared by the few-token NVFP4 kernels: exact dequantization of E2M1
// codes to bf16 MFMA operands, device-scope publication of data that another workgroup
// of the same launch will read, and the bounded wait for such data.
#pragma once

#include "common.hpp"

namespace ql {

// 8 E2M1 codes (one dword) times one block scale -> 8 exact bf16 values.
__device__ __forceinline__ bf16x8 gv_dequant8(uint32_t c, float sc) {
  const f32x2 p0 = e2m1_unpack2<0>(c), p1 = e2m1_unpack2<1>(c), p2 = e2m1_unpack2<2>(c),
              p3 = e2m1_unpack2<3>(c);
  i32x4 o = {(int)pack_exact_bf16(p0.x * sc, p0.y * sc), (int)pack_exact_bf16(p1.x * sc, p1.y * sc),
             (int)pack_exact_bf16(p2.x * sc, p2.y * sc), (int)pack_exact_bf16(p3.x * sc, p3.y * sc)};
  return __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ bf16x8 gv_zero8() {
  i32x4 z = {0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

// Cross-workgroup publication.  Data another workgroup will read is stored with
// device-scope (write-through, "sc1") stores and read with device-scope loads, so no
// L2-wide write-back or invalidate is needed; s_waitcnt 0 makes sure those stores have
// completed before the counter or flag that announces them is touched.
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// 16-byte loads with the same cache policy as the device-scope loads above (sc1), through
// a raw buffer descriptor over `base` (byte offsets below 2^31): one instruction per 16
// bytes, so that a thread can keep many partial tiles in flight at once.
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_dev4v(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, kCpolSc1));
}
// The matching 16-byte store (same sc1 policy as st_dev_u32):
// partial tiles leave as whole 16-byte pieces.
__device__ __forceinline__ void st_dev4v(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), rs, (int)byte_off, 0, kCpolSc1);
}

// Bounded wait for a flag raised by another workgroup of the same launch.  Thread 0 polls
// with device-scope loads for at most kWaitTicks ticks of the 100 MHz real-time counter
// (250 ms; a launch whose workgroups all make progress never comes near it) and
// broadcasts whether it saw the flag through `seen`.  Every thread of the workgroup calls
// it.  A wait that gives up is reported by the caller (status word, NaN outputs), never
// passed over silently.
constexpr uint64_t kWaitTicks = 25000000;
__device__ __forceinline__ bool wait_flag_bounded(const uint32_t* f, int* seen) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = ld_dev_u32(f) != 0u;
    while (!ok && __builtin_amdgcn_s_memrealtime() - t0 < kWaitTicks) {
      __builtin_amdgcn_s_sleep(4);
      ok = ld_dev_u32(f) != 0u;
    }
    *seen = ok;
  }
  __syncthreads();
  return *seen != 0;
}

}  // namespace ql
