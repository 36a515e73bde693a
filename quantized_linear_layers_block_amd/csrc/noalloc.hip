// qlinear_forward_noalloc: qlinear_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// Instead of a caller-provided workspace it uses `scratch`, a file-scope device array of
// QLINEAR_NOALLOC_MAX_BYTES laid out exactly like a forward workspace (status word and
// counters in the first QLINEAR_WS_RESERVED_BYTES, scratch after them).  Each GPU the
// library runs on holds its own copy until the process ends.  In host code the array's
// name is only a host-side stand-in, so its device address is taken once per device with
// hipGetSymbolAddress and only that address is ever handed to kernels.  The counters must
// be zero before the first call: the set-up clears the reserved region once (the array
// starts zeroed when the code object loads; the clear makes it independent of that), and
// every call returns the counters it used to zero, so nothing is cleared per call.
#include <mutex>

#include "../../include/qlinear.h"
#include "launch.hpp"

namespace ql {

constexpr size_t kNoAllocBytes = QLINEAR_NOALLOC_MAX_BYTES;
static_assert(kNoAllocBytes > kWsReserved, "the array holds the reserved region and scratch");

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once set up
}  // namespace

}  // namespace ql

extern "C" qlinear_status qlinear_forward_noalloc(const qlinear_qweight* w, const uint16_t* x,
                                                  int64_t m, const uint16_t* lora_a,
                                                  const uint16_t* lora_b, int32_t rank,
                                                  float lora_scale, void* y, int32_t out_dtype,
                                                  void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ql::kMaxDevices) return QL_ERR_HIP;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(ql::g_mu);
    ptr = ql::g_ptr[dev];
    if (!ptr) {
      // Set-up on this device: not under stream capture (the clear below is synchronous).
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) return QL_ERR_HIP;
      if (cs != hipStreamCaptureStatusNone) return QL_ERR_ARG;
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(ql::scratch)) != hipSuccess || !p) return QL_ERR_HIP;
      if (hipMemset(p, 0, ql::kWsReserved) != hipSuccess) return QL_ERR_HIP;
      ql::g_ptr[dev] = p;
      ptr = p;
    }
  }
  // Same checks and kernels as qlinear_forward, on the array: a call whose workspace
  // query exceeds the array returns QL_ERR_WORKSPACE having enqueued nothing.
  return ql::forward_impl(w, x, m, lora_a, lora_b, rank, lora_scale, y, out_dtype, ptr,
                          ql::kNoAllocBytes, stream);
}
