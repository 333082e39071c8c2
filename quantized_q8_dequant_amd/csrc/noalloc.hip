// The Q8_0 linear for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// qwen3_q8_0_linear takes its scratch (the activation rows quantised per
// 32-block: int8 codes, then f32 scales) from the caller.  This variant
// takes it from a fixed array in device memory instead, so it needs no
// buffer and allocates nothing; it runs the same kernels through that entry
// point.  Each GPU the library runs on holds its own copy of the array until
// the process ends.  Every call on one GPU uses that GPU's copy: two calls
// that overlap on one GPU (for instance on two streams) race.  Nothing in it
// needs to start at zero: the quantiser writes every byte the linear reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qwen3_q8.h"
#include "errors.h"

namespace {

constexpr size_t kScratchBytes = QWEN3_LINEAR_NOALLOC_SCRATCH_BYTES;

// Host code must not pass this name to a kernel: on the host it is only a
// stand-in.  The device address, per device, comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device

// The current device's address of `scratch`, resolved once per device (with
// that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return q8rt::set_error(QWEN3_E_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return q8rt::set_error(QWEN3_E_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return q8rt::set_error(QWEN3_E_DEVICE, "hipGetSymbolAddress of the scratch array failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return QWEN3_OK;
}

}  // namespace

extern "C" int qwen3_q8_0_linear_noalloc(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs,
                                         const uint16_t* d_scale, int64_t n, float* d_y, void* stream) {
  void* work = nullptr;
  if (m > 1 && k > 0) {
    // m * k is bounded before it is formed
    if (m > (int64_t)kScratchBytes || k > (int64_t)kScratchBytes ||
        qwen3_linear_work_bytes(m, k) > kScratchBytes)
      return q8rt::set_error(QWEN3_E_INVALID_ARGUMENT,
                             "m x k too large for the fixed scratch (qwen3_linear_work_bytes(m, k) must not exceed "
                             "QWEN3_LINEAR_NOALLOC_SCRATCH_BYTES)");
    const int rc = scratch_address(&work);
    if (rc != QWEN3_OK) return rc;
  }
  return qwen3_q8_0_linear(d_x, m, k, d_qs, d_scale, n, d_y, work, stream);
}
