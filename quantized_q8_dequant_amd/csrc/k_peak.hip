// Achievable-peak probes for gfx950, the figures the roofline fractions are
// also read against: a streaming copy (HBM read plus write), a streaming
// read, and a loop of int8 MFMAs (v_mfma_i32_32x32x32_i8) on operands held
// in registers.  The streams use nontemporal loads and stores and 8192
// workgroups, the fastest of the forms measured (plain accesses, eight
// loads in flight, 2048 to 65536 workgroups).
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kStreamGrid = 8192;
constexpr int kMfmaChains = 4;  // independent accumulators per wavefront

// dst[i] = src[i] over n 16-byte words, grid-stride, four loads in flight per
// thread before their stores
__global__ void __launch_bounds__(kThreads) k_copy_peak(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                        int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    v4i r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(r[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// The wrapping sum of the 32-bit words of n 16-byte words, one partial per
// wavefront in out[4 * blockIdx.x + wave] (four loads in flight per thread)
__global__ void __launch_bounds__(kThreads) k_read_peak(const v4i* __restrict__ src, int64_t n, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n; i += 4 * stride) {
    v4i r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += (uint32_t)r[u].x + (uint32_t)r[u].y + (uint32_t)r[u].z + (uint32_t)r[u].w;
  }
  for (; i < n; i += stride) {
    const v4i r = src[i];
    acc += (uint32_t)r.x + (uint32_t)r.y + (uint32_t)r.z + (uint32_t)r.w;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc += (uint32_t)__shfl_xor((int)acc, o);
  if (threadIdx.x % kWave == 0) out[(int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave] = acc;
}

// iters rounds of kMfmaChains independent 32x32x32 int8 MFMAs per wavefront,
// every operand byte equal to the low byte of `fill`; each lane writes the
// sum of its accumulator elements (so the work is not dead code and the
// result is checkable: 4 chains x 16 elements x 32 * fill_byte^2 * iters)
__global__ void __launch_bounds__(kThreads) k_mfma_peak(int32_t* __restrict__ out, int iters, int fill) {
  const int b = fill & 0xFF;
  const int w = b | (b << 8) | (b << 16) | (b << 24);
  const v4i x = {w, w, w, w};
  v16i c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x, x, c[k], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[k][e];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

namespace q8k {

hipError_t copy_peak(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t want = (n + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kStreamGrid ? want : kStreamGrid);
  hipLaunchKernelGGL(k_copy_peak, dim3(grid), dim3(kThreads), 0, s, static_cast<const v4i*>(src),
                     static_cast<v4i*>(dst), n);
  return hipGetLastError();
}

int read_peak_partials() { return kStreamGrid * (kThreads / kWave); }

hipError_t read_peak(const void* src, size_t bytes, uint32_t* out, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t want = (n + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < kStreamGrid ? want : kStreamGrid);
  hipLaunchKernelGGL(k_read_peak, dim3(grid), dim3(kThreads), 0, s, static_cast<const v4i*>(src), n, out);
  return hipGetLastError();
}

double mfma_peak_ops(int workgroups, int iters) {
  return (double)workgroups * (kThreads / kWave) * kMfmaChains * (double)iters * (32.0 * 32.0 * 32.0 * 2.0);
}

hipError_t mfma_peak(int32_t* out, int workgroups, int iters, int fill, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(workgroups), dim3(kThreads), 0, s, out, iters, fill);
  return hipGetLastError();
}

}  // namespace q8k
