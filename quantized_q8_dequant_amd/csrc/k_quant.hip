// Q8_0 encode / repack / embedding gather / row quantisation kernels (gfx950).
//
// Q8_0 block format and encoder: Fucina course, "Model files and
// quantization", section 11.7.  Embedding gather: Fucina course, "A
// transformer from scratch", section 12.3.1 (rows dequantised on the fly).
// RMSNorm: the same page, section 12.3.2.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

// f32 values -> Q8_0 wire blocks (34 bytes: f16 d, 32 x int8).  One 8-lane
// group per block, 4 values per lane.
__global__ void __launch_bounds__(256) k_encode_q8_0(const float* __restrict__ x, int64_t nblocks,
                                                     uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  const bool live = blk < nblocks;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float4 t = *reinterpret_cast<const float4*>(x + blk * 32 + sub * 4);
    v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
  }
  float d;
  const int packed = quant4_group8(v, &d);  // all 8 lanes of a group share liveness
  if (live) {
    uint8_t* b = out + blk * 34;
    if (sub == 0) {
      const uint16_t h = f32_to_f16_bits(d);
      b[0] = (uint8_t)(h & 0xFF);
      b[1] = (uint8_t)(h >> 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) b[2 + sub * 4 + i] = (uint8_t)((packed >> (8 * i)) & 0xFF);
  }
}

__global__ void k_encode_bf16(const float* __restrict__ x, int64_t n, uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = f32_to_bf16_bits(x[i]);
}

// Wire blocks -> planes: qs int8 [rows, k] at row stride k, scales f16 [rows, k/32].
// dst_row0 lets the runtime stack several matrices into one plane;
// interleave_off >= 0 places source row r at stacked row
// dst_row0 + (r / 32) * 64 + interleave_off + r % 32
// (gate/up pairing: each 64-row group = 32 gate rows then 32 up rows).
__global__ void k_repack_q8_0(const uint8_t* __restrict__ src, int64_t rows, int64_t k, int8_t* __restrict__ qs,
                              uint16_t* __restrict__ sc, int64_t dst_row0, int interleave_off) {
  const int64_t nb = k / 32;
  const int64_t total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb, b = i % nb;
    int64_t dr = dst_row0 + r;
    if (interleave_off >= 0) dr = dst_row0 + (r / 32) * 64 + interleave_off + (r % 32);
    const uint8_t* s = src + i * 34;
    sc[dr * nb + b] = (uint16_t)(s[0] | (s[1] << 8));
    int8_t* q = qs + dr * k + b * 32;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) q[j] = (int8_t)s[2 + j];
  }
}

// bf16 rows copied into a stacked plane (same stacking rules as above).
__global__ void k_repack_bf16(const uint16_t* __restrict__ src, int64_t rows, int64_t k, uint16_t* __restrict__ dst,
                              int64_t dst_row0, int interleave_off) {
  const int64_t total = rows * k;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / k, c = i % k;
    int64_t dr = dst_row0 + r;
    if (interleave_off >= 0) dr = dst_row0 + (r / 32) * 64 + interleave_off + (r % 32);
    dst[dr * k + c] = src[i];
  }
}

// Embedding gather: x[t, :] = dequant(token_embd[tok[t], :]) (exact in f32).
// Token ids are clamped into [0, vocab) (device-side ids cannot be checked
// on the host without a synchronisation).
__global__ void __launch_bounds__(256) k_embed_q8_0(const int32_t* __restrict__ tok, int vocab, int H,
                                                    const int8_t* __restrict__ qs, const uint16_t* __restrict__ sc,
                                                    float* __restrict__ x) {
  const int t = blockIdx.x;
  int id = tok[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  const int8_t* row = qs + (int64_t)id * H;
  const uint16_t* srow = sc + (int64_t)id * (H / 32);
  for (int c = threadIdx.x; c < H; c += blockDim.x)
    x[(int64_t)t * H + c] = f16_bits_to_f32(srow[c >> 5]) * (float)row[c];
}

__global__ void __launch_bounds__(256) k_embed_bf16(const int32_t* __restrict__ tok, int vocab, int H,
                                                    const uint16_t* __restrict__ w, float* __restrict__ x) {
  const int t = blockIdx.x;
  int id = tok[t];
  id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
  for (int c = threadIdx.x; c < H; c += blockDim.x)
    x[(int64_t)t * H + c] = bf16_bits_to_f32(w[(int64_t)id * H + c]);
}

// Row-wise (optional RMSNorm) + Q8_0 quantisation: one workgroup per row.
// x [T, K] f32 -> qa int8 [T, K], da f32 [T, K/32] (the f32 value of f16(d)).
// norm_w == nullptr skips the norm.  K % 32 == 0.
__global__ void __launch_bounds__(256) k_rows_quant(const float* __restrict__ x, int K, const float* __restrict__ norm_w,
                                                    float eps, int8_t* __restrict__ qa, float* __restrict__ da,
                                                    uint16_t* __restrict__ da_bits, int blocked) {
  __shared__ double s_red[4];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * K;
  double r = 1.0;
  if (norm_w) {
    double ss = 0.0;
    for (int c = threadIdx.x * 4; c < K; c += 256 * 4) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
    ss = block_sum_d<256>(ss, s_red);
    r = rms_scale(ss, K, eps);
  }
  // every thread takes part in each pass (groups of 8 lanes stay uniform)
  for (int base = 0; base < K; base += 256 * 4) {
    const int c = base + threadIdx.x * 4;
    const bool live = c < K;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      const float4 t4 = *reinterpret_cast<const float4*>(xr + c);
      v[0] = t4.x, v[1] = t4.y, v[2] = t4.z, v[3] = t4.w;
      if (norm_w) {
        const float4 w4 = *reinterpret_cast<const float4*>(norm_w + c);
        v[0] = rms_apply(v[0], r, w4.x), v[1] = rms_apply(v[1], r, w4.y);
        v[2] = rms_apply(v[2], r, w4.z), v[3] = rms_apply(v[3], r, w4.w);
      }
    }
    float d;
    const int packed = quant4_group8(v, &d);
    if (live) {
      const int64_t T = gridDim.x, b = c / 32;
      *reinterpret_cast<int*>(qa + (blocked ? (b * T + t) * 32 + c % 32 : t * K + c)) = packed;
      if ((threadIdx.x & 7) == 0) {
        const int64_t bi = blocked ? b * T + t : t * (K / 32) + b;
        if (da) da[bi] = f16_round(d);
        if (da_bits) da_bits[bi] = f32_to_f16_bits(d);
      }
    }
  }
}

// KV slab export: [nkv][cap][hd] (f32 or bf16) rows [0, len) -> f32 [nkv][len][hd].
// (KV_Q8_0: code times its block's f16 scale, exact in f32.)
__global__ void k_kv_export(const void* src, const uint16_t* __restrict__ srcs, int kvt, int nkv, int cap, int len,
                            int hd, float* __restrict__ dst) {
  const int64_t total = (int64_t)nkv * len * hd;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = i / ((int64_t)len * hd), rem = i % ((int64_t)len * hd);
    const int64_t si = g * (int64_t)cap * hd + rem;
    float v;
    if (kvt == KV_BF16)
      v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(src)[si]);
    else if (kvt == KV_Q8_0)
      v = (float)reinterpret_cast<const int8_t*>(src)[si] * f16_bits_to_f32(srcs[si / 32]);
    else
      v = reinterpret_cast<const float*>(src)[si];
    dst[i] = v;
  }
}

// ---- launchers -------------------------------------------------------------------------
namespace q8k {

hipError_t encode_q8_0(const float* x, int64_t n, void* out, hipStream_t s) {
  const int64_t nb = n / 32;
  if (nb == 0) return hipSuccess;
  const int64_t threads = nb * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(k_encode_q8_0, dim3((unsigned)grid), dim3(256), 0, s, x, nb, (uint8_t*)out);
  return hipGetLastError();
}

hipError_t encode_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_encode_bf16, dim3((unsigned)grid), dim3(256), 0, s, x, n, out);
  return hipGetLastError();
}

hipError_t repack_q8_0(const void* src, int64_t rows, int64_t k, int8_t* qs, uint16_t* sc, int64_t dst_row0,
                       int interleave_off, hipStream_t s) {
  const int64_t total = rows * (k / 32);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_repack_q8_0, dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t*)src, rows, k, qs, sc,
                     dst_row0, interleave_off);
  return hipGetLastError();
}

hipError_t repack_bf16(const void* src, int64_t rows, int64_t k, uint16_t* dst, int64_t dst_row0, int interleave_off,
                       hipStream_t s) {
  const int64_t total = rows * k;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_repack_bf16, dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)src, rows, k, dst,
                     dst_row0, interleave_off);
  return hipGetLastError();
}

hipError_t embed(const int32_t* tok, int T, int vocab, int H, const void* w, const uint16_t* sc, bool bf16, float* x,
                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(k_embed_bf16, dim3(T), dim3(256), 0, s, tok, vocab, H, (const uint16_t*)w, x);
  else
    hipLaunchKernelGGL(k_embed_q8_0, dim3(T), dim3(256), 0, s, tok, vocab, H, (const int8_t*)w, sc, x);
  return hipGetLastError();
}

hipError_t kv_export(const void* src, const uint16_t* srcs, int kvt, int nkv, int cap, int len, int hd, float* dst,
                     hipStream_t s) {
  const int64_t total = (int64_t)nkv * len * hd;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(k_kv_export, dim3((unsigned)grid), dim3(256), 0, s, src, srcs, kvt, nkv, cap, len, hd, dst);
  return hipGetLastError();
}

// Greedy pick of every row of f32 logits [T, V] ("A transformer from
// scratch", section 12.6: the argmax over the vocabulary; among equal maxima
// the lowest index, as in the other argmax epilogues).  Grid (slices, T):
// each workgroup scans one slice of a row (lanes in ascending strided order,
// then a (value, index) reduction), folds its best into the row's 64-bit key
// with an atomic max (order-preserving value bits above, inverted index
// below), and the last workgroup of the row writes the index and clears the
// key and counter for the next launch.
constexpr int kArgmaxSlice = 4096;  // logits per workgroup

__device__ __forceinline__ void argmax_take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) bv = v, bi = i;
}

__global__ void __launch_bounds__(256) k_rows_argmax(const float* __restrict__ x, int V, int32_t* __restrict__ out,
                                                     unsigned long long* key, unsigned* counter, int32_t* len,
                                                     const int32_t* row_seq, int len_add) {
  __shared__ float s_v[256 / kWave];
  __shared__ int s_i[256 / kWave];
  const int row = blockIdx.y;
  const float* xr = x + (int64_t)row * V;
  const int c0 = blockIdx.x * kArgmaxSlice, c1 = min(V, c0 + kArgmaxSlice);
  float bv = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  if ((V & 3) == 0) {
    const float4* x4 = reinterpret_cast<const float4*>(xr);
    for (int c = c0 / 4 + threadIdx.x; c < c1 / 4; c += 256) {
      const float4 t = x4[c];
      argmax_take(bv, bi, t.x, 4 * c);
      argmax_take(bv, bi, t.y, 4 * c + 1);
      argmax_take(bv, bi, t.z, 4 * c + 2);
      argmax_take(bv, bi, t.w, 4 * c + 3);
    }
  } else {
    for (int c = c0 + threadIdx.x; c < c1; c += 256) argmax_take(bv, bi, xr[c], c);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    argmax_take(bv, bi, ov, oi);
  }
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) s_v[wave] = bv, s_i[wave] = bi;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 256 / kWave; ++w) argmax_take(bv, bi, s_v[w], s_i[w]);
    const uint32_t u = __float_as_uint(bv + 0.0f);  // -0 -> +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const unsigned long long k = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)bi);
    __hip_atomic_fetch_max(key + row, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_memory();
    const unsigned prev = arrive(counter + row);
    if (prev == gridDim.x - 1) {  // last workgroup of this row
      const unsigned long long best =
          __hip_atomic_fetch_add(key + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      out[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
      st_coherent(key + row, 0ull);
      st_coherent(counter + row, 0u);
      if (len) len[row_seq ? row_seq[row] : row] += len_add;  // the step's row is in the cache
    }
  }
}

hipError_t rows_quant(const float* x, int T, int K, const float* norm_w, float eps, int8_t* qa, float* da,
                      uint16_t* da_bits, hipStream_t s, bool blocked) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rows_quant, dim3(T), dim3(256), 0, s, x, K, norm_w, eps, qa, da, da_bits, blocked ? 1 : 0);
  return hipGetLastError();
}

hipError_t rows_argmax(const float* x, int T, int V, int32_t* out, unsigned long long* key, unsigned* counter,
                       hipStream_t s, int32_t* len, const int32_t* row_seq, int len_add) {
  if (T == 0) return hipSuccess;
  if (V <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((V + kArgmaxSlice - 1) / kArgmaxSlice), (unsigned)T);
  hipLaunchKernelGGL(k_rows_argmax, grid, dim3(256), 0, s, x, V, out, key, counter, len, row_seq, len_add);
  return hipGetLastError();
}

}  // namespace q8k
