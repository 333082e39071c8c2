// Linear layers of models stored with bf16 weights, for prefill and batched
// decode: C[M, N] = X[M, K] . W[N, K]^T with f32 activations and bf16 weights
// widened exactly (the weight binding of the Fucina reference page "The LLM
// stack: fucina_llm", section 13, widens bf16 in registers; the activations
// are not rounded).  Every product of a bf16 and an f32 value is exact in
// f64, so the kernel runs on the f64 matrix cores (v_mfma_f64_16x16x4f64)
// and rounds each sum to f32 once, in the epilogue.
//
// Tiling: a 256-thread workgroup owns a BM x 64 tile of C; its four waves
// own (BM/2) x 32 quadrants made of 16 x 16 MFMA blocks.  K advances in
// 32-wide slabs staged through double-buffered LDS (both operands held as
// f32 rows of 36 words, so the fragment reads of a wave hit 64 distinct
// banks).  The epilogue goes through LDS: the tile is rounded to f32 there
// and then stored, added to the residual stream, paired into SwiGLU outputs
// (the gate/up plane interleaves 32 gate rows with the 32 matching up rows),
// or reduced to the greedy argmax.
//
// Split K: while the tile grid is under two workgroups per CU (the batched
// decode step's 64-row products have 16 to 96 tiles), K is cut into slices of
// whole slabs over grid.z; each slice writes its f64 tile sums to a scratch
// plane and k_gemm_reduce adds the planes in slice order, rounds once to f32
// and applies the epilogue.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;
constexpr int kLds = kBK + 4;  // f32 words per staged row
constexpr int kBN = 64;
constexpr int kEpiPartial = 7;  // f64 sums of one K slice to the scratch plane

struct Best {
  float v;
  int i;
};
QDEV Best better(Best a, Best b) {  // larger value; ties -> lower index
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

template <int BM, int EPI>
__global__ void __launch_bounds__(256) k_gemm_bf16(GemmBf16Args a) {
  constexpr int BN = kBN;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int STAGE = (BM + BN) * kLds;
  constexpr int CST = BN + 1;
  constexpr int SMEM = (2 * STAGE > BM * CST) ? 2 * STAGE : BM * CST;
  constexpr int A_PER = BM * (kBK / 4) / 256;  // float4 per thread per slab
  constexpr int B_PER = BN * (kBK / 8) / 256;  // 8-bf16 chunks per thread per slab
  static_assert(A_PER >= 1 && B_PER >= 1, "tile too small for the staging map");
  __shared__ __align__(16) float smem[SMEM];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm0 = (wave / 2) * WM, wn0 = (wave % 2) * WN;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int M = a.M, N = a.N, K = a.K;

  float4 ra[A_PER];
  v4i rb[B_PER];
  auto load = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int idx = tid + i * 256;
      const int row = idx / (kBK / 4), c4 = idx % (kBK / 4);
      const int64_t m = m0 + row;
      ra[i] = m < M ? *reinterpret_cast<const float4*>(a.x + m * a.lda + k0 + c4 * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int idx = tid + i * 256;
      const int row = idx / (kBK / 8), c8 = idx % (kBK / 8);
      const int64_t n = n0 + row;
      rb[i] = n < N ? *reinterpret_cast<const v4i*>(a.w + n * (int64_t)K + k0 + c8 * 8) : v4i{0, 0, 0, 0};
    }
  };
  auto store = [&](float* st) {
    float* sa = st;
    float* sb = st + BM * kLds;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int idx = tid + i * 256;
      const int row = idx / (kBK / 4), c4 = idx % (kBK / 4);
      *reinterpret_cast<float4*>(sa + row * kLds + c4 * 4) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int idx = tid + i * 256;
      const int row = idx / (kBK / 8), c8 = idx % (kBK / 8);
      float4 lo, hi;  // bf16 pairs: element 2j in the low half of word j
      lo.x = __uint_as_float((uint32_t)rb[i][0] << 16), lo.y = __uint_as_float((uint32_t)rb[i][0] & 0xFFFF0000u);
      lo.z = __uint_as_float((uint32_t)rb[i][1] << 16), lo.w = __uint_as_float((uint32_t)rb[i][1] & 0xFFFF0000u);
      hi.x = __uint_as_float((uint32_t)rb[i][2] << 16), hi.y = __uint_as_float((uint32_t)rb[i][2] & 0xFFFF0000u);
      hi.z = __uint_as_float((uint32_t)rb[i][3] << 16), hi.w = __uint_as_float((uint32_t)rb[i][3] & 0xFFFF0000u);
      *reinterpret_cast<float4*>(sb + row * kLds + c8 * 8) = lo;
      *reinterpret_cast<float4*>(sb + row * kLds + c8 * 8 + 4) = hi;
    }
  };

  v4d acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};

  // this workgroup's slabs [kt0, kt1): slice blockIdx.z of gridDim.z (the
  // slice count divides the slab count)
  const int nk = K / kBK;
  const int kt0 = (int)blockIdx.z * nk / (int)gridDim.z, kt1 = ((int)blockIdx.z + 1) * nk / (int)gridDim.z;
  load(kt0);
  store(smem);
  __syncthreads();
  const int fr = lane % 16, fk = lane / 16;
  for (int kt = kt0; kt < kt1; ++kt) {
    const float* sa = smem + ((kt - kt0) & 1) * STAGE;
    const float* sb = sa + BM * kLds;
    if (kt + 1 < kt1) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 4) {
      double af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = (double)sa[(wm0 + 16 * i + fr) * kLds + kk + fk];
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = (double)sb[(wn0 + 16 * j + fr) * kLds + kk + fk];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < kt1) store(smem + ((kt + 1 - kt0) & 1) * STAGE);
    __syncthreads();
  }

  if constexpr (EPI == kEpiPartial) {
    // the slice's f64 sums, unrounded: block (i, j) item t is
    // C[wm0 + 16i + 4t + lane/16][wn0 + 16j + lane%16]
    double* pp = a.part + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t m = m0 + wm0 + 16 * i + 4 * t + fk, n = n0 + wn0 + 16 * j + fr;
          if (m < M && n < N) pp[m * N + n] = acc[i][j][t];
        }
    return;
  }

  // round once to f32 into the LDS tile: block (i, j) item t holds
  // C[wm0 + 16i + 4t + lane/16][wn0 + 16j + lane%16]
  float* sc = smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) sc[(wm0 + 16 * i + 4 * t + fk) * CST + wn0 + 16 * j + fr] = (float)acc[i][j][t];
  __syncthreads();

  if (EPI == EPI_STORE || EPI == EPI_RESIDUAL) {
    for (int idx = tid; idx < BM * BN; idx += 256) {
      const int row = idx / BN, col = idx % BN;
      const int64_t m = m0 + row, n = n0 + col;
      if (m < M && n < N) {
        float* o = a.out + m * a.ldc + n;
        const float y = sc[row * CST + col];
        *o = EPI == EPI_RESIDUAL ? *o + y : y;
      }
    }
  } else if (EPI == EPI_SWIGLU) {
    // columns [0, 32) of the tile are gate rows, [32, 64) the matching up rows
    for (int idx = tid; idx < BM * (BN / 2); idx += 256) {
      const int row = idx / (BN / 2), c = idx % (BN / 2);
      const int64_t m = m0 + row;
      if (m < M && n0 + c < N) a.out[m * a.ldc + n0 / 2 + c] = swiglu_f64(sc[row * CST + c], sc[row * CST + c + 32]);
    }
  } else {  // EPI_ARGMAX: logits and the (max, lowest index) key of each row
    for (int row = wave; row < BM; row += 4) {
      const int64_t m = m0 + row;
      if (m >= M) break;  // rows ascend: uniform for the wave
      const int64_t n = n0 + lane;
      Best b{-INFINITY, 0x7FFFFFFF};
      if (n < N) {
        const float y = sc[row * CST + lane];
        if (a.logits) a.logits[m * (int64_t)N + n] = y;
        b = Best{y, (int)n};
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        Best c;
        c.v = __shfl_xor(b.v, o);
        c.i = __shfl_xor(b.i, o);
        b = better(b, c);
      }
      if (lane == 0) {
        const uint32_t u = __float_as_uint(b.v + 0.0f);  // -0 -> +0
        const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        const unsigned long long key = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)b.i);
        __hip_atomic_fetch_max(a.best_key + m, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    wait_memory();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = arrive(a.counter + blockIdx.y);
      if (prev == gridDim.x - 1) {  // last workgroup of this row tile
        for (int row = 0; row < BM && m0 + row < M; ++row) {
          const int64_t m = m0 + row;
          const unsigned long long k =
              __hip_atomic_fetch_add(a.best_key + m, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (a.argmax) a.argmax[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
          st_coherent(a.best_key + m, 0ull);
          if (a.len_ptr) {
            const int seq = a.len_seq ? a.len_seq[m] : 0;
            a.len_ptr[seq] += a.len_add;
          }
        }
        st_coherent(a.counter + blockIdx.y, 0u);
      }
    }
  }
}

// y[t] = RMSNorm(x[t]) * w, each row's sum of squares in f64 ("A transformer
// from scratch", section 12.3.2), rounded to f32 once per element.
__global__ void __launch_bounds__(256) k_rows_norm(const float* __restrict__ x, int64_t ldx, int K,
                                                   const float* __restrict__ w, float eps, float* __restrict__ y,
                                                   int64_t ldy) {
  __shared__ double s_red[4];
  const float* xr = x + (int64_t)blockIdx.x * ldx;
  float* yr = y + (int64_t)blockIdx.x * ldy;
  double ss = 0.0;
  for (int c = threadIdx.x * 4; c < K; c += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(xr + c);
    ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  ss = block_sum_d<256>(ss, s_red);
  const double r = rms_scale(ss, K, eps);
  for (int c = threadIdx.x * 4; c < K; c += 256 * 4) {
    const float4 v = *reinterpret_cast<const float4*>(xr + c);
    const float4 g = *reinterpret_cast<const float4*>(w + c);
    float4 o;
    o.x = rms_apply(v.x, r, g.x), o.y = rms_apply(v.y, r, g.y);
    o.z = rms_apply(v.z, r, g.z), o.w = rms_apply(v.w, r, g.w);
    *reinterpret_cast<float4*>(yr + c) = o;
  }
}

// K slices for a grid of `tiles` workgroups (the rule of the Q8_0 GEMM):
// doubled while the grid is under two workgroups per CU, the slices stay
// whole slabs and the planes fit the scratch; never for the argmax epilogue.
int bf16_splits(const GemmBf16Args& a, int bm, int epi) {
  if (!a.part || epi == EPI_ARGMAX) return 1;
  const int tiles = ((a.N + kBN - 1) / kBN) * ((a.M + bm - 1) / bm);
  const int nk = a.K / kBK;
  int sp = 1;
  while (tiles * sp < 512 && nk % (2 * sp) == 0 && (size_t)2 * sp * a.M * a.N * 8 <= a.part_bytes) sp *= 2;
  return sp;
}

template <int BM>
hipError_t launch_bm(const GemmBf16Args& a, int epi, hipStream_t s) {
  const int sp = bf16_splits(a, BM, epi);
  if (sp > 1) {
    const dim3 grid((unsigned)((a.N + kBN - 1) / kBN), (unsigned)((a.M + BM - 1) / BM), (unsigned)sp);
    hipLaunchKernelGGL((k_gemm_bf16<BM, kEpiPartial>), grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return q8k::gemm_reduce(a.part, sp, a.M, a.N, a.out, a.ldc, epi, s);
  }
  const dim3 grid((unsigned)((a.N + kBN - 1) / kBN), (unsigned)((a.M + BM - 1) / BM));
#define BF_CASE(E)                                                                 \
  if (epi == E) {                                                                  \
    hipLaunchKernelGGL((k_gemm_bf16<BM, E>), grid, dim3(256), 0, s, a);            \
    return hipGetLastError();                                                      \
  }
  BF_CASE(EPI_STORE)
  BF_CASE(EPI_RESIDUAL)
  BF_CASE(EPI_SWIGLU)
  BF_CASE(EPI_ARGMAX)
#undef BF_CASE
  return hipErrorInvalidValue;
}

}  // namespace

namespace q8k {

hipError_t gemm_bf16(const GemmBf16Args& a, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0 || a.K % kBK || a.lda % 4) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && a.N % kBN) return hipErrorInvalidValue;
  return a.M > 64 ? launch_bm<128>(a, epi, s) : launch_bm<64>(a, epi, s);
}

hipError_t rows_norm(const float* x, int64_t ldx, int T, int K, const float* w, float eps, float* y, int64_t ldy,
                     hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (K % 4 || ldx % 4 || ldy % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rows_norm, dim3((unsigned)T), dim3(256), 0, s, x, ldx, K, w, eps, y, ldy);
  return hipGetLastError();
}

}  // namespace q8k
