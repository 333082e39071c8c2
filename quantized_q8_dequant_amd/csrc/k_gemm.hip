// Prefill Q8_0 GEMM for gfx950 on int8 MFMA (v_mfma_i32_32x32x32_i8).
//
// C[m, n] = sum_b d_a[m, b] * d_w[n, b] * S_b[m, n] where S_b is the exact
// integer dot of 32-block b (Fucina course, "Model files and quantization",
// section 11.9).  One 32x32x32 MFMA covers exactly one Q8_0 block, so its
// int32 result IS S_b for a 32x32 tile; it is converted and rescaled by the
// product of the two f16 scales (exact in f32) into an f64 accumulator (every
// term is exact in f64) that is rounded to f32 once.
//
// Tiling: a 256-thread workgroup owns a 128 (tokens) x 64 (outputs) tile;
// its 4 wavefronts each own 32 x 64 = 1 x 2 MFMA tiles.  K advances in
// stages of 4 blocks (128 bytes); A/B stages are double-buffered in LDS
// (rows padded by 16 bytes against bank conflicts), the next stage's global
// loads are issued before the current stage's MFMAs.
//
// Epilogues: store, residual add into C, and SwiGLU of the paired gate/up
// columns (the weight stack interleaves 32 gate rows and 32 up rows, so a
// wavefront's 64 columns are one gate tile and its up tile).
//
// Split K: when the tile grid alone would leave most of the 256 CUs idle
// (short prompts, narrow outputs), blockIdx.z takes a contiguous slice of the
// K stages and the tile's f64 sums go to a scratch plane; k_gemm_reduce adds
// the planes in slice order, rounds once to f32 and applies the epilogue.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

// A 128 (tokens) x 64 (outputs) tile per workgroup: wavefront w owns rows
// 32w .. 32w+31 and all 64 columns (two 32x32 MFMA tiles), so the SwiGLU
// epilogue finds a gate tile and its up tile in one wavefront.  The small
// per-wavefront tile keeps the kernel within 256 registers per lane and its
// LDS within 64 KB, so two workgroups share a CU: the f64 epilogue of one
// wavefront then runs while the other waits for LDS or memory.
constexpr int BM = 128, BN = 64;
constexpr int KB = 4;            // 32-blocks per stage
constexpr int SK = KB * 32;      // bytes of K per stage
constexpr int LDS_ROW = SK + 16; // padded row stride (bytes)
constexpr int AL = BM * SK / 16 / 256;  // 16-byte loads of A per thread per stage (4)
constexpr int BL = BN * SK / 16 / 256;  // ... of B (2)

struct Stage {  // loaded values as they are in memory (converted when staged)
  v4i a[AL], b[BL];
  float da[BM * KB / 256];
  uint16_t dw[BN * KB / 256 > 0 ? BN * KB / 256 : 1];  // f16 bits
};

QDEV void gemm_lstore(const Stage& r, int8_t* sA, int8_t* sB, double (*sDa)[BM], double (*sDw)[BN]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / 8, c16 = idx % 8;
    *reinterpret_cast<v4i*>(&sA[row * LDS_ROW + c16 * 16]) = r.a[i];
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / 8, c16 = idx % 8;
    *reinterpret_cast<v4i*>(&sB[row * LDS_ROW + c16 * 16]) = r.b[i];
  }
#pragma unroll
  for (int i = 0; i < BM * KB / 256; ++i) {
    const int idx = tid + 256 * i;
    sDa[idx % KB][idx / KB] = (double)r.da[i];  // widened once here, not per use
  }
  if (tid < BN * KB) sDw[tid % KB][tid / KB] = (double)f16_bits_to_f32(r.dw[0]);
}

QDEV void gemm_gload(const GemmArgs& a, Stage& r, int st, int m0, int n0, int nblk) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / 8, c16 = idx % 8;
    const int gm = min(m0 + row, a.M - 1);
    r.a[i] = *reinterpret_cast<const v4i*>(a.qa + (int64_t)gm * a.K + st * SK + c16 * 16);
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / 8, c16 = idx % 8;
    const int gn = min(n0 + row, a.N - 1);
    r.b[i] = *reinterpret_cast<const v4i*>(a.qs + (int64_t)gn * a.K + st * SK + c16 * 16);
  }
#pragma unroll
  for (int i = 0; i < BM * KB / 256; ++i) {
    const int idx = tid + 256 * i;
    const int gm = min(m0 + idx / KB, a.M - 1);
    r.da[i] = a.da[(int64_t)gm * nblk + st * KB + idx % KB];
  }
  {
    const int idx = tid % (BN * KB);
    const int gn = min(n0 + idx / KB, a.N - 1);
    r.dw[0] = a.sc[(int64_t)gn * nblk + st * KB + idx % KB];
  }
}

constexpr int EPI_PARTIAL = 7;  // f64 sums of one K slice to the scratch plane

template <int EPI>
__global__ void __launch_bounds__(256, 2) k_gemm_q8(GemmArgs a) {
  __shared__ __align__(16) int8_t sA[2][BM * LDS_ROW];
  __shared__ __align__(16) int8_t sB[2][BN * LDS_ROW];
  __shared__ __align__(16) double sDa[2][KB][BM];  // scales widened to f64 when staged
  __shared__ __align__(16) double sDw[2][KB][BN];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nblk = a.K / 32;
  const int nslice = a.K / SK / gridDim.z;  // K stages of this workgroup's slice
  const int st0 = blockIdx.z * nslice;

  // block terms d_a * d_w * S are exact in f64; the sum is rounded to f32
  // once, in the epilogue
  double acc[2][16];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[ni][j] = 0.0;

  const int lr = lane % 32, lg = lane / 32;
  // one stage of K from LDS buffer buf into the accumulators
  auto compute = [&](int buf) {
#pragma unroll 2
    for (int kb = 0; kb < KB; ++kb) {
      const v4i af = *reinterpret_cast<const v4i*>(&sA[buf][(wave * 32 + lr) * LDS_ROW + kb * 32 + lg * 16]);
      v4i bf[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bf[ni] = *reinterpret_cast<const v4i*>(&sB[buf][(ni * 32 + lr) * LDS_ROW + kb * 32 + lg * 16]);
      // the two block products (S = the exact int32 dots of 32-block kb),
      // then their scaled f64 accumulation: d_a * d_w is exact in f64 as in
      // f32, and every term S * d_a * d_w is exact in f64
      v16i S[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const v16i zero = {};
        S[ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf[ni], zero, 0, 0, 0);
      }
      double dw[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) dw[ni] = sDw[buf][kb][ni * 32 + lr];
      double da[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const double* d = &sDa[buf][kb][wave * 32 + 8 * g4 + 4 * lg];
        const double2 lo = *reinterpret_cast<const double2*>(d), hi = *reinterpret_cast<const double2*>(d + 2);
        da[4 * g4 + 0] = lo.x, da[4 * g4 + 1] = lo.y, da[4 * g4 + 2] = hi.x, da[4 * g4 + 3] = hi.y;
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[ni][j] += (double)S[ni][j] * (da[j] * dw[ni]);
    }
  };

  // Stages go global -> registers two stages ahead of their use, then
  // registers -> LDS one stage ahead, so each global load has a whole stage
  // of compute more to land.  The two register sets take turns (the loop
  // steps two stages at a time); loads past the slice re-read its last
  // stage, so every load is issued unconditionally (a load under a branch
  // would make the compiler drain all loads at the join).
  Stage ra, rb;
  const int last = st0 + nslice - 1;
  gemm_gload(a, ra, st0, m0, n0, nblk);
  gemm_gload(a, rb, min(st0 + 1, last), m0, n0, nblk);
  gemm_lstore(ra, sA[0], sB[0], sDa[0], sDw[0]);
  __syncthreads();
  // stage si is in LDS buffer si & 1; `next` holds stage si + 1; `free`
  // receives stage si + 2
  auto step = [&](int si, Stage& free, Stage& next) {
    gemm_gload(a, free, min(st0 + si + 2, last), m0, n0, nblk);
    compute(si & 1);
    if (si + 1 < nslice) gemm_lstore(next, sA[(si + 1) & 1], sB[(si + 1) & 1], sDa[(si + 1) & 1], sDw[(si + 1) & 1]);
    __syncthreads();
  };
  for (int si = 0; si < nslice; si += 2) {
    step(si, ra, rb);
    if (si + 1 < nslice) step(si + 1, rb, ra);
  }

  // epilogue: element j of tile ni is row 8*(j/4) + 4*lg + j%4, column lr
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int m = m0 + wave * 32 + 8 * (j / 4) + 4 * lg + (j % 4);
    if (m >= a.M) continue;
    if (EPI == EPI_PARTIAL) {
      double* pp = a.part + (int64_t)blockIdx.z * a.M * a.N + (int64_t)m * a.N;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + ni * 32 + lr;
        if (n < a.N) pp[n] = acc[ni][j];
      }
    } else if (EPI == EPI_SWIGLU) {
      if (n0 >= a.N) continue;
      const int unit = (n0 / 64) * 32 + lr;
      a.out[(int64_t)m * a.ldc + unit] = swiglu_f64((float)acc[0][j], (float)acc[1][j]);
    } else {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + ni * 32 + lr;
        if (n >= a.N) continue;
        float* p = a.out + (int64_t)m * a.ldc + n;
        const float y = (float)acc[ni][j];
        if (EPI == EPI_STORE) *p = y;
        if (EPI == EPI_RESIDUAL) *p = *p + y;
      }
    }
  }
}

// Sum of the split planes in split order, rounded once to f32, then the
// epilogue; one thread per output (per hidden unit for SwiGLU).
template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_reduce(const double* __restrict__ part, int splits, int M, int N,
                                                     float* out, int64_t ldc) {
  const int NO = EPI == EPI_SWIGLU ? N / 2 : N;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * NO) return;
  const int m = (int)(idx / NO), c = (int)(idx % NO);
  const int64_t plane = (int64_t)M * N;
  const double* p = part + (int64_t)m * N;
  if (EPI == EPI_SWIGLU) {
    const int ng = (c / 32) * 64 + c % 32;  // gate column; its up column is ng + 32
    double g = 0.0, u = 0.0;
    for (int z = 0; z < splits; ++z) {
      g += p[z * plane + ng];
      u += p[z * plane + ng + 32];
    }
    out[(int64_t)m * ldc + c] = swiglu_f64((float)g, (float)u);
  } else {
    double acc = 0.0;
    for (int z = 0; z < splits; ++z) acc += p[z * plane + c];
    float* o = out + (int64_t)m * ldc + c;
    if (EPI == EPI_STORE) *o = (float)acc;
    else *o = *o + (float)acc;
  }
}

}  // namespace

namespace q8k {

// K slices for a grid of `tiles` workgroups: doubled while the grid is under
// two workgroups per CU, the slices stay whole stages and the planes fit.
int gemm_splits(int M, int N, int K, size_t part_bytes) {
  const int tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  const int nstage = K / SK;
  int sp = 1;
  while (tiles * sp < 512 && nstage % (2 * sp) == 0 && (size_t)2 * sp * M * N * 8 <= part_bytes) sp *= 2;
  return sp;
}

hipError_t gemm_reduce(const double* part, int splits, int M, int N, float* out, int64_t ldc, int epi, hipStream_t s) {
  const int NO = epi == EPI_SWIGLU ? N / 2 : N;
  const dim3 rg((unsigned)(((int64_t)M * NO + 255) / 256));
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(k_gemm_reduce<EPI_STORE>, rg, dim3(256), 0, s, part, splits, M, N, out, ldc); break;
    case EPI_RESIDUAL: hipLaunchKernelGGL(k_gemm_reduce<EPI_RESIDUAL>, rg, dim3(256), 0, s, part, splits, M, N, out, ldc); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_reduce<EPI_SWIGLU>, rg, dim3(256), 0, s, part, splits, M, N, out, ldc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const int sp = a.part ? gemm_splits(a.M, a.N, a.K, a.part_bytes) : 1;
  if (sp > 1) {
    const dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, sp);
    hipLaunchKernelGGL(k_gemm_q8<EPI_PARTIAL>, grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return gemm_reduce(a.part, sp, a.M, a.N, a.out, a.ldc, epi, s);
  }
  const dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(k_gemm_q8<EPI_STORE>, grid, dim3(256), 0, s, a); break;
    case EPI_RESIDUAL: hipLaunchKernelGGL(k_gemm_q8<EPI_RESIDUAL>, grid, dim3(256), 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_q8<EPI_SWIGLU>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q8k
