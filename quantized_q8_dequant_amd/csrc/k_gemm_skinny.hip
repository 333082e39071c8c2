// Small-M Q8_0 GEMM for gfx950 on int8 MFMA (v_mfma_i32_16x16x32_i8): the
// projections of a batched decode step (one row per stream) and of short
// prefill chunks (M <= 64 rows), in M tiles of 16 or 32 rows per workgroup.
//
// C[m, n] = sum_b d_a[m, b] * d_w[n, b] * S_b[m, n], S_b the exact integer dot
// of 32-block b (Fucina course, "Model files and quantization", section
// 11.9); one 16x16x32 MFMA is exactly one block for a 16 x 16 tile, every
// term S_b * d_a * d_w is exact in f64 and the sum is rounded to f32 once.
// Reading the weights from HBM once for all rows (the M tiles of a weight
// unit run on one XCD and share its L2) is what makes a batch of streams
// cheaper than the streams one by one (the same page, section 11.6, and "A
// transformer from scratch", section 12.5: decode is weight-bandwidth-bound,
// and the batched decode step reads the weights once for all of its streams).
//
// Work split: a workgroup owns 16 * NT weight rows (for SwiGLU 16 gate rows
// and their 16 up rows) against all M rows (MT tiles of 16); its KW
// wavefronts take KW equal slices of K and add their f64 sums in slice order
// at the end (through LDS), so the sum order is fixed for a given matrix.
// The small units spread even narrow matrices (1024 outputs) over 64
// workgroups, times the 16-row M tiles; the vocabulary projection
// gets 64-row units and all M rows per workgroup.  KW is chosen so
// that a slice is at most eight blocks: a wavefront then issues every load
// of its slice at once and waits one memory round trip (longer slices take
// their chunks of eight in turn).  Operands come straight from global memory
// in the MFMA's lane layout (lane (r, g) holds bytes 8g..8g+7 of a block of
// row r): the weights once, the activation rows from L2.  The activations
// may be stored block-major (the 32 codes of block b of every row together),
// so that a load instruction's 16 rows are 512 contiguous bytes: row-major,
// they are 16 pieces of 32 bytes K apart, and a workgroup's loads were
// measured a third slower.  The activation
// scales of a chunk are staged in the wavefront's own LDS, where each lane
// reads those of the four rows it accumulates.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef int v4i_acc __attribute__((ext_vector_type(4)));

// MT: 16-row M tiles per workgroup (1 or 2); NT: 16-row weight tiles per workgroup (for
// SwiGLU the gate tile and its up tile); KW: wavefronts (slices of K).
template <int MT, int NT, int KW, int EPI>
__global__ void __launch_bounds__(64 * KW) k_gemm_skinny(GemmArgs a) {
  static_assert(EPI != EPI_SWIGLU || NT == 2, "SwiGLU pairs a gate tile with its up tile");
  constexpr int UG = 8;  // blocks per chunk
  constexpr int MR = 16 * MT;
  constexpr int RV = MT * 4;                        // f64 values per lane per weight tile
  __shared__ __align__(16) float s_da[KW][UG][MR];  // per wavefront: scales of its chunk
  __shared__ double s_red[KW - 1][RV][kWave];

  const int units = EPI == EPI_SWIGLU ? a.N / 32 : (a.N + 16 * NT - 1) / (16 * NT);
  // workgroup -> (weight unit, M tile): workgroups are dealt to the eight
  // XCDs in turn, so id % 8 is the XCD; on each XCD the M tiles of a unit
  // are consecutive, run together and share the unit's weights in its L2
  const int mtiles = (a.M + MR - 1) / MR;
  const int wid = blockIdx.x / 8;
  const int unit = (wid / mtiles) * 8 + blockIdx.x % 8, mtile = wid % mtiles;
  if (unit >= units) return;  // units rounded up to a multiple of eight
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int lc = lane % 16, lk = lane / 16;
  const int K = a.K, nblk = K / 32;
  const int nq = nblk / KW;  // blocks of each slice
  const int kb0 = w * nq;
  const int nch = (nq + UG - 1) / UG;
  // weight rows of this workgroup; SwiGLU: the stack interleaves 32 gate and
  // 32 up rows, and unit u takes 16 of each
  int64_t wrow[NT];
  int n0;
  if (EPI == EPI_SWIGLU) {
    const int g = unit / 2, h = unit % 2;
    n0 = 64 * g + 16 * h;
    wrow[0] = min(n0 + lc, a.N - 1);
    wrow[NT - 1] = min(n0 + 32 + lc, a.N - 1);
  } else {
    n0 = unit * 16 * NT;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wrow[nt] = min(n0 + 16 * nt + lc, a.N - 1);
  }
  const int m0 = mtile * MR;  // first row of this workgroup's M tile
  int64_t arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(m0 + mt * 16 + lc, a.M - 1);
  const int64_t drow = min(m0 + lane, a.M - 1);  // the scale row this lane stages (lane < MR)

  struct Chunk {
    long b[NT][UG];
    uint16_t dw[NT][UG];
    long x[MT][UG];
    float d[UG];
  };
  // every load is issued whatever the chunk's length (blocks past the
  // slice re-read its last block, never used), so the count is fixed
  auto load = [&](Chunk& c, int ci) {
    const int kbc = kb0 + ci * UG;
#pragma unroll
    for (int i = 0; i < UG; ++i) {
      const int kb = min(kbc + i, kb0 + nq - 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        c.b[nt][i] = *reinterpret_cast<const long*>(a.qs + wrow[nt] * K + kb * 32 + 8 * lk);
        c.dw[nt][i] = a.sc[wrow[nt] * nblk + kb];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        c.x[mt][i] = *reinterpret_cast<const long*>(a.qa + (a.a_blocked ? ((int64_t)kb * a.M + arow[mt]) * 32 : arow[mt] * K + kb * 32) + 8 * lk);
      c.d[i] = a.da[a.a_blocked ? (int64_t)kb * a.M + drow : drow * nblk + kb];
    }
  };

  double acc[NT][MT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[nt][mt][q] = 0.0;

  auto compute = [&](const Chunk& c, int ci) {
    // the chunk's activation scales to this wavefront's LDS rows; LDS
    // accesses of one wavefront complete in order, so its own lanes read
    // them back below without a workgroup barrier
    if (lane < MR) {
#pragma unroll
      for (int i = 0; i < UG; ++i) s_da[w][i][lane] = c.d[i];
    }
    __builtin_amdgcn_wave_barrier();
    const int cnt = min(UG, nq - ci * UG);
#pragma unroll
    for (int i = 0; i < UG; ++i) {
      if (i < cnt) {  // uniform across the wavefront
        double dw[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) dw[nt] = (double)f16_bits_to_f32(c.dw[nt][i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // element q of a tile is row 4*lk + q (of the tile), column lc
          const float4 d4 = *reinterpret_cast<const float4*>(&s_da[w][i][mt * 16 + 4 * lk]);
          const double da[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const v4i_acc zero = {};
            const v4i_acc S = __builtin_amdgcn_mfma_i32_16x16x32_i8(c.x[mt][i], c.b[nt][i], zero, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[nt][mt][q] += (double)S[q] * (da[q] * dw[nt]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // K slices are sized so that a slice is one chunk on the model shapes
  // (every load of the slice in flight at once); longer slices take their
  // chunks one after the other
  for (int ci = 0; ci < nch; ++ci) {
    Chunk c;
    load(c, ci);
    compute(c, ci);
  }

  // the slices' sums, added in slice order by wavefront 0, one weight tile
  // at a time
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (nt > 0) __syncthreads();  // the previous tile's values consumed
    if (w > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) s_red[w - 1][mt * 4 + q][lane] = acc[nt][mt][q];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          double t = acc[nt][mt][q];
#pragma unroll
          for (int v = 0; v < KW - 1; ++v) t += s_red[v][mt * 4 + q][lane];
          acc[nt][mt][q] = t;
        }
    }
  }
  if (w != 0) return;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + mt * 16 + 4 * lk + q;
      if (m >= a.M) continue;
      if (EPI == EPI_SWIGLU) {
        const int unit = (n0 / 64) * 32 + (n0 % 64) + lc;  // hidden unit of gate row n0 + lc
        a.out[(int64_t)m * a.ldc + unit] = swiglu_f64((float)acc[0][mt][q], (float)acc[NT - 1][mt][q]);
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + 16 * nt + lc;
          if (n >= a.N) continue;
          float* p = a.out + (int64_t)m * a.ldc + n;
          const float y = (float)acc[nt][mt][q];
          if (EPI == EPI_STORE) *p = y;
          if (EPI == EPI_RESIDUAL) *p = *p + y;
        }
      }
    }
}

// One workgroup per (weight unit, M tile of 16 * MT rows), the units
// rounded up to a multiple of eight (see the kernel's mapping).
template <int MT, int NT, int KW, int EPI>
hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
  const unsigned mtiles = (unsigned)((a.M + 16 * MT - 1) / (16 * MT));
  const unsigned units = EPI == EPI_SWIGLU ? (unsigned)(a.N / 32) : (unsigned)((a.N + 16 * NT - 1) / (16 * NT));
  const unsigned grid = (units + 7) / 8 * 8 * mtiles;
  hipLaunchKernelGGL((k_gemm_skinny<MT, NT, KW, EPI>), dim3(grid), dim3(64 * KW), 0, s, a);
  return hipGetLastError();
}

// Shape choice: 64-row units when even they give several workgroups per CU
// (the vocabulary projection), else 16-row units (gate + up for SwiGLU).  K
// slices: the fewest of 4, 8, 16 that make a slice at most one chunk and
// divide the blocks evenly; more rows per wavefront cap them (registers and
// LDS of the slice reduction).
template <int MT, int NT, int EPI>
hipError_t launch_nt(const GemmArgs& a, hipStream_t s) {
  const int nblk = a.K / 32;
  constexpr int KWMAX = MT >= 4 || NT >= 4 ? 4 : (MT >= 2 || NT >= 2 ? 8 : 16);
  if constexpr (KWMAX >= 8) {
    if (nblk % 8 == 0 && nblk / 4 > 8) {
      if constexpr (KWMAX >= 16)
        if (nblk % 16 == 0 && nblk / 8 > 8) return launch_one<MT, NT, 16, EPI>(a, s);
      return launch_one<MT, NT, 8, EPI>(a, s);
    }
  }
  return launch_one<MT, NT, 4, EPI>(a, s);
}

template <int MT>
hipError_t launch_mt(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE:
      if constexpr (MT <= 2)
        if ((a.N + 63) / 64 >= 1024) return launch_nt<MT, 4, EPI_STORE>(a, s);
      return launch_nt<MT, 1, EPI_STORE>(a, s);
    case EPI_RESIDUAL:
      return launch_nt<MT, 1, EPI_RESIDUAL>(a, s);
    case EPI_SWIGLU:  // a.N % 64 == 0: N / 32 units of 16 gate + 16 up rows
      return launch_nt<MT, 2, EPI_SWIGLU>(a, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

namespace q8k {

bool gemm_skinny_supported(int M, int K) { return M >= 1 && M <= kSkinnyMaxRows && K >= 128 && K % 128 == 0; }

hipError_t gemm_skinny(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (!gemm_skinny_supported(a.M, a.K) || a.N <= 0 || (epi == EPI_SWIGLU && a.N % 64 != 0))
    return hipErrorInvalidValue;
  // M goes over workgroups in tiles (grid.y): a workgroup's loads bound
  // these launches, and every workgroup reads all of its rows' activations,
  // so fewer rows per workgroup and more workgroups win.  Narrow matrices
  // (fewer than 1024 16-row weight units) take 16-row tiles; the vocabulary
  // projection takes 32-row tiles of 64-row weight units (at most two tiles
  // reading each unit, on one XCD).
  if (a.M <= 16 || (a.N + 15) / 16 < 1024) return launch_mt<1>(a, epi, s);
  return launch_mt<2>(a, epi, s);
}

}  // namespace q8k
