// Decode-step Q8_0 GEMV for gfx950: y[n] = sum_b d_w[n,b] * d_a[b] * S[n,b],
// S the exact integer dot of one 32-block (Fucina course, "Model files and
// quantization", section 11.9), with the activation quantised per 32-block
// on the fly (same page, section 11.7).
//
// Layout: the weight matrix is two planes -- int8 codes [N][K] (row r is
// output r) and f16 scales [N][K/32].  A wavefront streams rows with 128-bit
// loads: LPR lanes cover one row and each lane owns whole 32-byte blocks
// b = lane + j*LPR (two 16-byte loads; the pair of load instructions covers
// the row's bytes contiguously), so S is formed in one lane by 8 x v_dot4.
// The activation is loaded first and the first two tiles' weights next
// (weights do not depend on the activation), so the prologue, which
// quantises the activation into LDS, waits for the activation alone.
//
// Prologues: RMSNorm + quantise (the norm of "A transformer from scratch",
// section 12.3.2) or quantise only.  Epilogues: store, residual add (section
// 12.3.7), SwiGLU of paired gate/up rows (section 12.3.6), and the tied
// lm_head with the first pass of the greedy argmax (per-workgroup (max,
// lowest index)); the last workgroup to finish runs the second pass.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {


// Quantise the activation [K] (optionally RMSNorm'd with w) into LDS: s_qa
// [K] bytes, s_da [K/32] f32 (the value of f16(d)).  The activation and the
// norm weights arrive in registers: chunk i of thread t holds elements
// 4 * (t + i * NT) .. + 3 (XN chunks; those past K are unused).
template <bool NORM, int NT, int XN>
QDEV void prologue_quant(const float4 (&xv)[XN], const float4 (&wv)[XN], float eps, int K, int8_t* s_qa,
                              float* s_da, double* s_red) {
  double r = 1.0;
  if (NORM) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      const int c = 4 * ((int)threadIdx.x + i * NT);
      if (c < K) {
        const float4 v = xv[i];
        ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
      }
    }
    ss = block_sum_d<NT>(ss, s_red);
    r = rms_scale(ss, K, eps);
  }
#pragma unroll
  for (int i = 0; i < XN; ++i) {
    const int c = 4 * ((int)threadIdx.x + i * NT);
    const bool live = c < K;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      v[0] = xv[i].x, v[1] = xv[i].y, v[2] = xv[i].z, v[3] = xv[i].w;
      if (NORM) {
        v[0] = rms_apply(v[0], r, wv[i].x), v[1] = rms_apply(v[1], r, wv[i].y);
        v[2] = rms_apply(v[2], r, wv[i].z), v[3] = rms_apply(v[3], r, wv[i].w);
      }
    }
    float d;
    const int packed = quant4_group8(v, &d);
    if (live) {
      *reinterpret_cast<int*>(s_qa + c) = packed;
      if ((threadIdx.x & 7) == 0) s_da[c >> 5] = f16_round(d);
    }
  }
  __syncthreads();
}

struct ArgBest {
  float v;
  int i;
};
QDEV ArgBest better(ArgBest a, ArgBest b) {  // larger value; ties -> lower index
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}
QDEV ArgBest wave_best(ArgBest a) {  // over the 64 lanes
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    ArgBest b;
    b.v = __shfl_xor(a.v, o);
    b.i = __shfl_xor(a.i, o);
    a = better(a, b);
  }
  return a;
}

// LPR lanes per row, BPL 32-value blocks per lane per row (K = 32*LPR*BPL),
// ROWS rows per lane group.  For EPI_SWIGLU the first ROWS/2 rows are gate
// rows and the last ROWS/2 the matching up rows.
template <int LPR, int BPL, int ROWS, int WAVES, bool NORM, int EPI>
__global__ void __launch_bounds__(64 * WAVES) k_gemv(GemvArgs a) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kWaves = WAVES;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ double s_red[kWaves];
  __shared__ ArgBest s_best[kWaves];
  constexpr int K = 32 * LPR * BPL;
  constexpr int GPW = kWave / LPR;  // lane groups per wave
  int8_t* s_qa = reinterpret_cast<int8_t*>(smem);
  float* s_da = reinterpret_cast<float*>(smem + K);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int li = lane % LPR, grp = lane / LPR;
  const int groups_per_wg = kWaves * GPW;
  const int64_t nb = K / 32;

  // rows of the activation batch: blockIdx.y selects one batch row
  const float* src = a.src + (int64_t)blockIdx.y * a.src_stride;
  float* out = a.out ? a.out + (int64_t)blockIdx.y * a.out_stride : nullptr;

  ArgBest best{-INFINITY, 0x7FFFFFFF};

  // weights of one tile in registers; two buffers so that the next tile's
  // loads are in flight while the current tile is reduced
  struct WTile {
    v4i w0[ROWS][BPL], w1[ROWS][BPL];
    uint16_t ws[ROWS][BPL];
  };
  auto tile_rows = [&](int tile, int (&rows)[ROWS]) {
    const int gg = tile * groups_per_wg + wave * GPW + grp;  // global lane-group index
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (EPI == EPI_SWIGLU) {
        constexpr int P = ROWS / 2;
        const int n = gg * P + (r % P);
        rows[r] = (n / 32) * 64 + (r < P ? 0 : 32) + (n % 32);
      } else {
        rows[r] = gg * ROWS + r;
      }
    }
  };
  auto load = [&](WTile& t, int tile) {
    int rows[ROWS];
    tile_rows(tile, rows);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int64_t row = rows[r] < a.N ? rows[r] : a.N - 1;
      const int8_t* wr = a.qs + row * (int64_t)K;
      const uint16_t* sr = a.sc + row * nb;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        const int b = li + j * LPR;
        t.w0[r][j] = *reinterpret_cast<const v4i*>(wr + b * 32);
        t.w1[r][j] = *reinterpret_cast<const v4i*>(wr + b * 32 + 16);
        t.ws[r][j] = sr[b];
      }
    }
  };
  auto compute = [&](const WTile& t, int tile) {
    int rows[ROWS];
    tile_rows(tile, rows);
    const int gg = tile * groups_per_wg + wave * GPW + grp;
    // block terms d_w * d_a * S are exact in f64; their sum is rounded to
    // f32 once, in the epilogue
    double acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = 0.0;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const int b = li + j * LPR;
      const v4i a0 = *reinterpret_cast<const v4i*>(s_qa + b * 32);
      const v4i a1 = *reinterpret_cast<const v4i*>(s_qa + b * 32 + 16);
      const float da = s_da[b];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int S = dot32_i8(t.w0[r][j], t.w1[r][j], a0, a1);
        acc[r] += (double)S * (double)(f16_bits_to_f32(t.ws[r][j]) * da);
      }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = group_sum_d<LPR>(acc[r]);

    if (li == LPR - 1) {  // the lane holding the row sums
      if (EPI == EPI_SWIGLU) {
        constexpr int P = ROWS / 2;
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int n = gg * P + i;
          if (n < a.N / 2) {
            out[n] = swiglu_f64((float)acc[i], (float)acc[P + i]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const int row = rows[r];
          if (row < a.N) {
            const float y = (float)acc[r];
            if (EPI == EPI_STORE) out[row] = y;
            if (EPI == EPI_RESIDUAL) out[row] = out[row] + y;
            if (EPI == EPI_ARGMAX) {
              if (a.logits) a.logits[(int64_t)blockIdx.y * a.N + row] = y;
              best = better(best, ArgBest{y, row});
            }
          }
        }
      }
    }
  };

  // grid-stride over tiles: the activation is quantised once per workgroup
  // (weights of the first two tiles already in flight), later tiles' weights
  // are loaded one tile ahead
  // (the prefetch is issued unconditionally -- past the last tile it
  // re-reads a tile already loaded, a cache hit -- so that the compiler keeps
  // it in flight while it waits for the older tile)
  int tile = blockIdx.x;
  if (tile < a.ntiles) {
    WTile A, B;
    // the activation first, then the first two tiles' weights: loads
    // complete in order, so the prologue waits for the activation alone
    // while both tiles are in flight
    constexpr int XN = (K + 4 * kThreads - 1) / (4 * kThreads);
    float4 xv[XN], wv[XN];
#pragma unroll
    for (int i = 0; i < XN; ++i) {
      const int c = 4 * ((int)threadIdx.x + i * kThreads);
      const int cc = c < K ? c : 0;
      xv[i] = *reinterpret_cast<const float4*>(src + cc);
      wv[i] = NORM ? *reinterpret_cast<const float4*>(a.norm_w + cc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    load(A, tile);
    if (tile + (int)gridDim.x >= a.ntiles) {  // one tile
      prologue_quant<NORM, kThreads, XN>(xv, wv, a.eps, K, s_qa, s_da, s_red);
      compute(A, tile);
    } else {
      load(B, tile + (int)gridDim.x);
      prologue_quant<NORM, kThreads, XN>(xv, wv, a.eps, K, s_qa, s_da, s_red);
      // A holds tile, B tile + G: the next tile's loads are in flight while
      // one is reduced
      for (;;) {
        const int t1 = tile + gridDim.x, t2 = t1 + gridDim.x, t3 = t2 + gridDim.x;
        compute(A, tile);
        if (t1 >= a.ntiles) break;
        load(A, t2 < a.ntiles ? t2 : t1);
        compute(B, t1);
        if (t2 >= a.ntiles) break;
        load(B, t3 < a.ntiles ? t3 : t2);
        tile = t2;
      }
    }
  }

  if (EPI == EPI_ARGMAX) {
    // first pass: this workgroup's (max, lowest index), folded into one
    // 64-bit key per batch row with an atomic max (order-preserving float
    // bits above, inverted index below, so equal maxima keep the lowest
    // index); second pass: the last workgroup reads the key
    best = wave_best(best);
    if (lane == 0) s_best[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      ArgBest b = s_best[0];
      for (int i = 1; i < kWaves; ++i) b = better(b, s_best[i]);
      const uint32_t u = __float_as_uint(b.v + 0.0f);  // -0 -> +0
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const unsigned long long key = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)b.i);
      __hip_atomic_fetch_max(a.best_key + blockIdx.y, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_memory();
      const unsigned prev = arrive(a.counter + blockIdx.y);
      if (prev == gridDim.x - 1) {  // last workgroup of this batch row
        const unsigned long long k =
            __hip_atomic_fetch_add(a.best_key + blockIdx.y, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (a.argmax) a.argmax[blockIdx.y] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        st_coherent(a.best_key + blockIdx.y, 0ull);  // ready for the next launch
        st_coherent(a.counter + blockIdx.y, 0u);
        if (a.len_ptr) {
          const int seq = a.len_seq ? a.len_seq[blockIdx.y] : 0;
          a.len_ptr[seq] += a.len_add;
        }
      }
    }
  }
}

// Test hook: S[t][n][b] with the same per-lane block dot as the GEMV.
// One wavefront per (t, n) pair, one lane per block.
constexpr int kBdThreads = 256;
__global__ void __launch_bounds__(kBdThreads) k_block_dots(const int8_t* __restrict__ qa, const int8_t* __restrict__ qs,
                                                        int K, int N, int64_t pairs, int32_t* __restrict__ S) {
  const int lane = threadIdx.x % kWave;
  const int64_t pair = (int64_t)blockIdx.x * (kBdThreads / kWave) + threadIdx.x / kWave;
  if (pair >= pairs) return;  // uniform per wavefront
  const int t = (int)(pair / N), n = (int)(pair % N);
  const int nblocks = K / 32;
  for (int b = lane; b < nblocks; b += kWave) {
    const int8_t* w = qs + (int64_t)n * K + b * 32;
    const int8_t* x = qa + (int64_t)t * K + b * 32;
    const int s = dot32_i8(*reinterpret_cast<const v4i*>(w), *reinterpret_cast<const v4i*>(w + 16),
                           *reinterpret_cast<const v4i*>(x), *reinterpret_cast<const v4i*>(x + 16));
    S[((int64_t)t * N + n) * nblocks + b] = s;
  }
}

template <int LPR, int BPL, int ROWS, int WAVES, bool NORM, int EPI>
hipError_t launch_one(const GemvArgs& a, int grid_x, int grid_y, hipStream_t s) {
  constexpr int K = 32 * LPR * BPL;
  const size_t shm = K + (K / 32) * sizeof(float);
  hipLaunchKernelGGL((k_gemv<LPR, BPL, ROWS, WAVES, NORM, EPI>), dim3(grid_x, grid_y), dim3(64 * WAVES), shm, s, a);
  return hipGetLastError();
}

constexpr int rows_per_tile(int lpr, int rows, int waves) { return waves * (64 / lpr) * rows; }
constexpr int kMaxGrid = 1024;

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Workgroups of one launch.  Small matrices: one tile each (up to 1024, the
// tail strides).  Large matrices: one 512-thread workgroup per CU at most,
// with the tiles spread evenly, so the activation is quantised a few hundred
// times rather than once per tile.
int grid_for(int ntiles, bool large) {
  if (!large) return ntiles < kMaxGrid ? ntiles : kMaxGrid;
  const int cus = cu_count();
  const int per = (ntiles + cus - 1) / cus;
  return (ntiles + per - 1) / per;
}

template <int LPR, int BPL, int ROWS, int WAVES>
hipError_t launch_epi(GemvArgs& a, bool norm, int epi, int grid_y, bool large, hipStream_t s) {
  const int rpt = rows_per_tile(LPR, ROWS, WAVES);
  a.ntiles = (a.N + rpt - 1) / rpt;
  const int grid = grid_for(a.ntiles, large);
#define Q8_CASE(NORM_, EPI_) \
  if (norm == NORM_ && epi == EPI_) return launch_one<LPR, BPL, ROWS, WAVES, NORM_, EPI_>(a, grid, grid_y, s);
  Q8_CASE(true, EPI_STORE)
  Q8_CASE(false, EPI_STORE)
  Q8_CASE(false, EPI_RESIDUAL)
  if constexpr (ROWS % 2 == 0) {
    Q8_CASE(true, EPI_SWIGLU)
  }
  Q8_CASE(true, EPI_ARGMAX)
  Q8_CASE(false, EPI_ARGMAX)
#undef Q8_CASE
  return hipErrorInvalidValue;
}

// Launch shapes per K (LPR = lanes per row, BPL = blocks per lane, ROWS per
// lane group, WAVES per workgroup): small-N matrices get few rows per
// workgroup so that every launch spreads over all 256 CUs.
#define Q8_SHAPES(X)                                                                     \
  X(256, 8, 1, 2, 4) X(512, 16, 1, 2, 4) X(768, 8, 3, 2, 4)                            \
  X(1024, 32, 1, 2, 4) X(2048, 64, 1, 2, 4) X(3072, 32, 3, 2, 4) X(4096, 64, 2, 2, 4)  \
  X(6144, 64, 3, 2, 4) X(8192, 64, 4, 2, 4) X(12288, 64, 6, 2, 4)
#define Q8_SMALL(X) X(2048, 64, 1, 1, 4) X(3072, 32, 3, 1, 2) X(4096, 64, 2, 1, 4) X(6144, 64, 3, 1, 4) \
  X(8192, 64, 4, 1, 4) X(12288, 64, 6, 1, 4)
#define Q8_ARGMAX(X) X(1024, 32, 1, 8, 4) X(4096, 64, 2, 4, 4)
// matrices of at least kLargeElems weights (8B-class layers): 8 waves
#define Q8_LARGE(X) X(4096, 64, 2, 1, 8) X(6144, 64, 3, 1, 8) X(8192, 64, 4, 1, 8) X(12288, 64, 6, 1, 8)
#define Q8_LARGE_SW(X) X(2048, 64, 1, 2, 8) X(4096, 64, 2, 2, 8)
constexpr int64_t kLargeElems = 16ll << 20;

}  // namespace

namespace q8k {

namespace {
// shape used for (K, epilogue): ARGMAX on K=1024 takes 32-row tiles, the
// other non-SwiGLU launches the single-row shapes where they exist
struct Shape {
  int lpr, bpl, rows, waves;
  bool large;
};
bool pick(int K, int64_t N, int epi, Shape* sh) {
#define Q8_PICK(K_, L_, B_, R_, W_) \
  if (K == K_) { *sh = Shape{L_, B_, R_, W_, false}; found = true; }
#define Q8_PICK_L(K_, L_, B_, R_, W_) \
  if (K == K_) { *sh = Shape{L_, B_, R_, W_, true}; found = true; }
  bool found = false;
  if (epi != EPI_ARGMAX && N * K >= kLargeElems) {
    if (epi == EPI_SWIGLU) {
      Q8_LARGE_SW(Q8_PICK_L)
    } else {
      Q8_LARGE(Q8_PICK_L)
    }
    if (found) return true;
  }
  Q8_SHAPES(Q8_PICK)
  if (epi != EPI_SWIGLU) { Q8_SMALL(Q8_PICK) }
  if (epi == EPI_ARGMAX) { Q8_ARGMAX(Q8_PICK) }
#undef Q8_PICK
#undef Q8_PICK_L
  return found;
}
}  // namespace

int gemv_argmax_grid(int N, int K) {
  Shape sh;
  if (!pick(K, N, EPI_ARGMAX, &sh)) return 0;
  const int rpt = sh.waves * (64 / sh.lpr) * sh.rows;
  const int ntiles = (N + rpt - 1) / rpt;
  return ntiles < kMaxGrid ? ntiles : kMaxGrid;
}

hipError_t gemv(GemvArgs a, bool norm, int epi, int grid_y, hipStream_t s) {
  Shape sh;
  if (!pick(a.K, a.N, epi, &sh)) return hipErrorInvalidValue;
#define Q8_GO(K_, L_, B_, R_, W_) \
  if (a.K == K_ && sh.lpr == L_ && sh.bpl == B_ && sh.rows == R_ && sh.waves == W_) \
    return launch_epi<L_, B_, R_, W_>(a, norm, epi, grid_y, sh.large, s);
  Q8_SHAPES(Q8_GO)
  Q8_SMALL(Q8_GO)
  Q8_ARGMAX(Q8_GO)
  Q8_LARGE(Q8_GO)
  Q8_LARGE_SW(Q8_GO)
#undef Q8_GO
  return hipErrorInvalidValue;
}

bool gemv_supported_k(int K) {
  Shape sh;
  return pick(K, 0, EPI_STORE, &sh);
}

hipError_t block_dots(const int8_t* qa, const int8_t* qs, int M, int K, int N, int32_t* S, hipStream_t s) {
  const int64_t pairs = (int64_t)M * N;
  const int64_t grid = (pairs + kBdThreads / kWave - 1) / (kBdThreads / kWave);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_dots, dim3((unsigned)grid), dim3(kBdThreads), 0, s, qa, qs, K, N, pairs, S);
  return hipGetLastError();
}

}  // namespace q8k
