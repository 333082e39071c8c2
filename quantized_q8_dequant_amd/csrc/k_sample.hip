// Sampling pipeline for gfx950: one token per row of f32 logits, in the
// order of Fucina course, "A transformer from scratch", section 12.6 and
// Fucina reference, "The LLM stack (fucina_llm)", section 13.6:
// penalties (in place) -> greedy shortcut -> top-k -> temperature softmax ->
// top-p -> min-p -> one draw.
//
// k_penalties: one workgroup per row; each distinct token of the row's last
// repeat_last_n history tokens (counted c times there) has its logit divided
// (positive) or multiplied (negative) by repeat_penalty, then c * freq +
// presence subtracted, in f64, rounded back to f32 once.
//
// k_sample_slices: one workgroup per (4096-logit slice, row): the slice's
// max (lowest index on ties), its partial softmax denominator (exact
// nucleus) and its list of keys at or above its W1-th best, by a radix
// select on order-preserving 32-bit keys (four 8-bit passes of LDS
// histograms: the counts are exact, so the cut is too).
//
// k_sample: one 1024-thread workgroup per row.
//   - max and argmax from the slices': the greedy answer when temperature <= 0;
//   - the W best candidates (W = min(top_k, 256), or the exact-nucleus window
//     256, 1024, 4096, 16384, 65536, ... up to the vocabulary when top_k == 0),
//     descending logit, ties by lower id.
//     The union of the slices' lists holds every key at or above the highest
//     cut T* of a partial list; a union of up to 8192 keys is copied to LDS.
//     Per window a radix select over that copy (else over the union in
//     memory; over the whole row when the union may miss keys of the
//     window) gives the W-th key, a gather takes the keys at or above it
//     (ties in id order) and a bitonic sort held in registers orders them.
//     A window of more than 4096 candidates lives in the caller's scratch:
//     the row's keys at or above the W-th are gathered in id order and put
//     in descending order by a stable radix sort (4-bit digits), so ties
//     stay in id order, and the cumulative p go to the scratch too;
//   - p_i = exp((l_i - l_max) / T) / Z in f64, Z over the W candidates
//     (top_k > 0) or over the whole row (top_k == 0), an inclusive f64 scan,
//     the top-p prefix, the min-p prefix, and the inverse-CDF draw of the
//     row's uniform against the kept total.
// Each scan adds non-negative terms, so the cumulative values are monotone
// and every "first index where" search has one answer.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxCand = 256;      // top_k cap (the pages' candidate limit)
constexpr int kMaxWindow = 4096;   // windows up to this size live in LDS
constexpr int kUnionCap = 8192;    // slice-list union copied to LDS
constexpr int kHists = kWaves / 2; // radix histograms (fewer same-bin atomics per copy)

// Stage-1 results: per (row, slice) the max, its lowest index, the partial
// denominator and the candidate list (kSlice slots, cnt used).
struct SliceScratch {
  unsigned long long* cand;
  unsigned long long* wide;  // per row V more slots: the exact nucleus's wide window
  double* z;
  float* m;
  int* am;
  int* cnt;
  unsigned* thr;  // the list's cut (its W1-th best key), 0 when it holds the whole slice
  int S;
};

QDEV uint32_t okey(float v) {  // order-preserving bits; -0 and +0 tie
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
QDEV float okey_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__global__ void __launch_bounds__(256) k_penalties(float* __restrict__ logits, int V, const int32_t* __restrict__ hist,
                                                   int hstride, const int32_t* __restrict__ hlen, SampleArgs a) {
#pragma clang fp contract(off)
  const int row = blockIdx.x;
  const int len = min(max(hlen[row], 0), hstride);
  const int win = min(len, a.repeat_last_n);
  const int32_t* h = hist + (int64_t)row * hstride + (len - win);
  for (int t = threadIdx.x; t < win; t += 256) {
    const int tok = h[t];
    if (tok < 0 || tok >= V) continue;
    bool first = true;
    int c = 0;
    for (int j = 0; j < win; ++j) {
      if (h[j] == tok) {
        if (j < t) first = false;
        ++c;
      }
    }
    if (!first) continue;  // the token's first occurrence applies it once
    float* p = logits + (int64_t)row * V + tok;
    double v = (double)*p;
    v = v > 0 ? v / (double)a.repeat_penalty : v * (double)a.repeat_penalty;
    v = v - ((double)c * (double)a.freq_penalty + (double)a.presence_penalty);
    *p = (float)v;
  }
}

// f(j, l[j], valid) for every j < V, by all threads of the workgroup; every
// thread calls f the same number of times (valid == false past the row), so
// f may ballot.  With V a multiple of 4 (rows 16-byte aligned) each thread
// keeps four float4 loads in flight per step: one load at a time would leave
// every pass waiting out the memory latency once per element group.
template <typename F>
QDEV void for_row(const float* __restrict__ l, int V, F&& f) {
  const int tid = threadIdx.x;
  if ((V & 3) == 0) {
    const float4* l4 = reinterpret_cast<const float4*>(l);
    const int V4 = V / 4;
    for (int base = 0; base < V4; base += 4 * kThreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kThreads + tid;
        v[u] = i < V4 ? l4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kThreads + tid;
        const bool ok = i < V4;
        f(4 * i, v[u].x, ok);
        f(4 * i + 1, v[u].y, ok);
        f(4 * i + 2, v[u].z, ok);
        f(4 * i + 3, v[u].w, ok);
      }
    }
  } else {
    for (int base = 0; base < V; base += kThreads) {
      const int j = base + tid;
      f(j, j < V ? l[j] : 0.f, j < V);
    }
  }
}

// A slot in an LDS list for each lane whose `take` is set: one atomic per
// wavefront (its lanes' count), each lane offset by the taking lanes below it.
QDEV int claim_slot(bool take, int* counter) {
  const int lane = threadIdx.x % kWave;
  const unsigned long long m = __ballot(take);
  if (m == 0ull) return -1;
  const int leader = __ffsll((long long)m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, leader);
  return take ? base + __popcll(m & ((1ull << lane) - 1ull)) : -1;
}

// Counts one key into bin `bin` of an LDS histogram for each lane whose
// `take` is set.  The keys of a radix pass crowd into few bins (the best
// logits share their sign and exponent), and lanes adding to one address
// are served one at a time: so the lanes of the two most common bins of the
// wavefront are counted with one atomic each, the rest lane by lane.
QDEV void hist_add(unsigned* h, unsigned bin, bool take) {
  const int lane = threadIdx.x % kWave;
  unsigned long long rem = __ballot(take);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (rem == 0ull) return;
    const int leader = __ffsll((long long)rem) - 1;
    const unsigned b0 = __shfl(bin, leader);
    const unsigned long long same = __ballot(bin == b0) & rem;
    if (lane == leader) atomicAdd(&h[b0], (unsigned)__popcll(same));
    rem &= ~same;
  }
  if ((rem >> lane) & 1ull) atomicAdd(&h[bin], 1u);
}

// The bin (8 bits at `shift`) of the rem-th largest counted key, for radix
// select: every thread of the workgroup calls it; thread t < 256 takes bin
// 255 - t, so a prefix scan over t counts the keys in the bins above.  One
// bin satisfies above < rem <= above + count; it writes the prefix, the rank
// left within it and its count to s_sel.
template <int NW>
QDEV void pick_bin(const unsigned* hist, unsigned* s_w, unsigned* s_sel, int shift) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const unsigned rem = s_sel[1], prefix = s_sel[0];
  const unsigned c = tid < 256 ? hist[255 - tid] : 0u;
  unsigned inc = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) s_w[wave] = inc;
  __syncthreads();
  unsigned before = 0u;  // bins live in the first 256 threads (four wavefronts)
  if (tid < 256)
    for (int w = 0; w < wave && w < NW; ++w) before += s_w[w];
  const unsigned above = before + inc - c;
  __syncthreads();  // every thread has read s_sel and s_w
  if (tid < 256 && above < rem && above + c >= rem) {
    s_sel[0] = prefix | ((unsigned)(255 - tid) << shift);
    s_sel[1] = rem - above;
    s_sel[2] = c;
  }
}

// Block-wide exclusive scan of one value per thread (order: thread index);
// returns the exclusive prefix, *total gets the sum.  T: int or double.
template <typename T>
QDEV T block_exclusive_scan(T v, T* s_w, T* total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  T inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == kWave - 1) s_w[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T acc = 0;
    for (int w = 0; w < kWaves; ++w) {
      const T t = s_w[w];
      s_w[w] = acc;
      acc += t;
    }
    s_w[kWaves] = acc;
  }
  __syncthreads();
  const T ex = s_w[wave] + inc - v;
  *total = s_w[kWaves];
  __syncthreads();  // s_w reusable
  return ex;
}

template <typename T>
QDEV T block_sum(T v, T* s_w) {  // fixed order: lanes by halving, then waves in order
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  T t = 0;
  for (int w = 0; w < kWaves; ++w) t += s_w[w];
  __syncthreads();
  return t;
}

// Bitonic sort, descending, of s[0, n) padded with zeros (below every key)
// to n2, a power of two of at most E * kThreads, by the whole workgroup.  Thread t holds the E consecutive
// elements from E t in registers: compare distances below E stay in the
// thread, those below E * 64 are lane exchanges within the wavefront, and
// only the wider ones go through LDS (two barriers each).  At distance jj
// in a merge of size k, element i keeps the larger of itself and i ^ jj
// when (i & jj == 0) equals (i & k == 0).
template <int E>
QDEV void sort_desc(unsigned long long* s, int n, int n2) {
  const int i0 = threadIdx.x * E;
  unsigned long long v[E];
#pragma unroll
  for (int q = 0; q < E; ++q) v[q] = i0 + q < n ? s[i0 + q] : 0ull;
  auto settle = [&](int q, unsigned long long y, int jj, int k) {
    const int i = i0 + q;
    const bool keep_max = ((i & jj) == 0) == ((i & k) == 0);
    v[q] = keep_max ? (v[q] > y ? v[q] : y) : (v[q] < y ? v[q] : y);
  };
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= E * kWave) {
        __syncthreads();  // earlier reads of s are done
#pragma unroll
        for (int q = 0; q < E; ++q)
          if (i0 + q < n2) s[i0 + q] = v[q];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < E; ++q)
          if (i0 + q < n2) settle(q, s[(i0 + q) ^ jj], jj, k);
      } else if (jj >= E) {
        const int lm = jj / E;
#pragma unroll
        for (int q = 0; q < E; ++q) settle(q, __shfl_xor(v[q], lm), jj, k);
      } else {
        // jj < E: partners in this thread's registers (indices fixed at
        // compile time, so the array stays in registers)
        unsigned long long w[E];
#pragma unroll
        for (int q = 0; q < E; ++q) w[q] = v[q];
#pragma unroll
        for (int d = 1; d < E; d <<= 1)
          if (d == jj) {
#pragma unroll
            for (int q = 0; q < E; ++q) settle(q, w[q ^ d], jj, k);
          }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < E; ++q)
    if (i0 + q < n2) s[i0 + q] = v[q];
  __syncthreads();
}

QDEV void sort_window(unsigned long long* s, int n) {
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  if (n2 > 2 * kThreads) sort_desc<4>(s, n, n2);
  else if (n2 > kThreads) sort_desc<2>(s, n, n2);
  else sort_desc<1>(s, n, n2);
}

// Stable sort, descending by key (the high 32 bits), of the n elements at a,
// with b (n slots) as the other buffer: one pass per 4-bit digit from bit 0
// up to the digit at top_shift (the keys agree above it; top_shift < 0: all
// keys are equal and a is already in order).  Each thread takes a contiguous
// chunk, counts its digits into its own column of s_cnt (16 x kThreads),
// the counts are scanned in (digit, thread) order, and the chunk is
// scattered in its order, so equal digits keep their order.  Returns the
// buffer that holds the result.
QDEV unsigned long long* radix_sort_desc(unsigned long long* a, unsigned long long* b, int n, int top_shift,
                                         unsigned* s_cnt, int* s_iw) {
  const int tid = threadIdx.x;
  const int C = (n + kThreads - 1) / kThreads;
  const int j0 = min(n, tid * C), j1 = min(n, j0 + C);
  for (int shift = 0; shift <= top_shift; shift += 4) {
#pragma unroll
    for (int d = 0; d < 16; ++d) s_cnt[d * kThreads + tid] = 0u;
    for (int j = j0; j < j1; ++j) {
      const unsigned d = 15u - (unsigned)((a[j] >> (32 + shift)) & 15ull);
      s_cnt[d * kThreads + tid] += 1u;
    }
    __syncthreads();
    unsigned loc[16];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      loc[q] = s_cnt[16 * tid + q];
      sum += (int)loc[q];
    }
    int total;
    unsigned run = (unsigned)block_exclusive_scan(sum, s_iw, &total);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      s_cnt[16 * tid + q] = run;
      run += loc[q];
    }
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
      const unsigned long long e = a[j];
      const unsigned d = 15u - (unsigned)((e >> (32 + shift)) & 15ull);
      const unsigned pos = s_cnt[d * kThreads + tid];
      s_cnt[d * kThreads + tid] = pos + 1u;
      b[pos] = e;
    }
    __syncthreads();  // b is whole before the next pass reads it
    unsigned long long* t = a;
    a = b;
    b = t;
  }
  return a;
}

// Stage 1: one 256-thread workgroup per (slice of kSlice logits, row): the
// slice's max and its lowest index, its partial denominator relative to its
// own max (exact nucleus), and every logit at or above the slice's W1-th
// best (radix select on 16 keys per thread), written as (key << 32) | ~id,
// with that cut (0 when the list holds the whole slice).
constexpr int kSlice = 4096;
constexpr int kSliceThreads = 256;
constexpr int kSliceWaves = kSliceThreads / kWave;

__global__ void __launch_bounds__(kSliceThreads) k_sample_slices(const float* __restrict__ logits, int V, SampleArgs a,
                                                                 int W1, SliceScratch ss) {
  __shared__ unsigned s_hist[kSliceWaves][256];
  __shared__ float s_bv[kSliceWaves];
  __shared__ int s_bi[kSliceWaves];
  __shared__ double s_dz[kSliceWaves];
  __shared__ unsigned s_sel[3];
  __shared__ unsigned s_uw[kSliceWaves];
  __shared__ int s_n;
  const int sl = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int j0 = sl * kSlice;
  const int n = min(kSlice, V - j0);
  const float* l = logits + (int64_t)row * V + j0;
  constexpr int PER = kSlice / kSliceThreads;  // 16
  float v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * kSliceThreads;
    v[k] = i < n ? l[i] : -__builtin_inff();
  }
  float bv = -__builtin_inff();
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * kSliceThreads;
    if (i < n && (v[k] > bv || (v[k] == bv && j0 + i < bi))) bv = v[k], bi = j0 + i;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) bv = ov, bi = oi;
  }
  if (lane == 0) s_bv[wave] = bv, s_bi[wave] = bi;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSliceWaves; ++w)
      if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) bv = s_bv[w], bi = s_bi[w];
    const int64_t o = (int64_t)row * ss.S + sl;
    ss.m[o] = bv;
    ss.am[o] = bi;
    s_bv[0] = bv;
  }
  __syncthreads();
  if (!(a.temperature > 0.f)) return;  // greedy: the maxima are all stage 2 needs
  const float ms = s_bv[0];
  if (a.top_k == 0) {
    double z = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + k * kSliceThreads < n) z += exp(((double)v[k] - (double)ms) / (double)a.temperature);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0) s_dz[wave] = z;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w = 0; w < kSliceWaves; ++w) t += s_dz[w];
      ss.z[(int64_t)row * ss.S + sl] = t;
    }
  }
  // the slice's W1-th best key
  const int w1 = min(W1, n);
  uint32_t key[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) key[k] = tid + k * kSliceThreads < n ? okey(v[k]) : 0u;
  if (tid == 0) s_sel[0] = 0u, s_sel[1] = (unsigned)w1, s_n = 0;
  unsigned mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < kSliceWaves * 256; b += kSliceThreads) s_hist[b / 256][b % 256] = 0u;
    __syncthreads();
    const unsigned prefix = s_sel[0];
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + k * kSliceThreads < n && (key[k] & mask) == prefix) atomicAdd(&s_hist[wave][(key[k] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 256) {
      unsigned t = 0u;
      for (int w = 0; w < kSliceWaves; ++w) t += s_hist[w][tid];
      s_hist[0][tid] = t;
    }
    __syncthreads();
    pick_bin<kSliceWaves>(s_hist[0], s_uw, s_sel, shift);
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = s_sel[0];
  unsigned long long* dst = ss.cand + ((int64_t)row * ss.S + sl) * kSlice;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * kSliceThreads;
    const bool take = i < n && key[k] >= thr;
    const int slot = claim_slot(take, &s_n);
    if (take) dst[slot] = ((unsigned long long)key[k] << 32) | (0xFFFFFFFFu - (uint32_t)(j0 + i));
  }
  __syncthreads();
  if (tid == 0) {
    ss.cnt[(int64_t)row * ss.S + sl] = s_n;
    ss.thr[(int64_t)row * ss.S + sl] = n > W1 ? thr : 0u;
  }
}

// Stage 2: one 1024-thread workgroup per row.
__global__ void __launch_bounds__(kThreads) k_sample(const float* __restrict__ logits, int V, SampleArgs a,
                                                     const float* __restrict__ uni, int32_t* __restrict__ out,
                                                     SliceScratch ss) {
  __shared__ unsigned long long s_u[kUnionCap];      // the union of the slices' lists
  __shared__ unsigned long long s_cand[kMaxWindow];  // (key << 32) | ~id of the window, sorted descending
  __shared__ double s_cum[kMaxWindow];               // inclusive cumulative p of the window
  __shared__ unsigned s_hist[kHists][256];           // one histogram per pair of wavefronts
  __shared__ int s_cnt[2];
  __shared__ int s_iw[kWaves + 1];
  __shared__ double s_dw[kWaves + 1];
  __shared__ float s_bv[kWaves];
  __shared__ int s_bi[kWaves];
  __shared__ unsigned s_sel[3];  // prefix, remaining rank, the bin's count
  __shared__ unsigned s_uw[kWaves];
  __shared__ unsigned s_ut[kWaves];
  __shared__ unsigned s_lo;
  __shared__ int s_pos[2];  // top-p and min-p prefix lengths, then the pick
  __shared__ double s_z[1];  // the softmax denominator of the candidates

  const int row = blockIdx.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const float* l = logits + (int64_t)row * V;
  const int64_t r0 = (int64_t)row * ss.S;

  // max and the lowest index of it, from the slices' maxima; the union's
  // size U and the highest cut T* among the slices whose list is partial
  float bv = -__builtin_inff();
  int bi = 0x7FFFFFFF, U = 0;
  unsigned tstar = 0u;
  for (int sl = tid; sl < ss.S; sl += kThreads) {
    const float v = ss.m[r0 + sl];
    const int j = ss.am[r0 + sl];
    if (v > bv || (v == bv && j < bi)) bv = v, bi = j;
    U += ss.cnt[r0 + sl];
    tstar = max(tstar, ss.thr[r0 + sl]);
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) bv = ov, bi = oi;
    U += __shfl_xor(U, o);
    tstar = max(tstar, (unsigned)__shfl_xor((int)tstar, o));
  }
  if (lane == 0) s_bv[wave] = bv, s_bi[wave] = bi, s_iw[wave] = U, s_ut[wave] = tstar;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) {
      if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) bv = s_bv[w], bi = s_bi[w];
      U += s_iw[w];
      tstar = max(tstar, s_ut[w]);
    }
    s_bv[0] = bv, s_bi[0] = bi, s_iw[kWaves] = U, s_ut[0] = tstar;
  }
  __syncthreads();
  const float fmax = s_bv[0];
  if (!(a.temperature > 0.f)) {  // greedy
    if (tid == 0) out[row] = s_bi[0];
    return;
  }
  U = s_iw[kWaves];
  tstar = s_ut[0];
  const double lmax = (double)fmax, T = (double)a.temperature;
  const double top_p = (double)a.top_p;

  // the whole-row denominator of the exact nucleus: the slices' partials,
  // each rescaled from its own max to the row's
  double zfull = 0.0;
  if (a.top_k == 0) {
    double zt = 0.0;
    for (int sl = tid; sl < ss.S; sl += kThreads) zt += ss.z[r0 + sl] * exp(((double)ss.m[r0 + sl] - lmax) / T);
    zfull = block_sum(zt, s_dw);
  }

  // The union of the slices' lists holds every key >= T* of the row (a
  // partial list holds all of its slice's keys >= its cut), so the union's
  // best W are the row's best W when W <= NV, the union's count of keys
  // >= T*.  A union that fits LDS is copied there once.
  const unsigned long long* crow = ss.cand + r0 * kSlice;
  const int* nrow = ss.cnt + r0;
  enum { kFromLds, kFromUnion, kFromRow };
  int src = U <= kUnionCap ? kFromLds : kFromUnion;
  int NV = 0;
  unsigned ulo = 0u;  // the union's lowest key
  if (src == kFromLds) {
    if (tid == 0) s_cnt[0] = 0, s_cnt[1] = 0, s_lo = 0xFFFFFFFFu;
    __syncthreads();
    for (int sl = wave; sl < ss.S; sl += kWaves) {
      const int c = nrow[sl];
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_cnt[0], c);
      base = __shfl(base, 0);
      for (int i = lane; i < c; i += kWave) s_u[base + i] = crow[(int64_t)sl * kSlice + i];
    }
    __syncthreads();
    int nv = 0;
    unsigned lo = 0xFFFFFFFFu;
    for (int i = tid; i < U; i += kThreads) {
      const uint32_t k = (uint32_t)(s_u[i] >> 32);
      nv += k >= tstar;
      lo = min(lo, k);
    }
    for (int o = kWave / 2; o > 0; o >>= 1) {
      nv += __shfl_xor(nv, o);
      lo = min(lo, (unsigned)__shfl_xor((int)lo, o));
    }
    if (lane == 0) atomicAdd(&s_cnt[1], nv), atomicMin(&s_lo, lo);
    __syncthreads();
    NV = s_cnt[1];
    ulo = s_lo;
    __syncthreads();
  }

  // f(key, id, valid) over the source's elements; every lane of a wavefront
  // calls f the same number of times (valid == false past the end)
  auto for_elems = [&](auto&& f) {
    if (src == kFromLds) {
      for (int base = 0; base < U; base += 2 * kThreads) {
        unsigned long long e[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = base + u * kThreads + tid;
          e[u] = i < U ? s_u[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
          f((uint32_t)(e[u] >> 32), (int)(0xFFFFFFFFu - (uint32_t)(e[u] & 0xFFFFFFFFull)),
            base + u * kThreads + tid < U);
      }
    } else if (src == kFromUnion) {
      for (int sl = wave; sl < ss.S; sl += kWaves) {
        const int c = nrow[sl];
        const unsigned long long* p = crow + (int64_t)sl * kSlice;
        for (int base = 0; base < c; base += 4 * kWave) {
          unsigned long long e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = base + u * kWave + lane;
            e[u] = i < c ? p[i] : 0ull;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            f((uint32_t)(e[u] >> 32), (int)(0xFFFFFFFFu - (uint32_t)(e[u] & 0xFFFFFFFFull)),
              base + u * kWave + lane < c);
        }
      }
    } else {
      for_row(l, V, [&](int j, float v, bool valid) { f(okey(v), j, valid); });
    }
  };

  int W = a.top_k > 0 ? min(min(a.top_k, kMaxCand), V) : min(kMaxCand, V);
  const int C = (V + kThreads - 1) / kThreads;  // contiguous chunk per thread (keeps ids in order)
  // the window and its cumulative p: in LDS, or for a wide exact-nucleus
  // window in the caller's scratch (the row's list slots and V more)
  unsigned long long* cand = s_cand;
  double* cum = s_cum;
  unsigned long long* const gA = ss.cand + r0 * kSlice;  // S * kSlice >= V slots
  unsigned long long* const gB = ss.wide + (int64_t)row * V;
  for (;;) {
    const bool wide = W > kMaxWindow;
    if (wide) src = kFromRow;
    if (src == kFromLds && W > NV) src = kFromRow;  // past what the union is sure to hold
    // radix select: the key of the W-th best candidate (pairs of wavefronts
    // count into their own histogram; the bins are then summed).  The
    // union's keys lie in [ulo, okey(max)]: the leading bytes those share
    // are every key's, so the passes start at the first byte that differs
    // (the last pass always runs: it counts the ties).
    int start = 24;
    unsigned mask = 0u;
    if (src == kFromLds) {
      const unsigned d = ulo ^ okey(fmax);
      start = d >= (1u << 24) ? 24 : d >= (1u << 16) ? 16 : d >= (1u << 8) ? 8 : 0;
      mask = start == 24 ? 0u : 0xFFFFFFFFu << (start + 8);
    }
    if (tid == 0) s_sel[0] = okey(fmax) & mask, s_sel[1] = (unsigned)W;
    for (int shift = start; shift >= 0; shift -= 8) {
      for (int b = tid; b < kHists * 256; b += kThreads) s_hist[b / 256][b % 256] = 0u;
      __syncthreads();
      const unsigned prefix = s_sel[0];
      for_elems([&](uint32_t k, int, bool valid) {
        hist_add(s_hist[wave / 2], (k >> shift) & 255u, valid && (k & mask) == prefix);
      });
      __syncthreads();
      if (tid < 256) {
        unsigned t = 0u;
        for (int w = 0; w < kHists; ++w) t += s_hist[w][tid];
        s_hist[0][tid] = t;
      }
      __syncthreads();
      pick_bin<kWaves>(s_hist[0], s_uw, s_sel, shift);  // s_sel[2]: after the last pass, the ties
      mask |= 255u << shift;
      __syncthreads();
    }
    const uint32_t thr = s_sel[0];
    const int need_eq = (int)s_sel[1];  // >= 1 candidates with key == thr, in id order
    const int cnt_gt = W - need_eq;
    const int all_eq = (int)s_sel[2];
    if (src != kFromRow && (thr < tstar || cnt_gt + all_eq > kMaxWindow)) {
      // the union may miss keys of the window, or too many ties for the
      // window: redo over the row
      src = kFromRow;
      __syncthreads();
      continue;
    }

    // gather.  Usually every key equal to the threshold fits in the window:
    // then all of them are taken into slots from a counter, the sort orders
    // them (ties by id) and the first W are kept.  Otherwise (and always for
    // a wide window) each thread scans its own contiguous chunk of the row,
    // so equal keys are taken in id order.
    cand = wide ? gA : s_cand;
    cum = s_cum;
    int NC = W;  // candidates gathered
    if (!wide && cnt_gt + all_eq <= kMaxWindow) {
      NC = cnt_gt + all_eq;
      if (tid == 0) s_cnt[0] = 0;
      __syncthreads();
      for_elems([&](uint32_t k, int j, bool valid) {
        const bool take = valid && k >= thr;
        const int slot = claim_slot(take, &s_cnt[0]);
        if (take) s_cand[slot] = ((unsigned long long)k << 32) | (0xFFFFFFFFu - (uint32_t)j);
      });
    } else {
      int ngt = 0, neq = 0;
      const int j0 = tid * C, j1 = min(V, j0 + C);
      for (int j = j0; j < j1; ++j) {
        const uint32_t k = okey(l[j]);
        ngt += k > thr;
        neq += k == thr;
      }
      int tot;
      int ogt = block_exclusive_scan(ngt, s_iw, &tot);
      int oeq = block_exclusive_scan(neq, s_iw, &tot);
      for (int j = j0; j < j1; ++j) {
        const uint32_t k = okey(l[j]);
        const unsigned long long c = ((unsigned long long)k << 32) | (0xFFFFFFFFu - (uint32_t)j);
        if (k > thr) {
          cand[ogt++] = c;
        } else if (k == thr) {
          if (oeq < need_eq) cand[cnt_gt + oeq] = c;
          ++oeq;
        }
      }
    }
    __syncthreads();

    double z = zfull;
    if (!wide) {
      sort_window(s_cand, NC);
      // p_i in f64, then the inclusive scan (4 consecutive candidates per thread)
      double pv[4];
      double loc = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * tid + q;
        pv[q] = i < W ? exp(((double)okey_value((uint32_t)(s_cand[i] >> 32)) - lmax) / T) : 0.0;
      }
      if (a.top_k > 0) {
        double zs = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) zs += pv[q];
        z = block_sum(zs, s_dw);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pv[q] = pv[q] / z;
        loc += pv[q];
        pv[q] = loc;  // running local sum
      }
      double dtot;
      const double off = block_exclusive_scan(loc, s_dw, &dtot);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * tid + q;
        if (i < W) s_cum[i] = off + pv[q];
      }
    } else {
      // the keys of the window agree above the highest bit where the W-th
      // key and the maximum differ: the sort needs only the digits below
      const unsigned dk = thr ^ okey(fmax);
      const int top_shift = dk == 0u ? -4 : ((31 - __builtin_clz(dk)) / 4) * 4;
      cand = radix_sort_desc(gA, gB, W, top_shift, reinterpret_cast<unsigned*>(s_u), s_iw);
      cum = reinterpret_cast<double*>(cand == gA ? gB : gA);
      // p_i in f64 and the inclusive scan, a contiguous chunk per thread
      const int C2 = (W + kThreads - 1) / kThreads;
      const int j0 = min(W, tid * C2), j1 = min(W, j0 + C2);
      double loc = 0.0;
      for (int j = j0; j < j1; ++j) loc += exp(((double)okey_value((uint32_t)(cand[j] >> 32)) - lmax) / T) / z;
      double dtot;
      double run = block_exclusive_scan(loc, s_dw, &dtot);
      for (int j = j0; j < j1; ++j) {
        run += exp(((double)okey_value((uint32_t)(cand[j] >> 32)) - lmax) / T) / z;
        cum[j] = run;
      }
    }
    if (tid == 0) s_z[0] = z;
    __syncthreads();
    if (a.top_k == 0 && top_p < 1.0 && cum[W - 1] < top_p && W < V) {
      W = min(4 * W, V);
      __syncthreads();
      continue;
    }
    break;
  }

  // top-p, then min-p: each cuts a descending prefix
  if (tid == 0) s_pos[0] = W, s_pos[1] = W;
  __syncthreads();
  if (top_p < 1.0) {
    for (int i = tid; i < W; i += kThreads)
      if (cum[i] >= top_p && (i == 0 || cum[i - 1] < top_p)) s_pos[0] = i + 1;
  }
  if (a.min_p > 0.f) {
    // p_i recomputed exactly as above; p descends, so p_i < min_p * p_0
    // first holds at one index
    const double z = s_z[0];
    auto p_of = [&](int i) { return exp(((double)okey_value((uint32_t)(cand[i] >> 32)) - lmax) / T) / z; };
    const double thr = (double)a.min_p * p_of(0);
    for (int i = tid; i < W; i += kThreads)
      if (p_of(i) < thr && (i == 0 || !(p_of(i - 1) < thr))) s_pos[1] = i;
  }
  __syncthreads();
  const int keep = max(1, min(s_pos[0], s_pos[1]));
  const double r = (double)uni[row] * cum[keep - 1];
  if (tid == 0) s_pos[0] = keep - 1;
  __syncthreads();
  for (int i = tid; i < keep; i += kThreads)
    if (cum[i] > r && (i == 0 || !(cum[i - 1] > r))) s_pos[0] = i;
  __syncthreads();
  if (tid == 0) out[row] = (int)(0xFFFFFFFFu - (uint32_t)(cand[s_pos[0]] & 0xFFFFFFFFull));
}

}  // namespace

namespace q8k {

size_t sample_work_bytes(int n, int V) {
  const size_t S = (size_t)((V + kSlice - 1) / kSlice);
  return (size_t)n * S * ((size_t)kSlice * 8 + 8 + 4 + 4 + 4 + 4) + (size_t)n * V * 8 + 256;
}

hipError_t sample(float* logits, int n, int V, const SampleArgs& a, const int32_t* hist, int hstride,
                  const int32_t* hlen, const float* uni, int32_t* out, void* work, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool penalise = hist && hlen && a.repeat_last_n > 0 &&
                        (a.repeat_penalty != 1.f || a.freq_penalty != 0.f || a.presence_penalty != 0.f);
  if (penalise) hipLaunchKernelGGL(k_penalties, dim3(n), dim3(256), 0, s, logits, V, hist, hstride, hlen, a);
  const int S = (V + kSlice - 1) / kSlice;
  SliceScratch ss{};
  ss.S = S;
  uint8_t* w = static_cast<uint8_t*>(work);
  const size_t rs = (size_t)n * S;
  ss.cand = reinterpret_cast<unsigned long long*>(w);
  w += rs * kSlice * 8;
  ss.wide = reinterpret_cast<unsigned long long*>(w);
  w += (size_t)n * V * 8;
  ss.z = reinterpret_cast<double*>(w);
  ss.m = reinterpret_cast<float*>(w + rs * 8);
  ss.am = reinterpret_cast<int*>(w + rs * 12);
  ss.cnt = reinterpret_cast<int*>(w + rs * 16);
  ss.thr = reinterpret_cast<unsigned*>(w + rs * 20);
  // Each slice lists its best W1, sized so the union fits the LDS copy
  // (W1 <= kUnionCap / S); for top-k no more than min(top_k, 256) are needed
  const int W1 = max(1, min(a.top_k > 0 ? min(a.top_k, kMaxCand) : kUnionCap, kUnionCap / S));
  hipLaunchKernelGGL(k_sample_slices, dim3(S, n), dim3(kSliceThreads), 0, s, logits, V, a, W1, ss);
  hipLaunchKernelGGL(k_sample, dim3(n), dim3(kThreads), 0, s, logits, V, a, uni, out, ss);
  return hipGetLastError();
}

}  // namespace q8k
