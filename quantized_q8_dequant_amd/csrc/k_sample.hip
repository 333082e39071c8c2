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
// k_sample: one 1024-thread workgroup per row.
//   - max and argmax (lowest index): the greedy answer when temperature <= 0;
//   - the W best candidates (W = min(top_k, 256), or the exact-nucleus window
//     256, 1024, 4096 when top_k == 0) by a radix select on order-preserving
//     32-bit keys (four 8-bit passes of LDS histograms; counts are exact, so
//     the threshold is too), then a gather that keeps equal keys in token
//     order, then a bitonic sort of (key, inverted id) in LDS: descending
//     logit, ties by lower id;
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
constexpr int kMaxWindow = 4096;   // exact-nucleus window cap (LDS)
constexpr int kHists = kWaves / 2; // radix histograms (fewer same-bin atomics per copy)

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

__global__ void __launch_bounds__(kThreads) k_sample(const float* __restrict__ logits, int V, SampleArgs a,
                                                     const float* __restrict__ uni, int32_t* __restrict__ out) {
  __shared__ unsigned long long s_cand[kMaxWindow];  // (key << 32) | ~id; after the sort, the f64 cumulative p
  __shared__ int s_id[kMaxWindow];
  __shared__ unsigned s_hist[kHists][256];  // one histogram per pair of wavefronts
  __shared__ int s_cnt[2];
  __shared__ int s_iw[kWaves + 1];
  __shared__ double s_dw[kWaves + 1];
  __shared__ float s_bv[kWaves];
  __shared__ int s_bi[kWaves];
  __shared__ unsigned s_sel[3];  // prefix, remaining, found bin
  __shared__ int s_pos[2];       // top-p and min-p prefix lengths, then the pick
  __shared__ double s_z[1];      // the softmax denominator of the candidates
  double* s_cum = reinterpret_cast<double*>(s_cand);

  const int row = blockIdx.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const float* l = logits + (int64_t)row * V;

  // max and the lowest index of it
  float bv = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  for (int j = tid; j < V; j += kThreads) {
    const float v = l[j];
    if (v > bv || (v == bv && j < bi)) bv = v, bi = j;
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
    for (int w = 1; w < kWaves; ++w)
      if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) bv = s_bv[w], bi = s_bi[w];
    s_bv[0] = bv, s_bi[0] = bi;
  }
  __syncthreads();
  const float fmax = s_bv[0];
  if (!(a.temperature > 0.f)) {  // greedy
    if (tid == 0) out[row] = s_bi[0];
    return;
  }
  const double lmax = (double)fmax, T = (double)a.temperature;
  const double top_p = (double)a.top_p;

  // the whole-row denominator of the exact nucleus
  double zfull = 0.0;
  if (a.top_k == 0) {
    double z = 0.0;
    for (int j = tid; j < V; j += kThreads) z += exp(((double)l[j] - lmax) / T);
    zfull = block_sum(z, s_dw);
  }

  int W = a.top_k > 0 ? min(min(a.top_k, kMaxCand), V) : min(kMaxCand, V);
  const int C = (V + kThreads - 1) / kThreads;  // contiguous chunk per thread (keeps ids in order)
  for (;;) {
    // radix select: the key of the W-th best candidate (pairs of wavefronts
    // count into their own histogram; the bins are then summed in order)
    if (tid == 0) s_sel[0] = 0u, s_sel[1] = (unsigned)W;
    unsigned mask = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < kHists * 256; b += kThreads) s_hist[b / 256][b % 256] = 0u;
      __syncthreads();
      const unsigned prefix = s_sel[0];
      for (int j = tid; j < V; j += kThreads) {
        const uint32_t k = okey(l[j]);
        if ((k & mask) == prefix) atomicAdd(&s_hist[wave / 2][(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        unsigned t = 0u;
        for (int w = 0; w < kHists; ++w) t += s_hist[w][tid];
        s_hist[0][tid] = t;
      }
      __syncthreads();
      if (tid == 0) {
        unsigned rem = s_sel[1], acc = 0u;
        int b = 255;
        for (; b > 0; --b) {
          if (acc + s_hist[0][b] >= rem) break;
          acc += s_hist[0][b];
        }
        s_sel[0] = prefix | ((unsigned)b << shift);
        s_sel[1] = rem - acc;
        s_sel[2] = s_hist[0][b];  // after the last pass: the count of keys equal to the threshold
      }
      mask |= 255u << shift;
      __syncthreads();
    }
    const uint32_t thr = s_sel[0];
    const int need_eq = (int)s_sel[1];  // >= 1 candidates with key == thr, in id order
    const int cnt_gt = W - need_eq;
    const int all_eq = (int)s_sel[2];

    // gather.  Usually every key equal to the threshold fits in the window:
    // then all of them are taken with strided (coalesced) reads into slots
    // from a counter, the sort orders them (ties by id) and the first W are
    // kept.  Otherwise each thread scans its own contiguous chunk, so equal
    // keys are taken in id order.
    int NC = W;  // candidates gathered
    if (cnt_gt + all_eq <= kMaxWindow) {
      NC = cnt_gt + all_eq;
      if (tid == 0) s_cnt[0] = 0;
      __syncthreads();
      for (int j = tid; j < V; j += kThreads) {
        const uint32_t k = okey(l[j]);
        if (k >= thr) s_cand[atomicAdd(&s_cnt[0], 1)] = ((unsigned long long)k << 32) | (0xFFFFFFFFu - (uint32_t)j);
      }
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
          s_cand[ogt++] = c;
        } else if (k == thr) {
          if (oeq < need_eq) s_cand[cnt_gt + oeq] = c;
          ++oeq;
        }
      }
    }
    int W2 = 1;
    while (W2 < NC) W2 <<= 1;
    __syncthreads();
    for (int i = NC + tid; i < W2; i += kThreads) s_cand[i] = 0ull;
    __syncthreads();

    // bitonic sort, descending
    for (int k = 2; k <= W2; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < W2; i += kThreads) {
          const int p = i ^ jj;
          if (p > i) {
            const unsigned long long x = s_cand[i], y = s_cand[p];
            const bool up = (i & k) == 0;
            if ((x < y) == up) s_cand[i] = y, s_cand[p] = x;
          }
        }
        __syncthreads();
      }
    }

    // p_i in f64, then the inclusive scan (4 consecutive candidates per thread)
    double pv[4];
    double loc = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      pv[q] = 0.0;
      if (i < W) {
        const unsigned long long c = s_cand[i];
        s_id[i] = (int)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFull));
        pv[q] = exp(((double)okey_value((uint32_t)(c >> 32)) - lmax) / T);
      }
    }
    double z = zfull;
    if (a.top_k > 0) {
      double zs = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) zs += pv[q];
      z = block_sum(zs, s_dw);
    }
    if (tid == 0) s_z[0] = z;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pv[q] = pv[q] / z;
      loc += pv[q];
      pv[q] = loc;  // running local sum
    }
    double dtot;
    const double off = block_exclusive_scan(loc, s_dw, &dtot);
    __syncthreads();  // every s_cand read above is done before s_cum overwrites it
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * tid + q;
      if (i < W) s_cum[i] = off + pv[q];
    }
    __syncthreads();
    const int cap = min(V, kMaxWindow);
    if (a.top_k == 0 && top_p < 1.0 && s_cum[W - 1] < top_p && W < cap) {
      W = min(4 * W, cap);
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
      if (s_cum[i] >= top_p && (i == 0 || s_cum[i - 1] < top_p)) s_pos[0] = i + 1;
  }
  if (a.min_p > 0.f) {
    // p_i recomputed exactly as above; p descends, so p_i < min_p * p_0
    // first holds at one index
    const double z = s_z[0];
    auto p_of = [&](int i) { return exp(((double)l[s_id[i]] - lmax) / T) / z; };
    const double thr = (double)a.min_p * p_of(0);
    for (int i = tid; i < W; i += kThreads)
      if (p_of(i) < thr && (i == 0 || !(p_of(i - 1) < thr))) s_pos[1] = i;
  }
  __syncthreads();
  const int keep = max(1, min(s_pos[0], s_pos[1]));
  const double r = (double)uni[row] * s_cum[keep - 1];
  if (tid == 0) s_pos[0] = keep - 1;
  __syncthreads();
  for (int i = tid; i < keep; i += kThreads)
    if (s_cum[i] > r && (i == 0 || !(s_cum[i - 1] > r))) s_pos[0] = i;
  __syncthreads();
  if (tid == 0) out[row] = s_id[s_pos[0]];
}

}  // namespace

namespace q8k {

hipError_t sample(float* logits, int n, int V, const SampleArgs& a, const int32_t* hist, int hstride,
                  const int32_t* hlen, const float* uni, int32_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool penalise = hist && hlen && a.repeat_last_n > 0 &&
                        (a.repeat_penalty != 1.f || a.freq_penalty != 0.f || a.presence_penalty != 0.f);
  if (penalise) hipLaunchKernelGGL(k_penalties, dim3(n), dim3(256), 0, s, logits, V, hist, hstride, hlen, a);
  hipLaunchKernelGGL(k_sample, dim3(n), dim3(kThreads), 0, s, logits, V, a, uni, out);
  return hipGetLastError();
}

}  // namespace q8k
