// Decode-step attention for gfx950: per-head Q/K RMSNorm + NeoX RoPE + KV
// append + split-K ("flash decoding") grouped-query attention over the KV
// cache, staged in LDS, with the split combine done by the last workgroup.
//
// What is computed (Fucina course, "A transformer from scratch"):
//   q_h = rope(rmsnorm(q_h, q_norm), p), k = rope(rmsnorm(k, k_norm), p)
//     (per-head norm before RoPE: section 12.3.2 and minfer "Qwen3 Support
//     Plan" section 2.2; NeoX half-layout rotation: section 12.3.4);
//   K (post-RoPE) and V rows are written at cache row p = len (section 12.4;
//     V is never roped);
//   for query head h reading KV head g = h / (nh/nkv) (section 12.3.5):
//     s_j = (q_h . K_j) / sqrt(hd) over j <= p, softmax, o_h = sum_j w_j V_j.
//
// Grid (nsplit_max, nkv, nrows): workgroup (split, g, row) serves the G query
// heads of KV head g, so each K/V row is read once for all of them.  The
// positions [0, p] are cut into min(nsplit_max, ceil((p+1)/min_rows)) equal
// ranges; each workgroup keeps an online softmax (running max m, sum l,
// unnormalised o) and writes it as a partial; the last workgroup to arrive
// (atomic counter) merges the partials and writes the normalised output.
// The position is read on the device, so a captured graph replays unchanged.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int TJ = 64;  // cache rows per LDS tile

template <bool BF16>
QDEV float load_kv(const void* base, int64_t idx) {
  if (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

template <int HD, int G, bool BF16>
__global__ void __launch_bounds__(kThreads) k_attn_decode(AttnDecodeArgs a) {
  __shared__ float s_qf[G][HD];
  __shared__ double s_q[G][HD];
  __shared__ float s_knew[HD];
  __shared__ float s_vnew[HD];
  __shared__ float s_k[TJ][HD + 1];
  __shared__ float s_v[TJ][HD];
  __shared__ double s_p[G][TJ];
  __shared__ double s_alpha[G];
  __shared__ int s_last;

  const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int seq = a.row_seq ? a.row_seq[row] : 0;
  const int p = a.len[seq];
  const int ctx = p + 1;
  int nsplit = (ctx + a.min_rows - 1) / a.min_rows;
  if (nsplit > a.nsplit_max) nsplit = a.nsplit_max;
  if (split >= nsplit) return;  // uniform per workgroup; not counted below
  const int chunk = (ctx + nsplit - 1) / nsplit;
  const int j0 = split * chunk;
  const int j1 = min(ctx, j0 + chunk);

  const int cap = a.seq_cap[seq];
  const int nkv = a.nkv;
  const int64_t head_elems = (int64_t)cap * HD;
  const int64_t kbase = a.seq_base[seq] + ((int64_t)a.layer * 2 * nkv + g) * head_elems;
  const int64_t vbase = kbase + (int64_t)nkv * head_elems;
  const float* qkv = a.qkv + (int64_t)row * a.qkv_stride;
  const int nh = nkv * G;
  const double* cs = a.rope_cos + (int64_t)p * (HD / 2);
  const double* sn = a.rope_sin + (int64_t)p * (HD / 2);

  // stage raw q (G heads), and the new k / v of head g
  for (int e = threadIdx.x; e < G * HD; e += kThreads) s_qf[e / HD][e % HD] = qkv[(int64_t)(g * G) * HD + e];
  const bool has_new = j1 == ctx;  // this split holds position p
  if (has_new) {
    for (int d = threadIdx.x; d < HD; d += kThreads) {
      s_knew[d] = qkv[(int64_t)nh * HD + (int64_t)g * HD + d];
      s_vnew[d] = qkv[(int64_t)(nh + nkv) * HD + (int64_t)g * HD + d];
    }
  }
  __syncthreads();
  for (int h = wave; h < G; h += kWaves) norm_rope_wave<HD>(s_qf[h], a.q_norm, a.eps, cs, sn);
  if (has_new && wave == kWaves - 1) norm_rope_wave<HD>(s_knew, a.k_norm, a.eps, cs, sn);
  __syncthreads();
  for (int e = threadIdx.x; e < G * HD; e += kThreads) s_q[e / HD][e % HD] = (double)s_qf[e / HD][e % HD];
  if (has_new) {
    // append: the cache stores post-RoPE K and raw V (bf16 caches round here,
    // and the rounded values are the ones attended below)
    for (int d = threadIdx.x; d < HD; d += kThreads) {
      const int64_t ki = kbase + (int64_t)p * HD + d, vi = vbase + (int64_t)p * HD + d;
      if (BF16) {
        const uint16_t kb = f32_to_bf16_bits(s_knew[d]), vb = f32_to_bf16_bits(s_vnew[d]);
        reinterpret_cast<uint16_t*>(a.kv)[ki] = kb;
        reinterpret_cast<uint16_t*>(a.kv)[vi] = vb;
        s_knew[d] = bf16_bits_to_f32(kb);
        s_vnew[d] = bf16_bits_to_f32(vb);
      } else {
        reinterpret_cast<float*>(a.kv)[ki] = s_knew[d];
        reinterpret_cast<float*>(a.kv)[vi] = s_vnew[d];
      }
    }
  }
  __syncthreads();

  // online softmax in f64: wave h (< G) owns head h's (m, l); outputs are
  // spread over threads as e = tid + 256*i -> (head e / HD, dim e % HD)
  constexpr int OUT_PER_T = (G * HD + kThreads - 1) / kThreads;
  double o[OUT_PER_T];
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) o[i] = 0.0;
  constexpr int HPW = (G + kWaves - 1) / kWaves;  // heads per wavefront
  double m_run[HPW], l_run[HPW];  // head wave + kWaves*i, held by that wavefront
#pragma unroll
  for (int i = 0; i < HPW; ++i) m_run[i] = -INFINITY, l_run[i] = 0.0;
  const double scale = a.scale;

  for (int t0 = j0; t0 < j1; t0 += TJ) {
    const int nrow = min(TJ, j1 - t0);
    // stage K and V rows t0 .. t0+nrow-1 (row p comes from LDS)
    for (int e = threadIdx.x; e < TJ * HD; e += kThreads) {
      const int r = e / HD, d = e % HD;
      const int j = t0 + r;
      float kv_k = 0.f, kv_v = 0.f;
      if (r < nrow) {
        if (j == p) {
          kv_k = s_knew[d];
          kv_v = s_vnew[d];
        } else {
          kv_k = load_kv<BF16>(a.kv, kbase + (int64_t)j * HD + d);
          kv_v = load_kv<BF16>(a.kv, vbase + (int64_t)j * HD + d);
        }
      }
      s_k[r][d] = kv_k;
      s_v[r][d] = kv_v;
    }
    __syncthreads();
    // scores (f64): thread -> (row r = tid % TJ, head h = tid / TJ)
    for (int e = threadIdx.x; e < G * TJ; e += kThreads) {
      const int r = e % TJ, h = e / TJ;
      double s = -INFINITY;
      if (r < nrow) {
        s = 0.0;
#pragma unroll 8
        for (int d = 0; d < HD; ++d) s += s_q[h][d] * (double)s_k[r][d];
        s *= scale;
      }
      s_p[h][r] = s;
    }
    __syncthreads();
    // per-head max / exp / sum: wave h handles head h (TJ == wavefront size)
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = wave + i * kWaves;
      if (h < G) {
        const double s = s_p[h][lane];
        const double mt = wave_max_d<kWave>(s);
        const double m_new = fmax(m_run[i], mt);
        const double pr = (s == -INFINITY) ? 0.0 : exp(s - m_new);
        const double lt = wave_sum_d<kWave>(pr);
        const double alpha = (m_run[i] == -INFINITY) ? 0.0 : exp(m_run[i] - m_new);
        l_run[i] = l_run[i] * alpha + lt;
        m_run[i] = m_new;
        s_p[h][lane] = pr;
        if (lane == 0) s_alpha[h] = alpha;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OUT_PER_T; ++i) {
      const int e = threadIdx.x + i * kThreads;
      if (e < G * HD) {
        const int h = e / HD, d = e % HD;
        double acc = o[i] * s_alpha[h];
        for (int r = 0; r < nrow; ++r) acc += s_p[h][r] * (double)s_v[r][d];
        o[i] = acc;
      }
    }
    __syncthreads();
  }

  // write this split's partial: [row][g][split][h][0..HD-1] = o, [HD] = m, [HD+1] = l
  const int64_t pstride = (int64_t)G * (HD + 2);
  double* part = a.part + (((int64_t)row * nkv + g) * a.nsplit_max + split) * pstride;
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) {
    const int e = threadIdx.x + i * kThreads;
    if (e < G * HD) part[(e / HD) * (HD + 2) + (e % HD)] = o[i];
  }
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + i * kWaves;
    if (h < G && lane == 0) {
      part[h * (HD + 2) + HD] = m_run[i];
      part[h * (HD + 2) + HD + 1] = l_run[i];
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = a.counter + (int64_t)row * nkv + g;
    const unsigned prev = atomicAdd(cnt, 1u);
    s_last = prev == (unsigned)(nsplit - 1);
    if (s_last) *cnt = 0u;  // every split of this launch has arrived
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // merge the nsplit partials of the G heads (f64), round once to f32
  const double* pb = a.part + (((int64_t)row * nkv + g) * a.nsplit_max) * pstride;
  for (int e = threadIdx.x; e < G * HD; e += kThreads) {
    const int h = e / HD, d = e % HD;
    double M = -INFINITY;
    for (int sidx = 0; sidx < nsplit; ++sidx)
      M = fmax(M, __builtin_nontemporal_load(pb + sidx * pstride + h * (HD + 2) + HD));
    double L = 0.0, O = 0.0;
    for (int sidx = 0; sidx < nsplit; ++sidx) {
      const double* ps = pb + sidx * pstride + h * (HD + 2);
      const double ms = __builtin_nontemporal_load(ps + HD);
      if (ms == -INFINITY) continue;
      const double wgt = exp(ms - M);
      L += __builtin_nontemporal_load(ps + HD + 1) * wgt;
      O += __builtin_nontemporal_load(ps + d) * wgt;
    }
    a.out[(int64_t)row * a.out_stride + (int64_t)(g * G + h) * HD + d] = (float)(O / L);
  }
}

template <int HD, int G>
hipError_t launch(const AttnDecodeArgs& a, bool bf16, int nrows, hipStream_t s) {
  const dim3 grid(a.nsplit_max, a.nkv, nrows);
  if (bf16)
    hipLaunchKernelGGL((k_attn_decode<HD, G, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_decode<HD, G, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

__global__ void k_set_len(int32_t* len, int seq, int value) { len[seq] = value; }

}  // namespace

namespace q8k {

bool attn_decode_supported(int hd, int group) {
  return (hd == 64 || hd == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t attn_decode(const AttnDecodeArgs& a, int hd, int group, bool kv_bf16, int nrows, hipStream_t s) {
#define Q8_ATT(HD_, G_) \
  if (hd == HD_ && group == G_) return launch<HD_, G_>(a, kv_bf16, nrows, s);
  Q8_ATT(64, 1)
  Q8_ATT(64, 2)
  Q8_ATT(64, 4)
  Q8_ATT(64, 8)
  Q8_ATT(128, 1)
  Q8_ATT(128, 2)
  Q8_ATT(128, 4)
  Q8_ATT(128, 8)
#undef Q8_ATT
  return hipErrorInvalidValue;
}

hipError_t set_len(int32_t* len, int seq, int value, hipStream_t s) {
  hipLaunchKernelGGL(k_set_len, dim3(1), dim3(1), 0, s, len, seq, value);
  return hipGetLastError();
}

}  // namespace q8k
