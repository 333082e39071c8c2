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
constexpr int TJ = 32;  // cache rows per tile
constexpr int kMaxSplit = 128;  // bound of nsplit_max

// One tile of K and V rows staged through registers: every thread issues
// all of its 16-byte loads for the tile at once (one memory round trip),
// and the next tile's loads are in flight while the current tile is used.
template <int HD, bool BF16>
struct TileRegs {
  static constexpr int ELEMS = TJ * HD;                  // per matrix
  static constexpr int PER_LOAD = BF16 ? 8 : 4;           // elements per 16 bytes
  static constexpr int LOADS = ELEMS / PER_LOAD / kThreads;  // per thread per matrix
  int4 k[LOADS], v[LOADS];
};

template <int HD, bool BF16>
QDEV void tile_load(TileRegs<HD, BF16>& t, const void* kv, int64_t kbase, int64_t vbase, int row0, int nrow) {
  constexpr int PER = TileRegs<HD, BF16>::PER_LOAD;
  constexpr int ESZ = BF16 ? 2 : 4;
#pragma unroll
  for (int i = 0; i < TileRegs<HD, BF16>::LOADS; ++i) {
    const int e = (threadIdx.x + i * kThreads) * PER;  // element index in the tile
    const int r = e / HD;
    if (r < nrow) {
      const int64_t off = (int64_t)(row0 + r) * HD + (e % HD);
      t.k[i] = *reinterpret_cast<const int4*>(static_cast<const uint8_t*>(kv) + (kbase + off) * ESZ);
      t.v[i] = *reinterpret_cast<const int4*>(static_cast<const uint8_t*>(kv) + (vbase + off) * ESZ);
    } else {
      t.k[i] = int4{0, 0, 0, 0};
      t.v[i] = int4{0, 0, 0, 0};
    }
  }
}

template <int HD, bool BF16>
QDEV void tile_store(const TileRegs<HD, BF16>& t, float (*s_k)[HD + 1], float (*s_v)[HD + 1]) {
  constexpr int PER = TileRegs<HD, BF16>::PER_LOAD;
#pragma unroll
  for (int i = 0; i < TileRegs<HD, BF16>::LOADS; ++i) {
    const int e = (threadIdx.x + i * kThreads) * PER;
    const int r = e / HD, d = e % HD;
    if (BF16) {
      const uint32_t kw[4] = {(uint32_t)t.k[i].x, (uint32_t)t.k[i].y, (uint32_t)t.k[i].z, (uint32_t)t.k[i].w};
      const uint32_t vw[4] = {(uint32_t)t.v[i].x, (uint32_t)t.v[i].y, (uint32_t)t.v[i].z, (uint32_t)t.v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s_k[r][d + 2 * j] = __uint_as_float(kw[j] << 16);
        s_k[r][d + 2 * j + 1] = __uint_as_float(kw[j] & 0xFFFF0000u);
        s_v[r][d + 2 * j] = __uint_as_float(vw[j] << 16);
        s_v[r][d + 2 * j + 1] = __uint_as_float(vw[j] & 0xFFFF0000u);
      }
    } else {
      s_k[r][d] = __int_as_float(t.k[i].x), s_k[r][d + 1] = __int_as_float(t.k[i].y);
      s_k[r][d + 2] = __int_as_float(t.k[i].z), s_k[r][d + 3] = __int_as_float(t.k[i].w);
      s_v[r][d] = __int_as_float(t.v[i].x), s_v[r][d + 1] = __int_as_float(t.v[i].y);
      s_v[r][d + 2] = __int_as_float(t.v[i].z), s_v[r][d + 3] = __int_as_float(t.v[i].w);
    }
  }
}

template <int HD, int G, bool BF16>
__global__ void __launch_bounds__(kThreads) k_attn_decode(AttnDecodeArgs a) {
  // score work split: thread -> (row r, head h, d-part) with NP parts of HD/NP
  constexpr int NP = kThreads / (TJ * G) > 0 ? kThreads / (TJ * G) : 1;
  constexpr int DPP = HD / NP;  // dims per part
  constexpr int SC_PASSES = (TJ * G * NP + kThreads - 1) / kThreads;
  constexpr bool QREG = DPP <= 32;  // query slice in registers, else read from LDS
  __shared__ float s_qf[G][HD];
  __shared__ double s_qd[QREG ? 1 : G][HD];
  __shared__ float s_knew[HD];
  __shared__ float s_vnew[HD];
  __shared__ float s_k[TJ][HD + 1];
  __shared__ float s_v[TJ][HD + 1];
  __shared__ double s_part[NP][G][TJ];
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

  // first cache tile in flight before anything else (rows < p only; row p
  // comes from this step's projections)
  TileRegs<HD, BF16> tr;
  const int cache_end = min(j1, p);  // rows [j0, cache_end) are read from the cache
  if (j0 < cache_end) tile_load<HD, BF16>(tr, a.kv, kbase, vbase, j0, min(TJ, cache_end - j0));

  // stage raw q (G heads), and the new k / v of head g
  for (int e = threadIdx.x; e < G * HD; e += kThreads) s_qf[e / HD][e % HD] = qkv[(int64_t)(g * G) * HD + e];
  const bool has_new = j0 < j1 && j1 == ctx;  // this split holds position p
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

  // this thread's query slice, in f64 (registers when it is small)
  int sc_r[SC_PASSES], sc_h[SC_PASSES], sc_pt[SC_PASSES];
  double qreg[QREG ? SC_PASSES : 1][QREG ? DPP : 1];
#pragma unroll
  for (int ps = 0; ps < SC_PASSES; ++ps) {
    const int e = threadIdx.x + ps * kThreads;
    sc_r[ps] = e % TJ;
    sc_h[ps] = (e / TJ) % G;
    sc_pt[ps] = e / (TJ * G);
    if (QREG) {
#pragma unroll
      for (int i = 0; i < (QREG ? DPP : 1); ++i)
        qreg[QREG ? ps : 0][i] = (e < TJ * G * NP) ? (double)s_qf[sc_h[ps]][sc_pt[ps] * DPP + i] : 0.0;
    }
  }
  if (!QREG)
    for (int e = threadIdx.x; e < G * HD; e += kThreads) s_qd[QREG ? 0 : e / HD][e % HD] = (double)s_qf[e / HD][e % HD];

  // online softmax in f64: wave h (< G) owns head h's (m, l); outputs are
  // spread over threads as e = tid + 256*i -> (head e / HD, dim e % HD)
  constexpr int OUT_PER_T = (G * HD + kThreads - 1) / kThreads;
  double o[OUT_PER_T];
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) o[i] = 0.0;
  constexpr int HPW = (G + kWaves - 1) / kWaves;  // heads per wavefront
  double m_run[HPW], l_run[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) m_run[i] = -INFINITY, l_run[i] = 0.0;
  const double scale = a.scale;

  for (int t0 = j0; t0 < j1; t0 += TJ) {
    const int nrow = min(TJ, j1 - t0);
    __syncthreads();  // previous tile fully consumed
    if (t0 < cache_end) tile_store<HD, BF16>(tr, s_k, s_v);
    if (t0 + nrow > p) {  // the tile holds row p: take it from this step's values
      __syncthreads();    // (after the tile store, which zero-fills that row)
      const int r = p - t0;
      for (int d = threadIdx.x; d < HD; d += kThreads) {
        s_k[r][d] = s_knew[d];
        s_v[r][d] = s_vnew[d];
      }
    }
    __syncthreads();
    const int tn = t0 + TJ;  // prefetch the next tile while this one is used
    if (tn < cache_end) tile_load<HD, BF16>(tr, a.kv, kbase, vbase, tn, min(TJ, cache_end - tn));
    // partial scores over each thread's d slice (f64)
#pragma unroll
    for (int ps = 0; ps < SC_PASSES; ++ps) {
      const int e = threadIdx.x + ps * kThreads;
      if (e < TJ * G * NP) {
        double acc = 0.0;
        const float* kr = &s_k[sc_r[ps]][sc_pt[ps] * DPP];
        if (QREG) {
#pragma unroll
          for (int i = 0; i < (QREG ? DPP : 1); ++i) acc += qreg[QREG ? ps : 0][i] * (double)kr[i];
        } else {
          const double* qd = &s_qd[QREG ? 0 : sc_h[ps]][sc_pt[ps] * DPP];
#pragma unroll 16
          for (int i = 0; i < DPP; ++i) acc += qd[i] * (double)kr[i];
        }
        s_part[sc_pt[ps]][sc_h[ps]][sc_r[ps]] = acc;
      }
    }
    __syncthreads();
    // per-head scores, max / exp / sum: wave handles heads wave + 4i, half-waves
    // share one head's 32 rows
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = wave + i * kWaves;
      if (h < G) {
        const int r = lane % TJ;
        double s = 0.0;
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) s += s_part[pt][h][r];
        s = (r < nrow) ? s * scale : -INFINITY;
        const double mt = wave_max_d<TJ>(s);
        const double m_new = fmax(m_run[i], mt);
        const double pr = (s == -INFINITY) ? 0.0 : exp(s - m_new);
        const double lt = wave_sum_d<TJ>(pr);
        const double alpha = (m_run[i] == -INFINITY) ? 0.0 : exp(m_run[i] - m_new);
        l_run[i] = l_run[i] * alpha + lt;
        m_run[i] = m_new;
        if (lane < TJ) s_p[h][r] = pr;
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
  }

  // write this split's partial: [row][g][split][h][0..HD-1] = o, [HD] = m, [HD+1] = l
  const int64_t pstride = (int64_t)G * (HD + 2);
  double* part = a.part + (((int64_t)row * nkv + g) * a.nsplit_max + split) * pstride;
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) {
    const int e = threadIdx.x + i * kThreads;
    if (e < G * HD) st_coherent(part + (e / HD) * (HD + 2) + (e % HD), o[i]);
  }
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + i * kWaves;
    if (h < G && lane == 0) {
      st_coherent(part + h * (HD + 2) + HD, m_run[i]);
      st_coherent(part + h * (HD + 2) + HD + 1, l_run[i]);
    }
  }
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = a.counter + (int64_t)row * nkv + g;
    const unsigned prev = arrive(cnt);
    s_last = prev == (unsigned)(nsplit - 1);
    if (s_last) st_coherent(cnt, 0u);  // every split of this launch has arrived
  }
  __syncthreads();
  if (!s_last) return;
  // merge the nsplit partials of the G heads (f64), round once to f32.  All
  // loads of a phase are issued together (each one crosses the device-wide
  // fence, so a load-per-iteration loop would pay that latency nsplit times).
  const double* pb = a.part + (((int64_t)row * nkv + g) * a.nsplit_max) * pstride;
  __shared__ double s_w[G][kMaxSplit];
  __shared__ double s_l[G][kMaxSplit];
  __shared__ double s_L[G];
  for (int e = threadIdx.x; e < G * nsplit; e += kThreads) {
    const int h = e / nsplit, sidx = e % nsplit;
    s_w[h][sidx] = ld_coherent(pb + sidx * pstride + h * (HD + 2) + HD);
    s_l[h][sidx] = ld_coherent(pb + sidx * pstride + h * (HD + 2) + HD + 1);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    double M = -INFINITY;
    for (int sidx = 0; sidx < nsplit; ++sidx) M = fmax(M, s_w[h][sidx]);
    s_alpha[h] = M;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * nsplit; e += kThreads) {
    const int h = e / nsplit, sidx = e % nsplit;
    const double ms = s_w[h][sidx];
    s_w[h][sidx] = (ms == -INFINITY) ? 0.0 : exp(ms - s_alpha[h]);
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    double L = 0.0;
    for (int sidx = 0; sidx < nsplit; ++sidx) L += s_w[h][sidx] * s_l[h][sidx];
    s_L[h] = L;
  }
  double O[OUT_PER_T];
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) {
    const int e = threadIdx.x + i * kThreads;
    O[i] = 0.0;
    if (e < G * HD) {
      const int h = e / HD, d = e % HD;
      int sidx = 0;
      for (; sidx + 16 <= nsplit; sidx += 16) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = ld_coherent(pb + (sidx + u) * pstride + h * (HD + 2) + d);
#pragma unroll
        for (int u = 0; u < 16; ++u) O[i] += s_w[h][sidx + u] * v[u];
      }
      for (; sidx < nsplit; ++sidx) O[i] += s_w[h][sidx] * ld_coherent(pb + sidx * pstride + h * (HD + 2) + d);
    }
  }
  __syncthreads();  // s_L ready
#pragma unroll
  for (int i = 0; i < OUT_PER_T; ++i) {
    const int e = threadIdx.x + i * kThreads;
    if (e < G * HD) {
      const int h = e / HD, d = e % HD;
      a.out[(int64_t)row * a.out_stride + (int64_t)(g * G + h) * HD + d] = (float)(O[i] / s_L[h]);
    }
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
