// Prefill attention path for gfx950.
//
// k_qk_rope_append: per (token, head) -- per-head RMSNorm of q and k, NeoX
// RoPE at the token's absolute position, q written as f16 for the MFMA
// kernel, post-RoPE k and raw v appended to the KV cache (Fucina course, "A
// transformer from scratch", sections 12.3.2, 12.3.4, 12.4; minfer "Qwen3
// Support Plan", section 2.2).
//
// k_attn_prefill: causal grouped-query flash attention (section 12.3.5) on
// f16 MFMA (v_mfma_f32_32x32x16_f16) with an f32 online softmax.  A
// wavefront owns 32 queries of one head and computes S^T = K Q^T, so its
// accumulator holds the scores of ONE query per lane (lane % 32) over 16 keys;
// the row max / sum need a single exchange with lane ^ 32, and the
// probabilities are already in the B-operand layout of O^T = V^T P^T (the
// V tile is staged transposed in LDS with the matching key order).  The
// workgroup's waves share one KV head, so a K/V tile staged in LDS serves
// all of its query heads.
#include "kernels.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <bool BF16>
QDEV float ld_kv(const void* base, int64_t idx) {
  if (BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

template <int HD, bool BF16>
__global__ void __launch_bounds__(64) k_qk_rope_append(QkRopeArgs a) {
  __shared__ float x[HD];
  const int t = blockIdx.x, h = blockIdx.y;
  const int pos = a.pos0 + t;
  const float* row = a.qkv + (int64_t)t * a.qkv_stride;
  const float* cs = a.rope_cos + (int64_t)pos * (HD / 2);
  const float* sn = a.rope_sin + (int64_t)pos * (HD / 2);
  if (h < a.nh) {
    for (int d = threadIdx.x; d < HD; d += 64) x[d] = row[(int64_t)h * HD + d];
    __syncthreads();
    norm_rope_wave<HD>(x, a.q_norm, a.eps, cs, sn, 1.0f);
    __syncthreads();
    for (int d = threadIdx.x; d < HD; d += 64) a.q16[((int64_t)t * a.nh + h) * HD + d] = (_Float16)x[d];
  } else {
    const int g = h - a.nh;
    for (int d = threadIdx.x; d < HD; d += 64) x[d] = row[(int64_t)(a.nh + g) * HD + d];
    __syncthreads();
    norm_rope_wave<HD>(x, a.k_norm, a.eps, cs, sn, 1.0f);
    __syncthreads();
    const int64_t head_elems = (int64_t)a.cap * HD;
    const int64_t kb = a.kbase + g * head_elems + (int64_t)pos * HD;
    const int64_t vb = kb + (int64_t)a.nkv * head_elems;
    for (int d = threadIdx.x; d < HD; d += 64) {
      const float v = row[(int64_t)(a.nh + a.nkv + g) * HD + d];
      if (BF16) {
        reinterpret_cast<uint16_t*>(a.kv)[kb + d] = f32_to_bf16_bits(x[d]);
        reinterpret_cast<uint16_t*>(a.kv)[vb + d] = f32_to_bf16_bits(v);
      } else {
        reinterpret_cast<float*>(a.kv)[kb + d] = x[d];
        reinterpret_cast<float*>(a.kv)[vb + d] = v;
      }
    }
  }
}

constexpr int KT = 64;  // keys per LDS tile

template <int HD, int G, bool BF16>
__global__ void __launch_bounds__(256) k_attn_prefill(AttnPrefillArgs a) {
  constexpr int HW = G < 4 ? G : 4;  // query heads per workgroup
  constexpr int TPW = 4 / HW;        // 32-token sub-tiles per workgroup
  constexpr int QT = 32 * TPW;       // tokens per workgroup
  constexpr int KROW = HD + 8;       // halves per K row in LDS
  constexpr int VROW = KT + 8;       // halves per transposed V row
  constexpr int NDT = HD / 32;       // 32-wide d tiles
  constexpr int NST = HD / 16;       // K=16 steps over head_dim
  __shared__ __align__(16) _Float16 sK[KT * KROW];
  __shared__ __align__(16) _Float16 sVt[HD * VROW];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lq = lane % 32, lg = lane / 32;
  const int hb_per_g = G / HW;
  const int g = blockIdx.y / hb_per_g, hb = blockIdx.y % hb_per_g;
  const int h = g * G + hb * HW + (wave % HW);
  const int t0 = blockIdx.x * QT;
  const int tw0 = t0 + (wave / HW) * 32;  // first token of this wavefront
  const int T = a.T;

  // this lane's query (clamped so padded lanes stay finite; never stored)
  const int tq = min(tw0 + lq, T - 1);
  const int qpos = a.pos0 + tq;
  v8h qf[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st)
    qf[st] = *reinterpret_cast<const v8h*>(a.q16 + ((int64_t)tq * a.nh + h) * HD + st * 16 + lg * 8);

  const int64_t head_elems = (int64_t)a.cap * HD;
  const int64_t kb0 = a.kbase + (int64_t)g * head_elems;
  const int64_t vb0 = kb0 + (int64_t)a.nkv * head_elems;
  const int kend = a.pos0 + min(T, t0 + QT);  // keys [0, kend) matter for this workgroup

  v16f o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kbase = 0; kbase < kend; kbase += KT) {
    __syncthreads();
    for (int e = tid; e < KT * HD; e += 256) {
      const int kr = e / HD, d = e % HD;
      const int key = kbase + kr;
      float kval = 0.f, vval = 0.f;
      if (key < kend) {
        kval = ld_kv<BF16>(a.kv, kb0 + (int64_t)key * HD + d);
        vval = ld_kv<BF16>(a.kv, vb0 + (int64_t)key * HD + d);
      }
      sK[kr * KROW + d] = (_Float16)kval;
      sVt[d * VROW + kr] = (_Float16)vval;
    }
    __syncthreads();

    // S^T tiles: keys kt*32 + (8*(j/4) + 4*lg + j%4), query lq
    v16f s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kt][j] = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const v8h kf = *reinterpret_cast<const v8h*>(&sK[(kt * 32 + lq) * KROW + st * 16 + lg * 8]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[st], s[kt], 0, 0, 0);
      }
    }
    float rmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kbase + kt * 32 + 8 * (j / 4) + 4 * lg + (j % 4);
        const float v = (key <= qpos) ? s[kt][j] * a.scale : -INFINITY;
        s[kt][j] = v;
        rmax = fmaxf(rmax, v);
      }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float m_new = fmaxf(m_run, rmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    float rsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = (s[kt][j] == -INFINITY) ? 0.f : expf(s[kt][j] - m_new);
        s[kt][j] = p;
        rsum += p;
      }
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;

    // O^T += V^T P^T; half hf of key tile kt covers keys kt*32 + 16*hf + {4lg..4lg+3, 8+4lg..8+4lg+3}
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        v8h pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (_Float16)s[kt][8 * hf + i];
        const int kofs = kt * 32 + 16 * hf + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const _Float16* vr = &sVt[(dt * 32 + lq) * VROW + kofs];
          const v4h lo = *reinterpret_cast<const v4h*>(vr);
          const v4h hi = *reinterpret_cast<const v4h*>(vr + 8);
          const v8h va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[dt], 0, 0, 0);
        }
      }
    }
  }

  const int tout = tw0 + lq;
  if (tout < T) {
    const float inv = 1.0f / l_run;
    float* orow = a.out + (int64_t)tout * a.nh * HD + (int64_t)h * HD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) orow[dt * 32 + 8 * (j / 4) + 4 * lg + (j % 4)] = o[dt][j] * inv;
  }
}

template <int HD, int G>
hipError_t launch_attn(const AttnPrefillArgs& a, bool bf16, hipStream_t s) {
  constexpr int HW = G < 4 ? G : 4;
  constexpr int QT = 32 * (4 / HW);
  const dim3 grid((a.T + QT - 1) / QT, a.nkv * (G / HW));
  if (bf16)
    hipLaunchKernelGGL((k_attn_prefill<HD, G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_prefill<HD, G, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

namespace q8k {

hipError_t qk_rope_append(const QkRopeArgs& a, int T, int hd, bool kv_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(T, a.nh + a.nkv);
  if (hd == 64) {
    if (kv_bf16) hipLaunchKernelGGL((k_qk_rope_append<64, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((k_qk_rope_append<64, false>), grid, dim3(64), 0, s, a);
  } else if (hd == 128) {
    if (kv_bf16) hipLaunchKernelGGL((k_qk_rope_append<128, true>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((k_qk_rope_append<128, false>), grid, dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool attn_prefill_supported(int hd, int group) {
  return (hd == 64 || hd == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t attn_prefill(const AttnPrefillArgs& a, int hd, int group, bool kv_bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
#define Q8_AP(HD_, G_) \
  if (hd == HD_ && group == G_) return launch_attn<HD_, G_>(a, kv_bf16, s);
  Q8_AP(64, 1)
  Q8_AP(64, 2)
  Q8_AP(64, 4)
  Q8_AP(64, 8)
  Q8_AP(128, 1)
  Q8_AP(128, 2)
  Q8_AP(128, 4)
  Q8_AP(128, 8)
#undef Q8_AP
  return hipErrorInvalidValue;
}

}  // namespace q8k
