// Prefill attention path for gfx950.
//
// k_qk_rope_append: per (token, head) -- per-head RMSNorm of q and k, NeoX
// RoPE at the token's absolute position, q written (f32) for the MFMA
// kernel, post-RoPE k and raw v appended to the KV cache (Fucina course, "A
// transformer from scratch", sections 12.3.2, 12.3.4, 12.4; minfer "Qwen3
// Support Plan", section 2.2).
//
// k_attn_prefill: causal grouped-query flash attention (section 12.3.5) on
// f64 MFMA (v_mfma_f64_16x16x4_f64) with an f64 online softmax; the output
// is rounded to f32 once.  The attention output is quantised to Q8_0 right
// after, so it must round exactly like a reference that reduces in f64: an
// f32-accurate attention flips a share of those codes and moves the logits
// by several 1e-3 of their range.  (On gfx950 the f64 matrix and vector
// rates are equal, so MFMA is used for its register-fed operands.)
//
// A wavefront owns 16 queries of one head and computes S^T = K Q^T: lane
// (g = lane/16, q = lane%16) then holds the scores of query q for keys
// 4*item + g, so the row max / sum need two lane exchanges and each item is
// already the B operand of one O^T += V^T P^T step (keys 4*item .. +3).  The
// workgroup's waves share one KV head, so a K/V tile staged in LDS serves all
// of its query heads.
//
// Short prompts leave most CUs idle with one 32-query block per workgroup,
// and the causal triangle makes the last blocks the longest; there (KS = 2)
// the two waves of a query head take the two halves of every staged tile and
// merge their (max, sum, output) through LDS at the end, which doubles the
// workgroups and halves the longest one.  Blocks are issued longest first.
//
// Few query blocks over a long cache (a short verify pass after a long
// prompt, the last blocks of a causal prompt) leave the launch bound by its
// longest workgroup; there the keys of a block are also cut across
// workgroups into runs of whole 64-key tiles, each run leaves its
// unnormalised (O, max, sum) per (token, head), and k_attn_merge combines the
// runs in order, in f64.
#include "kernels.h"
#include "qdevice.h"

#include <algorithm>

using namespace q8;

namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

// Q8_0 round trip of one head row in LDS, by all 64 threads of the
// workgroup: per 32-block the activation encoder (scale max|x|/127, codes
// rounded to nearest even), the codes and f16 scale bits to `codes` /
// `scales` when given, the dequantised values (exact in f32) back into x.
// Each thread touches only its own four values.
template <int HD>
QDEV void q8_row(float* x, int8_t* codes, uint16_t* scales) {
  const int t = threadIdx.x;
  const bool live = t < HD / 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = x[4 * t + i];
  }
  float d;
  const int packed = quant4_group8(v, &d);  // groups of 8 lanes: one block each
  if (live) {
    const float df = f16_round(d);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * t + i] = (float)(int8_t)((packed >> (8 * i)) & 0xFF) * df;
    if (codes) *reinterpret_cast<int*>(codes + 4 * t) = packed;
    if (scales && (t & 7) == 0) scales[t / 8] = f32_to_f16_bits(d);
  }
}

template <int HD, int KVT>
__global__ void __launch_bounds__(64) k_qk_rope_append(QkRopeArgs a) {
  __shared__ float x[HD];
  __shared__ float xv[HD];
  const int t = blockIdx.x, h = blockIdx.y;
  const int pos = a.pos0 + t;
  const float* row = a.qkv + (int64_t)t * a.qkv_stride;
  const double* cs = a.rope_cos + (int64_t)pos * (HD / 2);
  const double* sn = a.rope_sin + (int64_t)pos * (HD / 2);
  if (h < a.nh) {
    for (int d = threadIdx.x; d < HD; d += 64) x[d] = row[(int64_t)h * HD + d];
    __syncthreads();
    norm_rope_wave<HD>(x, a.q_norm, a.eps, cs, sn);
    __syncthreads();
    if (KVT == KV_Q8_0 && a.quant_q) {  // the integer score path of a single-token step
      q8_row<HD>(x, nullptr, nullptr);
      __syncthreads();
    }
    for (int d = threadIdx.x; d < HD; d += 64) a.q32[((int64_t)t * a.nh + h) * HD + d] = x[d];
  } else {
    const int g = h - a.nh;
    for (int d = threadIdx.x; d < HD; d += 64) x[d] = row[(int64_t)(a.nh + g) * HD + d];
    __syncthreads();
    norm_rope_wave<HD>(x, a.k_norm, a.eps, cs, sn);
    __syncthreads();
    const int64_t head_elems = (int64_t)a.cap * HD;
    const int64_t kb = a.kbase + g * head_elems + (int64_t)pos * HD;
    const int64_t vb = kb + (int64_t)a.nkv * head_elems;
    if (KVT == KV_Q8_0) {
      for (int d = threadIdx.x; d < HD; d += 64) xv[d] = row[(int64_t)(a.nh + a.nkv + g) * HD + d];
      __syncthreads();
      int8_t* codes = reinterpret_cast<int8_t*>(a.kv);
      q8_row<HD>(x, codes + kb, a.kvs + kb / 32);
      q8_row<HD>(xv, codes + vb, a.kvs + vb / 32);
      return;
    }
    for (int d = threadIdx.x; d < HD; d += 64) {
      const float v = row[(int64_t)(a.nh + a.nkv + g) * HD + d];
      if (KVT == KV_BF16) {
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

// One K/V tile (KT rows of HD) in registers: 16-byte loads, the same count
// for every tile (rows past `kend` re-read row kend - 1: finite values whose
// scores are masked and whose probabilities are 0).  KV_Q8_0: a load is 16
// codes of one row (half a block) plus that block's f16 scale; the codes are
// widened exactly (code times scale) when the tile is staged.
template <int HD, int KVT>
struct KVTile {
  static constexpr int ESZ = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
  static constexpr int PER = 16 / ESZ;  // elements per 16-byte load
  static constexpr int LOADS = KT * HD / PER / 256;
  static_assert(LOADS >= 1 && LOADS * PER * 256 == KT * HD, "tile map");
  v4i k[LOADS], v[LOADS];
  uint16_t ks[KVT == KV_Q8_0 ? LOADS : 1], vs[KVT == KV_Q8_0 ? LOADS : 1];
  QDEV void load(const void* kv, const uint16_t* kvs, int64_t kb0, int64_t vb0, int kbase, int kend) {
    const uint8_t* base = static_cast<const uint8_t*>(kv);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (threadIdx.x + i * 256) * PER;
      const int key = min(kbase + e / HD, kend - 1);
      const int64_t off = (int64_t)key * HD + (e % HD);
      k[i] = *reinterpret_cast<const v4i*>(base + (kb0 + off) * ESZ);
      v[i] = *reinterpret_cast<const v4i*>(base + (vb0 + off) * ESZ);
      if (KVT == KV_Q8_0) {
        ks[i] = kvs[(kb0 + off) / 32];
        vs[i] = kvs[(vb0 + off) / 32];
      }
    }
  }
  QDEV static void widen_q8(v4i w, float sc, float* dst) {  // 16 codes -> 16 floats
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = w[j];
      float4 f;
      f.x = (float)(int8_t)(c & 0xFF) * sc;
      f.y = (float)(int8_t)((c >> 8) & 0xFF) * sc;
      f.z = (float)(int8_t)((c >> 16) & 0xFF) * sc;
      f.w = (float)(int8_t)((c >> 24) & 0xFF) * sc;
      *reinterpret_cast<float4*>(dst + 4 * j) = f;
    }
  }
  QDEV void store(float* sK, int krow, float* sV, int vrow) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (threadIdx.x + i * 256) * PER;
      const int r = e / HD, d = e % HD;
      if (KVT == KV_Q8_0) {
        widen_q8(k[i], f16_bits_to_f32(ks[i]), sK + r * krow + d);
        widen_q8(v[i], f16_bits_to_f32(vs[i]), sV + r * vrow + d);
      } else if (KVT == KV_BF16) {
        float4 a0, a1, b0, b1;
        a0.x = __uint_as_float((uint32_t)k[i][0] << 16), a0.y = __uint_as_float((uint32_t)k[i][0] & 0xFFFF0000u);
        a0.z = __uint_as_float((uint32_t)k[i][1] << 16), a0.w = __uint_as_float((uint32_t)k[i][1] & 0xFFFF0000u);
        a1.x = __uint_as_float((uint32_t)k[i][2] << 16), a1.y = __uint_as_float((uint32_t)k[i][2] & 0xFFFF0000u);
        a1.z = __uint_as_float((uint32_t)k[i][3] << 16), a1.w = __uint_as_float((uint32_t)k[i][3] & 0xFFFF0000u);
        b0.x = __uint_as_float((uint32_t)v[i][0] << 16), b0.y = __uint_as_float((uint32_t)v[i][0] & 0xFFFF0000u);
        b0.z = __uint_as_float((uint32_t)v[i][1] << 16), b0.w = __uint_as_float((uint32_t)v[i][1] & 0xFFFF0000u);
        b1.x = __uint_as_float((uint32_t)v[i][2] << 16), b1.y = __uint_as_float((uint32_t)v[i][2] & 0xFFFF0000u);
        b1.z = __uint_as_float((uint32_t)v[i][3] << 16), b1.w = __uint_as_float((uint32_t)v[i][3] & 0xFFFF0000u);
        *reinterpret_cast<float4*>(sK + r * krow + d) = a0;
        *reinterpret_cast<float4*>(sK + r * krow + d + 4) = a1;
        *reinterpret_cast<float4*>(sV + r * vrow + d) = b0;
        *reinterpret_cast<float4*>(sV + r * vrow + d + 4) = b1;
      } else {
        *reinterpret_cast<v4i*>(sK + r * krow + d) = k[i];
        *reinterpret_cast<v4i*>(sV + r * vrow + d) = v[i];
      }
    }
  }
};

// An LDS pointer for the global-to-LDS loads.
QDEV __attribute__((address_space(3))) void* lds_ptr(float* p) {
  return (__attribute__((address_space(3))) void*)p;
}

// Two workgroups per CU (eight waves, two per SIMD): while one waits for a
// tile or runs its softmax, the other's MFMAs keep the SIMD busy.
template <int HD, int G, int KVT, int KS>
__global__ void __launch_bounds__(256, 2) k_attn_prefill(AttnPrefillArgs a) {
  constexpr int HW = G < 4 ? G : 4;  // query heads per workgroup
  static_assert(HW * KS <= 4, "waves");
  constexpr int TPW = 4 / (HW * KS);  // 16-token sub-tiles per workgroup
  constexpr int QT = 16 * TPW;        // tokens per workgroup
  constexpr int KTW = KT / KS;        // keys of each staged tile this wave scores
  // An f32 cache goes to LDS as it is, straight from memory (no staging
  // registers); other caches are widened in registers first.
  constexpr bool DMA = KVT == KV_F32;
  constexpr int KROW = HD + 4;   // f32 per K row in LDS (padded: the 16 x 4 lanes of
                                 // a K operand read hit 64 distinct banks)
  constexpr int VROW = HD + 16;  // f32 per V row in LDS (padded)
  constexpr int NST = HD / 4;        // k=4 steps over head_dim
  constexpr int NDT = HD / 16;       // 16-wide d tiles of the output
  // K and V tiles in one array (the merge of key halves reuses all of it)
  __shared__ __align__(16) float sKV[KT * KROW + KT * VROW];
  float* const sK = sKV;
  float* const sV = sKV + KT * KROW;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lq = lane % 16, lg = lane / 16;
  // one-dimensional grid, head groups fastest, then the runs of a query
  // block, then the blocks from the last (longest) to the first: workgroups
  // are dispatched in about decreasing length, whatever the head count
  const int ny = a.nkv * (G / HW);
  const int gy = blockIdx.x % ny;
  const int run = (blockIdx.x / ny) % a.nz;
  const int qrev = blockIdx.x / ny / a.nz;
  const int hb_per_g = G / HW;
  const int g = gy / hb_per_g, hb = gy % hb_per_g;
  const int h = g * G + hb * HW + (wave % HW);
  const int kpar = (wave / HW) % KS;  // which part of every tile this wave takes
  const int t0 = (a.nqb - 1 - qrev) * QT;
  const int tw0 = t0 + (wave / (HW * KS)) * 16;       // first token of this wavefront
  const int T = a.T;

  // this lane's query (clamped so padded lanes stay finite; never stored)
  const int tq = min(tw0 + lq, T - 1);
  const int qpos = a.pos0 + tq;
  // the query stays f32 in registers and is widened at each use (an f64
  // copy would cost NST more registers than two waves per SIMD leave)
  float qf[NST];
  const float* qrow = a.q32 + ((int64_t)tq * a.nh + h) * HD;
#pragma unroll
  for (int st = 0; st < NST; ++st) qf[st] = qrow[4 * st + lg];

  const int64_t head_elems = (int64_t)a.cap * HD;
  const int64_t kb0 = a.kbase + (int64_t)g * head_elems;
  const int64_t vb0 = kb0 + (int64_t)a.nkv * head_elems;
  const int kend = a.pos0 + min(T, t0 + QT);  // keys [0, kend) matter for this block
  // this workgroup's run of key tiles: [k_lo, k_hi) (the whole range unsplit)
  const int ntq = (kend + KT - 1) / KT;
  const int ns = a.tps > 0 ? (ntq + a.tps - 1) / a.tps : 1;
  if (run >= ns) return;  // uniform per workgroup, before any barrier
  const int k_lo = a.tps > 0 ? run * a.tps * KT : 0;
  const int k_hi = a.tps > 0 ? min(kend, k_lo + a.tps * KT) : kend;

  v4d o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = v4d{0.0, 0.0, 0.0, 0.0};
  double m_run = -INFINITY, l_run = 0.0;

  // widened caches: the next tile's loads are issued right after the current
  // tile is staged, so they land while the current tile is used
  KVTile<HD, DMA ? KV_BF16 : KVT> tile;
  if (!DMA) tile.load(a.kv, a.kvs, kb0, vb0, k_lo, kend);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  for (int kbase = k_lo; kbase < k_hi; kbase += KT) {
    __syncthreads();
    if constexpr (DMA) {
      // rows [kbase, kbase + KT) of K and V (rows past kend re-read row
      // kend - 1: finite, masked, probability 0).  One load of a wave writes
      // 64 consecutive 16-byte chunks of LDS, one per lane, so each lane
      // fetches the chunk that belongs at its place in the padded rows (a
      // padding chunk fetches the row's first chunk, never read)
      const float* kvf = static_cast<const float*>(a.kv);
      auto fill = [&](float* dst, int64_t base, int rowf) {
        const int cpr = rowf / 4;      // chunks per padded row
        const int nld = KT * cpr / kWave;  // loads for the whole tile
        for (int j = wv; j < nld; j += 4) {
          const int L = j * kWave + lane;
          const int r = L / cpr, pc = L % cpr;
          const int64_t key = min(kbase + r, kend - 1);
          __builtin_amdgcn_global_load_lds(kvf + base + key * HD + (pc < HD / 4 ? 4 * pc : 0),
                                           lds_ptr(dst + j * kWave * 4), 16, 0, 0);
        }
      };
      static_assert(KT * (KROW / 4) % kWave == 0 && KT * (VROW / 4) % kWave == 0, "whole loads");
      fill(sK, kb0, KROW);
      fill(sV, vb0, VROW);
      __builtin_amdgcn_s_waitcnt(0);  // the loads have written LDS
    } else {
      tile.store(sK, KROW, sV, VROW);
      tile.load(a.kv, a.kvs, kb0, vb0, kbase + KT < k_hi ? kbase + KT : kbase, kend);
    }
    __syncthreads();

    // scores S^T for the sub-tiles of 16 keys of this wave's part; lane holds
    // keys 4*item + lg of each
    const int kw0 = kpar * KTW;  // first key of the part within the tile
    v4d s[KTW / 16];
#pragma unroll
    for (int st = 0; st < NST; ++st) asm volatile("" : "+v"(qf[st]));  // widened per tile, not kept in f64
#pragma unroll
    for (int kt = 0; kt < KTW / 16; ++kt) {
      s[kt] = v4d{0.0, 0.0, 0.0, 0.0};
      const float* kr = &sK[(kw0 + kt * 16 + lq) * KROW + lg];
#pragma unroll
      for (int st = 0; st < NST; ++st)
        s[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)kr[4 * st], (double)qf[st], s[kt], 0, 0, 0);
    }
    double rmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KTW / 16; ++kt)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int key = kbase + kw0 + kt * 16 + 4 * it + lg;
        const double v = (key <= qpos) ? s[kt][it] * a.scale : -INFINITY;
        s[kt][it] = v;
        rmax = fmax(rmax, v);
      }
    rmax = fmax(rmax, __shfl_xor(rmax, 16));
    rmax = fmax(rmax, __shfl_xor(rmax, 32));
    const double m_new = fmax(m_run, rmax);
    const double alpha = (m_run == -INFINITY) ? 0.0 : exp(m_run - m_new);
    double rsum = 0.0;
#pragma unroll
    for (int kt = 0; kt < KTW / 16; ++kt)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const double p = (s[kt][it] == -INFINITY) ? 0.0 : exp(s[kt][it] - m_new);
        s[kt][it] = p;
        rsum += p;
      }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T: step (kt, it) covers keys kt*16 + 4*it + {0..3}; lane lg
    // supplies key kt*16 + 4*it + lg, which is exactly its score item it
#pragma unroll
    for (int kt = 0; kt < KTW / 16; ++kt) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float* vr = &sV[(kw0 + kt * 16 + 4 * it + lg) * VROW + lq];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)vr[16 * dt], s[kt][it], o[dt], 0, 0, 0);
      }
    }
  }

  // a query row whose keys all lie past its position (possible in a later
  // run) keeps m = -inf, l = 0, O = 0: it contributes nothing below
  const bool owner = KS == 1 || kpar == 0;  // the wave that holds the merged state
  if constexpr (KS == 2) {
    // merge the two halves: the second-half wave of each (head, token tile)
    // leaves (m, l, O) in LDS, the first-half wave rescales and adds
    static_assert(HW * TPW * 64 * (NDT * 4 + 2) * 8 <= (int)sizeof(sKV), "merge space");
    double* mo = reinterpret_cast<double*>(sKV);  // [HW * TPW slots][64 lanes][NDT * 4 + 2]
    const int slot = (wave % HW) + HW * (wave / (HW * KS));
    double* my = mo + ((int64_t)slot * 64 + lane) * (NDT * 4 + 2);
    __syncthreads();  // every wave is done with the tiles
    if (kpar == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int it = 0; it < 4; ++it) my[4 * dt + it] = o[dt][it];
      my[NDT * 4] = m_run;
      my[NDT * 4 + 1] = l_run;
    }
    __syncthreads();
    if (owner) {
      const double m1 = my[NDT * 4], l1 = my[NDT * 4 + 1];
      const double mx = fmax(m_run, m1);
      const double a0 = (m_run == -INFINITY) ? 0.0 : exp(m_run - mx);
      const double a1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - mx);
      l_run = l_run * a0 + l1 * a1;
      m_run = mx;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int it = 0; it < 4; ++it) o[dt][it] = o[dt][it] * a0 + my[4 * dt + it] * a1;
    }
  }

  // O^T layout: lane (lg, lq) holds d = 16*dt + 4*item + lg of query lq
  const int tout = tw0 + lq;
  if (ns == 1) {
    if (owner && tout < T) {
      float* orow = a.out + (int64_t)tout * a.nh * HD + (int64_t)h * HD;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int it = 0; it < 4; ++it) orow[16 * dt + 4 * it + lg] = (float)(o[dt][it] / l_run);
    }
    return;
  }

  // key-split block: this run's unnormalised (O, m, l), merged by k_attn_merge
  constexpr int PS = HD + 2;
  if (owner && tout < T) {
    double* pr = a.part + ((int64_t)run * T * a.nh + (int64_t)tout * a.nh + h) * PS;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int it = 0; it < 4; ++it) pr[16 * dt + 4 * it + lg] = o[dt][it];
    if (lg == 0) pr[HD] = m_run, pr[HD + 1] = l_run;
  }
}

// Merge of the key-split runs: one workgroup per (token, head), one thread
// per output dimension.  The runs combine in run order (f64): with M the
// largest run maximum, O = sum_r exp(m_r - M) O_r and l = sum_r exp(m_r - M)
// l_r, and the output O / l is rounded once to f32.  Tokens of blocks that
// were not split were written by the attention kernel itself.
template <int HD>
__global__ void __launch_bounds__(HD) k_attn_merge(AttnPrefillArgs a, int QT) {
  constexpr int PS = HD + 2;
  const int t = blockIdx.x / a.nh, h = blockIdx.x % a.nh, d = threadIdx.x;
  const int kend = a.pos0 + min(a.T, (t / QT + 1) * QT);
  const int ns = ((kend + KT - 1) / KT + a.tps - 1) / a.tps;
  if (ns <= 1) return;
  const int64_t rstride = (int64_t)a.T * a.nh * PS;
  const double* pb = a.part + ((int64_t)t * a.nh + h) * PS;
  double M = -INFINITY;
  for (int r = 0; r < ns; ++r) M = fmax(M, pb[r * rstride + HD]);
  double O = 0.0, L = 0.0;
  for (int r = 0; r < ns; ++r) {
    const double* pr = pb + r * rstride;
    const double mr = pr[HD];
    const double w = (mr == -INFINITY) ? 0.0 : exp(mr - M);
    L += w * pr[HD + 1];
    O += w * pr[d];
  }
  a.out[(int64_t)t * a.nh * HD + (int64_t)h * HD + d] = (float)(O / L);
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Tiles per run of the key split.  Only launches whose unsplit grid leaves
// at least half of the CUs idle are split (measured on a 512-token prompt,
// 256 workgroups: splitting its long blocks made the launch slower).  One
// workgroup fills a CU, so a launch takes about max(longest run, total tiles
// / CUs) tile times; a split adds the merge (counted as one tile time).  The
// largest power of two that minimises that estimate, within the scratch for
// the runs' partials; 0 when not splitting is as good.
template <int HD, int QT>
int pick_tps(const AttnPrefillArgs& a, int ny) {
  if (!a.part) return 0;
  const int nqb = (a.T + QT - 1) / QT;
  if ((int64_t)nqb * ny * 2 > cu_count()) return 0;
  const int ntmax = (a.pos0 + a.T + KT - 1) / KT;
  int64_t total = 0;
  for (int q = 0; q < nqb; ++q) total += (a.pos0 + std::min(a.T, (q + 1) * QT) + KT - 1) / KT;
  total *= ny;
  const int cus = cu_count();
  auto est = [&](int64_t longest) { return std::max<int64_t>(longest, (total + cus - 1) / cus); };
  const int64_t plane = (int64_t)a.T * a.nh * (HD + 2) * 8;  // bytes of one run's partials
  int best = 0;
  int64_t best_t = est(ntmax);
  for (int tps = 1; tps < ntmax; tps *= 2) {
    const int64_t ns_max = (ntmax + tps - 1) / tps;
    if (ns_max * plane > (int64_t)a.part_bytes) continue;
    const int64_t t = est(tps) + 1;
    if (t <= best_t) best = tps, best_t = t;
  }
  return best;
}

template <int HD, int G, int KS>
hipError_t launch_attn_ks(const AttnPrefillArgs& a0, int kvt, hipStream_t s) {
  constexpr int HW = G < 4 ? G : 4;
  constexpr int QT = 16 * (4 / (HW * KS));
  const int ny = a0.nkv * (G / HW);
  AttnPrefillArgs a = a0;
  a.tps = pick_tps<HD, QT>(a0, ny);
  const int ntmax = (a.pos0 + a.T + KT - 1) / KT;
  a.nz = a.tps > 0 ? (ntmax + a.tps - 1) / a.tps : 1;
  a.nqb = (a.T + QT - 1) / QT;
  const int64_t nwg = (int64_t)a.nqb * a.nz * ny;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  switch (kvt) {
    case KV_F32: hipLaunchKernelGGL((k_attn_prefill<HD, G, KV_F32, KS>), grid, dim3(256), 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL((k_attn_prefill<HD, G, KV_BF16, KS>), grid, dim3(256), 0, s, a); break;
    case KV_Q8_0: hipLaunchKernelGGL((k_attn_prefill<HD, G, KV_Q8_0, KS>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.tps > 0) hipLaunchKernelGGL((k_attn_merge<HD>), dim3((unsigned)(a.T * a.nh)), dim3(HD), 0, s, a, QT);
  return hipGetLastError();
}

// Two key halves per head when one 32-query block per workgroup would give
// fewer than two workgroups per CU.
template <int HD, int G>
hipError_t launch_attn(const AttnPrefillArgs& a, int kvt, hipStream_t s) {
  constexpr int HW = G < 4 ? G : 4;
  if constexpr (HW <= 2) {
    if ((int64_t)((a.T + 31) / 32) * a.nkv * (G / HW) < 512) return launch_attn_ks<HD, G, 2>(a, kvt, s);
  }
  return launch_attn_ks<HD, G, 1>(a, kvt, s);
}

}  // namespace

namespace q8k {

template <int HD>
hipError_t launch_qk(const QkRopeArgs& a, dim3 grid, int kvt, hipStream_t s) {
  switch (kvt) {
    case KV_F32: hipLaunchKernelGGL((k_qk_rope_append<HD, KV_F32>), grid, dim3(64), 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL((k_qk_rope_append<HD, KV_BF16>), grid, dim3(64), 0, s, a); break;
    case KV_Q8_0: hipLaunchKernelGGL((k_qk_rope_append<HD, KV_Q8_0>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t qk_rope_append(const QkRopeArgs& a, int T, int hd, int kvt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(T, a.nh + a.nkv);
  if (hd == 64) return launch_qk<64>(a, grid, kvt, s);
  if (hd == 128) return launch_qk<128>(a, grid, kvt, s);
  return hipErrorInvalidValue;
}

bool attn_prefill_supported(int hd, int group) {
  return (hd == 64 || hd == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t attn_prefill(const AttnPrefillArgs& a, int hd, int group, int kvt, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
#define Q8_AP(HD_, G_) \
  if (hd == HD_ && group == G_) return launch_attn<HD_, G_>(a, kvt, s);
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
