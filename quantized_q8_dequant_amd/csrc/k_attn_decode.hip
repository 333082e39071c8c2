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

#include <type_traits>

using namespace q8;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// cache rows per staged tile: 16 KB of f32 K or V, 16 KB of bf16, 8 KB of
// Q8_0 codes
template <int KVT>
constexpr int kTileRows = KVT == KV_F32 ? 32 : 64;
constexpr int kMaxSplit = 64;    // bound of nsplit_max
constexpr int kScoreSlots = 4096;  // f64 scores a workgroup keeps: G heads x (4096 / G) rows
constexpr int kLdsRow = 4;       // padding of a staged row (keeps rows 16-byte aligned)
constexpr int kCombineRegs = 80; // f64 partial values a thread of the combine holds in flight

template <int G, int HD>
constexpr int direct_slots() { return G * HD; }

// One tile of K or V rows staged through registers: every thread issues all
// of its 16-byte loads for a tile at once; two tiles are in flight ahead of
// the one being used.
template <int HD, int KVT>
struct TileRegs {
  static constexpr int TJ = kTileRows<KVT>;
  static constexpr int PER_LOAD = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 8 : 16);  // elements per 16 bytes
  static constexpr int LOADS = TJ * HD / PER_LOAD / kThreads;                    // per thread
  static_assert(LOADS >= 1 && LOADS * PER_LOAD * kThreads == TJ * HD, "tile map");
  v4i x[LOADS];
  uint16_t sc[KVT == KV_Q8_0 ? LOADS : 1];  // Q8_0: the block scale of each 16-code load
};

// Every thread issues the same loads whatever the tile (rows past the end
// re-read the tile's last row and are never used), so the compiler can keep
// the older tile's loads in flight while waiting for the newer one.
template <int HD, int KVT>
QDEV void tile_load(TileRegs<HD, KVT>& t, const void* kv, const uint16_t* kvs, int64_t base, int row0, int nrow) {
  constexpr int PER = TileRegs<HD, KVT>::PER_LOAD;
  constexpr int ESZ = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);
#pragma unroll
  for (int i = 0; i < TileRegs<HD, KVT>::LOADS; ++i) {
    const int e = (threadIdx.x + i * kThreads) * PER;  // element index in the tile
    const int r = min(e / HD, nrow - 1);
    const int64_t off = (int64_t)(row0 + r) * HD + (e % HD);
    t.x[i] = *reinterpret_cast<const v4i*>(static_cast<const uint8_t*>(kv) + (base + off) * ESZ);
    if (KVT == KV_Q8_0) t.sc[i] = kvs[(base + off) / 32];
  }
}

template <int HD, int KVT>
QDEV void tile_store(const TileRegs<HD, KVT>& t, float (*s_t)[HD + kLdsRow]) {
  constexpr int PER = TileRegs<HD, KVT>::PER_LOAD;
#pragma unroll
  for (int i = 0; i < TileRegs<HD, KVT>::LOADS; ++i) {
    const int e = (threadIdx.x + i * kThreads) * PER;
    const int r = e / HD, d = e % HD;
    if (KVT == KV_Q8_0) {  // 16 codes widened exactly: code times the block scale
      const float sc = f16_bits_to_f32(t.sc[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t.x[i][j];
        float4 f;
        f.x = (float)(int8_t)(c & 0xFF) * sc;
        f.y = (float)(int8_t)((c >> 8) & 0xFF) * sc;
        f.z = (float)(int8_t)((c >> 16) & 0xFF) * sc;
        f.w = (float)(int8_t)((c >> 24) & 0xFF) * sc;
        *reinterpret_cast<float4*>(&s_t[r][d + 4 * j]) = f;
      }
    } else if (KVT == KV_BF16) {
      const uint32_t w[4] = {(uint32_t)t.x[i][0], (uint32_t)t.x[i][1], (uint32_t)t.x[i][2], (uint32_t)t.x[i][3]};
      float4 lo, hi;
      lo.x = __uint_as_float(w[0] << 16), lo.y = __uint_as_float(w[0] & 0xFFFF0000u);
      lo.z = __uint_as_float(w[1] << 16), lo.w = __uint_as_float(w[1] & 0xFFFF0000u);
      hi.x = __uint_as_float(w[2] << 16), hi.y = __uint_as_float(w[2] & 0xFFFF0000u);
      hi.z = __uint_as_float(w[3] << 16), hi.w = __uint_as_float(w[3] & 0xFFFF0000u);
      *reinterpret_cast<float4*>(&s_t[r][d]) = lo;
      *reinterpret_cast<float4*>(&s_t[r][d + 4]) = hi;
    } else {
      *reinterpret_cast<v4i*>(&s_t[r][d]) = t.x[i];
    }
  }
}

// RMSNorm (weights wa, wb) then NeoX RoPE (cos c, sin s) of one head whose
// rotation pairs (i, i + HD/2) sit in lanes i < HD/2 of the calling wave;
// the results go to dst[i] and dst[i + HD/2].  Same arithmetic as the
// LDS-staged form: f64 sum of squares, one f32 rounding per output.
template <int HD>
QDEV void norm_rope_pair(float xa, float xb, float wa, float wb, double c, double s, float eps, float* dst) {
#pragma clang fp contract(off)
  constexpr int H2 = HD / 2;
  const int lane = threadIdx.x % kWave;
  const double sq = lane < H2 ? (double)xa * (double)xa + (double)xb * (double)xb : 0.0;
  const double r = rms_scale(wave_total_d(sq), HD, eps);
  const double u = (double)rms_apply(xa, r, wa), v = (double)rms_apply(xb, r, wb);
  if (lane < H2) {
    dst[lane] = (float)(u * c - v * s);
    dst[lane + H2] = (float)(u * s + v * c);
  }
}

template <int HD, int G, int KVT>
__global__ void __launch_bounds__(kThreads) k_attn_decode(AttnDecodeArgs a) {
  constexpr int TJ = kTileRows<KVT>;
  // scores: thread -> (head h, d-part pt, row group rg of RPT rows); part pt
  // holds dims 4*pt + 4*NP*i + c (c < 4), interleaved so that the float4
  // reads of 16 lanes (4 rows x 4 parts, rows 132 or 68 floats apart) fall
  // on distinct LDS banks; the thread keeps its q dims in f64 registers
  constexpr int NP = (G == 1) ? 8 : 4;
  constexpr int DPP = HD / NP;
  constexpr int RPT = TJ * G * NP / kThreads;
  constexpr int RG = TJ / RPT;  // row groups
  static_assert(RPT >= 1 && RPT * kThreads == TJ * G * NP, "score map");
  // outputs: thread -> (head, DPT consecutive dims); threads >= OUT_T idle
  constexpr int DPT = (G * HD / kThreads) > 0 ? G * HD / kThreads : 1;
  constexpr int OUT_T = G * HD / DPT;
  constexpr int TPH = HD / DPT;  // output threads per head
  constexpr int MAXR = kScoreSlots / G;  // rows per split
  __shared__ float s_qf[G][HD];
  __shared__ float s_knew[HD];
  __shared__ float s_vnew[HD];
  __shared__ __align__(16) float s_t[TJ][HD + kLdsRow];
  __shared__ double s_s[G][MAXR];
  __shared__ double s_m[G];
  __shared__ double s_l[G];
  __shared__ int s_last;

  const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int seq = a.row_seq ? a.row_seq[row] : 0;
  const int p = a.len[seq];
  const int ctx = p + 1;
  int nsplit = (ctx + a.min_rows - 1) / a.min_rows;
  if (nsplit > a.nsplit_max) nsplit = a.nsplit_max;
  const int need = (ctx + MAXR - 1) / MAXR;  // the host keeps ctx <= kMaxSplit * MAXR
  if (nsplit < need) nsplit = need;
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

  // the split streams its K tiles, then its V tiles; stream index i < nt is
  // K tile i, i >= nt is V tile i - nt.  Rows >= p are not read from the
  // cache (row p comes from this step's projections).
  const int nt = j0 < j1 ? (j1 - j0 + TJ - 1) / TJ : 0;
  const int cache_end = min(j1, p);
  // loads of stream element i < 2 * nt; an element without cache rows (one
  // that holds only row p) reads its first row's slot instead, unused
  auto stream_load = [&](TileRegs<HD, KVT>& r, int i) {
    const bool isv = i >= nt;
    const int t0 = j0 + (isv ? i - nt : i) * TJ;
    const bool live = t0 < cache_end;
    tile_load<HD, KVT>(r, a.kv, a.kvs, isv ? vbase : kbase, live ? t0 : j0, live ? min(TJ, cache_end - t0) : 1);
  };
  // Prologue operands in registers, loaded before the first tiles so that
  // the prologue waits for them alone: wave w takes query heads w, w + 4, ...
  // and lane i the rotation pair (i, i + HD/2) (lanes past HD/2 repeat pair
  // 0 and write nothing); every wave also loads the new k and v of head g,
  // which the last wave normalises, ropes and stages.
  constexpr int H2 = HD / 2;
  constexpr int QH = (G + kWaves - 1) / kWaves;  // query heads per wave
  const int pi = lane < H2 ? lane : 0;
  const double c_rot = cs[pi], s_rot = sn[pi];
  const float qwa = a.q_norm[pi], qwb = a.q_norm[pi + H2];
  const float kwa = a.k_norm[pi], kwb = a.k_norm[pi + H2];
  float qa[QH], qb[QH];
#pragma unroll
  for (int k = 0; k < QH; ++k) {
    const int h = min(wave + k * kWaves, G - 1);
    qa[k] = qkv[(int64_t)(g * G + h) * HD + pi];
    qb[k] = qkv[(int64_t)(g * G + h) * HD + pi + H2];
  }
  const float* knew = qkv + (int64_t)nh * HD + (int64_t)g * HD;
  const float* vnew = qkv + (int64_t)(nh + nkv) * HD + (int64_t)g * HD;
  const float ka = knew[pi], kb = knew[pi + H2], va = vnew[pi], vb = vnew[pi + H2];

  TileRegs<HD, KVT> tA, tB;
  if (nt > 0) {  // 2 * nt >= 2 elements
    stream_load(tA, 0);
    stream_load(tB, 1);
  }

  const bool has_new = j0 < j1 && j1 == ctx;  // this split holds position p
#pragma unroll
  for (int k = 0; k < QH; ++k)
    if (wave + k * kWaves < G) norm_rope_pair<HD>(qa[k], qb[k], qwa, qwb, c_rot, s_rot, a.eps, s_qf[wave + k * kWaves]);
  if (has_new && wave == kWaves - 1) {
    norm_rope_pair<HD>(ka, kb, kwa, kwb, c_rot, s_rot, a.eps, s_knew);
    if (lane < H2) s_vnew[lane] = va, s_vnew[lane + H2] = vb;
  }
  __syncthreads();
  if (KVT == KV_Q8_0) {
    // the integer score path of a decode step ("The LLM stack (fucina_llm)",
    // section 13.4, the q8_0 option): each head's query is quantised per
    // 32-block like an activation; the dot of its exact dequantised values
    // with the widened K codes is sum_b d_q d_k S_b, as the integer dots give
    // it.  Every thread takes part in every pass (groups of 8 lanes = one
    // block of one head).
    for (int base = 0; base < G * HD; base += 4 * kThreads) {
      const int idx = base + 4 * tid;
      const bool live = idx < G * HD;
      float* q = &s_qf[live ? idx / HD : 0][live ? idx % HD : 0];
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (live) v[0] = q[0], v[1] = q[1], v[2] = q[2], v[3] = q[3];
      float d;
      const int packed = quant4_group8(v, &d);
      if (live) {
        const float df = f16_round(d);
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = (float)(int8_t)((packed >> (8 * c)) & 0xFF) * df;
      }
    }
    if (has_new && wave < 2) {
      // append: wave 0 encodes the new K row, wave 1 the new V row, into
      // codes and scales; the dequantised values are the ones attended below
      float* row = wave == 0 ? s_knew : s_vnew;
      const int64_t e0 = (wave == 0 ? kbase : vbase) + (int64_t)p * HD;
      const bool live = lane < HD / 4;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (live) v[0] = row[4 * lane], v[1] = row[4 * lane + 1], v[2] = row[4 * lane + 2], v[3] = row[4 * lane + 3];
      float d;
      const int packed = quant4_group8(v, &d);
      if (live) {
        *reinterpret_cast<int*>(reinterpret_cast<int8_t*>(a.kv) + e0 + 4 * lane) = packed;
        if ((lane & 7) == 0) a.kvs[e0 / 32 + lane / 8] = f32_to_f16_bits(d);
        const float df = f16_round(d);
#pragma unroll
        for (int c = 0; c < 4; ++c) row[4 * lane + c] = (float)(int8_t)((packed >> (8 * c)) & 0xFF) * df;
      }
    }
    __syncthreads();
  } else if (has_new) {
    // append: the cache stores post-RoPE K and raw V (bf16 caches round here,
    // and the rounded values are the ones attended below)
    for (int d = tid; d < HD; d += kThreads) {
      const int64_t ki = kbase + (int64_t)p * HD + d, vi = vbase + (int64_t)p * HD + d;
      if (KVT == KV_BF16) {
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

  // this thread's score role and q slice (f64)
  const int sc_pt = tid % NP, sc_rg = (tid / NP) % RG, sc_h = tid / (NP * RG);
  double qreg[DPP];
#pragma unroll
  for (int i = 0; i < DPP; ++i) qreg[i] = (double)s_qf[sc_h][4 * sc_pt + 4 * NP * (i / 4) + (i % 4)];
  // this thread's outputs
  const bool out_live = tid < OUT_T;
  const int o_h = out_live ? tid / TPH : 0, o_d = out_live ? (tid % TPH) * DPT : 0;
  double o[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) o[i] = 0.0;
  const double scale = a.scale;

  // softmax over the split's scores, once (f64): s_s becomes exp(s - m)
  auto softmax = [&]() {
    const int n = j1 - j0;
    for (int h = wave; h < G; h += kWaves) {
      double m = -INFINITY;
      for (int r = lane; r < n; r += kWave) m = fmax(m, s_s[h][r]);
      m = wave_max_all_d(m);
      double l = 0.0;
      for (int r = lane; r < n; r += kWave) {
        const double e = exp(s_s[h][r] - m);
        s_s[h][r] = e;
        l += e;
      }
      l = wave_total_d(l);
      if (lane == 0) s_m[h] = m, s_l[h] = l;
    }
  };

  // stream element i: stage it in LDS, start the load of element i + 2 into
  // the freed registers, then scores (K) or P.V (V)
  auto process = [&](TileRegs<HD, KVT>& tr, int i, auto prefetch) {
    constexpr bool PREFETCH = decltype(prefetch)::value;
    const bool isv = i >= nt;
    const int t0 = j0 + (isv ? i - nt : i) * TJ;
    const int nrow = min(TJ, j1 - t0);
    __syncthreads();  // previous tile (and, before the first V tile, the scores) consumed
    if (i == nt) {
      softmax();
      __syncthreads();
    }
    if (t0 < cache_end) tile_store<HD, KVT>(tr, s_t);
    if (PREFETCH) stream_load(tr, i + 2);
    if (t0 + nrow > p) {  // the tile holds row p: take it from this step's values
      __syncthreads();    // (after the tile store, which zero-fills that row)
      const int r = p - t0;
      const float* src = isv ? s_vnew : s_knew;
      for (int d = tid; d < HD; d += kThreads) s_t[r][d] = src[d];
    }
    __syncthreads();
    if (!isv) {
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const int r = sc_rg * RPT + j;
        const float* kr = &s_t[r][4 * sc_pt];
        double acc = 0.0;
#pragma unroll
        for (int d = 0; d < DPP; d += 4) {
          const float4 k4 = *reinterpret_cast<const float4*>(kr + NP * d);
          acc += qreg[d] * (double)k4.x;
          acc += qreg[d + 1] * (double)k4.y;
          acc += qreg[d + 2] * (double)k4.z;
          acc += qreg[d + 3] * (double)k4.w;
        }
        acc = group_sum_d<NP>(acc);
        if (sc_pt == NP - 1 && r < nrow) s_s[sc_h][t0 - j0 + r] = acc * scale;
      }
    } else if (out_live) {
      const double* pr = &s_s[o_h][t0 - j0];
      auto pv_row = [&](int r) {
        const double w = pr[r];
        const float* vr = &s_t[r][o_d];
        if (DPT == 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(vr);
          o[0] += w * (double)v4.x;
          o[DPT > 1 ? 1 : 0] += w * (double)v4.y;
          o[DPT > 2 ? 2 : 0] += w * (double)v4.z;
          o[DPT > 3 ? 3 : 0] += w * (double)v4.w;
        } else if (DPT == 2) {
          const float2 v2 = *reinterpret_cast<const float2*>(vr);
          o[0] += w * (double)v2.x;
          o[DPT > 1 ? 1 : 0] += w * (double)v2.y;
        } else {
          o[0] += w * (double)vr[0];
        }
      };
      // full tiles unrolled, so the LDS reads of many rows are in flight
      // together (row by row, each would wait out the LDS latency)
      if (nrow == TJ) {
#pragma unroll
        for (int r = 0; r < TJ; ++r) pv_row(r);
      } else {
#pragma unroll 8
        for (int r = 0; r < nrow; ++r) pv_row(r);
      }
    }
  };

  // pairs of elements with the pair after next in flight, then the last
  // pair (2 * nt is even); every load issued is used, and the number of
  // loads between two waits is fixed
  if (tid < G) s_m[tid] = -INFINITY, s_l[tid] = 0.0;  // an empty split contributes nothing
  int i = 0;
  for (; i + 2 < 2 * nt; i += 2) {
    process(tA, i, std::true_type{});
    process(tB, i + 1, std::true_type{});
  }
  if (nt > 0) {
    process(tA, i, std::false_type{});
    process(tB, i + 1, std::false_type{});
  }
  __syncthreads();

  // one split: its own o and l are the result (the combine below would
  // weigh it by exp(0) = 1 and divide by l, so the output is the same); o
  // goes through LDS to the combine's thread map, no memory round trip
  const bool direct = nsplit == 1;
  __shared__ double s_o[direct_slots<G, HD>()];
  if (direct) {
    if (out_live) {
#pragma unroll
      for (int i = 0; i < DPT; ++i) s_o[o_h * HD + o_d + i] = o[i];
    }
    __syncthreads();
  }

  // write this split's partial: [row][g][split][h][0..HD-1] = o, [HD] = m, [HD+1] = l
  const int64_t pstride = (int64_t)G * (HD + 2);
  double* part = a.part + (((int64_t)row * nkv + g) * a.nsplit_max + split) * pstride;
  if (!direct && out_live) {
#pragma unroll
    for (int i = 0; i < DPT; ++i) st_coherent(part + o_h * (HD + 2) + o_d + i, o[i]);
  }
  if (!direct && tid < G) {
    st_coherent(part + tid * (HD + 2) + HD, s_m[tid]);
    st_coherent(part + tid * (HD + 2) + HD + 1, s_l[tid]);
  }
  wait_memory();
  __syncthreads();
  if (direct) {
    if (tid == 0) s_last = 1;
  } else if (tid == 0) {
    unsigned* cnt = a.counter + (int64_t)row * nkv + g;
    const unsigned prev = arrive(cnt);
    s_last = prev == (unsigned)(nsplit - 1);
    if (s_last) st_coherent(cnt, 0u);  // every split of this launch has arrived
  }
  __syncthreads();
  if (!s_last) return;
  // combine the nsplit partials of the G heads (f64), rounded once to f32.
  // Every O load of a batch and the (m, l) loads are issued before any is
  // used (one memory round trip); wave w takes heads w, w + 4, ... and lane s
  // split s for the max and the weighted sum of l (nsplit <= 64 = lanes).
  // Thread map: E = G*HD output dims; with E >= 256 a thread owns dims
  // tid + 256k, otherwise dim tid % E for the splits = tid / E (mod NQ).
  const double* pb = a.part + (((int64_t)row * nkv + g) * a.nsplit_max) * pstride;
  constexpr int E = G * HD;
  constexpr int NQ = E >= kThreads ? 1 : kThreads / E;   // split phases
  constexpr int EPT = E >= kThreads ? E / kThreads : 1;  // dims per thread
  constexpr int SB = kCombineRegs / EPT < kMaxSplit / NQ ? kCombineRegs / EPT : kMaxSplit / NQ;  // splits per thread per batch
  const int cq = tid / (kThreads / NQ);
  const int ce = tid % (kThreads / NQ);
  __shared__ double s_w[G][kMaxSplit];
  __shared__ double s_L[G];
  __shared__ double s_red[NQ > 1 ? NQ : 1][NQ > 1 ? E : 1];
  int64_t eoff[EPT];
  int eh[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = ce + k * kThreads;
    eh[k] = e / HD;
    eoff[k] = (int64_t)eh[k] * (HD + 2) + e % HD;
  }
  double O[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) O[k] = 0.0;
  // batches of B splits per thread; B is the smallest of SB/4, SB/2, SB that
  // covers this thread's splits, so short caches issue few clamped repeats
  auto batches = [&](auto bsz) {
    constexpr int B = decltype(bsz)::value;
    for (int s0 = 0; s0 < nsplit; s0 += NQ * B) {
      double v[B][EPT];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int sidx = min(s0 + cq + NQ * j, nsplit - 1);
#pragma unroll
        for (int k = 0; k < EPT; ++k) v[j][k] = ld_coherent(pb + sidx * pstride + eoff[k]);
      }
      if (s0 == 0) {
        const int sl = min(lane, nsplit - 1);
        double m[QH], l[QH];
#pragma unroll
        for (int k = 0; k < QH; ++k) {
          const int h = min(wave + k * kWaves, G - 1);
          m[k] = ld_coherent(pb + sl * pstride + h * (HD + 2) + HD);
          l[k] = ld_coherent(pb + sl * pstride + h * (HD + 2) + HD + 1);
        }
#pragma unroll
        for (int k = 0; k < QH; ++k) {
          const int h = wave + k * kWaves;
          const bool live = lane < nsplit;
          const double M = wave_max_all_d(live ? m[k] : -INFINITY);
          const double w = live ? exp(m[k] - M) : 0.0;
          const double L = wave_total_d(w * l[k]);
          if (h < G) {
            s_w[h][lane] = w;
            if (lane == 0) s_L[h] = L;
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int sidx = s0 + cq + NQ * j;
        if (sidx < nsplit) {
#pragma unroll
          for (int k = 0; k < EPT; ++k) O[k] += s_w[eh[k]][sidx] * v[j][k];
        }
      }
    }
  };
  const int per_thread = (nsplit + NQ - 1) / NQ;
  if (direct) {
    if (cq == 0) {
#pragma unroll
      for (int k = 0; k < EPT; ++k) O[k] = s_o[ce + k * kThreads];
    }
    if (tid < G) s_L[tid] = s_l[tid];
    __syncthreads();
  } else if (per_thread <= SB / 4)
    batches(std::integral_constant<int, SB / 4>{});
  else if (per_thread <= SB / 2)
    batches(std::integral_constant<int, SB / 2>{});
  else
    batches(std::integral_constant<int, SB>{});
  if (NQ > 1 && !direct) {
    s_red[cq][ce] = O[0];
    __syncthreads();
    if (cq == 0) {
      double t = s_red[0][ce];
      for (int q = 1; q < NQ; ++q) t += s_red[q][ce];
      O[0] = t;
    }
  }
  if (cq == 0) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const float y = (float)(O[k] / s_L[eh[k]]);
      const int col = g * E + ce + k * kThreads;
      a.out[(int64_t)row * a.out_stride + col] = y;
      if (a.q_out) {
        // Q8_0 of the output row, block by block: a block's 32 values sit
        // in 32 consecutive lanes (E and g * E are multiples of 32); the
        // arithmetic is k_rows_quant's (max over the block, d = amax / 127,
        // codes rint(v / d) clamped, scale rounded to f16)
        float am = fabsf(y);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 32));
        const float d = am / 127.0f;
        const float inv = d == 0.f ? 0.f : 1.0f / d;
        const float q = fminf(fmaxf(rintf(y * inv), -127.f), 127.f);
        const int64_t bi = (int64_t)(col / 32) * gridDim.z + row;
        a.q_out[bi * 32 + col % 32] = (int8_t)(int)q;
        if (col % 32 == 0) a.q_scale[bi] = f16_round(d);
      }
    }
  }
}

template <int HD, int G>
hipError_t launch(const AttnDecodeArgs& a, int kvt, int nrows, hipStream_t s) {
  const dim3 grid(a.nsplit_max, a.nkv, nrows);
  switch (kvt) {
    case KV_F32: hipLaunchKernelGGL((k_attn_decode<HD, G, KV_F32>), grid, dim3(kThreads), 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL((k_attn_decode<HD, G, KV_BF16>), grid, dim3(kThreads), 0, s, a); break;
    case KV_Q8_0: hipLaunchKernelGGL((k_attn_decode<HD, G, KV_Q8_0>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void k_set_len(int32_t* len, int seq, int value) { len[seq] = value; }

}  // namespace

namespace q8k {

bool attn_decode_supported(int hd, int group) {
  return (hd == 64 || hd == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

int attn_decode_max_ctx(int group) { return kMaxSplit * (kScoreSlots / group); }

hipError_t attn_decode(const AttnDecodeArgs& a, int hd, int group, int kvt, int nrows, hipStream_t s) {
#define Q8_ATT(HD_, G_) \
  if (hd == HD_ && group == G_) return launch<HD_, G_>(a, kvt, nrows, s);
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
