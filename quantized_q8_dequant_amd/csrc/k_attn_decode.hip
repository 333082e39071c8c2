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
// Grid (nkv, nsplit_max, nrows): workgroup (g, split, row) serves the G query
// heads of KV head g, so each K/V row is read once for all of them; the KV
// head varies fastest, so the workgroups dispatched first (which run ahead
// of those sharing their CU) hold splits of every head.  The positions
// [0, p] are cut into about min(nsplit_max, ceil((p+1)/min_rows)) ranges of
// whole tiles; each workgroup computes its range's max m, sum l and unnormalised
// o (scores in LDS, one softmax, then P.V) and writes them as a partial; the
// last workgroup to arrive (atomic counter) merges the partials and writes
// the normalised output.  Within a workgroup a thread serves up to four
// query heads at once, so each K or V element is read from LDS and widened
// to f64 once for all of them.
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
constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int cmin(int x, int y) { return x < y ? x : y; }
typedef unsigned v4u __attribute__((ext_vector_type(4)));
// cache policy of the partials' 16-byte loads and stores: device scope (sc1),
// the policy of the agent-scope atomic loads and stores
constexpr int kCoherent = 16;

// The value of the lane whose index differs in bit M (M = 1, 2, 4, 8 with
// DPP moves inside a row of 16 lanes: the partner differs in bit M and
// possibly in lower bits, never in higher ones; otherwise an exact xor
// through the LDS permute).
template <int M, bool DPP>
QDEV double partner_d(double v) {
  if constexpr (DPP && M == 1) return dpp_move_d<0xB1>(v);   // quad_perm [1,0,3,2]
  else if constexpr (DPP && M == 2) return dpp_move_d<0x4E>(v);  // quad_perm [2,3,0,1]
  else if constexpr (DPP && M == 4) return dpp_move_d<0x141>(v);  // row_half_mirror
  else if constexpr (DPP && M == 8) return dpp_move_d<0x140>(v);  // row_mirror
  else return __shfl_xor(v, M);
}

// Sums of V slots over a group of NL lanes (lane masks M * S for M < NL),
// scattered: each halving step keeps the upper or lower half of the slots
// by the lane's bit M and adds the partner's values for that half, so that
// afterwards group member p holds in v[0 .. V/W - 1] (W = min(V, NL)) the
// totals of slots (p / (NL / W)) * (V / W) + u; when V < NL the last steps
// add whole totals, so the NL / W members of a block agree.
template <int M, int N, int NL, int V, int S, bool DPP>
QDEV void scatter_steps(double (&v)[V], int p) {
  constexpr int W = V < NL ? V : NL;
  if constexpr (M >= 1) {
    if constexpr (N > V / W) {
      constexpr int H = N / 2;
      const bool up = (p & M) != 0;
#pragma unroll
      for (int u = 0; u < H; ++u) {
        const double send = up ? v[u] : v[u + H];
        const double keep = up ? v[u + H] : v[u];
        v[u] = keep + partner_d<M * S, DPP>(send);
      }
      scatter_steps<M / 2, H, NL, V, S, DPP>(v, p);
    } else {
      v[0] += partner_d<M * S, DPP>(v[0]);
      scatter_steps<M / 2, N, NL, V, S, DPP>(v, p);
    }
  }
}
template <int NL, int V, int S, bool DPP>
QDEV void scatter_sum_d(double (&v)[V], int p) {
  scatter_steps<NL / 2, V, NL, V, S, DPP>(v, p);
}

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
  // A thread serves HG query heads at once: each K or V element it reads
  // from LDS is widened to f64 once and feeds HG products.
  constexpr int HG = G < 4 ? G : 4;  // query heads per thread
  constexpr int NHG = G / HG;        // head groups
  // scores: thread -> (head group, row group rg of RPT consecutive rows,
  // d-part pt); part pt holds dims 4*pt + 4*NP*i + c (c < 4), so the float4
  // reads of 8 consecutive lanes cover 128 consecutive bytes of one row (no
  // LDS bank conflict); the thread keeps the q dims of its heads in f64
  // registers and its HG x RPT partial dots are summed over the NP parts
  // scattered (one total per lane)
  constexpr int NP = cmax(cmax(8, HG * HD / 32), kThreads / (NHG * TJ));
  constexpr int DPP = HD / NP;
  constexpr int RG = kThreads / (NHG * NP);  // row groups
  constexpr int RPT = TJ / RG;
  constexpr int SV = HG * RPT;  // partial dots per thread, slot j * HG + k
  constexpr int SW = SV < NP ? SV : NP;
  static_assert(DPP % 4 == 0 && RPT >= 1 && NHG * NP * RG == kThreads && RG * RPT == TJ, "score map");
  // P.V: thread -> (head group, row group of RPV consecutive rows, d-chunk
  // dc); chunk dc holds dims 4*dc + 4*DC*i + c, the thread sums w_j V_j of
  // its rows for its HG heads; the row groups' sums are added once per split
  constexpr int DPV = cmin(cmin(16 / HG > 4 ? 16 / HG : 4, HD * NHG * TJ / kThreads), HD / 8);
  constexpr int DC = HD / DPV;
  constexpr int RGV = kThreads / (NHG * DC);
  constexpr int RPV = TJ / RGV;
  constexpr int OV = HG * DPV;    // sums per thread, slot k * DPV + i
  constexpr int RW = kWave / DC;  // row groups per wavefront
  constexpr int OW = OV < RW ? OV : RW;
  constexpr int WPG = kWaves / NHG;  // wavefronts per head group
  static_assert(DPV % 4 == 0 && RPV >= 1 && NHG * DC * RGV == kThreads && RGV * RPV == TJ && RW >= 1, "P.V map");
  constexpr int MAXR = kScoreSlots / G;  // rows per split
  __shared__ float s_qf[G][HD];
  __shared__ float s_knew[HD];
  __shared__ float s_vnew[HD];
  __shared__ __align__(16) float s_t[TJ][HD + kLdsRow];
  __shared__ double s_s[G][MAXR];
  __shared__ double s_m[G];
  __shared__ double s_l[G];
  __shared__ int s_last;

  const int g = blockIdx.x, split = blockIdx.y, row = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int seq = a.row_seq ? a.row_seq[row] : 0;
  const int p = a.len[seq];
  const int ctx = p + 1;
  int nsplit = (ctx + a.min_rows - 1) / a.min_rows;
  if (nsplit > a.nsplit_max) nsplit = a.nsplit_max;
  const int need = (ctx + MAXR - 1) / MAXR;  // the host keeps ctx <= kMaxSplit * MAXR
  if (nsplit < need) nsplit = need;
  // whole tiles per split: the range rounded up to a multiple of TJ rows and
  // the count recomputed (no more tile steps per split, fewer splits, so
  // fewer partials to combine); still at most MAXR rows, a multiple of TJ
  int chunk = (ctx + nsplit - 1) / nsplit;
  chunk = (chunk + TJ - 1) / TJ * TJ;
  nsplit = (ctx + chunk - 1) / chunk;
  if (split >= nsplit) return;  // uniform per workgroup; not counted below
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

  // this thread's score role and the q dims of its heads (f64)
  const int sc_pt = tid % NP, sc_rg = (tid / NP) % RG, sc_hg = tid / (NP * RG);
  double qreg[HG][DPP];
#pragma unroll
  for (int k = 0; k < HG; ++k)
#pragma unroll
    for (int i = 0; i < DPP; ++i) qreg[k][i] = (double)s_qf[sc_hg * HG + k][4 * sc_pt + 4 * NP * (i / 4) + (i % 4)];
  // this thread's P.V role and sums
  const int pv_dc = tid % DC, pv_rg = (tid / DC) % RGV, pv_hg = tid / (DC * RGV);
  double pv[OV];
#pragma unroll
  for (int i = 0; i < OV; ++i) pv[i] = 0.0;
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
      double acc[SV];
#pragma unroll
      for (int v = 0; v < SV; ++v) acc[v] = 0.0;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        const float* kr = &s_t[sc_rg * RPT + j][4 * sc_pt];
#pragma unroll
        for (int d = 0; d < DPP; d += 4) {
          const float4 k4 = *reinterpret_cast<const float4*>(kr + NP * d);
          const double kx = k4.x, ky = k4.y, kz = k4.z, kw = k4.w;
#pragma unroll
          for (int k = 0; k < HG; ++k) {
            double& s = acc[j * HG + k];
            s += qreg[k][d] * kx;
            s += qreg[k][d + 1] * ky;
            s += qreg[k][d + 2] * kz;
            s += qreg[k][d + 3] * kw;
          }
        }
      }
      // rows past nrow hold stale values; their slots are never written
      scatter_sum_d<NP, SV, 1, true>(acc, sc_pt);
      if (sc_pt % (NP / SW) == 0) {
#pragma unroll
        for (int u = 0; u < SV / SW; ++u) {
          const int v = (sc_pt / (NP / SW)) * (SV / SW) + u;
          const int r = sc_rg * RPT + v / HG;
          if (r < nrow) s_s[sc_hg * HG + v % HG][t0 - j0 + r] = acc[u] * scale;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPV; ++j) {
        const int r = pv_rg * RPV + j;
        if (r < nrow) {
          double w[HG];
#pragma unroll
          for (int k = 0; k < HG; ++k) w[k] = s_s[pv_hg * HG + k][t0 - j0 + r];
          const float* vr = &s_t[r][4 * pv_dc];
#pragma unroll
          for (int i = 0; i < DPV; i += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(vr + DC * i);
            const double vx = v4.x, vy = v4.y, vz = v4.z, vw = v4.w;
#pragma unroll
            for (int k = 0; k < HG; ++k) {
              pv[k * DPV + i] += w[k] * vx;
              pv[k * DPV + i + 1] += w[k] * vy;
              pv[k * DPV + i + 2] += w[k] * vz;
              pv[k * DPV + i + 3] += w[k] * vw;
            }
          }
        }
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

  // the P.V sums of the row groups: scattered over the row groups of each
  // wavefront, then the WPG wavefronts of a head group through LDS (the
  // score buffer, no longer read), added in wavefront order
  scatter_sum_d<RW, OV, DC, false>(pv, lane / DC);
  {
    double* buf = &s_s[0][0];  // [WPG][G][HD]
    const int rgw = lane / DC;
    if (rgw % (RW / OW) == 0) {
#pragma unroll
      for (int u = 0; u < OV / OW; ++u) {
        const int v = (rgw / (RW / OW)) * (OV / OW) + u;
        const int k = v / DPV, ii = v % DPV;
        const int d = 4 * pv_dc + DC * (ii / 4 * 4) + ii % 4;
        buf[((wave % WPG) * G + pv_hg * HG + k) * HD + d] = pv[u];
      }
    }
  }
  __syncthreads();
  // this split's o, in pairs of adjacent dims: pair pe of the E = G*HD
  // outputs is dims 2pe, 2pe + 1 of head 2pe / HD (HD is even, so a pair
  // never straddles two heads); thread tid owns pairs tid + 256k
  constexpr int E = G * HD;
  constexpr int P = E / 2;
  constexpr int PPT = P >= kThreads ? P / kThreads : 1;  // pairs per thread
  double o[PPT][2];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int pe = tid + k * kThreads;
    double t0 = 0.0, t1 = 0.0;
    if (pe < P) {
      const double* buf = &s_s[0][0];
      const int h = 2 * pe / HD, d = 2 * pe % HD;
#pragma unroll
      for (int w = 0; w < WPG; ++w) {
        t0 += buf[(w * G + h) * HD + d];
        t1 += buf[(w * G + h) * HD + d + 1];
      }
    }
    o[k][0] = t0, o[k][1] = t1;
  }

  // one split: its own o and l are the result (the combine below would
  // weigh it by exp(0) = 1 and divide by l, so the output is the same); o
  // goes through LDS to the combine's thread map, no memory round trip
  const bool direct = nsplit == 1;
  __shared__ double s_o[direct_slots<G, HD>()];
  if (direct) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pe = tid + k * kThreads;
      if (pe < P) s_o[2 * pe] = o[k][0], s_o[2 * pe + 1] = o[k][1];
    }
    __syncthreads();
  }

  // write this split's partial: [row][g][split][h][0..HD-1] = o, [HD] = m,
  // [HD+1] = l; every pair of doubles (o pairs, (m, l)) is one 16-byte store
  // with the device-scope policy (16-byte aligned: HD + 2 and the split
  // stride are even)
  const int pstride = G * (HD + 2);
  const int pbytes = a.nsplit_max * pstride * 8;  // one (row, KV head)'s partials
  double* pb = a.part + ((int64_t)row * nkv + g) * a.nsplit_max * pstride;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(pb, 0, pbytes, 0x00020000);
  auto put2 = [&](int idx, double x, double y) {  // doubles idx, idx + 1 of split `split`
    const v4u q = {(unsigned)__double2loint(x), (unsigned)__double2hiint(x), (unsigned)__double2loint(y),
                   (unsigned)__double2hiint(y)};
    __builtin_amdgcn_raw_buffer_store_b128(q, prs, (split * pstride + idx) * 8, 0, kCoherent);
  };
  if (!direct) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pe = tid + k * kThreads;
      if (pe < P) put2(2 * pe / HD * (HD + 2) + 2 * pe % HD, o[k][0], o[k][1]);
    }
    if (tid < G) put2(tid * (HD + 2) + HD, s_m[tid], s_l[tid]);
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
  // used (one memory round trip), 16 bytes (a pair) per load; wave w takes
  // heads w, w + 4, ... and lane s split s for the max and the weighted sum
  // of l (nsplit <= 64 = lanes).  Thread map: with P >= 256 pairs a thread
  // owns pairs tid + 256k, otherwise pair tid % P for the splits
  // = tid / P (mod NQ).
  constexpr int NQ = P >= kThreads ? 1 : kThreads / P;  // split phases
  constexpr int SB = cmin(kCombineRegs / (2 * PPT), kMaxSplit / NQ);  // splits per thread per batch
  const int cq = tid / (kThreads / NQ);
  const int ce = tid % (kThreads / NQ);
  __shared__ double s_w[G][kMaxSplit];
  __shared__ double s_L[G];
  __shared__ double s_red[NQ > 1 ? NQ : 1][NQ > 1 ? E : 1];
  int poff[PPT], ph[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int e0 = 2 * (ce + k * kThreads);
    ph[k] = e0 / HD;
    poff[k] = (ph[k] * (HD + 2) + e0 % HD) * 8;
  }
  double O[PPT][2];
#pragma unroll
  for (int k = 0; k < PPT; ++k) O[k][0] = O[k][1] = 0.0;
  auto lo_d = [](const v4u& v) { return __hiloint2double((int)v.y, (int)v.x); };
  auto hi_d = [](const v4u& v) { return __hiloint2double((int)v.w, (int)v.z); };
  // batches of B splits per thread; B is the smallest of SB/4, SB/2, SB that
  // covers this thread's splits, so short caches issue few clamped repeats
  auto batches = [&](auto bsz) {
    constexpr int B = decltype(bsz)::value;
    for (int s0 = 0; s0 < nsplit; s0 += NQ * B) {
      v4u v[B][PPT];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int sidx = min(s0 + cq + NQ * j, nsplit - 1);
#pragma unroll
        for (int k = 0; k < PPT; ++k)
          v[j][k] = __builtin_amdgcn_raw_buffer_load_b128(prs, sidx * pstride * 8 + poff[k], 0, kCoherent);
      }
      if (s0 == 0) {
        const int sl = min(lane, nsplit - 1);
        v4u ml[QH];
#pragma unroll
        for (int k = 0; k < QH; ++k) {
          const int h = min(wave + k * kWaves, G - 1);
          ml[k] = __builtin_amdgcn_raw_buffer_load_b128(prs, (sl * pstride + h * (HD + 2) + HD) * 8, 0, kCoherent);
        }
#pragma unroll
        for (int k = 0; k < QH; ++k) {
          const int h = wave + k * kWaves;
          const bool live = lane < nsplit;
          const double m = lo_d(ml[k]), l = hi_d(ml[k]);
          const double M = wave_max_all_d(live ? m : -INFINITY);
          const double w = live ? exp(m - M) : 0.0;
          const double L = wave_total_d(w * l);
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
          for (int k = 0; k < PPT; ++k) {
            const double w = s_w[ph[k]][sidx];
            O[k][0] += w * lo_d(v[j][k]);
            O[k][1] += w * hi_d(v[j][k]);
          }
        }
      }
    }
  };
  const int per_thread = (nsplit + NQ - 1) / NQ;
  if (direct) {
    if (cq == 0) {
#pragma unroll
      for (int k = 0; k < PPT; ++k) {
        const int e0 = 2 * (ce + k * kThreads);
        O[k][0] = s_o[e0], O[k][1] = s_o[e0 + 1];
      }
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
    s_red[cq][2 * ce] = O[0][0];
    s_red[cq][2 * ce + 1] = O[0][1];
    __syncthreads();
    if (cq == 0) {
      double t0 = s_red[0][2 * ce], t1 = s_red[0][2 * ce + 1];
      for (int q = 1; q < NQ; ++q) t0 += s_red[q][2 * ce], t1 += s_red[q][2 * ce + 1];
      O[0][0] = t0, O[0][1] = t1;
    }
  }
  if (cq == 0) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int col = g * E + 2 * (ce + k * kThreads);
      const float y0 = (float)(O[k][0] / s_L[ph[k]]);
      const float y1 = (float)(O[k][1] / s_L[ph[k]]);
      float* dst = a.out + (int64_t)row * a.out_stride + col;
      dst[0] = y0;
      dst[1] = y1;
      if (a.q_out) {
        // Q8_0 of the output row, block by block: a block's 32 values sit
        // in 16 consecutive lanes, two each (E and g * E are multiples of
        // 32); the arithmetic is k_rows_quant's (max over the block,
        // d = amax / 127, codes rint(v / d) clamped, scale rounded to f16)
        float am = fmaxf(fabsf(y0), fabsf(y1));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 16));
        const float d = am / 127.0f;
        const float inv = d == 0.f ? 0.f : 1.0f / d;
        const float q0 = fminf(fmaxf(rintf(y0 * inv), -127.f), 127.f);
        const float q1 = fminf(fmaxf(rintf(y1 * inv), -127.f), 127.f);
        const int64_t bi = (int64_t)(col / 32) * gridDim.z + row;
        a.q_out[bi * 32 + col % 32] = (int8_t)(int)q0;
        a.q_out[bi * 32 + col % 32 + 1] = (int8_t)(int)q1;
        if (col % 32 == 0) a.q_scale[bi] = f16_round(d);
      }
    }
  }
}

template <int HD, int G>
hipError_t launch(const AttnDecodeArgs& a, int kvt, int nrows, hipStream_t s) {
  const dim3 grid(a.nkv, a.nsplit_max, nrows);
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
