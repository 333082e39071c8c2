// One launch per decode step (single sequence, Q8_0 weights): a persistent
// grid of 256 workgroups, one per CU, runs every layer and the tied lm_head.
//
// What is computed is the decode step of the Fucina course page "A transformer
// from scratch" (sections 12.3-12.6) with the Q8_0 linears of "Model files and
// quantization" (sections 11.7 and 11.9), exactly as the per-kernel path
// computes it (same f64 reductions, same per-row block order):
//   x = embed(token); per layer:
//     A  qkv = W_qkv . quant(rmsnorm(x, attn_norm))
//     B  per KV head g: q/k norm + RoPE, append k/v at row p, attention over
//        rows 0..p split across workgroups; every workgroup then combines
//        the splits' partials for a slice of the head group's outputs
//     C  x = x + W_o . quant(att)
//     D  h = silu(W_gate . b) * (W_up . b), b = quant(rmsnorm(x, ffn_norm))
//     E  x = x + W_down . quant(h)
//   logits = W_emb . quant(rmsnorm(x, output_norm)); token = argmax.
//
// Between phases every workgroup needs values written by others.  Each
// activation word is stored as (f32 value, 32-bit epoch) in one 64-bit
// agent-coherent store; a reader polls the words it needs until all carry
// the epoch it expects, so the data is its own flag and no barrier or fence
// is used.  A phase issues the loads of its weight slice before it starts
// polling, so HBM streams while the workgroup waits (the placement of each
// slice and of the KV tiles is given where the slices are declared).  Each buffer is
// written once per layer with a new epoch, and the phase order guarantees
// that every reader of one epoch has finished before the next is written.
//
// Every wait is bounded: after a spin limit the workgroup sets an error word
// and leaves, the others see the word and leave too, the step's argmax is -1
// and the sequence length is not advanced.  The word is sticky: a step that
// starts with it set does nothing but write -1, until the host reads and
// clears it.  The grid must be co-resident: it is launched cooperatively, so
// a grid that cannot be resident fails to launch instead of waiting forever.
#include "persist.h"
#include "qdevice.h"

using namespace q8;

namespace {

typedef unsigned long long u64;
constexpr int NT = 256;        // threads per workgroup
constexpr int kWavesP = NT / kWave;
constexpr int TJ = 32;         // KV rows per staged tile
constexpr int kSpin = 1 << 21;  // poll rounds before a wait gives up

QDEV u64 tag_word(float v, unsigned tag) { return ((u64)tag << 32) | (u64)__float_as_uint(v); }
QDEV void put_tagged(u64* p, float v, unsigned tag) {
  __hip_atomic_store(p, tag_word(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
QDEV unsigned ld_err(const unsigned* err) { return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Polling.  A poll round re-reads the words it still waits for with
// device-coherent loads, and on this chip the cost of such a round grows with
// the number of load instructions, not with bytes: each load here takes two
// adjacent tagged words (16 bytes) through a buffer resource whose bounds
// are the polled vector's.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kCoherent = 16;  // cache policy of the loads: device scope (sc1)

// Each wavefront polls its own words, without a barrier per round: a round
// is its loads, one wait and a wavefront-wide check.  A wavefront stops when
// its words are all there, when the error word is set (checked every 64
// rounds) or at the spin limit (it then sets the error word, so the others
// stop too); then the workgroup meets once and fails if any wavefront did.
// Every wait is bounded, so every wavefront reaches that meeting.
QDEV bool wave_error(unsigned* err) { return __builtin_amdgcn_readfirstlane(ld_err(err)) != 0; }
QDEV bool block_failed(bool wave_bad) {  // wave_bad is wavefront-uniform
  __shared__ int s_bad[kWavesP];
  if (threadIdx.x % kWave == 0) s_bad[threadIdx.x / kWave] = wave_bad ? 1 : 0;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int w = 0; w < kWavesP; ++w) any |= s_bad[w];
  return any != 0;
}

// One wavefront's wait: rounds of loads (issue(j, r) loads slot j < PER of
// this thread into r) until every word carries `tag`; the words end in v.
// A slot whose pair has arrived is not read again (its tag cannot change
// before every reader of this epoch is done), so a round only fetches what
// is still missing; and while none of the wavefront's pairs has arrived, a
// round reads one pair only.  The device-coherent reads go to the memory
// side, where they compete with the weight streams.  False at the spin limit
// (the error word is then set) or when another workgroup has reported an
// error (checked every 64 rounds).
template <int PER, typename Issue>
QDEV bool poll_wave(Issue issue, unsigned tag, unsigned* err, v4u (&v)[PER]) {
  bool have[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) have[j] = false;
  bool started = true;  // the first round reads every pair
  for (int spin = 0;; ++spin) {
    // every load of the round is issued before any is checked, so one wait
    // covers them all.  While none of the wavefront's pairs has arrived, a
    // round re-reads only one pair (slot 0 of lane 0)
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (!have[j] && (started || (j == 0 && threadIdx.x % kWave == 0))) issue(j, v[j]);
    bool ok = true, any = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      have[j] = have[j] || (v[j].y == tag && v[j].w == tag);
      ok = ok && have[j];
      any = any || have[j];
    }
    if (__all(ok)) return true;
    started = __any(any);
    if ((spin & 63) == 63 && wave_error(err)) return false;
    if (spin == kSpin) {
      if (threadIdx.x % kWave == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

// Wait until the 2 * NPAIR words of the pairs at word offsets off(j) (even)
// of base[0, nwords) all carry `tag`; then the 32-bit payload of word
// 2j + h goes to *dst(2j + h).  False when the spin limit is reached or
// another workgroup has reported an error.
template <int NPAIR, typename Off, typename Dst>
QDEV bool poll_pairs(const u64* base, int nwords, Off off, Dst dst, unsigned tag, unsigned* err) {
  constexpr int PER = (NPAIR + NT - 1) / NT;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u64*>(base), 0, nwords * 8, 0x00020000);
  // slots past NPAIR re-read the last pair
  auto issue = [&](int j, v4u& r) {
    const int i = min((int)threadIdx.x + j * NT, NPAIR - 1);
    r = __builtin_amdgcn_raw_buffer_load_b128(rs, off(i) * 8, 0, kCoherent);
  };
  v4u v[PER];
  const bool bad = !poll_wave<PER>(issue, tag, err, v);
  if (block_failed(bad)) return false;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * NT;
    if (i < NPAIR) {
      *dst(2 * i) = v[j].x;
      *dst(2 * i + 1) = v[j].z;
    }
  }
  __syncthreads();
  return true;
}

// A Q8_0 block handed over quantised: 8 words of four codes, then the
// f16-valued scale in words 8 and 9 (one pair), padded to a 128-byte line so
// that no two workgroups write into one line (a shared partial line was seen
// much later by the readers).
constexpr int kBlockWords = 16;
constexpr int kBlockPairs = 5;
// Lane t < 8 of one 8-lane group stores code word t; lane 0 also the scale.
QDEV void put_block(u64* blk, int packed, float d16, unsigned tag) {
  const int t = threadIdx.x % 8;
  put_tagged(blk + t, __int_as_float(packed), tag);
  if (t == 0) {
    put_tagged(blk + 8, d16, tag);
    put_tagged(blk + 9, d16, tag);
  }
}
// Wait for the NB blocks at base, then their codes go to s_qa (block-major)
// and their scales to s_da.
template <int NB>
QDEV bool poll_blocks(const u64* base, unsigned tag, int8_t* s_qa, float* s_da, unsigned* err) {
  __shared__ unsigned s_spare;
  unsigned* qa = reinterpret_cast<unsigned*>(s_qa);
  unsigned* da = reinterpret_cast<unsigned*>(s_da);
  auto off = [](int j) { return (j / kBlockPairs) * kBlockWords + 2 * (j % kBlockPairs); };
  auto dst = [&](int i) {
    const int blk = i / (2 * kBlockPairs), w = i % (2 * kBlockPairs);
    return w < 8 ? qa + blk * 8 + w : w == 8 ? da + blk : &s_spare;
  };
  return poll_pairs<NB * kBlockPairs>(base, NB * kBlockWords, off, dst, tag, err);
}

// The N (even) contiguous words at src into dst (LDS) as floats.
template <int N>
QDEV bool poll_vec(const u64* src, unsigned tag, float* dst, unsigned* err) {
  static_assert(N % 2 == 0, "pairs");
  unsigned* d = reinterpret_cast<unsigned*>(dst);
  return poll_pairs<N / 2>(src, N, [](int j) { return 2 * j; }, [&](int i) { return d + i; }, tag, err);
}

// The N words at src into registers, in the layout the register quantiser
// takes: thread t receives words 1024 i + 4t .. 4t + 3 (i < N / 1024) as
// x[4 i .. 4 i + 3].  No LDS copy and no barrier after the wait.
template <int N>
QDEV bool poll_vec_regs(const u64* src, unsigned tag, float (&x)[N / NT], unsigned* err) {
  static_assert(N % (4 * NT) == 0, "whole passes of four words per thread");
  constexpr int PER = N / (2 * NT);  // pairs per thread
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<u64*>(src), 0, N * 8, 0x00020000);
  auto issue = [&](int j, v4u& r) {
    const int pair = (j / 2) * (2 * NT) + 2 * (int)threadIdx.x + (j % 2);
    r = __builtin_amdgcn_raw_buffer_load_b128(rs, pair * 16, 0, kCoherent);
  };
  v4u v[PER];
  const bool bad = !poll_wave<PER>(issue, tag, err, v);
  if (block_failed(bad)) return false;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    x[2 * j] = __uint_as_float(v[j].x);
    x[2 * j + 1] = __uint_as_float(v[j].z);
  }
  return true;
}

// An f64 as two tagged words (low half, then high half) at the even word
// offset `w` of base[0, nwords), written by one 16-byte store with the
// device-scope policy: each 8-byte half still carries its own tag, and the
// reader checks both, so the pair needs no atomicity beyond its halves; one
// store request per value instead of two.
QDEV void put_tagged_d(u64* base, int nwords, int w, double v, unsigned tag) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, nwords * 8, 0x00020000);
  const v4u q = {(unsigned)__double2loint(v), tag, (unsigned)__double2hiint(v), tag};
  __builtin_amdgcn_raw_buffer_store_b128(q, rs, w * 8, 0, kCoherent);
}

// A norm weight vector of K floats held in registers, one float4 per thread
// per pass of the 256 threads (loaded before a wait, used after it).
template <int K>
struct NormW {
  static constexpr int KI = (K + NT * 4 - 1) / (NT * 4);
  float4 w[KI];
  QDEV void load(const float* __restrict__ p) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int c = i * NT * 4 + threadIdx.x * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < K) {
        const v4i t = ld_global<v4i>(as_global(p) + c);
        v = make_float4(__int_as_float(t.x), __int_as_float(t.y), __int_as_float(t.z), __int_as_float(t.w));
      }
      w[i] = v;
    }
  }
};

// Quantise the K values in LDS (optionally RMSNorm'd with the weights nw) to Q8_0 codes
// and f16-valued scales in LDS; the same arithmetic and summation order as
// the decode GEMV's prologue.
template <int K, bool NORM>
QDEV void quantize_lds(const float* s_x, const NormW<K>* nw, float eps, int8_t* s_qa, float* s_da, double* s_red) {
  double r = 1.0;
  if (NORM) {
    double ss = 0.0;
    for (int c = threadIdx.x * 4; c < K; c += NT * 4) {
      const float4 v = *reinterpret_cast<const float4*>(s_x + c);
      ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
    ss = block_sum_d_open<NT>(ss, s_red);  // (the barrier at the end covers s_red)
    r = rms_scale(ss, K, eps);
  }
#pragma unroll
  for (int base = 0; base < K; base += NT * 4) {
    const int c = base + threadIdx.x * 4;
    const bool live = c < K;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      const float4 t = *reinterpret_cast<const float4*>(s_x + c);
      v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
      if (NORM) {
        const float4 w4 = nw->w[base / (NT * 4)];
        v[0] = rms_apply(v[0], r, w4.x), v[1] = rms_apply(v[1], r, w4.y);
        v[2] = rms_apply(v[2], r, w4.z), v[3] = rms_apply(v[3], r, w4.w);
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

// quantize_lds with the values in registers (thread t holds values
// 1024 i + 4t .. 4t + 3 as x[4 i ..]): the same arithmetic and summation
// order, without the LDS copy of x.
template <int K, bool NORM>
QDEV void quantize_regs(const float (&x)[K / NT], const NormW<K>* nw, float eps, int8_t* s_qa, float* s_da,
                        double* s_red) {
  static_assert(K % (4 * NT) == 0, "whole passes");
  double r = 1.0;
  if (NORM) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < K / (4 * NT); ++i) {
      const float* v = x + 4 * i;
      ss += (double)v[0] * v[0] + (double)v[1] * v[1] + (double)v[2] * v[2] + (double)v[3] * v[3];
    }
    ss = block_sum_d_open<NT>(ss, s_red);  // (the barrier at the end covers s_red)
    r = rms_scale(ss, K, eps);
  }
#pragma unroll
  for (int i = 0; i < K / (4 * NT); ++i) {
    const int c = i * NT * 4 + threadIdx.x * 4;
    float v[4] = {x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
    if (NORM) {
      const float4 w4 = nw->w[i];
      v[0] = rms_apply(v[0], r, w4.x), v[1] = rms_apply(v[1], r, w4.y);
      v[2] = rms_apply(v[2], r, w4.z), v[3] = rms_apply(v[3], r, w4.w);
    }
    float d;
    const int packed = quant4_group8(v, &d);
    *reinterpret_cast<int*>(s_qa + c) = packed;
    if ((threadIdx.x & 7) == 0) s_da[c >> 5] = f16_round(d);
  }
  __syncthreads();
}

// Wait for the K words at src, then quantise them (RMSNorm'd with nw when
// NORM) into s_qa / s_da: from registers where K fills whole passes of the
// grid, else through LDS.
template <int K, bool NORM>
QDEV bool poll_quantize(const u64* src, unsigned tag, float* s_x, const NormW<K>* nw, float eps, int8_t* s_qa,
                        float* s_da, double* s_red, unsigned* err) {
  if constexpr (K % (4 * NT) == 0) {
    float x[K / NT];
    if (!poll_vec_regs<K>(src, tag, x, err)) return false;
    quantize_regs<K, NORM>(x, nw, eps, s_qa, s_da, s_red);
  } else {
    if (!poll_vec<K>(src, tag, s_x, err)) return false;
    quantize_lds<K, NORM>(s_x, nw, eps, s_qa, s_da, s_red);
  }
  return true;
}

// A workgroup's slice of a Q8_0 matrix: R rows of K values.  LPR lanes share
// a row, each lane owns BPL whole blocks (the decode GEMV's layout for K, so
// the per-row summation order is the same); RPP rows per pass of the 256
// threads.
// LPR0 > 0 sets the lanes per row (fewer passes and shorter lane reductions
// for tall slices).
template <int K, int R, int LPR0 = 0>
struct Slice {
  static constexpr int NB = K / 32;
  static constexpr int LPR = LPR0 > 0 ? LPR0 : (NB % 64 == 0) ? 64 : (NB % 32 == 0) ? 32 : (NB % 16 == 0) ? 16 : 8;
  static constexpr int BPL = NB / LPR;
  static constexpr int RPP = NT / LPR;
  static constexpr int PASSES = (R + RPP - 1) / RPP;
  static_assert(NB % LPR == 0, "block count");
  v4i w0[PASSES][BPL], w1[PASSES][BPL];
  uint16_t ws[PASSES][BPL];

  // row(lr) maps a local row < R to a matrix row; rows past R load row(0).
  // Passes [p0, p1) only (all by default).
  template <typename RowOf>
  QDEV void load(const int8_t* __restrict__ qs, const uint16_t* __restrict__ sc, RowOf row, int p0 = 0,
                 int p1 = PASSES) {
    const int li = threadIdx.x % LPR;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      if (ps < p0 || ps >= p1) continue;
      const int lr = ps * RPP + threadIdx.x / LPR;
      const int64_t r = row(lr < R ? lr : 0);
      const QGLOBAL int8_t* wr = as_global(qs) + r * (int64_t)K;
      const QGLOBAL uint16_t* sr = as_global(sc) + r * (int64_t)NB;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        const int b = li + j * LPR;
        w0[ps][j] = ld_global<v4i>(wr + b * 32);
        w1[ps][j] = ld_global<v4i>(wr + b * 32 + 16);
        ws[ps][j] = sr[b];
      }
    }
  }

  // emit(lr, acc) runs on the last lane of each row with the row's f64 sum
  template <typename Emit>
  QDEV void compute(const int8_t* s_qa, const float* s_da, Emit emit) const {
    const int li = threadIdx.x % LPR;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < BPL; ++j) {
        const int b = li + j * LPR;
        const v4i a0 = *reinterpret_cast<const v4i*>(s_qa + b * 32);
        const v4i a1 = *reinterpret_cast<const v4i*>(s_qa + b * 32 + 16);
        const int S = dot32_i8(w0[ps][j], w1[ps][j], a0, a1);
        acc += (double)S * (double)(f16_bits_to_f32(ws[ps][j]) * s_da[b]);
      }
      acc = group_sum_d<LPR>(acc);
      const int lr = ps * RPP + threadIdx.x / LPR;
      if (li == LPR - 1 && lr < R) emit(lr, acc);
    }
  }
};

// KV rows of one tile in registers (16-byte loads, same count whatever the tile)
template <int HD, bool BF16>
struct KvTile {
  static constexpr int PER = BF16 ? 8 : 4;
  static constexpr int LOADS = (TJ * HD / PER + NT - 1) / NT;
  v4i x[LOADS];
  QDEV void load(const void* kv, int64_t base, int row0, int nrow) {
    constexpr int ESZ = BF16 ? 2 : 4;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = min((threadIdx.x + i * NT) * PER, TJ * HD - PER);
      const int r = min(e / HD, nrow - 1);
      const int64_t off = (int64_t)(row0 + r) * HD + (e % HD);
      x[i] = *reinterpret_cast<const v4i*>(static_cast<const uint8_t*>(kv) + (base + off) * ESZ);
    }
  }
  QDEV void store(float (*s_t)[HD + 4]) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (threadIdx.x + i * NT) * PER;
      if (e >= TJ * HD) continue;
      const int r = e / HD, d = e % HD;
      if (BF16) {
        float4 lo, hi;
        lo.x = __uint_as_float((uint32_t)x[i][0] << 16), lo.y = __uint_as_float((uint32_t)x[i][0] & 0xFFFF0000u);
        lo.z = __uint_as_float((uint32_t)x[i][1] << 16), lo.w = __uint_as_float((uint32_t)x[i][1] & 0xFFFF0000u);
        hi.x = __uint_as_float((uint32_t)x[i][2] << 16), hi.y = __uint_as_float((uint32_t)x[i][2] & 0xFFFF0000u);
        hi.z = __uint_as_float((uint32_t)x[i][3] << 16), hi.w = __uint_as_float((uint32_t)x[i][3] & 0xFFFF0000u);
        *reinterpret_cast<float4*>(&s_t[r][d]) = lo;
        *reinterpret_cast<float4*>(&s_t[r][d + 4]) = hi;
      } else {
        *reinterpret_cast<v4i*>(&s_t[r][d]) = x[i];
      }
    }
  }
};

// Register pins: one empty asm statement that takes every value of an array
// of LDS loads as an operand, so the compiler issues all of the loads before
// the first use and waits for them once (left alone, it interleaves each load
// with its use and waits after every one).
typedef float v4f __attribute__((ext_vector_type(4)));
QDEV void pin(v4f (&v)[4]) { asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])); }
QDEV void pin(v4f (&v)[8]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
QDEV void pin(double (&p)[8], float (&v)[8]) {
  asm volatile(""
               : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]), "+v"(p[7]),
                 "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}

struct ArgBest {
  float v;
  int i;
};
QDEV ArgBest better(ArgBest a, ArgBest b) {  // larger value; ties -> lower index
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

// H hidden, QW = heads * HD, F FFN width, S attention splits per KV head,
// MAXR rows per split at most.
template <int H, int QW, int F, int HD, int G, bool KVBF16, int S, int MAXR>
__global__ void __launch_bounds__(NT) k_decode_persistent(PersistArgs a) {
  constexpr int NKV = QW / (HD * G);
  constexpr int KVW = NKV * HD;
  constexpr int NQKV = QW + 2 * KVW;
  constexpr int NWG = kPersistWorkgroups;
  constexpr int RA = NQKV / NWG;  // QKV rows per workgroup
  constexpr int RC = H / NWG;     // hidden rows per workgroup (o_proj, down, embedding)
  constexpr int NUB = F / 32;     // FFN blocks: workgroup u < NUB owns FFN outputs 32u .. 32u+31
  static_assert(RA * NWG == NQKV && RC * NWG == H && NUB * 32 == F && NUB <= NWG,
                "shape does not split over the grid");
  static_assert(NKV * S <= NWG, "attention units exceed the grid");
  static_assert(NWG == NT, "one argmax key per thread");
  constexpr int XMAX = (H > QW ? (H > F ? H : F) : (QW > F ? QW : F));
  // attention maps (as the decode attention kernel)
  constexpr int NP = (G == 1) ? 8 : 4;
  constexpr int DPP = HD / NP;
  constexpr int RPT = TJ * G * NP / NT;
  constexpr int RG = TJ / RPT;
  static_assert(RPT >= 1 && RPT * NT == TJ * G * NP, "score map");
  constexpr int DPT = (G * HD / NT) > 0 ? G * HD / NT : 1;
  constexpr int OUT_T = G * HD / DPT;
  constexpr int TPH = HD / DPT;

  __shared__ __align__(16) float s_x[XMAX];
  __shared__ __align__(16) int8_t s_qa[XMAX];
  __shared__ float s_da[XMAX / 32];
  __shared__ double s_red[kWavesP];
  __shared__ float s_xkeep[RC];   // this workgroup's rows of x entering o_proj
  __shared__ float s_xckeep[RC];  // ... and entering the down projection
  __shared__ float s_gu[96];  // gate and up sums of an FFN block, then its SwiGLU values
  __shared__ float s_qf[G][HD];
  __shared__ float s_knew[HD];
  __shared__ float s_vnew[HD];
  __shared__ __align__(16) float s_t[TJ][HD + 4];
  __shared__ __align__(16) float s_tv[TJ][HD + 4];  // V tile of a one-tile split
  __shared__ double s_s[G][MAXR];
  __shared__ double s_m[G], s_l[G];
  // the combine: split s < NCB of KV head g also combines Q8_0 block s of
  // that head group's G * HD outputs (CPW = 32 of them), from every split's
  // (m, l) of the block's query head and its slice of o (WPS words of 32-bit
  // halves per split)
  constexpr int CPW = 32;
  constexpr int NCB = G * HD / CPW;  // combined blocks per KV head
  constexpr int WPS = 4 + 2 * CPW;
  constexpr int NOB = QW / 32;       // Q8_0 blocks of the attention output
  static_assert(NCB * CPW == G * HD && HD % CPW == 0 && NCB <= S && S <= kWave && NOB % 2 == 0, "combine map");
  __shared__ unsigned s_pw[S * WPS];
  __shared__ float s_att[CPW];
  __shared__ ArgBest s_best[kWavesP];
  __shared__ unsigned s_keys[2 * NWG];  // every workgroup's argmax key of the step (low, high halves)
  __shared__ u64 s_kmax[kWavesP];

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int seq = a.seq;
  const int p0 = a.len[seq];  // the first step appends row p0; step st appends row p0 + st
  const float eps = a.eps;

  // a failed earlier step leaves the error word set: do nothing
  if (ld_err(a.err) != 0) {
    if (b == 0 && tid == 0) a.argmax[0] = -1;
    return;
  }

  // attention unit of this workgroup; its rows [j0, j1) of the step's context
  const bool attn_unit = b < NKV * S;
  const int ag = b / S, asplit = b % S;
  int p, ctx, j0, j1, nt, cache_end;
  bool has_new;
  int next_tok = 0;  // the token the previous step chose (every workgroup forms it)
  unsigned T0;  // epoch of the step's layer 0
  const int64_t cap = a.seq_cap[seq];
  const int64_t head_elems = cap * HD;

  // Weight slices and KV tiles.  The QKV slice of the next layer is requested
  // during the down projection, ahead of its wait: a wait's loads complete, in order, after
  // everything issued before them, and that wait is long enough for the slice
  // to stream in, so the QKV phase finds it in registers instead of starting
  // its fetch after its own wait.  The gate/up slice (64 KB per workgroup,
  // the largest) is split: its first pass is requested with the o_proj
  // slice, ahead of that wait, its second at its own phase.  The other
  // slices are requested just before their own phase's wait, and the KV
  // tiles once the QKV phase has its input (ahead of that phase's compute,
  // not of its wait).  (Measured: issuing the whole gate/up slice, or the
  // o_proj or down slices, a phase early was slower: those windows already
  // carry the phase's own traffic, and the wait is then held until the
  // early slice has arrived.)
  using SA = Slice<H, RA, (H / 32 >= 32 && RA >= 16 ? 16 : 0)>;
  using SC = Slice<QW, RC>;
  using SD = Slice<H, 64, (H / 32 >= 32 ? 8 : 0)>;
  using SE = Slice<F, RC>;
  SA wA;
  SC wC;
  SD wD;
  SE wE;
  KvTile<HD, KVBF16> tA, tB;
  auto kbase_of = [&](int l) { return a.seq_base[seq] + ((int64_t)l * 2 * NKV + ag) * head_elems; };
  // stream element i < nt is K tile i, nt <= i < 2 nt is V tile i - nt
  auto stream_load = [&](KvTile<HD, KVBF16>& r, int i, int64_t kb) {
    const bool isv = i >= nt;
    const int t0 = j0 + (isv ? i - nt : i) * TJ;
    const bool live = t0 < cache_end;
    r.load(a.kv, isv ? kb + (int64_t)NKV * head_elems : kb, live ? t0 : 0, live ? min(TJ, cache_end - t0) : 1);
  };
  // layer l's QKV slice
  auto prefetch_layer = [&](int l) {
    const PLayer P = a.layers[l];
    wA.load(P.qkv_qs, P.qkv_sc, [&](int lr) { return b * RA + lr; });
  };

  // Greedy steps: each step is the decode step of the previous step's token.
  // Every workgroup publishes its rows' best (logit, index) key as a tagged
  // word, reads all of them and forms the argmax itself, so the next step
  // starts without a further hand-off.
  for (int st = 0; st < a.nsteps; ++st) {
  p = p0 + st;
  ctx = p + 1;
  T0 = (a.pstep + (unsigned)st) * (unsigned)(a.L + 1) + 1u;
  {
    const int chunk = (ctx + S - 1) / S;
    j0 = min(ctx, asplit * chunk);
    j1 = min(ctx, j0 + chunk);
    nt = j0 < j1 ? (j1 - j0 + TJ - 1) / TJ : 0;
    cache_end = min(j1, p);
    has_new = j0 < j1 && j1 == ctx;
  }

  // ---- embedding rows of this workgroup (exact f16(d) * q) ------------------
  {
    // a device token cannot be checked by the host: clamp it into [0, V)
    const int tok = st == 0 ? min(max(a.token[0], 0), a.V - 1) : next_tok;
    if (tid < RC) {
      const int n = b * RC + tid;
      const float x = f16_bits_to_f32(a.emb_sc[(int64_t)tok * (H / 32) + n / 32]) * (float)a.emb_qs[(int64_t)tok * H + n];
      put_tagged(a.xa + n, x, T0);
      s_xkeep[tid] = x;
    }
  }
  prefetch_layer(0);

  for (int l = 0; l < a.L; ++l) {
    const unsigned T = T0 + (unsigned)l;
    const PLayer P = a.layers[l];
    const int64_t kbase = kbase_of(l);
    const int64_t vbase = kbase + (int64_t)NKV * head_elems;

    // ---- A: QKV projection --------------------------------------------------
    {
      NormW<H> nw;
      nw.load(P.attn_norm);
      if (!poll_quantize<H, true>(a.xa, T, s_x, &nw, eps, s_qa, s_da, s_red, a.err)) goto fail;
      if (attn_unit && nt > 0) {
        stream_load(tA, 0, kbase);
        stream_load(tB, 1, kbase);
      }
      wA.compute(s_qa, s_da, [&](int lr, double acc) { put_tagged(a.qkv + b * RA + lr, (float)acc, T); });
    }

    // ---- B: attention of KV head ag over rows [j0, j1) -------------------------
    if (attn_unit) {
      // this lane's rotation pair and norm weights, loaded before the wait
      // (waves < G rotate the query heads, the last wave the new key)
      static_assert(G < kWavesP, "one wave per query head and one for the key");
      constexpr int H2 = HD / 2;
      const int rl = lane < H2 ? lane : 0;
      const double rcos = as_global(a.rope_cos)[(int64_t)p * H2 + rl];
      const double rsin = as_global(a.rope_sin)[(int64_t)p * H2 + rl];
      const QGLOBAL float* nwp = as_global(wave < G ? P.q_norm : P.k_norm);
      const float nwlo = nwp[rl], nwhi = nwp[rl + H2];
      // a split of at most one tile keeps its K and V tiles in LDS, stored
      // while the query is awaited
      const bool one_tile = nt <= 1;
      if (nt == 1 && j0 < cache_end) {
        tA.store(s_t);
        tB.store(s_tv);
      }
      {
        unsigned* qf = reinterpret_cast<unsigned*>(&s_qf[0][0]);
        unsigned* kn = reinterpret_cast<unsigned*>(s_knew);
        unsigned* vn = reinterpret_cast<unsigned*>(s_vnew);
        auto off = [&](int j) {  // word offset in qkv of pair j (q, then k, then v of head group ag)
          const int i = 2 * j;
          return i < G * HD ? ag * G * HD + i
                            : i < G * HD + HD ? QW + ag * HD + (i - G * HD) : QW + KVW + ag * HD + (i - G * HD - HD);
        };
        auto dst = [&](int i) { return i < G * HD ? qf + i : i < G * HD + HD ? kn + (i - G * HD) : vn + (i - G * HD - HD); };
        if (!poll_pairs<(G * HD + 2 * HD) / 2>(a.qkv, NQKV, off, dst, T, a.err)) goto fail;
      }
      if (wave < G) norm_rope_wave_reg<HD>(s_qf[wave], nwlo, nwhi, rcos, rsin, eps);
      if (has_new && wave == kWavesP - 1) norm_rope_wave_reg<HD>(s_knew, nwlo, nwhi, rcos, rsin, eps);
      if (one_tile) {
        // the new row: the key wave appends k/v to the cache and to the tiles
        if (has_new && wave == kWavesP - 1) {
          for (int d = lane; d < HD; d += kWave) {
            const int64_t ki = kbase + (int64_t)p * HD + d, vi = vbase + (int64_t)p * HD + d;
            float kf = s_knew[d], vf = s_vnew[d];
            if (KVBF16) {
              const uint16_t kb = f32_to_bf16_bits(kf), vb = f32_to_bf16_bits(vf);
              st_coherent(reinterpret_cast<uint16_t*>(a.kv) + ki, kb);
              st_coherent(reinterpret_cast<uint16_t*>(a.kv) + vi, vb);
              kf = bf16_bits_to_f32(kb), vf = bf16_bits_to_f32(vb);
            } else {
              st_coherent(reinterpret_cast<float*>(a.kv) + ki, kf);
              st_coherent(reinterpret_cast<float*>(a.kv) + vi, vf);
            }
            s_t[p - j0][d] = kf;
            s_tv[p - j0][d] = vf;
          }
        }
      }
      if (tid < G) s_m[tid] = -INFINITY, s_l[tid] = 0.0;
      __syncthreads();  // the rotated query (and the one-tile rows) in LDS
      const int sc_pt = tid % NP, sc_rg = (tid / NP) % RG, sc_h = tid / (NP * RG);
      double qreg[DPP];
      {
        v4f q4[DPP / 4];
#pragma unroll
        for (int i = 0; i < DPP / 4; ++i) q4[i] = *reinterpret_cast<const v4f*>(&s_qf[sc_h][4 * sc_pt + 4 * NP * i]);
        pin(q4);
#pragma unroll
        for (int i = 0; i < DPP / 4; ++i) {
          qreg[4 * i] = (double)q4[i].x, qreg[4 * i + 1] = (double)q4[i].y;
          qreg[4 * i + 2] = (double)q4[i].z, qreg[4 * i + 3] = (double)q4[i].w;
        }
      }
      const bool out_live = tid < OUT_T;
      const int o_h = out_live ? tid / TPH : 0, o_d = out_live ? (tid % TPH) * DPT : 0;
      double o[DPT];
#pragma unroll
      for (int i = 0; i < DPT; ++i) o[i] = 0.0;
      const double scale = a.scale;
      // scores of tile rows [0, nrow) starting at split row t0 - j0
      auto scores = [&](int t0, int nrow) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          const int r = sc_rg * RPT + j;
          const float* kr = &s_t[r][4 * sc_pt];
          v4f k4[DPP / 4];
#pragma unroll
          for (int d = 0; d < DPP; d += 4) k4[d / 4] = *reinterpret_cast<const v4f*>(kr + NP * d);
          pin(k4);
          double ax = 0.0, ay = 0.0, az = 0.0, aw = 0.0;  // four independent FMA chains
#pragma unroll
          for (int d = 0; d < DPP; d += 4) {
            ax += qreg[d] * (double)k4[d / 4].x;
            ay += qreg[d + 1] * (double)k4[d / 4].y;
            az += qreg[d + 2] * (double)k4[d / 4].z;
            aw += qreg[d + 3] * (double)k4[d / 4].w;
          }
          double acc = (ax + ay) + (az + aw);
          acc = group_sum_d<NP>(acc);
          if (sc_pt == NP - 1 && r < nrow) s_s[sc_h][t0 - j0 + r] = acc * scale;
        }
      };
      // one f64 softmax over the split's n scores of each query head
      auto softmax = [&]() {
        const int n = j1 - j0;
        for (int h = wave; h < G; h += kWavesP) {
          double m = -INFINITY;
          for (int r = lane; r < n; r += kWave) m = fmax(m, s_s[h][r]);
          m = wave_max_all_d(m);
          double lsum = 0.0;
          for (int r = lane; r < n; r += kWave) {
            const double e = exp(s_s[h][r] - m);
            s_s[h][r] = e;
            lsum += e;
          }
          lsum = wave_total_d(lsum);
          if (lane == 0) s_m[h] = m, s_l[h] = lsum;
        }
      };
      auto pv = [&](const float (*vt)[HD + 4], int t0, int nrow) {
        if (!out_live) return;
        const double* pr = &s_s[o_h][t0 - j0];
        double oa[4][DPT];  // rows r % 4 in independent FMA chains
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i2 = 0; i2 < DPT; ++i2) oa[c][i2] = 0.0;
        int r = 0;
        if constexpr (DPT == 1) {  // eight rows per batch of LDS loads (two groups of four, in order)
          for (; r + 8 <= nrow; r += 8) {
            double pp[8];
            float vv[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) pp[c] = pr[r + c], vv[c] = vt[r + c][o_d];
            pin(pp, vv);
#pragma unroll
            for (int c = 0; c < 8; ++c) oa[c % 4][0] += pp[c] * (double)vv[c];
          }
        }
        for (; r + 4 <= nrow; r += 4) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i2 = 0; i2 < DPT; ++i2) oa[c][i2] += pr[r + c] * (double)vt[r + c][o_d + i2];
        }
        for (; r < nrow; ++r)
#pragma unroll
          for (int i2 = 0; i2 < DPT; ++i2) oa[0][i2] += pr[r] * (double)vt[r][o_d + i2];
#pragma unroll
        for (int i2 = 0; i2 < DPT; ++i2) o[i2] += (oa[0][i2] + oa[1][i2]) + (oa[2][i2] + oa[3][i2]);
      };
      if (one_tile) {
        if (nt == 1) {
          scores(j0, j1 - j0);
          __syncthreads();
          softmax();
          __syncthreads();
          pv(s_tv, j0, j1 - j0);
        }
      } else {
        if (has_new) {
          for (int d = tid; d < HD; d += NT) {
            const int64_t ki = kbase + (int64_t)p * HD + d, vi = vbase + (int64_t)p * HD + d;
            if (KVBF16) {
              const uint16_t kb = f32_to_bf16_bits(s_knew[d]), vb = f32_to_bf16_bits(s_vnew[d]);
              st_coherent(reinterpret_cast<uint16_t*>(a.kv) + ki, kb);
              st_coherent(reinterpret_cast<uint16_t*>(a.kv) + vi, vb);
              s_knew[d] = bf16_bits_to_f32(kb);
              s_vnew[d] = bf16_bits_to_f32(vb);
            } else {
              st_coherent(reinterpret_cast<float*>(a.kv) + ki, s_knew[d]);
              st_coherent(reinterpret_cast<float*>(a.kv) + vi, s_vnew[d]);
            }
          }
        }
        // stream element i < nt is K tile i, nt <= i < 2 nt is V tile i - nt;
        // two tiles in flight
        auto process = [&](KvTile<HD, KVBF16>& tr, int i, bool prefetch) {
          const bool isv = i >= nt;
          const int t0 = j0 + (isv ? i - nt : i) * TJ;
          const int nrow = min(TJ, j1 - t0);
          __syncthreads();
          if (i == nt) {  // all scores written: softmax over the split, once
            softmax();
            __syncthreads();
          }
          if (t0 < cache_end) tr.store(s_t);
          if (prefetch) stream_load(tr, i + 2, kbase);
          if (t0 + nrow > p) {  // row p from this step's values (after the tile store)
            __syncthreads();
            const float* src = isv ? s_vnew : s_knew;
            for (int d = tid; d < HD; d += NT) s_t[p - t0][d] = src[d];
          }
          __syncthreads();
          if (!isv) scores(t0, nrow);
          else pv(s_t, t0, nrow);
        };
        int i = 0;
        for (; i + 2 < 2 * nt; i += 2) {
          process(tA, i, true);
          process(tB, i + 1, true);
        }
        process(tA, i, false);
        process(tB, i + 1, false);
      }
      __syncthreads();
      // partial (o, m, l) of this split as tagged words: no drain and no
      // counter, the words are their own flags
      constexpr int PWORDS = (HD + 2) * 2;  // words per (split, query head)
      u64* part = a.part + ((int64_t)ag * S + asplit) * G * PWORDS;
      if (out_live) {
#pragma unroll
        for (int i2 = 0; i2 < DPT; ++i2) put_tagged_d(part, G * PWORDS, o_h * PWORDS + 2 * (o_d + i2), o[i2], T);
      }
      if (tid < G) {
        put_tagged_d(part, G * PWORDS, tid * PWORDS + 2 * HD, s_m[tid], T);
        put_tagged_d(part, G * PWORDS, tid * PWORDS + 2 * (HD + 1), s_l[tid], T);
      }
      // ---- the combine of Q8_0 block asplit of the head group's outputs
      // (query head ch, dims cd0 ..) over the S splits:
      // O = sum_s w_s o_s / sum_s w_s l_s, w_s = exp(m_s - max m), each sum
      // taken in split order.  The block leaves quantised: o_proj's prologue
      // arithmetic, moved to the producer.
      if (asplit < NCB) {
        const int ch = (asplit * CPW) / HD, cd0 = (asplit * CPW) % HD;
        {
          const int pb = ag * S * G * PWORDS + ch * PWORDS;  // word offset of (split 0, head ch)
          auto off = [&](int j) {
            const int sp = (2 * j) / WPS, k = (2 * j) % WPS;
            return pb + sp * G * PWORDS + (k < 4 ? 2 * HD + k : 2 * cd0 + (k - 4));
          };
          auto dst = [&](int i) { return s_pw + i; };
          if (!poll_pairs<S * WPS / 2>(a.part, NKV * S * G * PWORDS, off, dst, T, a.err)) goto fail;
        }
        auto pw_d = [&](int sp, int k) {  // the f64 at words k, k + 1 of split sp
          return __hiloint2double((int)s_pw[sp * WPS + k + 1], (int)s_pw[sp * WPS + k]);
        };
        {  // thread (kk, sp) takes split sp's terms of outputs kk, kk + NT / S, ...
           // Every group of S lanes holds all splits, so it forms the weights
           // and L itself; the group sums are the same trees as a wavefront
           // sum over S live lanes.
          static_assert((S == 16 || S == 32) && CPW % (NT / S) == 0, "combine threads");
          const int sp = tid % S, kk = tid / S;
          const double ms = pw_d(sp, 0);
          const double M = group_max_all_d<S>(ms);
          const double wgt = ms != -INFINITY ? exp(ms - M) : 0.0;
          // all sums first, then the divisions, then one guarded store, so
          // the trees and the divisions of the outputs overlap
          constexpr int KPT = CPW / (NT / S);  // outputs per thread
          double v[KPT];
#pragma unroll
          for (int i = 0; i < KPT; ++i) v[i] = wgt * pw_d(sp, 4 + 2 * (kk + i * (NT / S)));
          const double L = group_sum_d<S>(wgt * pw_d(sp, 2));
#pragma unroll
          for (int i = 0; i < KPT; ++i) v[i] = group_sum_d<S>(v[i]);
          float o[KPT];
#pragma unroll
          for (int i = 0; i < KPT; ++i) o[i] = (float)(v[i] / L);
          if (sp == S - 1) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) s_att[kk + i * (NT / S)] = o[i];
          }
        }
        __syncthreads();
        if (tid < 8) {  // one 8-lane group: lane t quantises outputs 4t .. 4t+3
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = s_att[4 * tid + i];
          float d;
          const int packed = quant4_group8(v, &d);
          put_block(a.att + (ag * NCB + asplit) * kBlockWords, packed, f16_round(d), T);
        }
      }
    }

    // ---- C: o_proj + residual ----------------------------------------------------
    {
      wC.load(P.o_qs, P.o_sc, [&](int lr) { return b * RC + lr; });
      if (b < NUB) wD.load(P.gu_qs, P.gu_sc, [&](int lr) { return b * 64 + lr; }, 0, 1);
      // the attention output arrives quantised
      if (!poll_blocks<NOB>(a.att, T, s_qa, s_da, a.err)) goto fail;
      wC.compute(s_qa, s_da, [&](int lr, double acc) {
        const float xn = s_xkeep[lr] + (float)acc;
        put_tagged(a.xc + b * RC + lr, xn, T);
        s_xckeep[lr] = xn;
      });
    }

    // ---- D: gate/up + SwiGLU + the Q8_0 quantisation of h.  Workgroup u < F/32
    // owns FFN block u: gate rows 64u .. 64u+31 and up rows 64u+32 .. 64u+63 of
    // the interleaved matrix.  h leaves already quantised (the down
    // projection's prologue arithmetic) as one padded block (put_block).
    if (b < NUB) {
      wD.load(P.gu_qs, P.gu_sc, [&](int lr) { return b * 64 + lr; }, 1, SD::PASSES);
      NormW<H> nw;
      nw.load(P.ffn_norm);
      if (!poll_quantize<H, true>(a.xc, T, s_x, &nw, eps, s_qa, s_da, s_red, a.err)) goto fail;
      wD.compute(s_qa, s_da, [&](int lr, double acc) { s_gu[lr] = (float)acc; });
      __syncthreads();
      // the block's 32 SwiGLU values, one per lane (each is an f64 exp and
      // divide: spread over 32 lanes they cost one such chain, not four)
      if (tid < 32) s_gu[64 + tid] = swiglu_f64(s_gu[tid], s_gu[32 + tid]);
      __syncthreads();
      if (tid < 8) {  // one 8-lane group: lane t quantises h[4t .. 4t+3]
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = s_gu[64 + 4 * tid + i];
        float d;
        const int packed = quant4_group8(v, &d);
        put_block(a.h + b * kBlockWords, packed, f16_round(d), T);
      }
    }

    // ---- E: down + residual (x of the next layer) ----------------------------------
    {
      wE.load(P.dn_qs, P.dn_sc, [&](int lr) { return b * RC + lr; });
      if (l + 1 < a.L) prefetch_layer(l + 1);
      if (!poll_blocks<NUB>(a.h, T, s_qa, s_da, a.err)) goto fail;
      wE.compute(s_qa, s_da, [&](int lr, double acc) {
        const float xn = s_xckeep[lr] + (float)acc;
        put_tagged(a.xa + b * RC + lr, xn, T + 1u);
        s_xkeep[lr] = xn;
      });
    }
  }

  // ---- lm_head over rows [b*RV, ...) + greedy argmax ---------------------------------
  {
    using LS = Slice<H, Slice<H, 1>::RPP>;  // one pass of RPP rows per buffer
    constexpr int RPP = LS::RPP;
    const int V = a.V;
    const int RV = (V + NWG - 1) / NWG;
    const int r0 = b * RV;
    const int rend = min(V, r0 + RV);
    const int npass = r0 < rend ? (rend - r0 + RPP - 1) / RPP : 0;
    auto rowof = [&](int ps) { return [&, ps](int lr) { return min(r0 + ps * RPP + lr, V - 1); }; };
    LS wa, wb, wc, wd;
    if (npass > 0) wa.load(a.emb_qs, a.emb_sc, rowof(0));
    if (npass > 1) wb.load(a.emb_qs, a.emb_sc, rowof(1));
    if (npass > 2) wc.load(a.emb_qs, a.emb_sc, rowof(2));
    if (npass > 3) wd.load(a.emb_qs, a.emb_sc, rowof(3));
    NormW<H> nw;
    nw.load(a.out_norm);
    if (!poll_quantize<H, true>(a.xa, T0 + (unsigned)a.L, s_x, &nw, eps, s_qa, s_da, s_red, a.err)) goto fail;
    ArgBest best{-INFINITY, 0x7FFFFFFF};
    auto run = [&](const LS& w, int ps) {
      w.compute(s_qa, s_da, [&](int lr, double acc) {
        const int row = r0 + ps * RPP + lr;
        if (row < rend) {
          const float y = (float)acc;
          if (a.logits && st + 1 == a.nsteps) a.logits[row] = y;
          best = better(best, ArgBest{y, row});
        }
      });
    };
    // four passes in flight; past the end a buffer re-reads the last pass
    // (a cache hit), so every wait covers a fixed number of loads
    int ps = 0;
    for (; ps + 4 < npass; ps += 4) {
      run(wa, ps);
      wa.load(a.emb_qs, a.emb_sc, rowof(ps + 4));
      run(wb, ps + 1);
      wb.load(a.emb_qs, a.emb_sc, rowof(min(ps + 5, npass - 1)));
      run(wc, ps + 2);
      wc.load(a.emb_qs, a.emb_sc, rowof(min(ps + 6, npass - 1)));
      run(wd, ps + 3);
      wd.load(a.emb_qs, a.emb_sc, rowof(min(ps + 7, npass - 1)));
    }
    if (ps < npass) run(wa, ps);
    if (ps + 1 < npass) run(wb, ps + 1);
    if (ps + 2 < npass) run(wc, ps + 2);
    if (ps + 3 < npass) run(wd, ps + 3);
    // (max, lowest index) of the workgroup -> one 64-bit key; the last
    // workgroup to arrive writes the token and advances the length
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      ArgBest c;
      c.v = __shfl_xor(best.v, o);
      c.i = __shfl_xor(best.i, o);
      best = better(best, c);
    }
    if (lane == 0) s_best[wave] = best;
    // every wavefront's stores of this step (the new KV rows among them,
    // read by other workgroups in the next step) complete before the
    // workgroup publishes its key
    wait_memory();
    __syncthreads();
    // the key (order-preserving bits of the logit << 32 | ~index): the
    // largest key is the largest logit, ties going to the lowest index
    const unsigned Tk = T0 + (unsigned)(a.L + 1);
    if (tid == 0) {
      ArgBest bb = s_best[0];
      for (int i = 1; i < kWavesP; ++i) bb = better(bb, s_best[i]);
      const uint32_t u = __float_as_uint(bb.v + 0.0f);
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const u64 key = ((u64)ord << 32) | (0xFFFFFFFFu - (uint32_t)bb.i);
      put_tagged_d(a.keys, 2 * NWG, 2 * b, __longlong_as_double((long long)key), Tk);
    }
    // workgroup 0 reports the step; the others need the token only if a
    // step follows
    if (st + 1 < a.nsteps || b == 0) {
      if (!poll_pairs<NWG>(a.keys, 2 * NWG, [](int j) { return 2 * j; }, [&](int i) { return s_keys + i; }, Tk,
                           a.err))
        goto fail;
      u64 k = ((u64)s_keys[2 * tid + 1] << 32) | s_keys[2 * tid];
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const u64 c = __shfl_xor(k, o);
        k = c > k ? c : k;
      }
      if (lane == 0) s_kmax[wave] = k;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kWavesP; ++w) k = s_kmax[w] > k ? s_kmax[w] : k;
      next_tok = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
      if (b == 0 && tid == 0) {
        // every workgroup's key is there, so every workgroup finished the step
        if (a.tokens_out) a.tokens_out[st] = next_tok;
        if (st + 1 == a.nsteps) a.argmax[0] = next_tok;
        a.len[seq] = p + 1;
      }
    }
  }
  }  // greedy steps
  return;
fail:
  if (tid == 0) {
    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.argmax[0] = -1;
  }
}

}  // namespace

namespace q8k {

namespace {
template <int H, int QW, int F, int HD, int G, int S, int MAXR>
bool persist_try(const PersistShape& sh, bool kvbf16, const PersistArgs* a, hipStream_t s, hipError_t* err,
                 int* max_ctx) {
  if (sh.H != H || sh.QW != QW || sh.F != F || sh.HD != HD || sh.G != G) return false;
  if (max_ctx) *max_ctx = S * MAXR;
  if (!a) return true;
  // a cooperative launch is refused unless the whole grid can be resident
  // at once, which every hand-off between workgroups relies on
  PersistArgs arg = *a;
  void* params[] = {&arg};
  const void* fn = kvbf16 ? reinterpret_cast<const void*>(&k_decode_persistent<H, QW, F, HD, G, true, S, MAXR>)
                          : reinterpret_cast<const void*>(&k_decode_persistent<H, QW, F, HD, G, false, S, MAXR>);
  *err = hipLaunchCooperativeKernel(fn, dim3(kPersistWorkgroups), dim3(NT), params, 0, s);
  return true;
}

}  // namespace

// The shapes the persistent step is built for: Qwen3-0.6B and the tiny test
// model: every workgroup takes an attention split (32 per KV head for
// 0.6B, 16 for the tiny model), each of up to 512 rows.

int persist_max_ctx(const PersistShape& sh) {
  int mc = 0;
  if (persist_try<1024, 2048, 3072, 128, 2, 32, 512>(sh, false, nullptr, nullptr, nullptr, &mc)) return mc;
  if (persist_try<256, 256, 768, 64, 2, 16, 512>(sh, false, nullptr, nullptr, nullptr, &mc)) return mc;
  return 0;
}

int persist_occupancy(const PersistShape& sh, bool kvbf16) {
  int occ = 0;
  auto q = [&](auto kern) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, NT, 0) != hipSuccess) occ = 0;
  };
  if (sh.H == 1024 && sh.QW == 2048 && sh.F == 3072 && sh.HD == 128 && sh.G == 2) {
    if (kvbf16) q(k_decode_persistent<1024, 2048, 3072, 128, 2, true, 32, 512>);
    else q(k_decode_persistent<1024, 2048, 3072, 128, 2, false, 32, 512>);
  } else if (sh.H == 256 && sh.QW == 256 && sh.F == 768 && sh.HD == 64 && sh.G == 2) {
    if (kvbf16) q(k_decode_persistent<256, 256, 768, 64, 2, true, 16, 512>);
    else q(k_decode_persistent<256, 256, 768, 64, 2, false, 16, 512>);
  }
  return occ;
}

hipError_t decode_persistent(const PersistShape& sh, bool kvbf16, const PersistArgs& a, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (persist_try<1024, 2048, 3072, 128, 2, 32, 512>(sh, kvbf16, &a, s, &e, nullptr)) return e;
  if (persist_try<256, 256, 768, 64, 2, 16, 512>(sh, kvbf16, &a, s, &e, nullptr)) return e;
  return hipErrorInvalidValue;
}

}  // namespace q8k
