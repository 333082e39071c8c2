// Kernel launch interface between the C++ runtime and the gfx950 kernels.
// Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };

// KV cache element types.  KV_Q8_0: int8 codes at the element offsets (one
// byte each) and one f16 scale per 32 elements in a second plane (scale of
// element e at kvs[e / 32]); a (position, head) row is head_dim/32 blocks.
enum { KV_F32 = 0, KV_BF16 = 1, KV_Q8_0 = 2 };

// Arguments of the decode GEMV family (see k_gemv.hip).
struct GemvArgs {
  const float* src;  // activation rows f32 [grid_y][K] (row stride src_stride)
  int64_t src_stride;
  const float* norm_w;  // RMSNorm weight [K] (prologue with norm)
  float eps;
  const int8_t* qs;    // codes [N][K]
  const uint16_t* sc;  // f16 scales [N][K/32]
  int N;               // stacked rows (SWIGLU: 2 * hidden units)
  int K;
  int ntiles;          // set by the launcher
  float* out;          // STORE/RESIDUAL: [grid_y][N]; SWIGLU: [grid_y][N/2]
  int64_t out_stride;
  // ARGMAX epilogue (tied lm_head + two-pass argmax)
  float* logits;      // [grid_y][N] or null
  unsigned long long* best_key;  // [grid_y] running (max, lowest index) key, zero between launches
  unsigned* counter;  // [grid_y] zero between launches (the last workgroup resets it)
  int32_t* argmax;    // [grid_y] or null
  int32_t* len_ptr;   // KV lengths; the last workgroup adds len_add to len_ptr[seq]
  const int32_t* len_seq;  // [grid_y] sequence of each batch row (null: sequence 0)
  int32_t len_add;
};

// Decode attention over one layer's KV cache (see k_attn_decode.hip).
// Cache layout: sequence s occupies [num_layers][2 (K, V)][nkv][cap_s][hd]
// elements starting at element seq_base[s].
struct AttnDecodeArgs {
  const float* qkv;  // [nrows][qkv_stride] raw projections: q | k | v
  int64_t qkv_stride;
  const float* q_norm;  // [hd]
  const float* k_norm;  // [hd]
  float eps;
  const double* rope_cos;  // [max_pos][hd/2]
  const double* rope_sin;
  void* kv;                  // cache base
  uint16_t* kvs;             // KV_Q8_0: the scale plane
  const int64_t* seq_base;   // [max_seqs] element offset of each sequence
  const int32_t* seq_cap;    // [max_seqs] capacity (rows) of each sequence
  const int32_t* len;        // [max_seqs] KV lengths (position of the new token)
  const int32_t* row_seq;    // [nrows] sequence of each batch row (null: sequence 0)
  int layer;
  double* part;       // partials [nrows][nkv][nsplit_max][G][hd + 2]
  unsigned* counter;  // [nrows][nkv], zero between launches
  float* out;         // attention output [nrows][out_stride], head h at h*hd
  int64_t out_stride;
  // optional (null: off): the output rows quantised to Q8_0 block-major for
  // the small-M GEMM, codes q_out[(b * nrows + row) * 32 + j], scales
  // q_scale[b * nrows + row] (f16-rounded), exactly as k_rows_quant does
  int8_t* q_out;
  float* q_scale;
  int nkv, nsplit_max, min_rows;
  double scale;  // 1/sqrt(hd)
};

// Sampling pipeline (see k_sample.hip).
struct SampleArgs {
  float temperature;  // <= 0: greedy
  int top_k;          // 0: the exact nucleus (window grows up to the vocabulary)
  float top_p, min_p;
  float repeat_penalty, freq_penalty, presence_penalty;
  int repeat_last_n;
};

namespace q8k {

hipError_t encode_q8_0(const float* x, int64_t n, void* out, hipStream_t s);
hipError_t encode_bf16(const float* x, int64_t n, uint16_t* out, hipStream_t s);
// interleave_off < 0: plain stacking at dst_row0; >= 0: 32-row gate/up interleave
hipError_t repack_q8_0(const void* src, int64_t rows, int64_t k, int8_t* qs, uint16_t* sc, int64_t dst_row0,
                       int interleave_off, hipStream_t s);
hipError_t repack_bf16(const void* src, int64_t rows, int64_t k, uint16_t* dst, int64_t dst_row0, int interleave_off,
                       hipStream_t s);
hipError_t embed(const int32_t* tok, int T, int vocab, int H, const void* w, const uint16_t* sc, bool bf16, float* x,
                 hipStream_t s);
// src: the (sequence, layer) K or V block; srcs: its scales (KV_Q8_0)
hipError_t kv_export(const void* src, const uint16_t* srcs, int kvt, int nkv, int cap, int len, int hd, float* dst,
                     hipStream_t s);
// blocked: codes and scales block-major (qa[(b * T + t) * 32 + j], da[b * T + t]),
// the small-M GEMM's activation layout; else row-major ([T][K], [T][K/32]).
hipError_t rows_quant(const float* x, int T, int K, const float* norm_w, float eps, int8_t* qa, float* da,
                      uint16_t* da_bits, hipStream_t s, bool blocked = false);

bool gemv_supported_k(int K);
int gemv_argmax_grid(int N, int K);
hipError_t gemv(GemvArgs a, bool norm, int epi, int grid_y, hipStream_t s);
hipError_t block_dots(const int8_t* qa, const int8_t* qs, int M, int K, int N, int32_t* S, hipStream_t s);

bool attn_decode_supported(int hd, int group);
int attn_decode_max_ctx(int group);  // longest context (cache capacity) the decode attention takes
hipError_t attn_decode(const AttnDecodeArgs& a, int hd, int group, int kvt, int nrows, hipStream_t s);

// Sampling: penalties in place (when any is active and a history is given),
// then one token per row.
size_t sample_work_bytes(int n, int V);
hipError_t sample(float* logits, int n, int V, const SampleArgs& a, const int32_t* hist, int hstride,
                  const int32_t* hlen, const float* uni, int32_t* out, void* work, hipStream_t s);

// Row argmax of f32 [T, V] (lowest index among equal maxima) -> out [T];
// key [T] and counter [T] are zero between launches (and left so).  With
// len: len[row_seq[r]] (row_seq null: len[r]) += len_add once row r is done.
hipError_t rows_argmax(const float* x, int T, int V, int32_t* out, unsigned long long* key, unsigned* counter,
                       hipStream_t s, int32_t* len = nullptr, const int32_t* row_seq = nullptr, int len_add = 0);
hipError_t set_len(int32_t* len, int seq, int value, hipStream_t s);

}  // namespace q8k

// Prefill Q8_0 GEMM (see k_gemm.hip): C[M, N] from qa int8 [M][K] with
// per-block scales da f32 [M][K/32] and the weight planes.
struct GemmArgs {
  const int8_t* qa;
  const float* da;
  const int8_t* qs;
  const uint16_t* sc;
  int M, N, K;
  float* out;  // STORE/RESIDUAL: [M][ldc]; SWIGLU: [M][ldc] hidden units (N/2 of them)
  int64_t ldc;
  // split-K scratch: when the tile grid is small, K is split over `splits`
  // slices whose f64 sums go to part[split][M][N] and are added in split
  // order by a second kernel (0 or 1: no split)
  double* part;
  size_t part_bytes;
  // small-M form: qa/da block-major (qa[(b * M + m) * 32 + j], da[b * M + m])
  int a_blocked;
};

// Prefill per-token head work (see k_attn_prefill.hip).
struct QkRopeArgs {
  const float* qkv;  // [T][qkv_stride]
  int64_t qkv_stride;
  const float* q_norm;
  const float* k_norm;
  float eps;
  const double* rope_cos;
  const double* rope_sin;
  float* q32;  // [T][nh][hd] normalised + roped queries
  void* kv;
  uint16_t* kvs;  // KV_Q8_0: the scale plane
  int64_t kbase;  // element offset of this (sequence, layer) K block; V follows at + nkv*cap*hd
  int cap;
  int pos0;       // position of token 0
  int nh, nkv;
  int quant_q;    // KV_Q8_0 single-token step: q32 gets the Q8_0 round trip of each head's query
};

struct AttnPrefillArgs {
  const float* q32;  // [T][nh][hd]
  const void* kv;
  const uint16_t* kvs;  // KV_Q8_0 scale plane
  int64_t kbase;
  int cap;
  int pos0;  // position of query token 0 (cache rows [0, pos0 + T) are valid)
  int T;
  int nh, nkv;
  double scale;  // 1/sqrt(hd)
  float* out;  // [T][nh*hd]
  // key split across workgroups (tps = 0: none): a query block's keys are cut
  // into runs of tps 64-key tiles, one workgroup each; every run leaves
  // (o, m, l) per (token, head) in part [nsplit][T][nh][hd + 2], merged by a
  // second kernel
  int tps;
  double* part;
  size_t part_bytes;
  int nz, nqb;  // set at launch: runs per block (1 unsplit), query blocks
};

// Linear with bf16 weights (see k_gemm_bf16.hip): C[M, N] = X . W^T.
struct GemmBf16Args {
  const float* x;  // [M][lda] f32 activations
  int64_t lda;
  const uint16_t* w;  // [N][K] bf16 bits
  int M, N, K;
  float* out;  // STORE/RESIDUAL: [M][ldc]; SWIGLU: [M][ldc] hidden units (N/2 of them)
  int64_t ldc;
  // ARGMAX epilogue (as GemvArgs, one key per row, one counter per 64/128-row tile)
  float* logits;  // [M][N] or null
  unsigned long long* best_key;
  unsigned* counter;
  int32_t* argmax;
  int32_t* len_ptr;
  const int32_t* len_seq;
  int32_t len_add;
  // split-K scratch (f64 planes [splits][M][N]) or null for one pass
  double* part;
  size_t part_bytes;
};

namespace q8k {
hipError_t gemm(const GemmArgs& a, int epi, hipStream_t s);
// out (STORE, RESIDUAL, SWIGLU epilogue) from `splits` f64 planes [splits][M][N]
// added in slice order and rounded once (see k_gemm.hip).
hipError_t gemm_reduce(const double* part, int splits, int M, int N, float* out, int64_t ldc, int epi, hipStream_t s);
// Small-M form (see k_gemm_skinny.hip): M <= kSkinnyMaxRows, K % 128 == 0;
// STORE, RESIDUAL, SWIGLU; no scratch.
constexpr int kSkinnyMaxRows = 64;
bool gemm_skinny_supported(int M, int K);
hipError_t gemm_skinny(const GemmArgs& a, int epi, hipStream_t s);

// Achievable-peak probes (see k_peak.hip).
hipError_t copy_peak(const void* src, void* dst, size_t bytes, hipStream_t s);
int read_peak_partials();
hipError_t read_peak(const void* src, size_t bytes, uint32_t* out, hipStream_t s);
double mfma_peak_ops(int workgroups, int iters);
hipError_t mfma_peak(int32_t* out, int workgroups, int iters, int fill, hipStream_t s);
hipError_t gemm_bf16(const GemmBf16Args& a, int epi, hipStream_t s);
hipError_t rows_norm(const float* x, int64_t ldx, int T, int K, const float* w, float eps, float* y, int64_t ldy,
                     hipStream_t s);
hipError_t qk_rope_append(const QkRopeArgs& a, int T, int hd, int kvt, hipStream_t s);
hipError_t attn_prefill(const AttnPrefillArgs& a, int hd, int group, int kvt, hipStream_t s);
bool attn_prefill_supported(int hd, int group);
}  // namespace q8k

#include "persist.h"
