// Host runtime behind the C ABI in include/qwen3_q8.h: validation, the
// workspace plan (every device byte comes from the caller's workspace), the
// weight repack, the KV-cache bookkeeping, the launch sequences of prefill and
// decode, and HIP-graph capture of the decode step.
//
// Forward pass order: Fucina course, "A transformer from scratch", sections
// 12.3-12.5; the KV cache contract (append at len on every layer, advance
// once, reject pos0 != len and overflow): same page, section 12.4.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/qwen3_q8.h"
#include "errors.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

}  // namespace

int q8rt::set_error(int code, const char* msg) { return fail(code, msg); }

namespace {

#define HIP_TRY(expr)                                                                                   \
  do {                                                                                                  \
    hipError_t e_ = (expr);                                                                             \
    if (e_ != hipSuccess) return fail(QWEN3_E_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// checked multiply of non-negative sizes
bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// Bump allocator over the workspace; with base == nullptr it only measures.
struct Carver {
  uint8_t* base = nullptr;
  size_t off = 0;
  bool overflow = false;
  void* take(size_t bytes) {
    off = align_up(off);
    void* p = base ? base + off : nullptr;
    if (bytes > SIZE_MAX - off) overflow = true;
    else off += bytes;
    return p;
  }
  template <typename T>
  T* arr(size_t n) {
    size_t b;
    if (!mul_ok(n, sizeof(T), &b)) {
      overflow = true;
      return nullptr;
    }
    return static_cast<T*>(take(b));
  }
};

struct QPlane {  // repacked Q8_0 matrix, or bf16 rows
  int8_t* qs = nullptr;
  uint16_t* sc = nullptr;
  uint16_t* bf = nullptr;
  int64_t rows = 0, k = 0;
};

struct Layer {
  QPlane qkv, o, gateup, down;
  float *attn_norm = nullptr, *q_norm = nullptr, *k_norm = nullptr, *ffn_norm = nullptr;
};

// Splits of the decode attention per (batch row, KV head): about 512
// workgroups per launch (two per CU at its register use; 1024 and 2048 were
// measured slower on the 64-stream step, whose 512 (row, KV head) pairs then
// take one split each and skip the partial round trip), at most 64 by that
// rule (each split also keeps at least 64 rows, so short caches get fewer),
// and never fewer than the longest cache needs (a split holds at most
// 4096 / group rows).  The kernel then rounds a split's range up to whole
// K/V tiles, which can only lower the count.
int decode_splits_needed(int max_cap, int group) { return (max_cap + 4096 / group - 1) / (4096 / group); }
int decode_nsplit_max(int nkv, int nrows, int needed) {
  const int units = nkv * nrows;
  int n = (512 + units - 1) / units;
  if (n > 64) n = 64;
  if (n < needed) n = needed;
  return n;
}

}  // namespace

struct qwen3_model {
  qwen3_config cfg{};
  std::vector<int32_t> cap;
  int R = 0;  // max_batch_tokens
  int nh = 0, nkv = 0, hd = 0, H = 0, F = 0, V = 0, L = 0, G = 0, qw = 0, kvw = 0, nqkv = 0, kmax = 0;
  bool wbf16 = false, kvbf16 = false;
  int kvt = KV_F32;  // KV_F32 / KV_BF16 / KV_Q8_0
  uint16_t* kvs = nullptr;  // KV_Q8_0 scale plane (scale of element e at kvs[e / 32])
  int max_cap = 0;
  // device
  std::vector<Layer> layers;
  QPlane emb;
  float* out_norm = nullptr;
  double *rope_cos = nullptr, *rope_sin = nullptr;
  void* kv = nullptr;
  int64_t* d_seq_base = nullptr;
  int32_t* d_seq_cap = nullptr;
  int32_t* d_len = nullptr;
  int32_t* d_row_seq = nullptr;  // batch rows -> sequences
  int32_t* d_seq_ids = nullptr;  // constant 0 .. max_seqs-1 (row map of single-sequence steps)
  int32_t* d_tok = nullptr;
  float *x = nullptr, *qkv = nullptr, *attn = nullptr, *h = nullptr;
  int8_t* qa = nullptr;
  float* da = nullptr;
  float* q32 = nullptr;
  float* xn = nullptr;  // normalised rows (bf16-weight models: the norm is not fused)
  double* attn_part = nullptr;
  double* gemm_part = nullptr;  // split-K planes of the prefill GEMM; key-split attention partials
  float* blogits = nullptr;     // [kSkinnyMaxRows][V] logits of a batched step called without a logits buffer
  size_t gemm_part_bytes = 0;
  unsigned* attn_cnt = nullptr;
  unsigned long long* am_key = nullptr;
  unsigned* am_cnt = nullptr;
  // one-launch decode step (shapes it is built for; see k_decode_persistent.hip)
  PersistShape psh{};
  bool persist_capable = false, persist = false;
  PLayer* d_players = nullptr;
  unsigned long long *p_xa = nullptr, *p_xc = nullptr, *p_qkv = nullptr, *p_att = nullptr, *p_h = nullptr;
  unsigned long long* p_part = nullptr;
  unsigned* p_err = nullptr;
  unsigned long long* p_keys = nullptr;  // the workgroups' argmax keys of a one-launch step
  unsigned pstep = 0;
  size_t bytes = 0;
  // host
  std::vector<int64_t> seq_base;
  std::vector<int32_t> h_len;
  hipStream_t cap_stream = nullptr;
  bool use_graphs = true;
  std::map<std::tuple<int, const void*, const void*, const void*>, hipGraphExec_t> graphs;
  // batched steps, keyed by (n, d_tokens, d_logits, d_argmax); the row -> sequence
  // map is uploaded to d_row_seq before each replay
  std::map<std::tuple<int, const void*, const void*, const void*>, hipGraphExec_t> bgraphs;
};

namespace {

// Tagged attention-partial words of the one-launch step: every workgroup of
// its grid is at most one split, each split holds G heads of (o[hd], m, l) as
// two words per f64.
size_t persist_part_words(int64_t G, int64_t hd) { return (size_t)kPersistWorkgroups * G * (hd + 2) * 2; }

// Split-K planes of the prefill GEMM (f64 sums of K slices): enough for eight
// slices of a 1024 x 1024 output.  The key-split runs of prefill attention
// use the same scratch (the two never overlap on the stream).
constexpr size_t kGemmPartBytes = (size_t)64 << 20;

int validate(const qwen3_config* c) {
  if (!c) return fail(QWEN3_E_INVALID_ARGUMENT, "config is null");
  if (c->vocab_size <= 0 || c->hidden_size <= 0 || c->intermediate_size <= 0 || c->num_layers <= 0 ||
      c->num_attention_heads <= 0 || c->num_key_value_heads <= 0 || c->head_dim <= 0)
    return fail(QWEN3_E_INVALID_CONFIG, "every config integer must be positive");
  if (c->num_attention_heads % c->num_key_value_heads)
    return fail(QWEN3_E_INVALID_CONFIG, "num_attention_heads must be a multiple of num_key_value_heads");
  if (c->head_dim % 2) return fail(QWEN3_E_INVALID_CONFIG, "head_dim must be even (RoPE pairs)");
  if (!(c->rms_norm_eps > 0.f) || !std::isfinite(c->rms_norm_eps))
    return fail(QWEN3_E_INVALID_CONFIG, "rms_norm_eps must be positive");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta))
    return fail(QWEN3_E_INVALID_CONFIG, "rope_theta must be > 1");
  if (c->weight_type != QWEN3_W_Q8_0 && c->weight_type != QWEN3_W_BF16)
    return fail(QWEN3_E_UNSUPPORTED_WEIGHT_TYPE, "unknown weight_type");
  if (c->kv_type != QWEN3_KV_F32 && c->kv_type != QWEN3_KV_BF16 && c->kv_type != QWEN3_KV_Q8_0)
    return fail(QWEN3_E_UNSUPPORTED_WEIGHT_TYPE, "unknown kv_type");
  if (c->kv_type == QWEN3_KV_Q8_0 && c->head_dim % 32 != 0)
    return fail(QWEN3_E_INVALID_CONFIG, "a q8_0 KV cache needs head_dim % 32 == 0");
  const int qw = c->num_attention_heads * c->head_dim;
  if (c->hidden_size % 128 || qw % 128 || c->intermediate_size % 128)
    return fail(QWEN3_E_INVALID_CONFIG, "hidden_size, heads*head_dim and intermediate_size must be multiples of 128");
  const int G = c->num_attention_heads / c->num_key_value_heads;
  if (!q8k::attn_decode_supported(c->head_dim, G) || !q8k::attn_prefill_supported(c->head_dim, G))
    return fail(QWEN3_E_INVALID_CONFIG, "head_dim must be 64 or 128 and heads/kv_heads one of 1, 2, 4, 8");
  if (c->weight_type == QWEN3_W_Q8_0 &&
      (!q8k::gemv_supported_k(c->hidden_size) || !q8k::gemv_supported_k(qw) ||
       !q8k::gemv_supported_k(c->intermediate_size)))
    return fail(QWEN3_E_INVALID_CONFIG,
                "hidden_size, heads*head_dim and intermediate_size must each be one of 256, 512, 768, "
                "1024, 2048, 3072, 4096, 6144, 8192, 12288");
  if (c->max_seqs <= 0) return fail(QWEN3_E_INVALID_CONFIG, "max_seqs must be >= 1");
  if (!c->h_seq_capacity) return fail(QWEN3_E_INVALID_ARGUMENT, "h_seq_capacity is null");
  for (int i = 0; i < c->max_seqs; ++i)
    if (c->h_seq_capacity[i] <= 0) return fail(QWEN3_E_INVALID_CONFIG, "every seq_capacity must be >= 1");
  if (c->max_batch_tokens < 0) return fail(QWEN3_E_INVALID_CONFIG, "max_batch_tokens must be >= 0");
  for (int i = 0; i < c->max_seqs; ++i)
    if (c->h_seq_capacity[i] > q8k::attn_decode_max_ctx(G))
      return fail(QWEN3_E_INVALID_CONFIG, "a seq_capacity exceeds the decode attention limit of " +
                                              std::to_string(q8k::attn_decode_max_ctx(G)) + " rows");
  return QWEN3_OK;
}

// Lays out (or measures, with base == nullptr) the workspace.
int plan(qwen3_model* m, uint8_t* base, size_t* total) {
  const qwen3_config& c = m->cfg;
  Carver cv;
  cv.base = base;
  const int64_t H = c.hidden_size, F = c.intermediate_size, V = c.vocab_size, hd = c.head_dim;
  const int64_t nh = c.num_attention_heads, nkv = c.num_key_value_heads;
  const int64_t qw = nh * hd, kvw = nkv * hd, nqkv = qw + 2 * kvw;
  const int64_t R = m->R;
  auto plane = [&](QPlane& p, int64_t rows, int64_t k) {
    p.rows = rows;
    p.k = k;
    size_t n;
    if (!mul_ok((size_t)rows, (size_t)k, &n)) cv.overflow = true;
    if (m->wbf16) {
      p.bf = cv.arr<uint16_t>(n);
    } else {
      p.qs = cv.arr<int8_t>(n);
      p.sc = cv.arr<uint16_t>(n / 32);
    }
  };
  m->layers.assign(c.num_layers, Layer{});
  plane(m->emb, V, H);
  m->out_norm = cv.arr<float>(H);
  for (auto& ly : m->layers) {
    plane(ly.qkv, nqkv, H);
    plane(ly.o, H, qw);
    plane(ly.gateup, 2 * F, H);
    plane(ly.down, H, F);
    ly.attn_norm = cv.arr<float>(H);
    ly.q_norm = cv.arr<float>(hd);
    ly.k_norm = cv.arr<float>(hd);
    ly.ffn_norm = cv.arr<float>(H);
  }
  // RoPE table
  m->rope_cos = cv.arr<double>((size_t)m->max_cap * (hd / 2));
  m->rope_sin = cv.arr<double>((size_t)m->max_cap * (hd / 2));
  // KV cache: sequence s holds [layers][K, V][nkv][cap_s][hd]
  const size_t esz = m->kvt == KV_F32 ? 4 : (m->kvt == KV_BF16 ? 2 : 1);
  m->seq_base.assign(c.max_seqs, 0);
  size_t kv_elems = 0;
  for (int s = 0; s < c.max_seqs; ++s) {
    m->seq_base[s] = (int64_t)kv_elems;
    size_t per;
    if (!mul_ok((size_t)c.num_layers * 2 * nkv * hd, (size_t)m->cap[s], &per)) cv.overflow = true;
    if (per > SIZE_MAX - kv_elems) cv.overflow = true;
    else kv_elems += per;
  }
  size_t kv_bytes;
  if (!mul_ok(kv_elems, esz, &kv_bytes)) cv.overflow = true;
  m->kv = cv.take(kv_bytes);
  if (m->kvt == KV_Q8_0) m->kvs = cv.arr<uint16_t>(kv_elems / 32);
  m->d_seq_base = cv.arr<int64_t>(c.max_seqs);
  m->d_seq_cap = cv.arr<int32_t>(c.max_seqs);
  m->d_len = cv.arr<int32_t>(c.max_seqs);
  m->d_row_seq = cv.arr<int32_t>(R);
  m->d_seq_ids = cv.arr<int32_t>(c.max_seqs);
  m->d_tok = cv.arr<int32_t>(R);
  // activations (rows = R)
  m->x = cv.arr<float>(R * H);
  m->qkv = cv.arr<float>(R * nqkv);
  m->attn = cv.arr<float>(R * qw);
  m->h = cv.arr<float>(R * F);
  m->qa = cv.arr<int8_t>(R * m->kmax);
  m->da = cv.arr<float>(R * (m->kmax / 32));
  m->q32 = cv.arr<float>(R * qw);
  if (m->wbf16) m->xn = cv.arr<float>(R * H);
  // decode attention partials: rows * nkv * nsplit_max <= max(1024 + R * nkv, R * nkv * needed)
  const int64_t G = nh / nkv;
  const int64_t needed = decode_splits_needed(m->max_cap, (int)G);
  const int64_t slots = std::max<int64_t>(1024 + R * nkv, R * nkv * needed);
  m->attn_part = cv.arr<double>((size_t)slots * G * (hd + 2));
  m->gemm_part_bytes = kGemmPartBytes;
  m->gemm_part = cv.arr<double>(kGemmPartBytes / 8);
  if (!m->wbf16) m->blogits = cv.arr<float>((size_t)std::min<int64_t>(R, q8k::kSkinnyMaxRows) * V);
  m->attn_cnt = cv.arr<unsigned>(R * nkv);
  m->am_key = cv.arr<unsigned long long>(R);
  m->am_cnt = cv.arr<unsigned>(R);
  if (m->persist_capable) {
    m->d_players = cv.arr<PLayer>(c.num_layers);
    m->p_xa = cv.arr<unsigned long long>(H);
    m->p_xc = cv.arr<unsigned long long>(H);
    m->p_qkv = cv.arr<unsigned long long>(nqkv);
    m->p_att = cv.arr<unsigned long long>(qw / 32 * 16);  // Q8_0 blocks of 16 words (codes, scale, padding)
    m->p_h = cv.arr<unsigned long long>(F / 32 * 16);  // Q8_0 blocks of 16 words
    m->p_part = cv.arr<unsigned long long>(persist_part_words(G, hd));
    m->p_err = cv.arr<unsigned>(1);
    m->p_keys = cv.arr<unsigned long long>(2 * kPersistWorkgroups);
  }
  if (cv.overflow) return fail(QWEN3_E_INVALID_WEIGHT_SHAPE, "workspace size overflows");
  *total = align_up(cv.off);
  return QWEN3_OK;
}

int fill_model_shape(qwen3_model* m, const qwen3_config* cfg) {
  m->cfg = *cfg;
  m->cap.assign(cfg->h_seq_capacity, cfg->h_seq_capacity + cfg->max_seqs);
  m->cfg.h_seq_capacity = nullptr;
  m->R = cfg->max_batch_tokens > 0 ? cfg->max_batch_tokens : 1024;
  m->nh = cfg->num_attention_heads;
  m->nkv = cfg->num_key_value_heads;
  m->hd = cfg->head_dim;
  m->H = cfg->hidden_size;
  m->F = cfg->intermediate_size;
  m->V = cfg->vocab_size;
  m->L = cfg->num_layers;
  m->G = m->nh / m->nkv;
  m->qw = m->nh * m->hd;
  m->kvw = m->nkv * m->hd;
  m->nqkv = m->qw + 2 * m->kvw;
  m->kmax = std::max(m->H, std::max(m->qw, m->F));
  m->wbf16 = cfg->weight_type == QWEN3_W_BF16;
  m->kvbf16 = cfg->kv_type == QWEN3_KV_BF16;
  m->kvt = cfg->kv_type == QWEN3_KV_BF16 ? KV_BF16 : (cfg->kv_type == QWEN3_KV_Q8_0 ? KV_Q8_0 : KV_F32);
  m->max_cap = 0;
  for (int c : m->cap) m->max_cap = std::max(m->max_cap, c);
  m->psh = PersistShape{m->H, m->qw, m->F, m->hd, m->G};
  m->persist_capable = !m->wbf16 && m->kvt != KV_Q8_0 && q8k::persist_max_ctx(m->psh) > 0;
  return QWEN3_OK;
}

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

int repack(const void* src, QPlane& p, int64_t rows, int64_t row0, int inter, hipStream_t s) {
  if (!src) return fail(QWEN3_E_INVALID_ARGUMENT, "a weight pointer is null");
  if (p.bf)
    HIP_TRY(q8k::repack_bf16(src, rows, p.k, p.bf, row0, inter, s));
  else
    HIP_TRY(q8k::repack_q8_0(src, rows, p.k, p.qs, p.sc, row0, inter, s));
  return QWEN3_OK;
}

const void* plane_rows(const QPlane& p) { return p.bf ? (const void*)p.bf : (const void*)p.qs; }

GemmBf16Args bf16_args(const QPlane& p, const float* x, int64_t lda, int M, float* out, int64_t ldc) {
  GemmBf16Args g{};
  g.x = x;
  g.lda = lda;
  g.w = p.bf;
  g.M = M;
  g.N = (int)p.rows;
  g.K = (int)p.k;
  g.out = out;
  g.ldc = ldc;
  return g;
}

// ... with the model's scratch, for split-K on grids under two workgroups per CU
GemmBf16Args bf16_args_m(const qwen3_model* m, const QPlane& p, const float* x, int64_t lda, int M, float* out,
                         int64_t ldc) {
  GemmBf16Args g = bf16_args(p, x, lda, M, out, ldc);
  g.part = m->gemm_part;
  g.part_bytes = m->gemm_part_bytes;
  return g;
}

int copy_f32(float* dst, const void* src, int64_t n, hipStream_t s) {
  if (!src) return fail(QWEN3_E_INVALID_ARGUMENT, "a norm weight pointer is null");
  HIP_TRY(hipMemcpyAsync(dst, src, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
  return QWEN3_OK;
}

#define TRY(expr)           \
  do {                      \
    int r_ = (expr);        \
    if (r_ != QWEN3_OK) return r_; \
  } while (0)

// ---- launch sequences -----------------------------------------------------------------

GemvArgs gemv_args(const QPlane& p, const float* src, int64_t src_stride, const float* norm_w, float eps,
                   float* out, int64_t out_stride) {
  GemvArgs a{};
  a.src = src;
  a.src_stride = src_stride;
  a.norm_w = norm_w;
  a.eps = eps;
  a.qs = p.qs;
  a.sc = p.sc;
  a.N = (int)p.rows;
  a.K = (int)p.k;
  a.out = out;
  a.out_stride = out_stride;
  return a;
}

AttnDecodeArgs attn_args(const qwen3_model* m, const int32_t* d_row_seq, int nrows) {
  AttnDecodeArgs at{};
  at.qkv = m->qkv;
  at.qkv_stride = m->nqkv;
  at.eps = m->cfg.rms_norm_eps;
  at.rope_cos = m->rope_cos;
  at.rope_sin = m->rope_sin;
  at.kv = m->kv;
  at.kvs = m->kvs;
  at.seq_base = m->d_seq_base;
  at.seq_cap = m->d_seq_cap;
  at.len = m->d_len;
  at.row_seq = d_row_seq;
  at.part = m->attn_part;
  at.counter = m->attn_cnt;
  at.out = m->attn;
  at.out_stride = m->qw;
  at.nkv = m->nkv;
  at.nsplit_max = decode_nsplit_max(m->nkv, nrows, decode_splits_needed(m->max_cap, m->G));
  at.min_rows = 64;
  at.scale = 1.0 / std::sqrt((double)m->hd);
  return at;
}

// Batched decode steps of at least this many rows take the small-M GEMM
// (measured on the 0.6B shape at KV length 512: from 16 rows on it beats
// the per-row GEMV, which re-reads the weights for every row).
constexpr int kSkinnyMinBatch = 16;

// Q8_0 weights and rows the small-M GEMM takes (every K of the model a
// multiple of 128).
bool skinny_rows(const qwen3_model* m, int rows) {
  return !m->wbf16 && rows <= q8k::kSkinnyMaxRows && q8k::gemm_skinny_supported(rows, m->H) &&
         q8k::gemm_skinny_supported(rows, m->qw) && q8k::gemm_skinny_supported(rows, m->F);
}

// A batched decode step of nrows rows runs its projections on the small-M GEMM.
bool batched_small_m(const qwen3_model* m, int nrows) { return nrows >= kSkinnyMinBatch && skinny_rows(m, nrows); }

// Kernels of one decode step.  kind: 0 QKV GEMV, 1 attention, 2 o_proj,
// 3 gate/up SwiGLU, 4 down, 5 lm_head + argmax (len_add advances lengths).
int launch_decode_kernel(qwen3_model* m, int kind, int l, int nrows, const int32_t* d_row_seq, float* d_logits,
                         int32_t* d_argmax, int32_t len_add, hipStream_t s) {
  const float eps = m->cfg.rms_norm_eps;
  if (m->wbf16 && kind != 1) {
    // bf16 weights: RMSNorm rows (where the step has one), then the f64-MFMA linear
    const int64_t H = m->H;
    if (kind == 5) {
      HIP_TRY(q8k::rows_norm(m->x, H, nrows, m->H, m->out_norm, eps, m->xn, H, s));
      GemmBf16Args g = bf16_args_m(m, m->emb, m->xn, H, nrows, nullptr, 0);
      g.logits = d_logits;
      g.best_key = m->am_key;
      g.counter = m->am_cnt;
      g.argmax = d_argmax;
      g.len_ptr = len_add ? m->d_len : nullptr;
      g.len_seq = d_row_seq;
      g.len_add = len_add;
      HIP_TRY(q8k::gemm_bf16(g, EPI_ARGMAX, s));
      return QWEN3_OK;
    }
    const Layer& ly = m->layers[l];
    switch (kind) {
      case 0:
        HIP_TRY(q8k::rows_norm(m->x, H, nrows, m->H, ly.attn_norm, eps, m->xn, H, s));
        HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.qkv, m->xn, H, nrows, m->qkv, m->nqkv), EPI_STORE, s));
        break;
      case 2:
        HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.o, m->attn, m->qw, nrows, m->x, H), EPI_RESIDUAL, s));
        break;
      case 3:
        HIP_TRY(q8k::rows_norm(m->x, H, nrows, m->H, ly.ffn_norm, eps, m->xn, H, s));
        HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.gateup, m->xn, H, nrows, m->h, m->F), EPI_SWIGLU, s));
        break;
      case 4:
        HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.down, m->h, m->F, nrows, m->x, H), EPI_RESIDUAL, s));
        break;
      default:
        return fail(QWEN3_E_INVALID_ARGUMENT, "bad kernel kind");
    }
    return QWEN3_OK;
  }
  if (batched_small_m(m, nrows)) {
    // a batch of streams: quantise the rows once, one small-M GEMM pass over
    // each weight matrix for all of them (smaller batches: the per-row GEMV,
    // whose fused norm/quantise prologue saves the separate launches)
    const int64_t H = m->H;
    GemmArgs g{};
    g.qa = m->qa, g.da = m->da, g.M = nrows, g.a_blocked = 1;  // rows quantised block-major
    auto run = [&](const QPlane& p, int K, float* out, int64_t ldc, int epi) {
      g.qs = p.qs, g.sc = p.sc, g.N = (int)p.rows, g.K = K, g.out = out, g.ldc = ldc;
      return q8k::gemm_skinny(g, epi, s);
    };
    if (kind == 5) {
      float* lg = d_logits ? d_logits : m->blogits;
      HIP_TRY(q8k::rows_quant(m->x, nrows, m->H, m->out_norm, eps, m->qa, m->da, nullptr, s, true));
      HIP_TRY(run(m->emb, m->H, lg, m->V, EPI_STORE));
      HIP_TRY(q8k::rows_argmax(lg, nrows, m->V, d_argmax, m->am_key, m->am_cnt, s, len_add ? m->d_len : nullptr,
                               d_row_seq, len_add));
      return QWEN3_OK;
    }
    if (kind != 1) {
      const Layer& ly = m->layers[l];
      switch (kind) {
        case 0:
          HIP_TRY(q8k::rows_quant(m->x, nrows, m->H, ly.attn_norm, eps, m->qa, m->da, nullptr, s, true));
          HIP_TRY(run(ly.qkv, m->H, m->qkv, m->nqkv, EPI_STORE));
          break;
        case 2:  // the attention kernel wrote its output rows quantised to qa/da
          HIP_TRY(run(ly.o, m->qw, m->x, H, EPI_RESIDUAL));
          break;
        case 3:
          HIP_TRY(q8k::rows_quant(m->x, nrows, m->H, ly.ffn_norm, eps, m->qa, m->da, nullptr, s, true));
          HIP_TRY(run(ly.gateup, m->H, m->h, m->F, EPI_SWIGLU));
          break;
        case 4:
          HIP_TRY(q8k::rows_quant(m->h, nrows, m->F, nullptr, eps, m->qa, m->da, nullptr, s, true));
          HIP_TRY(run(ly.down, m->F, m->x, H, EPI_RESIDUAL));
          break;
        default:
          return fail(QWEN3_E_INVALID_ARGUMENT, "bad kernel kind");
      }
      return QWEN3_OK;
    }
  }
  if (kind == 5) {
    GemvArgs a = gemv_args(m->emb, m->x, m->H, m->out_norm, eps, nullptr, 0);
    a.logits = d_logits;
    a.best_key = m->am_key;
    a.counter = m->am_cnt;
    a.argmax = d_argmax;
    a.len_ptr = len_add ? m->d_len : nullptr;
    a.len_seq = d_row_seq;
    a.len_add = len_add;
    HIP_TRY(q8k::gemv(a, true, EPI_ARGMAX, nrows, s));
    return QWEN3_OK;
  }
  const Layer& ly = m->layers[l];
  switch (kind) {
    case 0:
      HIP_TRY(q8k::gemv(gemv_args(ly.qkv, m->x, m->H, ly.attn_norm, eps, m->qkv, m->nqkv), true, EPI_STORE, nrows, s));
      break;
    case 1: {
      AttnDecodeArgs at = attn_args(m, d_row_seq, nrows);
      at.q_norm = ly.q_norm;
      at.k_norm = ly.k_norm;
      at.layer = l;
      if (batched_small_m(m, nrows)) at.q_out = m->qa, at.q_scale = m->da;  // o_proj's input rows
      HIP_TRY(q8k::attn_decode(at, m->hd, m->G, m->kvt, nrows, s));
      break;
    }
    case 2:
      HIP_TRY(q8k::gemv(gemv_args(ly.o, m->attn, m->qw, nullptr, eps, m->x, m->H), false, EPI_RESIDUAL, nrows, s));
      break;
    case 3:
      HIP_TRY(q8k::gemv(gemv_args(ly.gateup, m->x, m->H, ly.ffn_norm, eps, m->h, m->F), true, EPI_SWIGLU, nrows, s));
      break;
    case 4:
      HIP_TRY(q8k::gemv(gemv_args(ly.down, m->h, m->F, nullptr, eps, m->x, m->H), false, EPI_RESIDUAL, nrows, s));
      break;
    default:
      return fail(QWEN3_E_INVALID_ARGUMENT, "bad kernel kind");
  }
  return QWEN3_OK;
}

// Enqueue one decode step for nrows batch rows (rows r -> sequence row_seq[r],
// token tok[r]); positions come from d_len on the device.
int enqueue_decode(qwen3_model* m, int nrows, const int32_t* d_tok, const int32_t* d_row_seq, float* d_logits,
                   int32_t* d_argmax, hipStream_t s) {
  HIP_TRY(q8k::embed(d_tok, nrows, m->V, m->H, plane_rows(m->emb), m->emb.sc, m->wbf16, m->x, s));
  for (int l = 0; l < m->L; ++l)
    for (int kind = 0; kind < 5; ++kind) TRY(launch_decode_kernel(m, kind, l, nrows, d_row_seq, nullptr, nullptr, 0, s));
  return launch_decode_kernel(m, 5, 0, nrows, d_row_seq, d_logits, d_argmax, 1, s);
}

// One prefill chunk: T tokens (already in m->d_tok) at positions pos0.. of seq.
// all_rows: the head runs on every row of the chunk, writing d_logits [T, V]
// (and d_argmax [T]) from the chunk's first row; else on row T-1 of the last chunk.
// quant_q: the call is a single-token step (a q8_0 cache then scores with the
// quantised query).
int enqueue_prefill_chunk(qwen3_model* m, int seq, int pos0, int T, bool last, float* d_logits, int32_t* d_argmax,
                          hipStream_t s, bool all_rows = false, bool quant_q = false) {
  const float eps = m->cfg.rms_norm_eps;
  // projections: the small-M GEMM for short chunks (no split-K pass), else the tiled one
  const bool small = skinny_rows(m, T);
  auto gemm = [&](const GemmArgs& g, int epi, hipStream_t st) {
    return small ? q8k::gemm_skinny(g, epi, st) : q8k::gemm(g, epi, st);
  };
  HIP_TRY(q8k::embed(m->d_tok, T, m->V, m->H, plane_rows(m->emb), m->emb.sc, m->wbf16, m->x, s));
  const int64_t head_elems = (int64_t)m->cap[seq] * m->hd;
  for (int l = 0; l < m->L; ++l) {
    const Layer& ly = m->layers[l];
    const int64_t kbase = m->seq_base[seq] + (int64_t)l * 2 * m->nkv * head_elems;
    GemmArgs g{};
    g.qa = m->qa;
    g.da = m->da;
    g.M = T;
    g.part = m->gemm_part;
    g.part_bytes = m->gemm_part_bytes;
    g.a_blocked = small ? 1 : 0;  // the small-M GEMM reads the rows block-major
    // attention input: RMSNorm + quantise, fused QKV GEMM
    if (m->wbf16) {
      HIP_TRY(q8k::rows_norm(m->x, m->H, T, m->H, ly.attn_norm, eps, m->xn, m->H, s));
      HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.qkv, m->xn, m->H, T, m->qkv, m->nqkv), EPI_STORE, s));
    } else {
      HIP_TRY(q8k::rows_quant(m->x, T, m->H, ly.attn_norm, eps, m->qa, m->da, nullptr, s, small));
      g.qs = ly.qkv.qs, g.sc = ly.qkv.sc, g.N = (int)ly.qkv.rows, g.K = m->H, g.out = m->qkv, g.ldc = m->nqkv;
      HIP_TRY(gemm(g, EPI_STORE, s));
    }
    QkRopeArgs qr{};
    qr.qkv = m->qkv;
    qr.qkv_stride = m->nqkv;
    qr.q_norm = ly.q_norm;
    qr.k_norm = ly.k_norm;
    qr.eps = eps;
    qr.rope_cos = m->rope_cos;
    qr.rope_sin = m->rope_sin;
    qr.q32 = m->q32;
    qr.kv = m->kv;
    qr.kvs = m->kvs;
    qr.quant_q = quant_q;
    qr.kbase = kbase;
    qr.cap = m->cap[seq];
    qr.pos0 = pos0;
    qr.nh = m->nh;
    qr.nkv = m->nkv;
    HIP_TRY(q8k::qk_rope_append(qr, T, m->hd, m->kvt, s));
    AttnPrefillArgs ap{};
    ap.q32 = m->q32;
    ap.kv = m->kv;
    ap.kvs = m->kvs;
    ap.kbase = kbase;
    ap.cap = m->cap[seq];
    ap.pos0 = pos0;
    ap.T = T;
    ap.nh = m->nh;
    ap.nkv = m->nkv;
    ap.scale = 1.0 / std::sqrt((double)m->hd);
    ap.out = m->attn;
    ap.part = m->gemm_part;
    ap.part_bytes = m->gemm_part_bytes;
    HIP_TRY(q8k::attn_prefill(ap, m->hd, m->G, m->kvt, s));
    if (m->wbf16) {
      const int64_t H = m->H;
      HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.o, m->attn, m->qw, T, m->x, H), EPI_RESIDUAL, s));
      HIP_TRY(q8k::rows_norm(m->x, H, T, m->H, ly.ffn_norm, eps, m->xn, H, s));
      HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.gateup, m->xn, H, T, m->h, m->F), EPI_SWIGLU, s));
      HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, ly.down, m->h, m->F, T, m->x, H), EPI_RESIDUAL, s));
      continue;
    }
    // o_proj + residual
    HIP_TRY(q8k::rows_quant(m->attn, T, m->qw, nullptr, eps, m->qa, m->da, nullptr, s, small));
    g.qs = ly.o.qs, g.sc = ly.o.sc, g.N = (int)ly.o.rows, g.K = m->qw, g.out = m->x, g.ldc = m->H;
    HIP_TRY(gemm(g, EPI_RESIDUAL, s));
    // FFN: RMSNorm + quantise, gate/up with SwiGLU, quantise, down + residual
    HIP_TRY(q8k::rows_quant(m->x, T, m->H, ly.ffn_norm, eps, m->qa, m->da, nullptr, s, small));
    g.qs = ly.gateup.qs, g.sc = ly.gateup.sc, g.N = (int)ly.gateup.rows, g.K = m->H, g.out = m->h, g.ldc = m->F;
    HIP_TRY(gemm(g, EPI_SWIGLU, s));
    HIP_TRY(q8k::rows_quant(m->h, T, m->F, nullptr, eps, m->qa, m->da, nullptr, s, small));
    g.qs = ly.down.qs, g.sc = ly.down.sc, g.N = (int)ly.down.rows, g.K = m->F, g.out = m->x, g.ldc = m->H;
    HIP_TRY(gemm(g, EPI_RESIDUAL, s));
  }
  if (all_rows) {
    // final RMSNorm + tied lm_head on all T rows as one GEMM, then the row argmax
    const int64_t H = m->H;
    if (m->wbf16) {
      HIP_TRY(q8k::rows_norm(m->x, H, T, m->H, m->out_norm, eps, m->xn, H, s));
      HIP_TRY(q8k::gemm_bf16(bf16_args_m(m, m->emb, m->xn, H, T, d_logits, m->V), EPI_STORE, s));
    } else {
      const bool head_small = skinny_rows(m, T);
      HIP_TRY(q8k::rows_quant(m->x, T, m->H, m->out_norm, eps, m->qa, m->da, nullptr, s, head_small));
      GemmArgs g{};
      g.qa = m->qa, g.da = m->da, g.M = T, g.a_blocked = head_small ? 1 : 0;
      g.part = m->gemm_part, g.part_bytes = m->gemm_part_bytes;
      g.qs = m->emb.qs, g.sc = m->emb.sc, g.N = m->V, g.K = m->H, g.out = d_logits, g.ldc = m->V;
      HIP_TRY(head_small ? q8k::gemm_skinny(g, EPI_STORE, s) : q8k::gemm(g, EPI_STORE, s));
    }
    if (d_argmax) HIP_TRY(q8k::rows_argmax(d_logits, T, m->V, d_argmax, m->am_key, m->am_cnt, s));
  } else if (last && (d_logits || d_argmax) && m->wbf16) {
    const int64_t H = m->H;
    HIP_TRY(q8k::rows_norm(m->x + (int64_t)(T - 1) * H, H, 1, m->H, m->out_norm, eps, m->xn, H, s));
    GemmBf16Args g = bf16_args_m(m, m->emb, m->xn, H, 1, nullptr, 0);
    g.logits = d_logits;
    g.best_key = m->am_key;
    g.counter = m->am_cnt;
    g.argmax = d_argmax;
    HIP_TRY(q8k::gemm_bf16(g, EPI_ARGMAX, s));
  } else if (last && (d_logits || d_argmax)) {
    GemvArgs a = gemv_args(m->emb, m->x + (int64_t)(T - 1) * m->H, m->H, m->out_norm, eps, nullptr, 0);
    a.logits = d_logits;
    a.best_key = m->am_key;
    a.counter = m->am_cnt;
    a.argmax = d_argmax;
    HIP_TRY(q8k::gemv(a, true, EPI_ARGMAX, 1, s));
  }
  HIP_TRY(q8k::set_len(m->d_len, seq, pos0 + T, s));
  return QWEN3_OK;
}

}  // namespace

extern "C" {

const char* qwen3_last_error(void) { return g_err.c_str(); }

int32_t qwen3_decode_launches(const qwen3_t* m) {
  if (!m) return -1;
  return m->persist ? 1 : 5 * m->L + 2;
}

size_t qwen3_workspace_bytes(const qwen3_config* cfg) {
  g_err.clear();
  if (validate(cfg) != QWEN3_OK) return 0;
  qwen3_model m;
  fill_model_shape(&m, cfg);
  size_t total = 0;
  if (plan(&m, nullptr, &total) != QWEN3_OK) return 0;
  return total;
}

int qwen3_create(const qwen3_config* cfg, const qwen3_weights* w, void* d_workspace, size_t workspace_bytes,
                 void* stream, qwen3_t** out) {
  g_err.clear();
  if (!out) return fail(QWEN3_E_INVALID_ARGUMENT, "out is null");
  *out = nullptr;
  TRY(validate(cfg));
  if (!w || !w->layers || !w->token_embd || !w->output_norm)
    return fail(QWEN3_E_INVALID_ARGUMENT, "weights (or a pointer in it) is null");
  for (int l = 0; l < cfg->num_layers; ++l) {
    const qwen3_layer_weights& ly = w->layers[l];
    const void* ps[] = {ly.attn_norm, ly.attn_q, ly.attn_k, ly.attn_v, ly.attn_output, ly.attn_q_norm,
                        ly.attn_k_norm, ly.ffn_norm, ly.ffn_gate, ly.ffn_up, ly.ffn_down};
    for (const void* p : ps)
      if (!p) return fail(QWEN3_E_INVALID_ARGUMENT, "layer " + std::to_string(l) + " has a null weight pointer");
  }
  if (!d_workspace) return fail(QWEN3_E_INVALID_ARGUMENT, "workspace is null");
  if (reinterpret_cast<uintptr_t>(d_workspace) % kAlign)
    return fail(QWEN3_E_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  auto* m = new qwen3_model();
  fill_model_shape(m, cfg);
  size_t need = 0;
  int rc = plan(m, nullptr, &need);
  if (rc != QWEN3_OK) {
    delete m;
    return rc;
  }
  if (workspace_bytes < need) {
    delete m;
    return fail(QWEN3_E_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, needs " + std::to_string(need));
  }
  plan(m, static_cast<uint8_t*>(d_workspace), &need);
  m->bytes = need;
  hipStream_t s = S(stream);
  auto body = [&]() -> int {
    const int64_t H = m->H, F = m->F, hd = m->hd;
    TRY(repack(w->token_embd, m->emb, m->V, 0, -1, s));
    TRY(copy_f32(m->out_norm, w->output_norm, H, s));
    for (int l = 0; l < m->L; ++l) {
      const qwen3_layer_weights& src = w->layers[l];
      Layer& ly = m->layers[l];
      TRY(repack(src.attn_q, ly.qkv, m->qw, 0, -1, s));
      TRY(repack(src.attn_k, ly.qkv, m->kvw, m->qw, -1, s));
      TRY(repack(src.attn_v, ly.qkv, m->kvw, m->qw + m->kvw, -1, s));
      TRY(repack(src.attn_output, ly.o, H, 0, -1, s));
      TRY(repack(src.ffn_gate, ly.gateup, F, 0, 0, s));
      TRY(repack(src.ffn_up, ly.gateup, F, 0, 32, s));
      TRY(repack(src.ffn_down, ly.down, H, 0, -1, s));
      TRY(copy_f32(ly.attn_norm, src.attn_norm, H, s));
      TRY(copy_f32(ly.q_norm, src.attn_q_norm, hd, s));
      TRY(copy_f32(ly.k_norm, src.attn_k_norm, hd, s));
      TRY(copy_f32(ly.ffn_norm, src.ffn_norm, H, s));
    }
    // RoPE table: angle(p, i) = p * theta^(-2i/hd), cos/sin kept in f64
    const int half = m->hd / 2;
    std::vector<double> cs((size_t)m->max_cap * half), sn((size_t)m->max_cap * half);
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)m->cfg.rope_theta, -2.0 * i / (double)m->hd);
      for (int p = 0; p < m->max_cap; ++p) {
        const double ang = (double)p * inv;
        cs[(size_t)p * half + i] = std::cos(ang);
        sn[(size_t)p * half + i] = std::sin(ang);
      }
    }
    HIP_TRY(hipMemcpyAsync(m->rope_cos, cs.data(), cs.size() * 8, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(m->rope_sin, sn.data(), sn.size() * 8, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(m->d_seq_base, m->seq_base.data(), m->seq_base.size() * 8, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(m->d_seq_cap, m->cap.data(), m->cap.size() * 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemsetAsync(m->d_len, 0, m->cap.size() * 4, s));
    {
      std::vector<int32_t> ids(m->cap.size());
      for (size_t i = 0; i < ids.size(); ++i) ids[i] = (int32_t)i;
      HIP_TRY(hipMemcpyAsync(m->d_seq_ids, ids.data(), ids.size() * 4, hipMemcpyHostToDevice, s));
      HIP_TRY(hipStreamSynchronize(s));  // ids is a host temporary
    }
    HIP_TRY(hipMemsetAsync(m->attn_cnt, 0, (size_t)m->R * m->nkv * 4, s));
    HIP_TRY(hipMemsetAsync(m->am_cnt, 0, (size_t)m->R * 4, s));
    HIP_TRY(hipMemsetAsync(m->am_key, 0, (size_t)m->R * 8, s));
    if (m->persist_capable) {
      std::vector<PLayer> tab(m->L);
      for (int l = 0; l < m->L; ++l) {
        const Layer& ly = m->layers[l];
        tab[l] = PLayer{ly.qkv.qs, ly.o.qs, ly.gateup.qs, ly.down.qs, ly.qkv.sc, ly.o.sc, ly.gateup.sc, ly.down.sc,
                        ly.attn_norm, ly.q_norm, ly.k_norm, ly.ffn_norm};
      }
      HIP_TRY(hipMemcpyAsync(m->d_players, tab.data(), tab.size() * sizeof(PLayer), hipMemcpyHostToDevice, s));
      HIP_TRY(hipMemsetAsync(m->p_xa, 0, (size_t)m->H * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_xc, 0, (size_t)m->H * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_qkv, 0, (size_t)m->nqkv * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_att, 0, (size_t)m->qw / 32 * 16 * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_h, 0, (size_t)m->F / 32 * 16 * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_part, 0, persist_part_words(m->G, m->hd) * 8, s));
      HIP_TRY(hipMemsetAsync(m->p_err, 0, 4, s));
      HIP_TRY(hipMemsetAsync(m->p_keys, 0, 2 * kPersistWorkgroups * 8, s));
      HIP_TRY(hipStreamSynchronize(s));  // tab is a host temporary
    }
    HIP_TRY(hipStreamSynchronize(s));
    HIP_TRY(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking));
    return QWEN3_OK;
  };
  rc = body();
  if (rc != QWEN3_OK) {
    delete m;
    return rc;
  }
  m->h_len.assign(m->cap.size(), 0);
  const char* ng = std::getenv("QWEN3_NO_GRAPH");
  m->use_graphs = !(ng && ng[0] == '1');
  // the one-launch decode step needs every workgroup of its grid resident at
  // once: at least kPersistWorkgroups CUs, and one workgroup fitting per CU
  if (m->persist_capable && m->max_cap <= q8k::persist_max_ctx(m->psh)) {
    const char* pe = std::getenv("QWEN3_PERSISTENT");
    int dev = 0, cus = 0;
    const bool on = !(pe && pe[0] == '0');
    if (on && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus >= kPersistWorkgroups && q8k::persist_occupancy(m->psh, m->kvbf16) >= 1)
      m->persist = true;
  }
  *out = m;
  return QWEN3_OK;
}

void qwen3_destroy(qwen3_t* m) {
  if (!m) return;
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  for (auto& kv : m->bgraphs) (void)hipGraphExecDestroy(kv.second);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  delete m;
}

int qwen3_kv_len(const qwen3_t* m, int32_t seq, int32_t* out) {
  if (!m || !out) return fail(QWEN3_E_INVALID_ARGUMENT, "null argument");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  *out = m->h_len[seq];
  return QWEN3_OK;
}

int qwen3_reset(qwen3_t* m, int32_t seq, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  HIP_TRY(q8k::set_len(m->d_len, seq, 0, S(stream)));
  m->h_len[seq] = 0;
  return QWEN3_OK;
}

int qwen3_step_status(qwen3_t* m, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (!m->p_err) return QWEN3_OK;  // no one-launch step on this handle
  hipStream_t s = S(stream);
  unsigned word = 0;
  HIP_TRY(hipMemcpyAsync(&word, m->p_err, 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (word == 0) return QWEN3_OK;
  // the failed steps advanced no device length: the host lengths follow them
  std::vector<int32_t> dl(m->h_len.size());
  HIP_TRY(hipMemcpyAsync(dl.data(), m->d_len, dl.size() * 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipMemsetAsync(m->p_err, 0, 4, s));
  HIP_TRY(hipStreamSynchronize(s));
  m->h_len = dl;
  return fail(QWEN3_E_DEVICE,
              "a one-launch decode step gave up waiting on another workgroup: it and every later one-launch step "
              "wrote token -1 and advanced no length");
}

int qwen3_inject_step_error(qwen3_t* m, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (!m->p_err) return fail(QWEN3_E_INVALID_ARGUMENT, "this handle has no one-launch decode step");
  HIP_TRY(hipMemsetAsync(m->p_err, 0xFF, 4, S(stream)));
  return QWEN3_OK;
}

int qwen3_prefill(qwen3_t* m, int32_t seq, const int32_t* h_tokens, int32_t n, float* d_logits, int32_t* d_argmax,
                  void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (n <= 0) return fail(QWEN3_E_INVALID_SEQUENCE_LENGTH, "prefill needs n >= 1 tokens");
  if (!h_tokens) return fail(QWEN3_E_INVALID_ARGUMENT, "h_tokens is null");
  const int len = m->h_len[seq];
  if ((int64_t)len + n > m->cap[seq])
    return fail(QWEN3_E_KV_CACHE_OVERFLOW, "len " + std::to_string(len) + " + " + std::to_string(n) +
                                               " exceeds capacity " + std::to_string(m->cap[seq]));
  for (int i = 0; i < n; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= m->V)
      return fail(QWEN3_E_TOKEN_OUT_OF_RANGE, "token " + std::to_string(i) + " = " + std::to_string(h_tokens[i]) +
                                                  " outside [0, vocab)");
  hipStream_t s = S(stream);
  for (int c0 = 0; c0 < n; c0 += m->R) {
    const int T = std::min(m->R, n - c0);
    HIP_TRY(hipMemcpyAsync(m->d_tok, h_tokens + c0, (size_t)T * 4, hipMemcpyHostToDevice, s));
    TRY(enqueue_prefill_chunk(m, seq, len + c0, T, c0 + T == n, d_logits, d_argmax, s, false, n == 1));
  }
  m->h_len[seq] = len + n;
  return QWEN3_OK;
}

int qwen3_prefill_all_logits(qwen3_t* m, int32_t seq, const int32_t* h_tokens, int32_t n, float* d_logits,
                             int32_t* d_argmax, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (n <= 0) return fail(QWEN3_E_INVALID_SEQUENCE_LENGTH, "prefill needs n >= 1 tokens");
  if (!h_tokens) return fail(QWEN3_E_INVALID_ARGUMENT, "h_tokens is null");
  if (!d_logits) return fail(QWEN3_E_INVALID_ARGUMENT, "d_logits is required");
  const int len = m->h_len[seq];
  if ((int64_t)len + n > m->cap[seq])
    return fail(QWEN3_E_KV_CACHE_OVERFLOW, "len " + std::to_string(len) + " + " + std::to_string(n) +
                                               " exceeds capacity " + std::to_string(m->cap[seq]));
  for (int i = 0; i < n; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= m->V)
      return fail(QWEN3_E_TOKEN_OUT_OF_RANGE, "token " + std::to_string(i) + " = " + std::to_string(h_tokens[i]) +
                                                  " outside [0, vocab)");
  hipStream_t s = S(stream);
  for (int c0 = 0; c0 < n; c0 += m->R) {
    const int T = std::min(m->R, n - c0);
    HIP_TRY(hipMemcpyAsync(m->d_tok, h_tokens + c0, (size_t)T * 4, hipMemcpyHostToDevice, s));
    TRY(enqueue_prefill_chunk(m, seq, len + c0, T, c0 + T == n, d_logits + (int64_t)c0 * m->V,
                              d_argmax ? d_argmax + c0 : nullptr, s, true, n == 1));
  }
  m->h_len[seq] = len + n;
  return QWEN3_OK;
}

int qwen3_truncate(qwen3_t* m, int32_t seq, int32_t keep_len, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (keep_len < 0) return fail(QWEN3_E_INVALID_ARGUMENT, "keep_len < 0");
  if (keep_len >= m->h_len[seq]) return QWEN3_OK;
  m->h_len[seq] = keep_len;
  HIP_TRY(q8k::set_len(m->d_len, seq, keep_len, S(stream)));
  return QWEN3_OK;
}

// Launch the decode step of nrows rows from the graph cached under `key`,
// capturing it on the model's capture stream the first time.
constexpr size_t kMaxCachedGraphs = 32;  // per cache; beyond it the cache starts over

static int replay_decode(qwen3_model* m, std::map<std::tuple<int, const void*, const void*, const void*>, hipGraphExec_t>& cache,
                         const std::tuple<int, const void*, const void*, const void*>& key, int nrows, const int32_t* d_tok,
                         const int32_t* d_row_seq, float* d_logits, int32_t* d_argmax, hipStream_t s) {
  auto it = cache.find(key);
  if (it == cache.end()) {
    hipGraph_t graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
    int rc = enqueue_decode(m, nrows, d_tok, d_row_seq, d_logits, d_argmax, m->cap_stream);
    hipError_t e = hipStreamEndCapture(m->cap_stream, &graph);
    if (rc != QWEN3_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return fail(QWEN3_E_DEVICE, std::string("graph capture: ") + hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(QWEN3_E_DEVICE, std::string("graph instantiate: ") + hipGetErrorString(e));
    if (cache.size() >= kMaxCachedGraphs) {  // callers that pass fresh buffers every step
      // a graph launched earlier on the stream may still run: wait for it first
      HIP_TRY(hipStreamSynchronize(s));
      for (auto& kv : cache) (void)hipGraphExecDestroy(kv.second);
      cache.clear();
    }
    it = cache.emplace(key, exec).first;
  }
  HIP_TRY(hipGraphLaunch(it->second, s));
  return QWEN3_OK;
}

// One launch of the one-launch decode step running n greedy steps.
static hipError_t launch_persistent(qwen3_model* m, int32_t seq, int n, const int32_t* d_token, int32_t* d_tokens_out,
                                    float* d_logits, int32_t* d_argmax, hipStream_t s) {
  PersistArgs a{};
  a.layers = m->d_players;
  a.L = m->L;
  a.V = m->V;
  a.eps = m->cfg.rms_norm_eps;
  a.scale = 1.0 / std::sqrt((double)m->hd);
  a.emb_qs = m->emb.qs;
  a.emb_sc = m->emb.sc;
  a.out_norm = m->out_norm;
  a.rope_cos = m->rope_cos;
  a.rope_sin = m->rope_sin;
  a.kv = m->kv;
  a.seq_base = m->d_seq_base;
  a.seq_cap = m->d_seq_cap;
  a.len = m->d_len;
  a.seq = seq;
  a.token = d_token;
  a.logits = d_logits;
  a.argmax = d_argmax;
  a.xa = m->p_xa, a.xc = m->p_xc, a.qkv = m->p_qkv, a.att = m->p_att, a.h = m->p_h;
  a.part = m->p_part;
  a.err = m->p_err;
  a.pstep = m->pstep;
  a.nsteps = n;
  a.tokens_out = d_tokens_out;
  a.keys = m->p_keys;
  const hipError_t e = q8k::decode_persistent(m->psh, m->kvbf16, a, s);
  if (e == hipSuccess) m->pstep += (unsigned)n;
  return e;
}

int qwen3_decode_step(qwen3_t* m, int32_t seq, const int32_t* d_token, float* d_logits, int32_t* d_argmax,
                      void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (!d_token || !d_argmax) return fail(QWEN3_E_INVALID_ARGUMENT, "d_token and d_argmax are required");
  if (m->h_len[seq] + 1 > m->cap[seq])
    return fail(QWEN3_E_KV_CACHE_OVERFLOW, "decode at len " + std::to_string(m->h_len[seq]) + " exceeds capacity");
  hipStream_t s = S(stream);
  if (m->persist) {
    HIP_TRY(launch_persistent(m, seq, 1, d_token, nullptr, d_logits, d_argmax, s));
    m->h_len[seq] += 1;
    return QWEN3_OK;
  }
  if (!m->use_graphs) {
    TRY(enqueue_decode(m, 1, d_token, m->d_seq_ids + seq, d_logits, d_argmax, s));
    m->h_len[seq] += 1;
    return QWEN3_OK;
  }
  auto key = std::make_tuple((int)seq, (const void*)d_token, (const void*)d_logits, (const void*)d_argmax);
  TRY(replay_decode(m, m->graphs, key, 1, d_token, m->d_seq_ids + seq, d_logits, d_argmax, s));
  m->h_len[seq] += 1;
  return QWEN3_OK;
}

int qwen3_decode_greedy(qwen3_t* m, int32_t seq, int32_t n, const int32_t* d_token, int32_t* d_tokens_out,
                        float* d_logits, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (n < 1) return fail(QWEN3_E_INVALID_ARGUMENT, "n must be at least 1");
  if (!d_token || !d_tokens_out) return fail(QWEN3_E_INVALID_ARGUMENT, "d_token and d_tokens_out are required");
  if ((int64_t)m->h_len[seq] + n > (int64_t)m->cap[seq])
    return fail(QWEN3_E_KV_CACHE_OVERFLOW, "decoding " + std::to_string(n) + " tokens at len " +
                                               std::to_string(m->h_len[seq]) + " exceeds capacity");
  hipStream_t s = S(stream);
  if (m->persist) {
    HIP_TRY(launch_persistent(m, seq, n, d_token, d_tokens_out, d_logits, d_tokens_out + n - 1, s));
    m->h_len[seq] += n;
    return QWEN3_OK;
  }
  // per-kernel steps, each fed the previous step's token (no graph: every
  // step has its own token pointer)
  for (int i = 0; i < n; ++i) {
    const int32_t* tok = i == 0 ? d_token : d_tokens_out + i - 1;
    TRY(enqueue_decode(m, 1, tok, m->d_seq_ids + seq, i + 1 == n ? d_logits : nullptr, d_tokens_out + i, s));
    m->h_len[seq] += 1;
  }
  return QWEN3_OK;
}

int qwen3_decode_batch(qwen3_t* m, const int32_t* h_seqs, int32_t n, const int32_t* d_tokens, float* d_logits,
                       int32_t* d_argmax, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (n <= 0) return fail(QWEN3_E_INVALID_SEQUENCE_LENGTH, "batch needs n >= 1");
  if (n > m->R) return fail(QWEN3_E_INVALID_ARGUMENT, "batch larger than max_batch_tokens");
  if (!h_seqs || !d_tokens || !d_argmax) return fail(QWEN3_E_INVALID_ARGUMENT, "null argument");
  std::vector<char> seen(m->h_len.size(), 0);
  for (int i = 0; i < n; ++i) {
    const int sq = h_seqs[i];
    if (sq < 0 || sq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
    if (seen[sq]) return fail(QWEN3_E_INVALID_ARGUMENT, "a sequence appears twice in one batch");
    seen[sq] = 1;
    if (m->h_len[sq] + 1 > m->cap[sq]) return fail(QWEN3_E_KV_CACHE_OVERFLOW, "a sequence is at capacity");
  }
  hipStream_t s = S(stream);
  HIP_TRY(hipMemcpyAsync(m->d_row_seq, h_seqs, (size_t)n * 4, hipMemcpyHostToDevice, s));
  if (m->use_graphs) {
    // a step is a few hundred small launches: replayed from a graph the host
    // no longer paces them
    auto key = std::make_tuple((int)n, (const void*)d_tokens, (const void*)d_logits, (const void*)d_argmax);
    TRY(replay_decode(m, m->bgraphs, key, n, d_tokens, m->d_row_seq, d_logits, d_argmax, s));
  } else {
    TRY(enqueue_decode(m, n, d_tokens, m->d_row_seq, d_logits, d_argmax, s));
  }
  for (int i = 0; i < n; ++i) m->h_len[h_seqs[i]] += 1;
  return QWEN3_OK;
}

int qwen3_replay_kernel(qwen3_t* m, int32_t seq, int32_t kind, int32_t layer, int32_t reps, void* stream) {
  g_err.clear();
  if (!m) return fail(QWEN3_E_INVALID_ARGUMENT, "null handle");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (kind < 0 || kind > 5 || layer < 0 || layer >= m->L || reps < 0)
    return fail(QWEN3_E_INVALID_ARGUMENT, "bad kernel kind, layer or reps");
  if (m->h_len[seq] + 1 > m->cap[seq]) return fail(QWEN3_E_KV_CACHE_OVERFLOW, "sequence is at capacity");
  for (int r = 0; r < reps; ++r)
    TRY(launch_decode_kernel(m, kind, layer, 1, m->d_seq_ids + seq, nullptr, nullptr, 0, S(stream)));
  return QWEN3_OK;
}

int qwen3_kv_export(const qwen3_t* m, int32_t seq, int32_t layer, float* d_k, float* d_v, void* stream) {
  g_err.clear();
  if (!m || !d_k || !d_v) return fail(QWEN3_E_INVALID_ARGUMENT, "null argument");
  if (seq < 0 || seq >= (int)m->h_len.size()) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sequence index");
  if (layer < 0 || layer >= m->L) return fail(QWEN3_E_INVALID_ARGUMENT, "bad layer index");
  const int cap = m->cap[seq], len = m->h_len[seq];
  const int64_t head_elems = (int64_t)cap * m->hd;
  const int64_t kbase = m->seq_base[seq] + (int64_t)layer * 2 * m->nkv * head_elems;
  const int64_t vbase = kbase + (int64_t)m->nkv * head_elems;
  const size_t esz = m->kvt == KV_F32 ? 4 : (m->kvt == KV_BF16 ? 2 : 1);
  const uint8_t* base = static_cast<const uint8_t*>(m->kv);
  const uint16_t* ks = m->kvs ? m->kvs + kbase / 32 : nullptr;
  const uint16_t* vs = m->kvs ? m->kvs + vbase / 32 : nullptr;
  HIP_TRY(q8k::kv_export(base + kbase * esz, ks, m->kvt, m->nkv, cap, len, m->hd, d_k, S(stream)));
  HIP_TRY(q8k::kv_export(base + vbase * esz, vs, m->kvt, m->nkv, cap, len, m->hd, d_v, S(stream)));
  return QWEN3_OK;
}

// ---- op-level entry points ---------------------------------------------------------------

int qwen3_peak_copy(const void* d_src, void* d_dst, size_t bytes, void* stream) {
  g_err.clear();
  if (bytes % 16) return fail(QWEN3_E_INVALID_ARGUMENT, "bytes must be a multiple of 16");
  if (bytes && (!d_src || !d_dst)) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  HIP_TRY(q8k::copy_peak(d_src, d_dst, bytes, S(stream)));
  return QWEN3_OK;
}

int qwen3_peak_read(const void* d_src, size_t bytes, uint32_t* d_out, void* stream) {
  g_err.clear();
  if (bytes % 16) return fail(QWEN3_E_INVALID_ARGUMENT, "bytes must be a multiple of 16");
  if (bytes && (!d_src || !d_out)) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  HIP_TRY(q8k::read_peak(d_src, bytes, d_out, S(stream)));
  return QWEN3_OK;
}

int32_t qwen3_peak_read_partials(void) { return q8k::read_peak_partials(); }

double qwen3_peak_mfma_i8_ops(int32_t workgroups, int32_t iters) {
  if (workgroups < 1 || iters < 1) return 0.0;
  return q8k::mfma_peak_ops(workgroups, iters);
}

int qwen3_peak_mfma_i8(int32_t* d_out, int32_t workgroups, int32_t iters, int32_t fill, void* stream) {
  g_err.clear();
  if (!d_out) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  if (workgroups < 1 || workgroups > 65536 || iters < 1)
    return fail(QWEN3_E_INVALID_ARGUMENT, "workgroups must be in [1, 65536], iters >= 1");
  HIP_TRY(q8k::mfma_peak(d_out, workgroups, iters, fill, S(stream)));
  return QWEN3_OK;
}

int qwen3_q8_0_encode(const float* d_x, int64_t n, void* d_blocks, void* stream) {
  g_err.clear();
  if (n < 0 || n % 32) return fail(QWEN3_E_INVALID_ARGUMENT, "n must be a non-negative multiple of 32");
  if (n && (!d_x || !d_blocks)) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  HIP_TRY(q8k::encode_q8_0(d_x, n, d_blocks, S(stream)));
  return QWEN3_OK;
}

int qwen3_bf16_encode(const float* d_x, int64_t n, uint16_t* d_out, void* stream) {
  g_err.clear();
  if (n < 0) return fail(QWEN3_E_INVALID_ARGUMENT, "n must be >= 0");
  if (n && (!d_x || !d_out)) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  HIP_TRY(q8k::encode_bf16(d_x, n, d_out, S(stream)));
  return QWEN3_OK;
}

int qwen3_q8_0_repack(const void* d_blocks, int64_t rows, int64_t k, int8_t* d_qs, uint16_t* d_scale, void* stream) {
  g_err.clear();
  if (rows < 0 || k <= 0 || k % 32) return fail(QWEN3_E_INVALID_ARGUMENT, "k must be a positive multiple of 32");
  if (rows && (!d_blocks || !d_qs || !d_scale)) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  HIP_TRY(q8k::repack_q8_0(d_blocks, rows, k, d_qs, d_scale, 0, -1, S(stream)));
  return QWEN3_OK;
}

size_t qwen3_linear_work_bytes(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return align_up((size_t)(m * k)) + align_up((size_t)(m * (k / 32)) * 4) + 4096;
}

int qwen3_q8_0_linear(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs, const uint16_t* d_scale, int64_t n,
                      float* d_y, void* d_work, void* stream) {
  g_err.clear();
  if (m <= 0 || n <= 0 || k <= 0) return fail(QWEN3_E_INVALID_ARGUMENT, "m, n, k must be positive");
  if (!d_x || !d_qs || !d_scale || !d_y) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  if (k % 128 || !q8k::gemv_supported_k((int)k)) return fail(QWEN3_E_INVALID_ARGUMENT, "unsupported k");
  if (m > 1 && !d_work) return fail(QWEN3_E_INVALID_ARGUMENT, "d_work is required for m > 1");
  if (m > INT32_MAX || n > INT32_MAX) return fail(QWEN3_E_INVALID_ARGUMENT, "size too large");
  hipStream_t s = S(stream);
  if (m == 1) {
    QPlane p;
    p.qs = const_cast<int8_t*>(d_qs);
    p.sc = const_cast<uint16_t*>(d_scale);
    p.rows = n;
    p.k = k;
    HIP_TRY(q8k::gemv(gemv_args(p, d_x, k, nullptr, 1e-6f, d_y, n), false, EPI_STORE, 1, s));
    return QWEN3_OK;
  }
  int8_t* qa = static_cast<int8_t*>(d_work);
  float* da = reinterpret_cast<float*>(static_cast<uint8_t*>(d_work) + align_up((size_t)(m * k)));
  const bool small = q8k::gemm_skinny_supported((int)m, (int)k);
  HIP_TRY(q8k::rows_quant(d_x, (int)m, (int)k, nullptr, 1e-6f, qa, da, nullptr, s, small));
  GemmArgs g{};
  g.a_blocked = small ? 1 : 0;
  g.qa = qa;
  g.da = da;
  g.qs = d_qs;
  g.sc = d_scale;
  g.M = (int)m;
  g.N = (int)n;
  g.K = (int)k;
  g.out = d_y;
  g.ldc = n;
  HIP_TRY(small ? q8k::gemm_skinny(g, EPI_STORE, s) : q8k::gemm(g, EPI_STORE, s));
  return QWEN3_OK;
}

int qwen3_q8_0_block_dots(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs, int64_t n, int8_t* d_qa,
                          uint16_t* d_da, int32_t* d_s, void* stream) {
  g_err.clear();
  if (m <= 0 || n <= 0 || k <= 0 || k % 32) return fail(QWEN3_E_INVALID_ARGUMENT, "bad sizes");
  if (!d_x || !d_qs || !d_qa || !d_da || !d_s) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return fail(QWEN3_E_INVALID_ARGUMENT, "size too large");
  hipStream_t s = S(stream);
  HIP_TRY(q8k::rows_quant(d_x, (int)m, (int)k, nullptr, 1e-6f, d_qa, nullptr, d_da, s));
  HIP_TRY(q8k::block_dots(d_qa, d_qs, (int)m, (int)k, (int)n, d_s, s));
  return QWEN3_OK;
}

size_t qwen3_sample_work_bytes(int32_t n, int32_t vocab) {
  if (n <= 0 || vocab <= 0) return 0;
  return q8k::sample_work_bytes(n, vocab);
}

int qwen3_sample(float* d_logits, int32_t n, int32_t vocab, const qwen3_sampler_config* cfg, const int32_t* d_history,
                 int32_t history_stride, const int32_t* d_history_len, const float* d_uniform, int32_t* d_tokens,
                 void* d_work, void* stream) {
  g_err.clear();
  if (!d_logits || !cfg || !d_tokens || !d_work) return fail(QWEN3_E_INVALID_ARGUMENT, "null argument");
  if (reinterpret_cast<uintptr_t>(d_work) % 256) return fail(QWEN3_E_INVALID_ARGUMENT, "d_work must be 256-byte aligned");
  if (n <= 0 || vocab <= 0) return fail(QWEN3_E_INVALID_ARGUMENT, "n and vocab must be positive");
  const qwen3_sampler_config& c = *cfg;
  if (!std::isfinite(c.temperature)) return fail(QWEN3_E_INVALID_ARGUMENT, "temperature is not finite");
  if (c.top_k < 0) return fail(QWEN3_E_INVALID_ARGUMENT, "top_k < 0");
  if (!(c.top_p > 0.f && c.top_p <= 1.f)) return fail(QWEN3_E_INVALID_ARGUMENT, "top_p outside (0, 1]");
  if (!(c.min_p >= 0.f && c.min_p <= 1.f)) return fail(QWEN3_E_INVALID_ARGUMENT, "min_p outside [0, 1]");
  if (!(c.repeat_penalty > 0.f) || !std::isfinite(c.repeat_penalty) || !std::isfinite(c.freq_penalty) ||
      !std::isfinite(c.presence_penalty))
    return fail(QWEN3_E_INVALID_ARGUMENT, "penalties must be finite and repeat_penalty > 0");
  if (c.repeat_last_n < 0 || c.repeat_last_n > 4096) return fail(QWEN3_E_INVALID_ARGUMENT, "repeat_last_n outside [0, 4096]");
  if (d_history && (!d_history_len || history_stride <= 0))
    return fail(QWEN3_E_INVALID_ARGUMENT, "a history needs its lengths and a positive stride");
  if (c.temperature > 0.f && !d_uniform) return fail(QWEN3_E_INVALID_ARGUMENT, "d_uniform is required when sampling");
  SampleArgs a{};
  a.temperature = c.temperature;
  a.top_k = c.top_k;
  a.top_p = c.top_p;
  a.min_p = c.min_p;
  a.repeat_penalty = c.repeat_penalty;
  a.freq_penalty = c.freq_penalty;
  a.presence_penalty = c.presence_penalty;
  a.repeat_last_n = c.repeat_last_n;
  HIP_TRY(q8k::sample(d_logits, n, vocab, a, d_history, history_stride, d_history_len, d_uniform, d_tokens, d_work,
                      S(stream)));
  return QWEN3_OK;
}

int qwen3_bf16_linear(const float* d_x, int64_t m, int64_t k, const uint16_t* d_w, int64_t n, float* d_y,
                      void* stream) {
  g_err.clear();
  if (m <= 0 || n <= 0 || k <= 0) return fail(QWEN3_E_INVALID_ARGUMENT, "m, n, k must be positive");
  if (k % 32) return fail(QWEN3_E_INVALID_ARGUMENT, "k must be a multiple of 32");
  if (!d_x || !d_w || !d_y) return fail(QWEN3_E_INVALID_ARGUMENT, "null pointer");
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return fail(QWEN3_E_INVALID_ARGUMENT, "size too large");
  QPlane p;
  p.bf = const_cast<uint16_t*>(d_w);
  p.rows = n;
  p.k = k;
  HIP_TRY(q8k::gemm_bf16(bf16_args(p, d_x, k, (int)m, d_y, n), EPI_STORE, S(stream)));
  return QWEN3_OK;
}

}  // extern "C"
