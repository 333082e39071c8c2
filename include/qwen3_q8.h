/*
 * qwen3_q8.h -- C ABI of the MI355X (gfx950) forward pass of a Qwen3 dense
 * decoder over GGUF-style Q8_0 weights (or bf16 weights).
 *
 * What is computed (sources are web pages, cited by title and section):
 *   - the forward pass: embedding rows, per layer RMSNorm -> Q/K/V
 *     projections -> per-head Q/K RMSNorm -> NeoX RoPE -> KV append ->
 *     causal grouped-query attention -> o_proj + residual -> RMSNorm ->
 *     SwiGLU FFN + residual; final RMSNorm -> tied lm_head -> greedy argmax
 *     (Fucina course, "A transformer from scratch", sections 12.3-12.6;
 *     minfer, "Qwen3 Support Plan", sections 1-2);
 *   - every Q8_0 linear quantises its f32 input row per 32-block to Q8_0 and
 *     sums integer block dots rescaled by d_w * d_a (Fucina course, "Model
 *     files and quantization", sections 11.7 and 11.9).
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device pointers (HIP), h_* are host pointers.
 *     The library never allocates device memory: everything it needs is
 *     carved from the caller's workspace (qwen3_workspace_bytes).
 *   - `stream` is a hipStream_t passed as void*.  Work is enqueued on it and
 *     the call returns without waiting (except where stated).  Results in
 *     device buffers are valid once the stream reaches that point.
 *   - Return value: QWEN3_OK (0) or a negative QWEN3_E_* code; on error
 *     qwen3_last_error() describes it (thread-local string) and the model
 *     state (KV lengths, cache contents) is unchanged.  Every argument and
 *     shape error is detected on the host before any launch.
 *   - A handle is single-stream mutable state; it is not thread-safe.
 */
#ifndef QWEN3_Q8_H
#define QWEN3_Q8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes -------------------------------------------------------- */
#define QWEN3_OK 0
#define QWEN3_E_INVALID_ARGUMENT (-1)        /* null pointer, bad seq index, bad size */
#define QWEN3_E_INVALID_CONFIG (-2)          /* zero/negative dims, heads not divisible, ... */
#define QWEN3_E_INVALID_WEIGHT_SHAPE (-3)    /* size arithmetic overflows */
#define QWEN3_E_UNSUPPORTED_WEIGHT_TYPE (-4) /* weight_type / kv_type not known */
#define QWEN3_E_WORKSPACE_TOO_SMALL (-5)
#define QWEN3_E_INVALID_SEQUENCE_LENGTH (-6) /* n <= 0 tokens */
#define QWEN3_E_KV_CACHE_OVERFLOW (-7)       /* len + n > the sequence's capacity */
#define QWEN3_E_TOKEN_OUT_OF_RANGE (-8)      /* a host token id outside [0, vocab) */
#define QWEN3_E_DEVICE (-9)                  /* a HIP call failed */

/* ---- element types -------------------------------------------------------- */
#define QWEN3_W_Q8_0 0 /* projections and embedding in Q8_0 blocks */
#define QWEN3_W_BF16 1 /* projections and embedding in bf16 */
#define QWEN3_KV_F32 0
#define QWEN3_KV_BF16 1
/* Q8_0 KV cache ("The LLM stack (fucina_llm)", section 13.4, the q8_0 option;
 * "A transformer from scratch", section 12.4): every (position, KV head) row
 * is head_dim/32 Q8_0 blocks, held as an int8 code plane plus an f16 scale
 * plane (1.0625 bytes per element).  A single-token step (decode, batched
 * decode, a one-token prefill) scores with the query quantised per head (the
 * integer score path); multi-token steps keep the f32 query against the
 * dequantised cache.  Needs head_dim % 32 == 0; decode runs the per-kernel
 * step (qwen3_decode_launches > 1). */
#define QWEN3_KV_Q8_0 2

/* Q8_0 block on the wire (Fucina course, "Model files and quantization",
 * section 11.7): the f16 bits of the scale d, then 32 signed bytes; 34 bytes,
 * no padding.  A row of K values is K/32 consecutive blocks. */
#define QWEN3_Q8_0_BLOCK_VALUES 32
#define QWEN3_Q8_0_BLOCK_BYTES 34

/* Model geometry and cache plan ("A transformer from scratch", section 12.1:
 * the config is nine numbers; head_dim is independent of hidden / heads,
 * minfer plan section 2.1).  Validation (QWEN3_E_INVALID_CONFIG): every
 * integer > 0; heads % kv_heads == 0; head_dim even and <= 256;
 * hidden_size, heads * head_dim and intermediate_size multiples of 128;
 * head_dim * heads/kv_heads <= 512; eps > 0; rope_theta > 1; max_seqs >= 1;
 * every seq_capacity[i] >= 1. */
typedef struct qwen3_config {
  int32_t vocab_size;
  int32_t hidden_size;
  int32_t intermediate_size;
  int32_t num_layers;
  int32_t num_attention_heads;
  int32_t num_key_value_heads;
  int32_t head_dim;
  float rms_norm_eps;
  float rope_theta;
  int32_t weight_type; /* QWEN3_W_* */
  int32_t kv_type;     /* QWEN3_KV_* */
  int32_t max_seqs;    /* independent KV caches held by the handle */
  const int32_t* h_seq_capacity; /* host [max_seqs]: KV rows of each sequence */
  int32_t max_batch_tokens; /* rows one pass may process; longer prompts are
                               prefilled in chunks of this many tokens.
                               Also the largest batch of qwen3_decode_batch.
                               0 selects 1024. */
} qwen3_config;

/* Device pointers to one layer's tensors, GGUF names (minfer plan section 1).
 * Projections are logical [out, in], row-major, `in` contiguous ("block row
 * r is output r", "Model files and quantization", section 11.9): Q8_0 rows
 * are in/32 blocks of 34 bytes; bf16 rows are `in` bf16 values.  Norm
 * weights are f32.  There are no biases (minfer plan section 5, item 7).
 *   attn_q [heads*hd, hidden]   attn_k, attn_v [kv_heads*hd, hidden]
 *   attn_output [hidden, heads*hd]   attn_q_norm, attn_k_norm [hd]
 *   ffn_gate, ffn_up [ffn, hidden]   ffn_down [hidden, ffn]
 *   attn_norm, ffn_norm [hidden] */
typedef struct qwen3_layer_weights {
  const void* attn_norm;
  const void* attn_q;
  const void* attn_k;
  const void* attn_v;
  const void* attn_output;
  const void* attn_q_norm;
  const void* attn_k_norm;
  const void* ffn_norm;
  const void* ffn_gate;
  const void* ffn_up;
  const void* ffn_down;
} qwen3_layer_weights;

/* token_embd [vocab, hidden] doubles as the lm_head (tied weights, "A
 * transformer from scratch", section 12.3.1).  `layers` is a HOST array of
 * num_layers entries holding DEVICE pointers. */
typedef struct qwen3_weights {
  const void* token_embd;
  const void* output_norm;
  const qwen3_layer_weights* layers;
} qwen3_weights;

typedef struct qwen3_model qwen3_t;

/* Bytes of device workspace a handle needs for `cfg` (weights repacked into
 * the library's layout, KV caches, RoPE table and activations).  The KV part
 * is layers * 2 * kv_heads * head_dim * element bytes per cached position of
 * every sequence ("A transformer from scratch", section 12.4, the cache's
 * bytes per position; "The LLM stack (fucina_llm)", section 13.4: the caller
 * sizes and owns the cache).  Returns 0 if cfg is invalid (qwen3_last_error
 * says why).  Host-only. */
size_t qwen3_workspace_bytes(const qwen3_config* cfg);

/* Build a handle ("The LLM stack (fucina_llm)", section 13.2: loaded weights
 * are copied into the engine's own layout, so the source may be freed;
 * section 13.4: a new cache has length 0; "A transformer from scratch",
 * section 12.3.4: the RoPE table is built once).  Copies and repacks the
 * weights (device pointers in the layout above) into `d_workspace`, builds
 * the RoPE table, and sets every sequence's KV length to 0.  The weight buffers are only read during this
 * call (enqueued on `stream`; the call synchronises the stream before
 * returning, so the caller may free them afterwards).  The workspace is owned
 * by the caller, must be at least qwen3_workspace_bytes(cfg) bytes, 256-byte
 * aligned, and must outlive the handle; the library never frees it. */
int qwen3_create(const qwen3_config* cfg, const qwen3_weights* w, void* d_workspace,
                 size_t workspace_bytes, void* stream, qwen3_t** out);

/* Destroy a handle (host state and captured graphs; no device frees). */
void qwen3_destroy(qwen3_t* h);

/* Prefill: append `n` tokens (host ids, validated) to sequence `seq` at its
 * current length L and run the forward pass over them ("A transformer from
 * scratch", section 12.5: the same forward serves prefill and decode).
 * Writes the logits of the LAST token to d_logits [vocab] (f32) and its
 * greedy argmax (lowest index among maxima) to d_argmax [1] (int32); either
 * may be NULL.  Afterwards the length is L + n.  Errors:
 * QWEN3_E_INVALID_SEQUENCE_LENGTH (n <= 0), QWEN3_E_KV_CACHE_OVERFLOW
 * (L + n > capacity), QWEN3_E_TOKEN_OUT_OF_RANGE. */
int qwen3_prefill(qwen3_t* h, int32_t seq, const int32_t* h_tokens, int32_t n, float* d_logits,
                  int32_t* d_argmax, void* stream);

/* Prefill returning every row's logits: the all-logits forward step ("A
 * transformer from scratch", sections 12.3.7 and 12.5, forwardStepAllLogits:
 * the same forward over the appended tokens, with the final norm and lm_head
 * applied to every position instead of the last only), the verify pass of
 * speculative decoding.  Appends the n tokens (host ids, validated) to `seq` at its length L
 * exactly as qwen3_prefill does, then applies the final RMSNorm and the tied
 * lm_head to all n rows.  d_logits [n, vocab] f32 (required, row-major);
 * d_argmax [n] int32 greedy argmax of each row (lowest index among maxima),
 * or NULL.  Length L -> L + n.  Errors as qwen3_prefill. */
int qwen3_prefill_all_logits(qwen3_t* h, int32_t seq, const int32_t* h_tokens, int32_t n, float* d_logits,
                             int32_t* d_argmax, void* stream);

/* Rewind sequence `seq` to its first keep_len positions in O(1) ("The LLM
 * stack (fucina_llm)", section 13.4, truncate; "A transformer from scratch",
 * section 12.4): only the length changes, the next append overwrites the
 * abandoned rows.  keep_len >= the current length is a no-op; keep_len < 0 is
 * QWEN3_E_INVALID_ARGUMENT.  The device length is set on `stream`. */
int qwen3_truncate(qwen3_t* h, int32_t seq, int32_t keep_len, void* stream);

/* One decode step of sequence `seq` ("A transformer from scratch", sections
 * 12.3-12.5: the cached forward of one token at position L, greedy argmax as
 * in section 12.6): the token id is read on the device from
 * d_token [1] (so the previous step's d_argmax can be passed straight back
 * and the step needs no host round trip).  Writes d_logits [vocab] (may be
 * NULL) and d_argmax [1] (required).  Length L -> L + 1; L + 1 > capacity is
 * QWEN3_E_KV_CACHE_OVERFLOW.  A device token outside [0, vocab) is clamped
 * into range (the host cannot check it without a synchronisation).  The
 * step is either one cooperative launch (qwen3_decode_launches == 1; its
 * device-side failure is reported by qwen3_step_status) or replayed from a
 * captured HIP graph keyed by (seq, d_token, d_logits, d_argmax); it
 * allocates nothing. */
int qwen3_decode_step(qwen3_t* h, int32_t seq, const int32_t* d_token, float* d_logits,
                      int32_t* d_argmax, void* stream);

/* n greedy decode steps of sequence `seq` in one call ("A transformer from
 * scratch", sections 12.5-12.6: each step is the cached forward of the
 * previous step's argmax, the generation loop of the greedy sampler): step 0
 * reads its token on the device from d_token [1] (clamped into [0, vocab)
 * like qwen3_decode_step); step i > 0 takes the token step i - 1 chose.
 * Writes the n chosen tokens to d_tokens_out [n] (device, required) and the
 * last step's logits to d_logits [vocab] (may be NULL).  Every step computes
 * exactly what qwen3_decode_step computes, so the tokens and the last logits
 * equal those of n qwen3_decode_step calls fed their own argmax.  Length L ->
 * L + n; L + n > capacity is QWEN3_E_KV_CACHE_OVERFLOW and n < 1 is
 * QWEN3_E_INVALID_ARGUMENT.  With the one-launch step (qwen3_decode_launches
 * == 1) all n steps are one cooperative launch, the token handed from step to
 * step on the device, so n - 1 launch gaps are saved; a device-side failure
 * at step k (see qwen3_step_status) leaves steps < k done and their tokens
 * written, writes -1 as the call's last token d_tokens_out[n - 1], leaves
 * slots k .. n - 2 unwritten, and qwen3_step_status then sets the host
 * length to L + k.  Otherwise the steps are n per-kernel steps enqueued on
 * `stream`.  Allocates nothing. */
int qwen3_decode_greedy(qwen3_t* h, int32_t seq, int32_t n, const int32_t* d_token, int32_t* d_tokens_out,
                        float* d_logits, void* stream);

/* Batched decode: one token for each of the `n` distinct sequences h_seqs
 * [n] (host) in one pass: weights are read once for all n rows, while RoPE
 * positions, KV appends and attention are per sequence ("A transformer from
 * scratch", section 12.5, batch decode).  d_tokens [n] (device),
 * d_logits [n, vocab] (may be NULL), d_argmax [n].  n <= max_batch_tokens.
 * The step is replayed from a captured HIP graph keyed by (n, d_tokens,
 * d_logits, d_argmax), h_seqs being uploaded before each replay; a handle
 * keeps at most 32 such graphs (then waits on `stream` and starts over). */
int qwen3_decode_batch(qwen3_t* h, const int32_t* h_seqs, int32_t n, const int32_t* d_tokens,
                       float* d_logits, int32_t* d_argmax, void* stream);

/* Set sequence `seq`'s KV length to 0 (buffers retained; "The LLM stack",
 * section 13.4, reset).  Enqueued on `stream`. */
int qwen3_reset(qwen3_t* h, int32_t seq, void* stream);

/* Outcome of the one-launch decode steps enqueued so far ("A transformer from
 * scratch", section 12.6 and "The LLM stack", section 13.4: a failing step
 * leaves the state it found valid).  The one-launch step (qwen3_decode_launches
 * == 1) hands activations between workgroups through bounded waits; a wait
 * that gives up (about 2 s) sets an error word on the device, and that step
 * and every later one-launch step of the handle write -1 to d_argmax and
 * advance no length, while qwen3_decode_step, which cannot see the device,
 * has already counted them.  This call waits for `stream`, reads the word,
 * and returns QWEN3_OK if it is clear; otherwise it sets every host length
 * back to the device's (the length before the first failed step), clears
 * the word, and returns QWEN3_E_DEVICE, after which steps run again.
 * QWEN3_OK at once for handles without the one-launch step. */
int qwen3_step_status(qwen3_t* h, void* stream);

/* Test hook for the failure path above: sets the error word on `stream`,
 * exactly as a wait that gave up would, so that the next one-launch step
 * fails without waiting.  QWEN3_E_INVALID_ARGUMENT for handles without the
 * one-launch step. */
int qwen3_inject_step_error(qwen3_t* h, void* stream);

/* Host-side KV length of `seq` ("The LLM stack (fucina_llm)", section 13.4:
 * the cache's len, the next append position); it counts every enqueued
 * append, so after a failed one-launch step it is right again only once
 * qwen3_step_status has reported the failure. */
int qwen3_kv_len(const qwen3_t* h, int32_t seq, int32_t* out);

/* Copy layer `layer` of sequence `seq`'s KV cache, positions [0, len), to
 * d_k and d_v, each f32 [kv_heads, len, head_dim] (bf16 caches are widened
 * exactly).  K rows are post-RoPE, V rows raw ("A transformer from scratch",
 * section 12.4).  Enqueued on `stream`; len is the host-side length. */
int qwen3_kv_export(const qwen3_t* h, int32_t seq, int32_t layer, float* d_k, float* d_v, void* stream);

/* Benchmark hook: enqueue `reps` launches of one kernel of sequence `seq`'s
 * decode step, in the step's own launch configuration at the sequence's
 * current length, so that its duration can be timed with events on
 * `stream`.  kind: 0 fused QKV GEMV, 1 decode attention, 2 o_proj GEMV,
 * 3 gate/up SwiGLU GEMV, 4 down GEMV (all of layer `layer`), 5 tied lm_head
 * with the argmax.  Side effects stay in the library's scratch buffers and
 * in cache row `len` (which the next decode step rewrites); no length is
 * advanced.  Enqueue after at least one decode step of `seq`. */
int qwen3_replay_kernel(qwen3_t* h, int32_t seq, int32_t kind, int32_t layer, int32_t reps, void* stream);

/* Achievable-peak probes, the measured figures the roofline fractions are
 * also given against (the vendor's peaks are the other).  qwen3_peak_copy:
 * copies `bytes` (a multiple of 16) from d_src to d_dst (device buffers that
 * do not overlap), a streaming kernel whose HBM traffic is 2 * bytes.
 * qwen3_peak_read: reads `bytes` (a multiple of 16) at d_src and writes
 * wrapping sums of its 32-bit words, one per wavefront, into d_out, which
 * holds qwen3_peak_read_partials() uint32 (entries past the launch's
 * wavefronts are left as they were; the partials' wrapping total is the
 * buffer's).  qwen3_peak_mfma_i8: `workgroups` workgroups of four wavefronts, each
 * wavefront `iters` rounds of four independent int8 MFMAs (32x32x32) on
 * operands every byte of which is the low byte of `fill` (b, read as a
 * signed 8-bit value); every lane writes 2048 * b * b * iters (wrapping as
 * int32) to d_out, which holds
 * 256 * workgroups int32.  qwen3_peak_mfma_i8_ops gives the int8 operations
 * of such a launch (two per multiply-add), 0 for invalid counts.  Both
 * launches are enqueued on `stream` to be timed with events there. */
int qwen3_peak_copy(const void* d_src, void* d_dst, size_t bytes, void* stream);
int qwen3_peak_read(const void* d_src, size_t bytes, uint32_t* d_out, void* stream);
int32_t qwen3_peak_read_partials(void);
int qwen3_peak_mfma_i8(int32_t* d_out, int32_t workgroups, int32_t iters, int32_t fill, void* stream);
double qwen3_peak_mfma_i8_ops(int32_t workgroups, int32_t iters);

/* Thread-local description of the last error ("" if none). */
const char* qwen3_last_error(void);

/* Kernel launches one qwen3_decode_step enqueues: 1 when the model's shape
 * has the one-launch (persistent) decode step and the device can hold its
 * grid resident (every CU holds one of its workgroups), else the per-kernel
 * step's count (one embedding launch, five launches per layer, one lm_head
 * launch).  Host-only; -1 on a null handle. */
int32_t qwen3_decode_launches(const qwen3_t* h);

/* ---- op-level entry points (kernel-boundary parity and input prep) ------- */

/* Q8_0 encoder ("Model files and quantization", section 11.7) of n f32
 * values (n a multiple of 32) into n/32 wire blocks (34 bytes each) at
 * d_blocks: amax; d = amax/127 (f32); inv = d == 0 ? 0 : 1/d (f32);
 * q = clamp(round-half-even(v*inv), -127, 127); stored scale f16(d) (RNE).
 * Non-finite input gives unspecified codes. */
int qwen3_q8_0_encode(const float* d_x, int64_t n, void* d_blocks, void* stream);

/* f32 -> bf16 (round half to even) of n values: input prep for bf16 models. */
int qwen3_bf16_encode(const float* d_x, int64_t n, uint16_t* d_out, void* stream);

/* Repack a Q8_0 matrix [rows, k] from wire blocks into the library's planes:
 * d_qs int8 [rows, k] and d_scale f16 [rows, k/32] (rows*k bytes and
 * rows*k/16 bytes).  k a multiple of 32. */
int qwen3_q8_0_repack(const void* d_blocks, int64_t rows, int64_t k, int8_t* d_qs,
                      uint16_t* d_scale, void* stream);

/* The Q8_0 linear on repacked planes: y[t, :] = linear(x[t, :]) for t < m,
 * x f32 [m, k], y f32 [m, n].  m == 1 runs the decode GEMV kernel, 2..64
 * rows the small-M GEMM, more rows the prefill GEMM (the same kernels the
 * model uses).  k % 128 == 0; for m > 64 also n % 128 == 0.  d_work:
 * scratch of qwen3_linear_work_bytes(m, k) bytes. */
size_t qwen3_linear_work_bytes(int64_t m, int64_t k);
int qwen3_q8_0_linear(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs,
                      const uint16_t* d_scale, int64_t n, float* d_y, void* d_work, void* stream);

/* The same Q8_0 linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no d_work argument; the scratch is a fixed array of
 * QWEN3_LINEAR_NOALLOC_SCRATCH_BYTES in device memory that each GPU holds
 * until the process ends.  Arguments, layouts and results are those of
 * qwen3_q8_0_linear (the same kernels run).  m > 1 with
 * qwen3_linear_work_bytes(m, k) above the limit is
 * QWEN3_E_INVALID_ARGUMENT, before any launch.  It calls no allocator.
 * Every call on one GPU uses that GPU's one array, so calls that overlap on
 * one GPU (two streams, two threads) race; calls in one stream do not. */
#define QWEN3_LINEAR_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int qwen3_q8_0_linear_noalloc(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs,
                              const uint16_t* d_scale, int64_t n, float* d_y, void* stream);

/* Test hook for the integer path: quantise x [m, k] the way the linears do
 * (d_qa int8 [m, k], d_da f16 bits [m, k/32]) and write every integer block
 * dot S[t, j, b] = sum_i qa[t, 32b+i] * qw[j, 32b+i] to d_s int32 [m, n, k/32],
 * using the same device code as the decode GEMV. */
int qwen3_q8_0_block_dots(const float* d_x, int64_t m, int64_t k, const int8_t* d_qs, int64_t n,
                          int8_t* d_qa, uint16_t* d_da, int32_t* d_s, void* stream);

/* The bf16-weight linear the bf16 models use (prefill and batched decode):
 * y[t, j] = f32( sum_i w[j, i] * x[t, i] ) for t < m, j < n, with x f32
 * [m, k] (row stride k), w bf16 bits [n, k] widened exactly, every product
 * and the sum in f64, rounded once (the exact in-register widening of the
 * "fucina_llm" reference page, section 13).  k % 32 == 0; y f32 [m, n]. */
int qwen3_bf16_linear(const float* d_x, int64_t m, int64_t k, const uint16_t* d_w, int64_t n,
                      float* d_y, void* stream);

/* ---- sampling ----------------------------------------------------------------
 * The sampling pipeline of Fucina course, "A transformer from scratch",
 * section 12.6 and Fucina reference, "The LLM stack (fucina_llm)", section
 * 13.6, on the device, in its fixed order: repetition / frequency / presence
 * penalties over the last repeat_last_n history tokens (each distinct token
 * once, with its count), the greedy shortcut (temperature <= 0: the argmax,
 * lowest id among equal maxima), top-k (at most 256 candidates), the
 * temperature softmax, top-p, min-p and one draw.  top_k == 0 is the exact
 * nucleus: probabilities carry the whole-vocabulary denominator and the
 * candidate window grows four-fold (256, 1024, 4096, 16384, 65536, ...) up
 * to the whole vocabulary until it holds the top_p mass, so no tail is cut.
 * Candidates are ordered by logit, ties by lower
 * id; the softmax and every sum are f64; the draw takes the first candidate
 * whose cumulative probability exceeds u times the kept total. */
typedef struct qwen3_sampler_config {
  float temperature;      /* <= 0: greedy */
  int32_t top_k;          /* 0: the exact nucleus; otherwise min(top_k, 256) candidates */
  float top_p;            /* (0, 1]; 1 disables */
  float min_p;            /* [0, 1]; 0 disables */
  float repeat_penalty;   /* > 0; 1 disables */
  float freq_penalty;     /* per-count subtraction */
  float presence_penalty; /* flat subtraction for a token present in the window */
  int32_t repeat_last_n;  /* penalty window, [0, 4096] */
} qwen3_sampler_config;

/* One token per row: d_logits f32 [n, vocab] (penalised in place, as the
 * pages' sampler does), d_history int32 [n, history_stride] with the first
 * d_history_len[r] entries of row r valid, most recent last (NULL: no
 * penalties), d_uniform f32 [n] one uniform in [0, 1) per row (the draw's
 * random number; unused when greedy, may then be NULL), d_tokens int32 [n]
 * out, d_work device scratch of qwen3_sample_work_bytes(n, vocab) bytes
 * (caller-owned, 256-byte aligned; each row's candidates per slice of 4096
 * logits, and 8 * vocab bytes per row for an exact-nucleus window wider than
 * 4096 candidates).  QWEN3_E_INVALID_ARGUMENT for a null or out-of-range
 * argument. */
size_t qwen3_sample_work_bytes(int32_t n, int32_t vocab);
int qwen3_sample(float* d_logits, int32_t n, int32_t vocab, const qwen3_sampler_config* cfg,
                 const int32_t* d_history, int32_t history_stride, const int32_t* d_history_len,
                 const float* d_uniform, int32_t* d_tokens, void* d_work, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QWEN3_Q8_H */
