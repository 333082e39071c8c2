// Launch interface of the one-launch decode step (k_decode_persistent.hip).
// Internal to the library (not part of the C ABI); kept apart from
// kernels.h so that the step's source is this header, the kernel file and
// qdevice.h alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// One-launch decode step (see k_decode_persistent.hip).
constexpr int kPersistWorkgroups = 256;
struct PLayer {  // a layer's repacked weights
  const int8_t *qkv_qs, *o_qs, *gu_qs, *dn_qs;
  const uint16_t *qkv_sc, *o_sc, *gu_sc, *dn_sc;
  const float *attn_norm, *q_norm, *k_norm, *ffn_norm;
};
struct PersistArgs {
  const PLayer* layers;  // device [L]
  int L, V;
  float eps;
  double scale;  // 1/sqrt(hd)
  const int8_t* emb_qs;
  const uint16_t* emb_sc;
  const float* out_norm;
  const double *rope_cos, *rope_sin;
  void* kv;
  const int64_t* seq_base;
  const int32_t* seq_cap;
  int32_t* len;
  int seq;
  const int32_t* token;  // device [1]
  float* logits;         // [V] or null
  int32_t* argmax;       // [1]
  unsigned long long *xa, *xc, *qkv, *att, *h;  // (value, epoch) words
  // attention partials of every split as (32-bit half, epoch) words:
  // [nkv][splits per KV head][G][hd + 2 (o..., m, l)][2 (low, high half)]
  unsigned long long* part;
  unsigned* err;         // set on a timed-out wait
  unsigned pstep;        // step counter (epochs) at the launch's first step
  int nsteps;            // greedy steps in this launch (>= 1)
  int32_t* tokens_out;   // [nsteps] the token of each step, or null
  // each workgroup's argmax key of the step as two (32-bit half, epoch) words
  unsigned long long* keys;  // [2 * kPersistWorkgroups]
};
struct PersistShape {
  int H, QW, F, HD, G;
};
namespace q8k {
int persist_max_ctx(const PersistShape& sh);  // 0: no persistent step for this shape
int persist_occupancy(const PersistShape& sh, bool kv_bf16);
hipError_t decode_persistent(const PersistShape& sh, bool kv_bf16, const PersistArgs& a, hipStream_t s);
}  // namespace q8k
