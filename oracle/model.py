"""The Qwen3 dense decoder forward pass (oracle; test infrastructure).

Order of operations ("A transformer from scratch", sections 12.3-12.4;
minfer "Qwen3 Support Plan", sections 2.1-2.2):

  x = embedding rows (Q8_0 rows dequantised exactly)
  per layer:
    a = rmsnorm(x, attn_norm)
    q, k, v = linear(a, Wq), linear(a, Wk), linear(a, Wv)
    q_h = rmsnorm(q_h, q_norm), k_g = rmsnorm(k_g, k_norm)   per head
    q, k = rope(q, pos), rope(k, pos)                        (v untouched)
    append k, v to this layer's cache rows [len, len + T)
    o = causal GQA attention of q over cache rows [0, len + T)
    x = x + linear(o, Wo)
    b = rmsnorm(x, ffn_norm)
    x = x + linear(swiglu(linear(b, Wgate), linear(b, Wup)), Wdown)
  len += T (once, after all layers)
  logits = linear(rmsnorm(x[last], output_norm), token_embd)  (tied head)
  token = lowest index of the maximum logit

`linear` is the Q8_0 linear (activations quantised per 32-block) for Q8_0
models, or the f32-activation x bf16-weight product for bf16 models.
"""

from __future__ import annotations

import numpy as np

from . import ops, q8_0


class InvalidSequenceLength(ValueError):
    pass


class KvCacheOverflow(ValueError):
    pass


class KVCache:
    """Per-layer post-RoPE K and raw V rows, [capacity, kv_heads, head_dim].

    Contract ("A transformer from scratch", section 12.4; "The LLM stack",
    section 13.4): every layer appends at the same base `len`; `advance(m)`
    runs once after all layers; `truncate(keep)` rewinds by lowering `len`;
    `reset()` sets len = 0.  kv_type "bf16" rounds rows to bf16 on store
    (widened on read); "f32" stores them as they are; "q8_0" stores each
    (position, head) row as head_dim/32 Q8_0 blocks ("A transformer from
    scratch", section 12.4, the q8_0 option; "The LLM stack (fucina_llm)",
    section 13.4), kept here as their exact dequantised values.
    """

    def __init__(self, num_layers: int, kv_heads: int, head_dim: int, capacity: int, kv_type: str = "f32"):
        if kv_type == "q8_0" and head_dim % q8_0.QK:
            raise ValueError("a q8_0 KV cache needs head_dim % 32 == 0")
        self.k = [np.zeros((capacity, kv_heads, head_dim), dtype=np.float32) for _ in range(num_layers)]
        self.v = [np.zeros((capacity, kv_heads, head_dim), dtype=np.float32) for _ in range(num_layers)]
        self.capacity = capacity
        self.kv_type = kv_type
        self.len = 0

    def _store(self, rows: np.ndarray) -> np.ndarray:
        return kv_store(rows, self.kv_type)

    def append_layer(self, layer: int, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        T = k_rows.shape[0]
        if self.len + T > self.capacity:
            raise KvCacheOverflow(f"len {self.len} + {T} > capacity {self.capacity}")
        if k_rows.shape[1:] != self.k[layer].shape[1:] or v_rows.shape != k_rows.shape:
            raise ValueError("KV row shape mismatch")
        self.k[layer][self.len : self.len + T] = self._store(k_rows)
        self.v[layer][self.len : self.len + T] = self._store(v_rows)

    def advance(self, m: int) -> None:
        self.len += m

    def truncate(self, keep_len: int) -> None:
        if keep_len < self.len:
            self.len = keep_len

    def reset(self) -> None:
        self.len = 0

    def k_slice(self, layer: int, n: int) -> np.ndarray:
        return self.k[layer][:n]

    def v_slice(self, layer: int, n: int) -> np.ndarray:
        return self.v[layer][:n]


def kv_store(rows: np.ndarray, kv_type: str) -> np.ndarray:
    """K or V rows [..., head_dim] as the cache holds them (f32 values)."""
    rows = np.asarray(rows, dtype=np.float32)
    if kv_type == "bf16":
        return ops.bf16_round(rows)
    if kv_type == "q8_0":
        return q8_0.decode(*q8_0.encode(rows))
    return rows


def attention_query(q: np.ndarray, kv_type: str) -> np.ndarray:
    """The query as the attention scores use it.  With a q8_0 cache a
    single-token step takes the integer score path: each head's query is
    quantised per 32-block like an activation and dotted with the cached K
    codes block by block, V dequantised as it is accumulated; a step of
    several tokens (prefill, the all-logits verify) keeps the dequantising
    path, its f32 query against the dequantised cache ("The LLM stack
    (fucina_llm)", section 13.4, the q8_0 option).  Since sum_b d_q,b d_k,b
    S_b is the dot of the two dequantised rows, the oracle uses the
    dequantised query (exact in f32) with the dequantised keys.  q is
    [T, heads, head_dim]; T == 1 is the single-token step."""
    if kv_type == "q8_0" and q.shape[0] == 1:
        return q8_0.decode(*q8_0.encode(q))
    return q


class Model:
    """Oracle model built from f32 generator weights (dict name -> array).

    Q8_0 models quantise every projection and the embedding with the Q8_0
    encoder; bf16 models round them to bf16.  Norm weights stay f32.
    """

    def __init__(self, shape, weights: dict, threads: int = 1, keep_f64: bool = False):
        """threads > 1 encodes the tensors in a thread pool (same results;
        the encoder is independent per tensor).  keep_f64 keeps every matrix
        also widened to f64 (8 bytes per weight), so that many decode steps
        do not widen the weights on every call; results are the same."""
        self.shape = shape
        if shape.weight_type not in ("q8_0", "bf16"):
            raise ValueError(shape.weight_type)

        def prep(arr):
            if arr.ndim == 1:
                return np.asarray(arr, dtype=np.float32)
            if shape.weight_type == "q8_0":
                return q8_0.Q8Weight(arr)
            return ops.bf16_round(arr)

        if threads > 1:
            import concurrent.futures as cf

            with cf.ThreadPoolExecutor(max_workers=threads) as ex:
                futs = {name: ex.submit(prep, arr) for name, arr in weights.items()}
                self.w = {name: f.result() for name, f in futs.items()}
        else:
            self.w = {name: prep(arr) for name, arr in weights.items()}
        if keep_f64:
            for name, w in self.w.items():
                if isinstance(w, q8_0.Q8Weight):
                    w.keep_f64()
                elif w.ndim == 2:
                    self.w[name] = w.astype(np.float64)

    # -- building blocks -------------------------------------------------
    def linear(self, x: np.ndarray, name: str) -> np.ndarray:
        w = self.w[name]
        if isinstance(w, q8_0.Q8Weight):
            return q8_0.linear(x, w)
        return ops.bf16_linear(x, w)

    def embed(self, tokens) -> np.ndarray:
        w = self.w["token_embd"]
        ids = np.asarray(tokens, dtype=np.int64)
        if np.any(ids < 0) or np.any(ids >= self.shape.vocab_size):
            raise ValueError("token id out of range")
        if isinstance(w, q8_0.Q8Weight):
            return w.rows(ids).astype(np.float32)
        return w[ids].astype(np.float32)

    def new_cache(self, capacity: int) -> KVCache:
        s = self.shape
        return KVCache(s.num_layers, s.num_key_value_heads, s.head_dim, capacity, s.kv_type)

    def qkv(self, layer: int, x: np.ndarray, positions):
        """Attention-input half of a layer: norm, projections, per-head norm,
        RoPE.  Returns q [T, nh, hd], k [T, nkv, hd] (post-RoPE), v."""
        s = self.shape
        p = f"blk.{layer}."
        a = ops.rmsnorm(x, self.w[p + "attn_norm"], s.rms_norm_eps)
        T = x.shape[0]
        q = self.linear(a, p + "attn_q").reshape(T, s.num_attention_heads, s.head_dim)
        k = self.linear(a, p + "attn_k").reshape(T, s.num_key_value_heads, s.head_dim)
        v = self.linear(a, p + "attn_v").reshape(T, s.num_key_value_heads, s.head_dim)
        q = ops.rmsnorm(q, self.w[p + "attn_q_norm"], s.rms_norm_eps)
        k = ops.rmsnorm(k, self.w[p + "attn_k_norm"], s.rms_norm_eps)
        q = ops.rope(q, positions, s.rope_theta)
        k = ops.rope(k, positions, s.rope_theta)
        return q, k, v

    def finish_layer(self, layer: int, x: np.ndarray, o: np.ndarray) -> np.ndarray:
        """o_proj + residual, then the SwiGLU FFN block + residual."""
        s = self.shape
        p = f"blk.{layer}."
        x = ops.add(x, self.linear(o, p + "attn_output"))
        b = ops.rmsnorm(x, self.w[p + "ffn_norm"], s.rms_norm_eps)
        h = ops.swiglu(self.linear(b, p + "ffn_gate"), self.linear(b, p + "ffn_up"))
        return ops.add(x, self.linear(h, p + "ffn_down"))

    def head(self, x_rows: np.ndarray) -> np.ndarray:
        """Final RMSNorm and the tied lm_head -> f32 logits [rows, V]."""
        h = ops.rmsnorm(x_rows, self.w["output_norm"], self.shape.rms_norm_eps)
        return self.linear(h, "token_embd")

    # -- entry points ------------------------------------------------------
    def forward(self, tokens, cache: KVCache, pos0: int | None = None, all_logits: bool = False) -> np.ndarray:
        """Cached forward step over `tokens` appended at cache.len.

        Requires pos0 == cache.len (else InvalidSequenceLength) and room in
        the cache (else KvCacheOverflow); on error the cache is unchanged.
        Returns logits [1, V] for the last token, or [T, V] if all_logits.
        """
        tokens = np.asarray(tokens, dtype=np.int64)
        T = tokens.shape[0]
        if T <= 0:
            raise InvalidSequenceLength("empty token list")
        if pos0 is not None and pos0 != cache.len:
            raise InvalidSequenceLength(f"pos0 {pos0} != cache len {cache.len}")
        if cache.len + T > cache.capacity:
            raise KvCacheOverflow(f"len {cache.len} + {T} > capacity {cache.capacity}")
        base = cache.len
        positions = np.arange(base, base + T)
        x = self.embed(tokens)
        for layer in range(self.shape.num_layers):
            q, k, v = self.qkv(layer, x, positions)
            cache.append_layer(layer, k, v)
            n = base + T
            q = attention_query(q, cache.kv_type)
            o = ops.attention(q, cache.k_slice(layer, n), cache.v_slice(layer, n), positions)
            x = self.finish_layer(layer, x, o)
        cache.advance(T)
        rows = x if all_logits else x[-1:]
        return self.head(rows)

    def forward_uncached(self, tokens, pos0: int = 0, all_logits: bool = False) -> np.ndarray:
        """Cacheless full recompute over `tokens` placed at positions
        pos0..pos0+T-1 (keys are the call's own tokens only)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        T = tokens.shape[0]
        positions = np.arange(pos0, pos0 + T)
        x = self.embed(tokens)
        for layer in range(self.shape.num_layers):
            q, k, v = self.qkv(layer, x, positions)
            kvt = self.shape.kv_type
            k, v, q = kv_store(k, kvt), kv_store(v, kvt), attention_query(q, kvt)
            o = ops.attention(q, k, v, positions, positions)
            x = self.finish_layer(layer, x, o)
        rows = x if all_logits else x[-1:]
        return self.head(rows)

    def generate(self, prompt, steps: int, cache: KVCache, keep_logits: bool = True):
        """Greedy protocol: one prefill of `prompt` (its argmax is generated
        token 1), then `steps` decode calls fed the previous argmax.
        Returns (tokens [steps + 1], list of logits [V])."""
        logits = self.forward(prompt, cache)[0]
        toks, outs = [], []
        for i in range(steps + 1):
            t = ops.argmax_lowest(logits)
            toks.append(t)
            if keep_logits:
                outs.append(logits)
            if i == steps:
                break
            logits = self.forward([t], cache)[0]
        return np.asarray(toks, dtype=np.int32), outs
