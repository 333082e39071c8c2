"""Pins of the oracle's whole forward pass (CPU only, tiny shape).

The model-level pins are invariants the architecture fixes, each chosen so
that a plausible wiring mistake fails it:
  * cached decode == cacheless recompute ("A transformer from scratch",
    12.4, third contract) -- catches KV append/advance/position bugs;
  * causality (12.3.5) -- later tokens never change earlier logits;
  * translation invariance of RoPE scores (12.3.4) -- shifting every
    position by s leaves the logits unchanged;
  * per-head Q/K RMSNorm (minfer plan 2.2) makes the model blind to the
    scale of Wq and Wk (control: Wv is not normalised);
  * SwiGLU gates with silu(gate), up is linear (12.3.6) -- scaling up by 2
    and down by 1/2 is invisible, scaling gate is not;
  * V and o_proj are linear -- scaling Wv by 2 and Wo by 1/2 is invisible;
  * the final norm weight scales the logits exactly;
  * with every block's output projection zeroed, the residual stream is the
    embedding and the tied head (12.3.1) scores the input token highest.
"""

import numpy as np
import pytest

from conftest import read_golden
from oracle import model as om
from synthetic import QWEN3_0_6B, QWEN3_8B, TINY, gen_prompt, gen_weights, tensor_specs


@pytest.fixture(scope="module")
def tiny_weights():
    return gen_weights(TINY, 101)


@pytest.fixture(scope="module")
def tiny(tiny_weights):
    return om.Model(TINY, tiny_weights)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / (np.max(b) - np.min(b))


def test_projection_widths():
    facts = {r[0]: int(float(r[1])) for r in read_golden("model_facts.txt")}
    spec = dict(tensor_specs(QWEN3_0_6B))
    assert spec["blk.0.attn_q"] == (facts["q_width"], 1024)
    assert spec["blk.0.attn_k"] == spec["blk.0.attn_v"] == (facts["kv_width"], 1024)
    assert spec["blk.0.attn_output"] == (facts["o_out"], facts["o_in"])
    assert spec["blk.0.attn_q_norm"] == (128,)
    t = dict(tensor_specs(TINY))
    assert t["blk.0.attn_q"] == (256, 256) and t["blk.0.attn_k"] == (128, 256)
    assert t["blk.1.attn_output"] == (256, 256) and t["blk.1.ffn_down"] == (256, 768)
    assert "output.weight" not in dict(tensor_specs(QWEN3_8B))  # tied head


def test_kv_bytes_per_position():
    facts = {r[0]: int(float(r[1])) for r in read_golden("model_facts.txt")}
    s = QWEN3_0_6B
    per_elem_positions = s.num_layers * 2 * s.num_key_value_heads * s.head_dim
    assert per_elem_positions * 2 == facts["kv_bytes_per_position_f16"]
    assert per_elem_positions * 4 == 229_376  # f32 cache
    c = om.KVCache(s.num_layers, s.num_key_value_heads, s.head_dim, 3)
    assert sum(a.nbytes for a in c.k + c.v) == 3 * per_elem_positions * 4


def test_kv_cache_contract_golden():
    rows = {r[0]: r[1:] for r in read_golden("kv_cache_contract.txt")}
    L, kvh, hd, cap = map(int, rows["geometry"])
    c = om.KVCache(L, kvh, hd, cap)
    n, kval, vval = int(rows["append"][0]), float(rows["append"][1]), float(rows["append"][2])
    c.append_layer(0, np.full((n, kvh, hd), kval, np.float32), np.full((n, kvh, hd), vval, np.float32))
    assert c.len == 0  # append does not advance
    c.advance(n)
    seq = read_golden("kv_cache_contract.txt")
    assert c.len == int(seq[2][1])
    assert c.k_slice(0, c.len).size == int(rows["slice_elements"][0])
    c.truncate(int(rows["truncate"][0]))
    assert c.len == int(seq[5][1])


def test_forward_error_contract(tiny):
    c = tiny.new_cache(8)
    with pytest.raises(om.InvalidSequenceLength):
        tiny.forward([1, 2], c, pos0=3)
    with pytest.raises(om.KvCacheOverflow):
        tiny.forward(list(range(9)), c)
    assert c.len == 0 and np.all(c.k[0] == 0)
    tiny.forward([1, 2, 3], c, pos0=0)
    assert c.len == 3


def test_cached_equals_recompute(tiny):
    toks = gen_prompt(TINY.vocab_size, 12, seed=5)
    full = tiny.forward_uncached(toks)[0]
    c = tiny.new_cache(16)
    one = tiny.forward(toks, c)[0]
    c2 = tiny.new_cache(16)
    tiny.forward(toks[:7], c2)
    for t in toks[7:-1]:
        tiny.forward([t], c2)
    split = tiny.forward(toks[-1:], c2)[0]
    assert _rel(one, full) <= 1e-6 and _rel(split, full) <= 1e-6
    assert np.argmax(one) == np.argmax(full) == np.argmax(split)


def test_causality(tiny):
    a = gen_prompt(TINY.vocab_size, 10, seed=6)
    b = a.copy()
    b[6:] = gen_prompt(TINY.vocab_size, 4, seed=7)
    la = tiny.forward_uncached(a, all_logits=True)
    lb = tiny.forward_uncached(b, all_logits=True)
    assert _rel(la[:6], lb[:6]) <= 1e-6
    assert _rel(la[6:], lb[6:]) > 1e-3


def test_position_shift_invariance(tiny):
    toks = gen_prompt(TINY.vocab_size, 9, seed=8)
    l0 = tiny.forward_uncached(toks, pos0=0, all_logits=True)
    for s in (1, 37, 3000):
        assert _rel(tiny.forward_uncached(toks, pos0=s, all_logits=True), l0) <= 2e-3


def _variant(weights, **scales):
    w = dict(weights)
    for key, factor in scales.items():
        for name in list(w):
            if name.endswith("." + key) or name == key:
                w[name] = (w[name] * np.float32(factor)).astype(np.float32)
    return om.Model(TINY, w)


@pytest.fixture(scope="module")
def tiny_logits(tiny):
    toks = gen_prompt(TINY.vocab_size, 10, seed=9)
    return toks, tiny.forward_uncached(toks, all_logits=True)


def test_qk_norm_removes_projection_scale(tiny_weights, tiny_logits):
    toks, ref = tiny_logits
    for key in ("attn_q", "attn_k"):
        got = _variant(tiny_weights, **{key: 2.0}).forward_uncached(toks, all_logits=True)
        assert _rel(got, ref) <= 1e-4
    control = _variant(tiny_weights, attn_v=2.0).forward_uncached(toks, all_logits=True)
    assert _rel(control, ref) > 1e-2


def test_swiglu_up_is_linear_gate_is_not(tiny_weights, tiny_logits):
    toks, ref = tiny_logits
    got = _variant(tiny_weights, ffn_up=2.0, ffn_down=0.5).forward_uncached(toks, all_logits=True)
    assert _rel(got, ref) <= 1e-6
    ctrl = _variant(tiny_weights, ffn_gate=2.0, ffn_down=0.5).forward_uncached(toks, all_logits=True)
    assert _rel(ctrl, ref) > 1e-3


def test_value_and_output_projection_are_linear(tiny_weights, tiny_logits):
    toks, ref = tiny_logits
    got = _variant(tiny_weights, attn_v=2.0, attn_output=0.5).forward_uncached(toks, all_logits=True)
    assert _rel(got, ref) <= 1e-6


def test_output_norm_scales_logits_exactly(tiny_weights, tiny_logits):
    toks, ref = tiny_logits
    got = _variant(tiny_weights, output_norm=2.0).forward_uncached(toks, all_logits=True)
    assert np.array_equal(got, ref * np.float32(2.0))


def test_zeroed_blocks_leave_embedding_and_tied_head(tiny_weights):
    m = _variant(tiny_weights, attn_output=0.0, ffn_down=0.0)
    toks = gen_prompt(TINY.vocab_size, 6, seed=10)
    logits = m.forward_uncached(toks, all_logits=True)
    direct = m.head(m.embed(toks))
    assert np.array_equal(logits, direct)
    assert list(np.argmax(logits, axis=1)) == list(toks)


def test_generate_protocol(tiny):
    prompt = gen_prompt(TINY.vocab_size, 5, seed=11)
    c = tiny.new_cache(16)
    toks, logits = tiny.generate(prompt, 3, c)
    assert len(toks) == 4 and c.len == 5 + 3
    assert toks[0] == np.argmax(tiny.forward_uncached(prompt)[0])
    seq = list(prompt) + list(toks[:3])
    assert toks[3] == np.argmax(tiny.forward_uncached(seq)[0])


def test_bf16_model_cached_equals_recompute():
    shape = TINY.with_(name="tiny-bf16", weight_type="bf16", kv_type="bf16")
    m = om.Model(shape, gen_weights(shape, 501))
    toks = gen_prompt(shape.vocab_size, 9, seed=12)
    full = m.forward_uncached(toks)[0]
    c = m.new_cache(12)
    m.forward(toks[:5], c)
    for t in toks[5:-1]:
        m.forward([t], c)
    got = m.forward(toks[-1:], c)[0]
    assert _rel(got, full) <= 1e-6
    # bf16 cache rows really are bf16 values
    k = c.k[0][: c.len]
    assert np.all((k.view(np.uint32) & 0xFFFF) == 0)


# ---- q8_0 KV cache ("The LLM stack (fucina_llm)", section 13.4; "A transformer
# from scratch", section 12.4) ------------------------------------------------------

TINY_Q8KV = TINY.with_(name="tiny-q8kv", kv_type="q8_0")


def _q8_exact_rows(shape, seed):
    """Rows that Q8_0 holds without loss: per 32-block an f16 scale d and int
    codes in [-127, 127] with one code at +-127 (so max|x| / 127 == d)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(-127, 128, size=shape).astype(np.int64)
    codes.reshape(-1, 32)[:, 0] = 127
    d = rng.uniform(0.01, 0.05, size=shape[:-1] + (shape[-1] // 32,)).astype(np.float16).astype(np.float32)
    return (codes.reshape(shape[:-1] + (shape[-1] // 32, 32)) * d[..., None]).reshape(shape).astype(np.float32)


def test_q8_kv_store_rounds_per_block():
    c = om.KVCache(1, 2, 64, 8, "q8_0")
    exact = _q8_exact_rows((3, 2, 64), 1)
    c.append_layer(0, exact, exact)
    assert np.array_equal(c.k[0][:3], exact)  # nothing lost for Q8_0-exact rows
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((2, 2, 64)).astype(np.float32)
    c.append_layer(0, rows, rows)  # overwrites rows 0..1 (len is still 0)
    got = c.k[0][:2].reshape(-1, 32).astype(np.float64)
    blocks = rows.reshape(-1, 32).astype(np.float64)
    d = np.max(np.abs(blocks), axis=1) / 127.0
    # per element within half a code step (plus the f16 rounding of d)
    assert np.all(np.abs(got - blocks) <= (0.5 + 127 * 2.0**-11) * d[:, None] * (1 + 1e-6))
    assert not np.array_equal(got, blocks)
    with pytest.raises(ValueError):
        om.KVCache(1, 2, 48, 8, "q8_0")  # head_dim must be whole 32-blocks


def test_q8_kv_integer_scores_are_the_dequantised_dot():
    """The integer score path (query quantised per 32-block, q8 x q8 block dots
    scaled by d_q * d_k) equals the dot of the dequantised rows."""
    from oracle import q8_0 as oq

    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 128)).astype(np.float32)
    keys = rng.standard_normal((40, 128)).astype(np.float32)
    qa, dq = oq.encode(q)
    kq, dk = oq.encode(keys)
    S = oq.block_dots(qa, kq)[0].astype(np.float64)  # [40, 4]
    integer = np.sum(S * dq.astype(np.float64)[0][None, :] * dk.astype(np.float64), axis=1)
    deq = oq.decode(kq, dk).astype(np.float64) @ oq.decode(qa, dq).astype(np.float64)[0]
    assert np.allclose(integer, deq, rtol=1e-13, atol=1e-13)
    # and the quantised query is what attention_query hands to the scores
    assert np.array_equal(om.attention_query(q.reshape(1, 1, 128), "q8_0").reshape(1, 128), oq.decode(qa, dq))


def test_q8_kv_attention_equals_f32_on_lossless_rows():
    """With queries, keys and values that Q8_0 holds exactly, a decode step over
    a q8_0 cache is the f32 cache's step, and a multi-token step keeps its f32
    query (the dequantising prefill path)."""
    from oracle import ops

    k = _q8_exact_rows((9, 2, 64), 4)
    v = _q8_exact_rows((9, 2, 64), 5)
    q1 = _q8_exact_rows((1, 4, 64), 6)
    for kvt in ("f32", "q8_0"):
        assert np.array_equal(om.kv_store(k, kvt), k)
    assert np.array_equal(om.attention_query(q1, "q8_0"), q1)
    qn = np.random.default_rng(7).standard_normal((3, 4, 64)).astype(np.float32)
    assert np.array_equal(om.attention_query(qn, "q8_0"), qn)  # T > 1: unquantised
    a = ops.attention(om.attention_query(q1, "q8_0"), om.kv_store(k, "q8_0"), om.kv_store(v, "q8_0"), [8])
    b = ops.attention(q1, k, v, [8])
    assert np.array_equal(a, b)


def test_q8_kv_model_decode_steps_quantise_the_query():
    """Model level: a q8_0-KV decode step equals attention over the dequantised
    cache with the quantised query, and prefill logits stay within the Q8_0
    loss of the f32-KV model (the cache differs, the tokens mostly do not)."""
    w = gen_weights(TINY_Q8KV, 101)
    m8 = om.Model(TINY_Q8KV, w)
    m32 = om.Model(TINY, w)
    toks = gen_prompt(TINY.vocab_size, 24, seed=9)
    c8, c32 = m8.new_cache(32), m32.new_cache(32)
    p8, p32 = m8.forward(toks, c8)[0], m32.forward(toks, c32)[0]
    assert 0 < _rel(p8, p32) <= 0.03
    # a single-token step: same as a step whose query is explicitly quantised
    # and whose attention reads the stored (dequantised) rows
    import copy

    c8b = copy.deepcopy(c8)
    tok = int(np.argmax(p8))
    d8 = m8.forward([tok], c8)[0]
    assert c8.len == 25 and np.all(np.isfinite(d8))
    orig = om.attention_query
    try:  # the same step with the query left unquantised differs
        om.attention_query = lambda q, kvt: q
        d8_plain = m8.forward([tok], c8b)[0]
    finally:
        om.attention_query = orig
    assert 0 < _rel(d8, d8_plain) <= 0.03
    # the cached K rows are Q8_0 round trips of the f32 model's K rows
    k32 = c32.k[0][:24]
    assert np.array_equal(c8.k[0][:24], om.kv_store(k32, "q8_0"))
