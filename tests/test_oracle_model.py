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
