"""The q8_0 KV cache on the GPU against the CPU oracle ("The LLM stack
(fucina_llm)", section 13.4, the q8_0 option; "A transformer from scratch",
section 12.4).

Each cached (position, KV head) row is head_dim/32 Q8_0 blocks; single-token
steps score with the query quantised per head (the integer score path),
multi-token steps with the f32 query against the dequantised cache.  The
bar is the model tests' one: logits within 1e-3 of the oracle's range,
greedy tokens identical; the exported cache rows are whole Q8_0 blocks
(every value a code times its block's f16 scale).
"""

import os

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, WORKLOADS, gen_lengths, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3
TINY_Q8KV = TINY.with_(name="tiny-q8kv", kv_type="q8_0")


def progress(msg):
    print(f"[{os.path.basename(__file__)}] {msg}", flush=True)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def gpu_generate(model, prompt, steps, seq=0):
    lg, am = model.prefill(prompt, seq=seq)
    toks, logits = [int(am.item())], [lg.cpu().numpy().copy()]
    for _ in range(steps):
        lg, am = model.decode_step(seq=seq)
        toks.append(int(am.item()))
        logits.append(lg.cpu().numpy().copy())
    return toks, logits


def check(toks, logits, rtoks, rlogits):
    errs = [rel_err(a, b) for a, b in zip(logits, rlogits)]
    assert max(errs) <= TOL, f"logit errors {['%.1e' % e for e in errs]}"
    assert toks == list(rtoks), f"tokens {toks} != oracle {list(rtoks)}"


def assert_q8_blocks(x):
    """Every 32-block of x (f32) is codes in [-127, 127] times one f16 scale,
    one code at +-127 (or an all-zero block)."""
    b = x.reshape(-1, 32).astype(np.float64)
    amax = np.max(np.abs(b), axis=1)
    d = amax / 127.0
    assert np.array_equal(d.astype(np.float16).astype(np.float64), d)
    nz = d > 0
    codes = b[nz] / d[nz][:, None]
    assert np.array_equal(codes, np.rint(codes))


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY_Q8KV, 101)


@pytest.fixture(scope="module")
def tiny_ref(tiny_w):
    return om.Model(TINY_Q8KV, tiny_w)


@pytest.mark.parametrize("mbt", [0, 16])  # one chunk; 16-row chunks with a ragged tail
def test_tiny_q8kv_prefill_and_decode(tiny_w, tiny_ref, mbt):
    wl = WORKLOADS["tiny"]
    prompt = gen_prompt(TINY.vocab_size, 45, wl.prompt_seed)
    gpu = make(TINY_Q8KV, tiny_w, [72], max_batch_tokens=mbt)
    assert gpu.decode_launches() > 1  # the per-kernel decode step
    toks, logits = gpu_generate(gpu, prompt, 16)
    rtoks, rlogits = tiny_ref.generate(prompt, 16, tiny_ref.new_cache(72))
    check(toks, logits, rtoks, rlogits)
    for layer in range(TINY.num_layers):
        k, v = gpu.kv_export(0, layer)
        assert_q8_blocks(k.cpu().numpy())
        assert_q8_blocks(v.cpu().numpy())


def test_tiny_q8kv_cache_rows_match_the_oracle(tiny_w, tiny_ref):
    prompt = gen_prompt(TINY.vocab_size, 30, 91)
    gpu = make(TINY_Q8KV, tiny_w, [40])
    gpu.prefill(prompt)
    gpu.decode_step()
    cache = tiny_ref.new_cache(40)
    t = tiny_ref.forward(prompt, cache)[0]
    tiny_ref.forward([int(np.argmax(t))], cache)
    for layer in range(TINY.num_layers):
        k, v = gpu.kv_export(0, layer)  # [kv_heads, len, hd]
        rk = np.transpose(cache.k[layer][:31], (1, 0, 2))
        rv = np.transpose(cache.v[layer][:31], (1, 0, 2))
        # the same rows up to a code at a rounding boundary: compare to one code step
        step = np.max(np.abs(rk.reshape(-1, 32)), axis=1) / 127.0
        assert np.all(np.abs(k.cpu().numpy().reshape(-1, 32) - rk.reshape(-1, 32)) <= 1.01 * step[:, None] + 1e-7)
        step = np.max(np.abs(rv.reshape(-1, 32)), axis=1) / 127.0
        assert np.all(np.abs(v.cpu().numpy().reshape(-1, 32) - rv.reshape(-1, 32)) <= 1.01 * step[:, None] + 1e-7)


def test_tiny_q8kv_single_token_prefill_quantises_the_query(tiny_w, tiny_ref):
    """A one-token prefill call is a single-token step: integer score path."""
    a, b = gen_prompt(TINY.vocab_size, 11, 92), gen_prompt(TINY.vocab_size, 1, 93)
    gpu = make(TINY_Q8KV, tiny_w, [16])
    gpu.prefill(a)
    lg, _ = gpu.prefill(b)
    cache = tiny_ref.new_cache(16)
    tiny_ref.forward(a, cache)
    ref = tiny_ref.forward(b, cache)[0]
    assert rel_err(lg.cpu().numpy(), ref) <= TOL


LONG_SHAPES = {
    "g2": TINY_Q8KV,
    "g4": TINY_Q8KV.with_(name="tiny-q8kv-g4", num_attention_heads=8, num_key_value_heads=2),
    "g1": TINY_Q8KV.with_(name="tiny-q8kv-g1", num_attention_heads=4, num_key_value_heads=4),
}


@pytest.mark.parametrize("name", list(LONG_SHAPES))
def test_tiny_q8kv_long_context_verify(name):
    """300-token all-logits prefill, a 12-token verify (key-split attention
    over Q8_0 tiles), a rewind and three decode steps."""
    shape = LONG_SHAPES[name]
    w = gen_weights(shape, 103)
    ref = om.Model(shape, w)
    prompt = gen_prompt(shape.vocab_size, 300, 94)
    draft = gen_prompt(shape.vocab_size, 12, 95)
    gpu = make(shape, w, [340], max_batch_tokens=320)
    lg_p, _ = gpu.prefill_all_logits(prompt)
    lg_v, am_v = gpu.prefill_all_logits(draft)
    gpu.truncate(304)
    tok = am_v[3:4].clone()
    steps = []
    for _ in range(3):
        lg, am = gpu.decode_step(token=tok)
        steps.append(lg.cpu().numpy().copy())
        tok = am
    cache = ref.new_cache(340)
    rp = ref.forward(prompt, cache, all_logits=True)
    rv = ref.forward(draft, cache, all_logits=True)
    for a, b in ((lg_p.cpu().numpy(), rp), (lg_v.cpu().numpy(), rv)):
        errs = np.max(np.abs(a - b), axis=1) / (np.max(b, axis=1) - np.min(b, axis=1))
        assert errs.max() <= TOL, errs.max()
    cache.truncate(304)
    t = int(np.argmax(rv[3]))
    for i in range(3):
        r = ref.forward([t], cache)[0]
        assert rel_err(steps[i], r) <= TOL
        t = int(np.argmax(r))


@pytest.mark.parametrize("n", [4, 20])  # per-row GEMV, small-M GEMM
def test_tiny_q8kv_batched_decode(tiny_w, tiny_ref, n):
    lengths = gen_lengths(n, 1, 60, 96 + n)
    prompts = [gen_prompt(TINY.vocab_size, int(L), 500 + s) for s, L in enumerate(lengths)]
    gpu = make(TINY_Q8KV, tiny_w, [64] * n)
    first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((n, TINY.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(n, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(3):
        gpu.decode_batch(list(range(n)), toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    for s, p in enumerate(prompts):
        rt, rl = tiny_ref.generate(p, 3, tiny_ref.new_cache(64))
        assert rt[0] == first[s]
        for i in range(3):
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL, (s, i)
            assert outs[i][1][s] == rt[i + 1], (s, i)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_q8kv_prefill_and_decode():
    wl = WORKLOADS["0.6b-decode"]
    shape = QWEN3_0_6B.with_(name="qwen3-0.6b-q8kv", kv_type="q8_0")
    w = gen_weights(shape, wl.weight_seed)
    prompt = gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed)
    steps = 6
    gpu = make(shape, w, [wl.prompt_len + steps + 1])
    progress("gpu")
    toks, logits = gpu_generate(gpu, prompt, steps)
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    progress("oracle")
    ref = om.Model(shape, w)
    del w
    rtoks, rlogits = ref.generate(prompt, steps, ref.new_cache(wl.prompt_len + steps + 1))
    check(toks, logits, rtoks, rlogits)
