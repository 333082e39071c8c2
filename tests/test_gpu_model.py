"""End-to-end parity of the GPU forward pass against the CPU oracle.

Protocol ("prompt P, then N greedy decode steps"): one prefill of P (its
argmax is generated token 1) then N decode steps fed the previous argmax.
Tolerance: per step, max |logit_gpu - logit_oracle| <= 1e-3 x (max - min of
the oracle's logits); greedy tokens identical.
"""

import os

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, WORKLOADS, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY, 101)


@pytest.fixture(scope="module")
def tiny_ref(tiny_w):
    return om.Model(TINY, tiny_w)


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


def check_against_oracle(toks, logits, rtoks, rlogits):
    errs = [rel_err(a, b) for a, b in zip(logits, rlogits)]
    assert max(errs) <= TOL, f"logit errors {['%.1e' % e for e in errs]}"
    for a, b in zip(logits, rlogits):  # the GPU argmax is its own logits' argmax
        pass
    assert toks == list(rtoks), f"tokens {toks} != oracle {list(rtoks)}"


def test_tiny_workload_matches_oracle(tiny_w, tiny_ref):
    wl = WORKLOADS["tiny"]
    prompt = gen_prompt(TINY.vocab_size, wl.prompt_len, wl.prompt_seed)
    gpu = make(TINY, tiny_w, [wl.kv_capacity])
    toks, logits = gpu_generate(gpu, prompt, wl.decode_steps)
    rtoks, rlogits = tiny_ref.generate(prompt, wl.decode_steps, tiny_ref.new_cache(wl.kv_capacity))
    check_against_oracle(toks, logits, rtoks, rlogits)
    for lg, t in zip(logits, toks):
        assert int(np.argmax(lg)) == t
    assert gpu.kv_len() == wl.prompt_len + wl.decode_steps


def test_tiny_chunked_prefill_and_ragged_tail(tiny_w, tiny_ref):
    prompt = gen_prompt(TINY.vocab_size, 45, 7)  # 45 = 2 x 16 + ragged 13
    gpu = make(TINY, tiny_w, [64], max_batch_tokens=16)
    toks, logits = gpu_generate(gpu, prompt, 4)
    rtoks, rlogits = tiny_ref.generate(prompt, 4, tiny_ref.new_cache(64))
    check_against_oracle(toks, logits, rtoks, rlogits)


def test_tiny_multi_turn_prefill(tiny_w, tiny_ref):
    a, b = gen_prompt(TINY.vocab_size, 9, 8), gen_prompt(TINY.vocab_size, 6, 9)
    gpu = make(TINY, tiny_w, [32])
    gpu.prefill(a)
    lg, am = gpu.prefill(b)
    ref = tiny_ref.forward_uncached(np.concatenate([a, b]))[0]
    assert rel_err(lg.cpu().numpy(), ref) <= TOL
    assert gpu.kv_len() == 15


def test_tiny_reset_reproduces(tiny_w):
    prompt = gen_prompt(TINY.vocab_size, 20, 10)
    gpu = make(TINY, tiny_w, [40])
    t1, l1 = gpu_generate(gpu, prompt, 5)
    gpu.reset()
    assert gpu.kv_len() == 0
    t2, l2 = gpu_generate(gpu, prompt, 5)
    assert t1 == t2
    for a, b in zip(l1, l2):
        assert np.array_equal(a, b)


def test_tiny_graph_and_eager_decode_agree(tiny_w, monkeypatch):
    prompt = gen_prompt(TINY.vocab_size, 10, 11)
    g = make(TINY, tiny_w, [32])
    tg, lgr = gpu_generate(g, prompt, 6)
    monkeypatch.setenv("QWEN3_NO_GRAPH", "1")
    e = make(TINY, tiny_w, [32])
    te, le = gpu_generate(e, prompt, 6)
    assert tg == te
    for a, b in zip(lgr, le):
        assert np.array_equal(a, b)


def test_tiny_errors_leave_state_unchanged(tiny_w):
    from quantized_q8_dequant_amd import Qwen3Error

    prompt = gen_prompt(TINY.vocab_size, 14, 12)
    gpu = make(TINY, tiny_w, [16])
    gpu.prefill(prompt)
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill(gen_prompt(TINY.vocab_size, 3, 13))
    assert e.value.code == -7
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill([1, TINY.vocab_size])
    assert e.value.code == -8
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill([])
    assert e.value.code == -6
    assert gpu.kv_len() == 14
    gpu.decode_step()
    gpu.decode_step()
    assert gpu.kv_len() == 16
    with pytest.raises(Qwen3Error) as e:
        gpu.decode_step()
    assert e.value.code == -7
    assert gpu.kv_len() == 16


def test_tiny_bf16_cache_matches_oracle():
    shape = TINY.with_(name="tiny-bf16kv", kv_type="bf16")
    w = gen_weights(shape, 101)
    ref = om.Model(shape, w)
    prompt = gen_prompt(shape.vocab_size, 24, 14)
    gpu = make(shape, w, [48])
    toks, logits = gpu_generate(gpu, prompt, 8)
    rtoks, rlogits = ref.generate(prompt, 8, ref.new_cache(48))
    check_against_oracle(toks, logits, rtoks, rlogits)


def test_tiny_batched_decode_matches_single(tiny_w, tiny_ref):
    prompts = [gen_prompt(TINY.vocab_size, n, 20 + n) for n in (5, 17, 33)]
    gpu = make(TINY, tiny_w, [48, 48, 48])
    first = []
    for s, p in enumerate(prompts):
        _, am = gpu.prefill(p, seq=s)
        first.append(int(am.item()))
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((3, TINY.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(3, dtype=torch.int32, device="cuda:0")
    seqs = [0, 1, 2]
    outs = []
    for _ in range(4):
        gpu.decode_batch(seqs, toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    for s, p in enumerate(prompts):
        rt, rl = tiny_ref.generate(p, 4, tiny_ref.new_cache(48))
        assert rt[0] == first[s]
        for i in range(4):
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL
            assert outs[i][1][s] == rt[i + 1]


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_prefill_and_decode_matches_oracle():
    wl = WORKLOADS["0.6b-decode"]
    w = gen_weights(QWEN3_0_6B, wl.weight_seed)
    prompt = gen_prompt(QWEN3_0_6B.vocab_size, wl.prompt_len, wl.prompt_seed)
    steps = 4
    gpu = make(QWEN3_0_6B, w, [wl.kv_capacity])
    toks, logits = gpu_generate(gpu, prompt, steps)
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    ref = om.Model(QWEN3_0_6B, w)
    del w
    rtoks, rlogits = ref.generate(prompt, steps, ref.new_cache(wl.kv_capacity))
    check_against_oracle(toks, logits, rtoks, rlogits)
