"""n greedy decode steps in one call (qwen3_decode_greedy) against n single
decode steps fed their own argmax.

The generation loop of the greedy sampler ("A transformer from scratch",
sections 12.5-12.6; "The LLM stack (fucina_llm)", section 13.6): every step
is the cached forward of the previous step's token.  One call runs the steps
back to back (with the one-launch step: one launch, the token handed between
steps on the device), so its tokens, its last logits and the KV rows it
appends are those of the single steps, bit for bit; both paths are checked,
and the tiny model against the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY, 101)


def singles(model, n, seq=0):
    toks = []
    lg = None
    for _ in range(n):
        lg, am = model.decode_step(seq=seq)
        toks.append(int(am.item()))
    return toks, lg.cpu().numpy().copy()


def kv_rows(model, shape, seq=0):
    return [tuple(t.cpu().numpy().copy() for t in model.kv_export(seq, layer)) for layer in range(shape.num_layers)]


@pytest.mark.parametrize("persistent", ["1", "0"])
@pytest.mark.parametrize("shape_name", ["tiny", "0.6b"])
def test_greedy_call_equals_single_steps(shape_name, persistent, tiny_w, monkeypatch):
    if shape_name == "0.6b" and persistent == "0":
        pytest.skip("the per-kernel path of the 0.6B shape is covered by the tiny shape and the model tests")
    monkeypatch.setenv("QWEN3_PERSISTENT", persistent)
    shape, w, plen, n = (TINY, tiny_w, 19, 13) if shape_name == "tiny" else (QWEN3_0_6B, gen_weights(QWEN3_0_6B, 201), 77, 24)
    prompt = gen_prompt(shape.vocab_size, plen, 61)
    a = make(shape, w, [plen + 2 * n + 4])
    b = make(shape, w, [plen + 2 * n + 4])
    assert (a.decode_launches() == 1) == (persistent == "1")
    a.prefill(prompt)
    b.prefill(prompt)
    toks, lg = a.decode_greedy(n)
    ta = [int(t) for t in toks.cpu().numpy()]
    la = lg.cpu().numpy().copy()
    tb, lb = singles(b, n)
    a.step_status()
    b.step_status()
    assert ta == tb
    assert np.array_equal(la, lb)
    assert a.kv_len() == b.kv_len() == plen + n
    for (ka, va), (kb, vb) in zip(kv_rows(a, shape), kv_rows(b, shape)):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    # a second call continues from the first one's last token, and single
    # steps continue from the second call's
    toks2, lg2 = a.decode_greedy(n // 2)
    a.decode_step()
    t2b, _ = singles(b, n // 2 + 1)
    ta2 = [int(t) for t in toks2.cpu().numpy()] + [int(a.io(0)[1].item())]
    assert ta2 == t2b
    assert a.kv_len() == b.kv_len() == plen + n + n // 2 + 1
    a.step_status()
    a.close()
    b.close()


def test_tiny_greedy_call_matches_oracle(tiny_w, monkeypatch):
    monkeypatch.setenv("QWEN3_PERSISTENT", "1")
    prompt = gen_prompt(TINY.vocab_size, 23, 62)
    gpu = make(TINY, tiny_w, [48])
    _, am = gpu.prefill(prompt)
    first = int(am.item())
    toks, lg = gpu.decode_greedy(10)
    gpu.step_status()
    got = [first] + [int(t) for t in toks.cpu().numpy()]
    ref = om.Model(TINY, tiny_w)
    rt, rl = ref.generate(prompt, 10, ref.new_cache(48))
    assert got == list(rt)
    assert rel_err(lg.cpu().numpy(), rl[-1]) <= TOL
    gpu.close()


def test_greedy_call_errors(tiny_w, monkeypatch):
    from quantized_q8_dequant_amd import Qwen3Error

    monkeypatch.setenv("QWEN3_PERSISTENT", "1")
    gpu = make(TINY, tiny_w, [20])
    gpu.prefill(gen_prompt(TINY.vocab_size, 9, 63))
    with pytest.raises(Qwen3Error) as e:
        gpu.decode_greedy(0)
    assert e.value.code == -1
    with pytest.raises(Qwen3Error) as e:
        gpu.decode_greedy(12)  # 9 + 12 > 20
    assert e.value.code == -7
    assert gpu.kv_len() == 9
    gpu.decode_greedy(11)  # exactly fills the cache
    gpu.step_status()
    assert gpu.kv_len() == 20
    gpu.close()


def test_failed_greedy_call_is_reported_and_leaves_lengths(tiny_w, monkeypatch):
    """With the error word set, the call writes -1 as its last token and
    nothing else, advances nothing on the device, and qwen3_step_status
    reports QWEN3_E_DEVICE and puts the host length back; the same call then
    gives the single steps' tokens."""
    from quantized_q8_dequant_amd import Qwen3Error

    monkeypatch.setenv("QWEN3_PERSISTENT", "1")
    prompt = gen_prompt(TINY.vocab_size, 15, 64)
    gpu = make(TINY, tiny_w, [40])
    ref = make(TINY, tiny_w, [40])
    gpu.prefill(prompt)
    ref.prefill(prompt)
    gpu.inject_step_error()
    out = torch.full((6,), 777, dtype=torch.int32, device="cuda:0")
    gpu.decode_greedy(6, out=out)
    got = out.cpu().numpy()
    assert got[5] == -1  # the launch's entry check writes -1 to the last slot, the token the call leaves
    assert np.all(got[:5] == 777)
    assert gpu.kv_len() == 15 + 6
    with pytest.raises(Qwen3Error) as e:
        gpu.step_status()
    assert e.value.code == -9
    assert gpu.kv_len() == 15
    # resume: step 0 is fed the prefill's argmax again (the failed call left -1 in the buffer)
    tok0 = torch.tensor([int(ref.io(0)[1].item())], dtype=torch.int32, device="cuda:0")
    toks, _ = gpu.decode_greedy(6, token=tok0)
    gpu.step_status()
    tb, _ = singles(ref, 6)
    assert [int(t) for t in toks.cpu().numpy()] == tb
    gpu.close()
    ref.close()
