"""The one-launch decode step at its edges: device tokens outside the
vocabulary, and a step whose hand-off between workgroups fails.

A failing call leaves the state it found valid ("A transformer from
scratch", section 12.6; "The LLM stack (fucina_llm)", section 13.4).  The
failure is forced from the host (the error word a timed-out wait would set),
so every workgroup leaves at once and no kernel waits on anything.
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


@pytest.mark.parametrize("shape_name", ["tiny", "0.6b"])
def test_out_of_range_device_tokens_are_clamped(shape_name, monkeypatch):
    """Ids -1 and V + 5 fed to the one-launch step give what the per-kernel
    step gives for them, which is the step of ids 0 and V - 1."""
    shape, wseed = (TINY, 101) if shape_name == "tiny" else (QWEN3_0_6B, 201)
    w = gen_weights(shape, wseed)
    V = shape.vocab_size
    prompt = gen_prompt(V, 19, 71)
    out = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("QWEN3_PERSISTENT", mode)
        m = make(shape, w, [32])
        assert (m.decode_launches() == 1) == (mode == "1")
        rows = []
        for bad, good in ((-1, 0), (V + 5, V - 1)):
            for tok in (bad, good):
                m.prefill(prompt)
                t = torch.tensor([tok], dtype=torch.int32, device="cuda:0")
                lg, am = m.decode_step(token=t)
                rows.append((lg.cpu().numpy().copy(), int(am.item())))
                assert m.kv_len() == len(prompt) + 1
                m.reset()
        m.step_status()
        m.close()
        out[mode] = rows
    for (lp, tp), (lk, tk) in zip(out["1"], out["0"]):
        assert tp == tk
        assert rel_err(lp, lk) <= TOL
    # clamped ids are the in-range ids' steps, bitwise on one path
    for mode in ("1", "0"):
        r = out[mode]
        assert np.array_equal(r[0][0], r[1][0]) and r[0][1] == r[1][1]
        assert np.array_equal(r[2][0], r[3][0]) and r[2][1] == r[3][1]


def test_failed_step_is_reported_and_leaves_lengths(tiny_w, monkeypatch):
    """After the error word is set: the step writes -1 and advances nothing,
    later steps do the same, qwen3_step_status reports QWEN3_E_DEVICE and
    puts the host length back, and decoding then resumes with the oracle's
    tokens."""
    from quantized_q8_dequant_amd import Qwen3Error

    monkeypatch.setenv("QWEN3_PERSISTENT", "1")
    prompt = gen_prompt(TINY.vocab_size, 23, 72)
    gpu = make(TINY, tiny_w, [48])
    assert gpu.decode_launches() == 1
    lg, am = gpu.prefill(prompt)
    toks = [int(am.item())]
    for _ in range(2):
        lg, am = gpu.decode_step()
        toks.append(int(am.item()))
    gpu.step_status()  # nothing failed so far
    assert gpu.kv_len() == len(prompt) + 2
    k_before, v_before = (t.cpu().clone() for t in gpu.kv_export(0, TINY.num_layers - 1))

    gpu.inject_step_error()
    fed = torch.tensor([toks[-1]], dtype=torch.int32, device="cuda:0")
    for _ in range(2):
        _, am = gpu.decode_step(token=fed)
        assert int(am.item()) == -1
    assert gpu.kv_len() == len(prompt) + 4  # the host counted both calls
    with pytest.raises(Qwen3Error) as e:
        gpu.step_status()
    assert e.value.code == -9
    assert gpu.kv_len() == len(prompt) + 2
    gpu.step_status()  # the word is clear again
    k_after, v_after = (t.cpu() for t in gpu.kv_export(0, TINY.num_layers - 1))
    assert torch.equal(k_before, k_after) and torch.equal(v_before, v_after)

    # decoding resumes where it stopped
    logits = []
    for _ in range(4):
        lg, am = gpu.decode_step(token=fed)
        t = int(am.item())
        toks.append(t)
        logits.append(lg.cpu().numpy().copy())
        fed = am.clone()
    gpu.step_status()
    ref = om.Model(TINY, tiny_w)
    rt, rl = ref.generate(prompt, 6, ref.new_cache(48))
    assert toks == list(rt)
    for a, b in zip(logits, rl[3:]):
        assert rel_err(a, b) <= TOL
    gpu.close()


def test_step_status_without_one_launch_step(tiny_w, monkeypatch):
    from quantized_q8_dequant_amd import Qwen3Error

    monkeypatch.setenv("QWEN3_PERSISTENT", "0")
    gpu = make(TINY, tiny_w, [16])
    gpu.prefill([1, 2, 3])
    gpu.decode_step()
    gpu.step_status()
    assert gpu.kv_len() == 4
    gpu.close()
    bf = TINY.with_(name="tiny-bf16", weight_type="bf16", kv_type="bf16")
    m = make(bf, gen_weights(bf, 101), [16])
    with pytest.raises(Qwen3Error) as e:
        m.inject_step_error()
    assert e.value.code == -1
    m.step_status()
    m.close()
