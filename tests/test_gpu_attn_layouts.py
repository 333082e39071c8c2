"""Decode attention over every head layout the kernel is built for, against
the oracle.

The decode step's attention ("A transformer from scratch", section 12.3.5:
query head h reads KV head h / (nh / nkv); section 12.4: the cached step
equals recomputation) is one kernel instantiated per head dim (64, 128) and
group size (1, 2, 4, 8).  Each instantiation has its own thread maps: a
thread serves up to four query heads of its group, the partial dots of a
tile are summed over the lanes of a row, the P.V sums over the row groups,
and the split partials travel as pairs of adjacent dims.  The model tests
reach the layouts of the three model shapes (64/2, 128/2, 128/4); this file
runs the others, on tiny-model variants, at three prompt lengths:
  - 40 tokens: one split per KV head (the output written straight from LDS);
  - 300: five splits of 64 rows (one combine batch);
  - 2700: 43 splits (several combine batches; the last split ragged).
Each case: chunked prefill, then 4 greedy decode steps on the per-kernel
path; tokens equal to the oracle's, logits within 1e-3 of the oracle's range.
A batched step of 17 ragged sequences covers the attention's quantised
output rows (from 16 rows on the small-M projection reads them).
"""

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import ops
from synthetic import TINY, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3
STEPS = 4

LAYOUTS = {
    "hd64-g1": TINY.with_(name="tiny-hd64-g1", num_attention_heads=4, num_key_value_heads=4),
    "hd64-g4": TINY.with_(name="tiny-hd64-g4", num_attention_heads=8, num_key_value_heads=2),
    "hd64-g8": TINY.with_(name="tiny-hd64-g8", num_attention_heads=16, num_key_value_heads=2),
    "hd128-g1": TINY.with_(name="tiny-hd128-g1", head_dim=128, num_attention_heads=2, num_key_value_heads=2),
    "hd128-g8": TINY.with_(name="tiny-hd128-g8", head_dim=128, num_attention_heads=16, num_key_value_heads=2),
    "hd128-g8-bf16kv": TINY.with_(
        name="tiny-hd128-g8-bf16kv", head_dim=128, num_attention_heads=16, num_key_value_heads=2, kv_type="bf16"
    ),
    "hd64-g4-q8kv": TINY.with_(name="tiny-hd64-g4-q8kv", num_attention_heads=8, num_key_value_heads=2, kv_type="q8_0"),
}


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def oracle_run(ref, prompt, steps, cap, chunk=300):
    """The oracle's chunked prefill then `steps` greedy steps: tokens and logits."""
    cache = ref.new_cache(cap)
    for i in range(0, len(prompt), chunk):
        lg = ref.forward(prompt[i : i + chunk], cache)[0]
    toks, logits = [int(ops.argmax_lowest(lg))], [lg]
    for _ in range(steps):
        lg = ref.forward([toks[-1]], cache)[0]
        toks.append(int(ops.argmax_lowest(lg)))
        logits.append(lg)
    return toks, logits


def weights_and_ref(name, cache={}):
    if name not in cache:
        shape = LAYOUTS[name]
        w = gen_weights(shape, 131)
        cache[name] = (w, om.Model(shape, w))
    return cache[name]


@pytest.mark.parametrize("plen", [40, 300, 2700])
@pytest.mark.parametrize("name", list(LAYOUTS))
def test_decode_attention_layout_matches_oracle(name, plen, monkeypatch):
    monkeypatch.setenv("QWEN3_PERSISTENT", "0")
    shape = LAYOUTS[name]
    w, ref = weights_and_ref(name)
    prompt = gen_prompt(shape.vocab_size, plen, 140 + plen)
    cap = plen + STEPS + 4
    print(f"[attn layouts] {name} prompt {plen}", flush=True)
    gpu = make(shape, w, [cap], max_batch_tokens=512)
    lg, am = gpu.prefill(prompt)
    toks, logits = [int(am.item())], [lg.cpu().numpy().astype(np.float64)]
    for _ in range(STEPS):
        lg, am = gpu.decode_step()
        toks.append(int(am.item()))
        logits.append(lg.cpu().numpy().astype(np.float64))
    gpu.close()
    rtoks, rlogits = oracle_run(ref, prompt, STEPS, cap)
    errs = [rel_err(a, b) for a, b in zip(logits, rlogits)]
    assert max(errs) <= TOL, f"logit errors {['%.1e' % e for e in errs]}"
    assert toks == rtoks


@pytest.mark.parametrize("name", ["hd64-g1", "hd64-g8", "hd128-g8"])
def test_batched_decode_attention_layout_matches_oracle(name):
    """17 sequences of 20..301 tokens stepped together: each row of the
    batched step against the oracle's own run of that sequence."""
    shape = LAYOUTS[name]
    w, ref = weights_and_ref(name)
    lens = tuple(20 + (281 * i) // 16 for i in range(17))
    prompts = [gen_prompt(shape.vocab_size, n, 150 + n) for n in lens]
    cap = max(lens) + STEPS + 4
    print(f"[attn layouts] batched {name}", flush=True)
    gpu = make(shape, w, [cap] * len(lens), max_batch_tokens=512)
    first = []
    for s, p in enumerate(prompts):
        _, am = gpu.prefill(p, seq=s)
        first.append(int(am.item()))
    n = len(lens)
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((n, shape.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(n, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(STEPS):
        gpu.decode_batch(list(range(n)), toks, logits, am)
        outs.append((logits.cpu().numpy().astype(np.float64), am.cpu().numpy().copy()))
        toks = am.clone()
    gpu.close()
    for s, p in enumerate(prompts):
        rtoks, rlogits = oracle_run(ref, p, STEPS, cap)
        assert rtoks[0] == first[s]
        for i in range(STEPS):
            assert rel_err(outs[i][0][s], rlogits[i + 1]) <= TOL
            assert int(outs[i][1][s]) == rtoks[i + 1]
