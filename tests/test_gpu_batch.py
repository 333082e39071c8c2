"""Batched Q8_0 decode against the CPU oracle: one step decodes one token for
each of N independent streams ("A transformer from scratch", section 12.5,
forwardStepBatch), the projections of all N rows in one small-M GEMM pass
over the weights, RoPE positions, KV appends and attention per stream.

Each stream must match the oracle run on that stream alone (logits within
1e-3 of the oracle's range, greedy tokens identical).  Batch sizes cover the
per-row GEMV path (below 16 rows), the three row tilings of the small-M GEMM
(up to 16, 32 and 64 rows) and ragged KV lengths; short prefill chunks (at
most 64 rows) run their projections through the same small-M GEMM.
"""

import os

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, gen_lengths, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3


def progress(msg):
    print(f"[{os.path.basename(__file__)}] {msg}", flush=True)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def run_batch(gpu, prompts, steps, with_logits=True):
    """Prefill each stream, then `steps` lockstep batched decode steps fed
    the previous argmax.  Returns per step (logits [n, V] or None, argmax [n])."""
    n = len(prompts)
    first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    V = gpu.cfg.vocab_size
    logits = torch.empty((n, V), dtype=torch.float32, device="cuda:0") if with_logits else None
    am = torch.empty(n, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(steps):
        gpu.decode_batch(list(range(n)), toks, logits, am)
        outs.append((logits.cpu().numpy().copy() if with_logits else None, am.cpu().numpy().copy()))
        toks = am.clone()
    return first, outs


def check_streams(ref, prompts, cap, steps, first, outs):
    for s, p in enumerate(prompts):
        rt, rl = ref.generate(p, steps, ref.new_cache(cap))
        assert rt[0] == first[s], s
        for i in range(steps):
            if outs[i][0] is not None:
                assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL, (s, i)
            assert outs[i][1][s] == rt[i + 1], (s, i)


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY, 101)


@pytest.fixture(scope="module")
def tiny_ref(tiny_w):
    return om.Model(TINY, tiny_w)


@pytest.mark.parametrize("n", [2, 15, 16, 17, 32, 33, 64])  # per-row GEMV below 16 rows
def test_tiny_batched_decode_row_tilings(tiny_w, tiny_ref, n):
    lengths = gen_lengths(n, 1, 90, 300 + n)
    prompts = [gen_prompt(TINY.vocab_size, int(L), 400 + s) for s, L in enumerate(lengths)]
    cap = 100
    gpu = make(TINY, tiny_w, [cap] * n)
    first, outs = run_batch(gpu, prompts, 3)
    check_streams(tiny_ref, prompts, cap, 3, first, outs)
    for s, p in enumerate(prompts):
        assert gpu.kv_len(s) == len(p) + 3


def test_tiny_batched_decode_without_logits_and_subsets(tiny_w, tiny_ref):
    """No logits buffer (the argmax alone), and batches over a subset of the
    sequences in an order of the caller's choosing."""
    n = 20
    prompts = [gen_prompt(TINY.vocab_size, 5 + 3 * s, 500 + s) for s in range(n)]
    gpu = make(TINY, tiny_w, [80] * n)
    first, outs = run_batch(gpu, prompts, 2, with_logits=False)
    check_streams(tiny_ref, prompts, 80, 2, first, outs)
    # the odd sequences, in reverse order, one more step
    sub = list(range(n - 1, 0, -2))
    toks = torch.tensor([int(outs[-1][1][s]) for s in sub], dtype=torch.int32, device="cuda:0")
    am = torch.empty(len(sub), dtype=torch.int32, device="cuda:0")
    logits = torch.empty((len(sub), TINY.vocab_size), dtype=torch.float32, device="cuda:0")
    gpu.decode_batch(sub, toks, logits, am)
    lg = logits.cpu().numpy()
    for i, s in enumerate(sub):
        rt, rl = tiny_ref.generate(prompts[s], 3, tiny_ref.new_cache(80))
        assert rel_err(lg[i], rl[3]) <= TOL and int(am[i].item()) == rt[3]
        assert gpu.kv_len(s) == len(prompts[s]) + 3
    for s in range(0, n, 2):
        assert gpu.kv_len(s) == len(prompts[s]) + 2


@pytest.mark.parametrize("T", [1, 15, 16, 33, 64])
def test_tiny_short_prefill_chunks(tiny_w, tiny_ref, T):
    """Prompts cut into chunks of T rows run their projections through the
    small-M GEMM; every chunk's cache rows feed the next."""
    prompt = gen_prompt(TINY.vocab_size, 150, 600 + T)
    gpu = make(TINY, tiny_w, [160], max_batch_tokens=T)
    lg, am = gpu.prefill(prompt)
    ref = tiny_ref.forward(prompt, tiny_ref.new_cache(160))[0]
    assert rel_err(lg.cpu().numpy(), ref) <= TOL
    assert int(am.item()) == int(np.argmax(lg.cpu().numpy()))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_batched_decode_matches_oracle():
    """Qwen3-0.6B, 24 streams with ragged prompts of 16..200 tokens, 3
    lockstep batched steps, every stream against the oracle."""
    n, steps = 24, 3
    w = gen_weights(QWEN3_0_6B, 201)
    lengths = gen_lengths(n, 16, 200, 700)
    prompts = [gen_prompt(QWEN3_0_6B.vocab_size, int(L), 800 + s) for s, L in enumerate(lengths)]
    cap = 210
    gpu = make(QWEN3_0_6B, w, [cap] * n)
    progress("gpu")
    first, outs = run_batch(gpu, prompts, steps)
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    progress("oracle")
    ref = om.Model(QWEN3_0_6B, w)
    del w
    check_streams(ref, prompts, cap, steps, first, outs)


@pytest.mark.parametrize("n", [4, 20])  # per-row GEMV, small-M GEMM
def test_graph_replays_equal_the_eager_step(tiny_w, n):
    """Batched steps replayed from a captured graph (same buffers every step)
    against a handle that launches every kernel eagerly: logits and tokens
    bitwise equal on every replay, with other device work and
    synchronisations between the replays."""
    lengths = gen_lengths(n, 1, 60, 900 + n)
    prompts = [gen_prompt(TINY.vocab_size, int(L), 950 + s) for s, L in enumerate(lengths)]
    os.environ["QWEN3_NO_GRAPH"] = "1"
    try:
        eager = make(TINY, tiny_w, [80] * n)
    finally:
        del os.environ["QWEN3_NO_GRAPH"]
    graph = make(TINY, tiny_w, [80] * n)
    outs = []
    for gpu in (eager, graph):
        first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
        am = torch.tensor(first, dtype=torch.int32, device="cuda:0")
        logits = torch.empty((n, TINY.vocab_size), dtype=torch.float32, device="cuda:0")
        steps = []
        for i in range(5):
            gpu.decode_batch(list(range(n)), am, logits, am)  # the same buffers each step
            noise = torch.randn(1 << 16, device="cuda:0").sum()  # unrelated device work between replays
            torch.cuda.synchronize()
            steps.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy(), float(noise)))
        outs.append(steps)
    for (le, ae, _), (lg, ag, _) in zip(*outs):
        assert np.array_equal(le, lg)
        assert np.array_equal(ae, ag)
