"""Greedy ties on every argmax path: the lowest index among equal maxima.

Greedy decoding takes the argmax of the last row's logits ("A transformer
from scratch", section 12.6; "The LLM stack (fucina_llm)", section 13.6, the
greedy example); where several logits share the maximum, the lowest index
is taken (the pages keep the first maximum of a strict-greater scan).

Ties are built, not hoped for: the tied embedding matrix is made periodic
(row r equals row r mod P, and inside a period rows 2i and 2i + 1 are equal),
so every logit value appears at 2 * V / P indices that lie in different
lanes, workgroups and vocabulary slices of every head kernel.  Feeding any
copy of a row gives the same forward pass, so the oracle's tokens stay
comparable; every argmax must be even and below P.

Paths: the decode GEMV's argmax epilogue (prefill's last row, per-kernel
decode, batches under 16 rows), the one-launch step's lm_head, the row
argmax after the small-M GEMM (batches from 16 rows, all-logits calls of at
most 64 rows) and after the MFMA GEMM (all-logits calls of more rows), and
the bf16 linear's argmax epilogue.
"""

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3
TINY_BF16 = TINY.with_(name="tiny-bf16", weight_type="bf16", kv_type="bf16")


def periodic(weights, period):
    """The weights with token_embd made periodic with `period` rows, rows
    paired inside a period."""
    w = dict(weights)
    e = np.array(w["token_embd"], dtype=np.float32, copy=True)
    V = e.shape[0]
    assert V % period == 0 and period % 2 == 0
    base = e[:period].copy()
    base[1::2] = base[0::2]
    w["token_embd"] = np.ascontiguousarray(np.tile(base, (V // period, 1)))
    return w


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / (np.max(b) - np.min(b)))


def check_row(logits, tok, period):
    """Copies of one logit are bitwise equal on the GPU, and the token is the
    lowest index of the maximum."""
    lg = np.asarray(logits, np.float32)
    V = lg.shape[0]
    per = lg.reshape(V // period, period // 2, 2)
    assert np.array_equal(per, np.broadcast_to(per[:1, :, :1], per.shape)), "copies differ"
    assert tok == int(np.argmax(lg)), (tok, int(np.argmax(lg)))
    assert tok % 2 == 0 and 0 <= tok < period


def canonical(tok, period):
    return (int(tok) % period) & ~1


@pytest.fixture(scope="module")
def tiny_tied():
    return periodic(gen_weights(TINY, 101), 1024)


@pytest.fixture(scope="module")
def tiny_tied_ref(tiny_tied):
    return om.Model(TINY, tiny_tied)


@pytest.mark.parametrize("persistent", ["1", "0"])
def test_single_sequence_greedy_ties(tiny_tied, tiny_tied_ref, persistent, monkeypatch):
    monkeypatch.setenv("QWEN3_PERSISTENT", persistent)
    prompt = gen_prompt(TINY.vocab_size, 21, 81)
    gpu = make(TINY, tiny_tied, [40])
    assert (gpu.decode_launches() == 1) == (persistent == "1")
    lg, am = gpu.prefill(prompt)
    toks, logits = [int(am.item())], [lg.cpu().numpy().copy()]
    for _ in range(6):
        lg, am = gpu.decode_step()
        toks.append(int(am.item()))
        logits.append(lg.cpu().numpy().copy())
    gpu.step_status()
    gpu.close()
    for lg, t in zip(logits, toks):
        check_row(lg, t, 1024)
    rt, rl = tiny_tied_ref.generate(prompt, 6, tiny_tied_ref.new_cache(40))
    assert toks == [canonical(t, 1024) for t in rt]
    for a, b in zip(logits, rl):
        assert rel_err(a, b) <= TOL


@pytest.mark.parametrize("n", [40, 100])
def test_all_logits_row_argmax_ties(tiny_tied, tiny_tied_ref, n):
    """n <= 64 rows: small-M GEMM head; more: the MFMA GEMM head; then the
    row argmax kernel."""
    prompt = gen_prompt(TINY.vocab_size, n, 82)
    gpu = make(TINY, tiny_tied, [128], max_batch_tokens=128)
    lg, am = gpu.prefill_all_logits(prompt)
    lg, am = lg.cpu().numpy(), am.cpu().numpy()
    gpu.close()
    for r in range(n):
        check_row(lg[r], int(am[r]), 1024)
    ref = tiny_tied_ref.forward(prompt, tiny_tied_ref.new_cache(128), all_logits=True)
    assert [int(t) for t in am] == [canonical(np.argmax(r), 1024) for r in ref]
    assert rel_err(lg, ref) <= TOL


@pytest.mark.parametrize("rows", [5, 20])
def test_batched_decode_argmax_ties(tiny_tied, tiny_tied_ref, rows):
    """5 rows: the per-row GEMV epilogue; 20 rows: the small-M GEMM and the
    row argmax."""
    prompts = [gen_prompt(TINY.vocab_size, 3 + 2 * s, 90 + s) for s in range(rows)]
    gpu = make(TINY, tiny_tied, [48] * rows)
    first = [int(gpu.prefill(p, seq=s)[1].item()) for s, p in enumerate(prompts)]
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    logits = torch.empty((rows, TINY.vocab_size), dtype=torch.float32, device="cuda:0")
    am = torch.empty(rows, dtype=torch.int32, device="cuda:0")
    outs = []
    for _ in range(3):
        gpu.decode_batch(list(range(rows)), toks, logits, am)
        outs.append((logits.cpu().numpy().copy(), am.cpu().numpy().copy()))
        toks = am.clone()
    gpu.close()
    for lg, a in outs:
        for r in range(rows):
            check_row(lg[r], int(a[r]), 1024)
    for s in (0, rows - 1):
        rt, rl = tiny_tied_ref.generate(prompts[s], 3, tiny_tied_ref.new_cache(48))
        assert first[s] == canonical(rt[0], 1024)
        for i in range(3):
            assert int(outs[i][1][s]) == canonical(rt[i + 1], 1024)
            assert rel_err(outs[i][0][s], rl[i + 1]) <= TOL


def test_bf16_weights_argmax_ties():
    w = periodic(gen_weights(TINY_BF16, 101), 1024)
    prompt = gen_prompt(TINY_BF16.vocab_size, 17, 83)
    gpu = make(TINY_BF16, w, [64, 64])
    lg, am = gpu.prefill(prompt)
    toks, logits = [int(am.item())], [lg.cpu().numpy().copy()]
    for _ in range(3):
        lg, am = gpu.decode_step()
        toks.append(int(am.item()))
        logits.append(lg.cpu().numpy().copy())
    for lg, t in zip(logits, toks):
        check_row(lg, t, 1024)
    lga, ama = gpu.prefill_all_logits(gen_prompt(TINY_BF16.vocab_size, 30, 84), seq=1)
    lga, ama = lga.cpu().numpy(), ama.cpu().numpy()
    for r in range(30):
        check_row(lga[r], int(ama[r]), 1024)
    gpu.close()
    ref = om.Model(TINY_BF16, w)
    rt, rl = ref.generate(prompt, 3, ref.new_cache(64))
    assert toks == [canonical(t, 1024) for t in rt]
    for a, b in zip(logits, rl):
        assert rel_err(a, b) <= TOL


@pytest.mark.slow
def test_0_6b_vocabulary_ties_one_launch_and_batched():
    """151,936 logits (period 37,984, four copies of each pair): the
    one-launch step's lm_head over 256 workgroups and the batched step's
    row argmax over 4096-logit slices."""
    P = QWEN3_0_6B.vocab_size // 4
    w = periodic(gen_weights(QWEN3_0_6B, 201), P)
    prompts = [gen_prompt(QWEN3_0_6B.vocab_size, 9 + s, 85 + s) for s in range(16)]
    gpu = make(QWEN3_0_6B, w, [32] * 16)
    assert gpu.decode_launches() == 1
    lg, am = gpu.prefill(prompts[0])
    check_row(lg.cpu().numpy(), int(am.item()), P)
    for _ in range(3):
        lg, am = gpu.decode_step()
        check_row(lg.cpu().numpy(), int(am.item()), P)
    gpu.step_status()
    for s in range(1, 16):
        gpu.prefill(prompts[s], seq=s)
    toks = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    for s in range(16):
        toks[s] = gpu.io(s)[1][0]
    logits = torch.empty((16, QWEN3_0_6B.vocab_size), dtype=torch.float32, device="cuda:0")
    am16 = torch.empty(16, dtype=torch.int32, device="cuda:0")
    for _ in range(2):
        gpu.decode_batch(list(range(16)), toks, logits, am16)
        lgh, amh = logits.cpu().numpy(), am16.cpu().numpy()
        for r in range(16):
            check_row(lgh[r], int(amh[r]), P)
        toks = am16.clone()
    gpu.close()
