"""The speculative-decoding seams against the CPU oracle: the all-logits
forward step (every appended position's logits, "A transformer from
scratch", sections 12.3.7 and 12.5) and the O(1) KV rewind ("The LLM stack
(fucina_llm)", section 13.4, truncate).

Tolerance as for the other model tests: per row, max |logit_gpu -
logit_oracle| <= 1e-3 x (max - min of the oracle row).  The argmax rows are
index work: each must be the lowest index of its own logits row's maximum
(bit-exact), and equal to the oracle's where the oracle's top two are
further apart than the logit tolerance.
"""

import os

import numpy as np
import pytest
import torch

from oracle import model as om
from synthetic import QWEN3_0_6B, TINY, WORKLOADS, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

TOL = 1e-3


def progress(msg):
    print(f"[{os.path.basename(__file__)}] {msg}", flush=True)


def row_errs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.max(np.abs(a - b), axis=1) / (np.max(b, axis=1) - np.min(b, axis=1))


def check_rows(lg, am, ref_rows):
    """lg [n, V] f32 and am [n] int32 from the GPU against oracle rows [n, V]."""
    errs = row_errs(lg, ref_rows)
    assert errs.max() <= TOL, f"worst row {int(errs.argmax())}: {errs.max():.2e}"
    if am is not None:
        assert np.array_equal(am, np.argmax(lg, axis=1).astype(np.int32))
        rng = np.max(ref_rows, axis=1) - np.min(ref_rows, axis=1)
        top2 = np.sort(ref_rows, axis=1)[:, -2:]
        clear = (top2[:, 1] - top2[:, 0]) > 2 * TOL * rng
        assert np.array_equal(am[clear], np.argmax(ref_rows, axis=1)[clear])


def make(shape, weights, caps, **kw):
    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    return Qwen3Model(Qwen3Config.from_shape(shape), weights, caps, **kw)


@pytest.fixture(scope="module")
def tiny_w():
    return gen_weights(TINY, 101)


@pytest.fixture(scope="module")
def tiny_ref(tiny_w):
    return om.Model(TINY, tiny_w)


@pytest.mark.parametrize("mbt", [0, 16])  # one chunk; 16-row chunks with a ragged tail
def test_tiny_all_logits_matches_oracle(tiny_w, tiny_ref, mbt):
    prompt = gen_prompt(TINY.vocab_size, 45, 71)
    gpu = make(TINY, tiny_w, [64], max_batch_tokens=mbt)
    lg, am = gpu.prefill_all_logits(prompt)
    lg, am = lg.cpu().numpy(), am.cpu().numpy()
    cache = tiny_ref.new_cache(64)
    ref = tiny_ref.forward(prompt, cache, all_logits=True)
    check_rows(lg, am, ref)
    assert gpu.kv_len() == 45
    # a second all-logits call continues the sequence at position 45
    more = gen_prompt(TINY.vocab_size, 7, 72)
    lg2, am2 = gpu.prefill_all_logits(more)
    check_rows(lg2.cpu().numpy(), am2.cpu().numpy(), tiny_ref.forward(more, cache, all_logits=True))
    assert gpu.kv_len() == 52


def test_tiny_all_logits_last_row_is_the_prefill_logits(tiny_w):
    """The all-logits step differs from the ordinary prefill only in how many
    rows reach the head: same cache, and its last row is the prefill's
    logits (different kernels, so within the tolerance)."""
    prompt = gen_prompt(TINY.vocab_size, 30, 73)
    a, b = make(TINY, tiny_w, [32]), make(TINY, tiny_w, [32])
    lg_all, am_all = a.prefill_all_logits(prompt)
    lg, am = b.prefill(prompt)
    last = lg_all[-1].cpu().numpy()[None]
    assert row_errs(last, lg.cpu().numpy()[None]).max() <= TOL
    assert int(am_all[-1].item()) == int(np.argmax(last))
    for layer in range(TINY.num_layers):
        ka, va = a.kv_export(0, layer)
        kb, vb = b.kv_export(0, layer)
        assert torch.equal(ka, kb) and torch.equal(va, vb)
    # without the argmax output
    c = make(TINY, tiny_w, [32])
    lg_c, am_c = c.prefill_all_logits(prompt, argmax=False)
    assert am_c is None and torch.equal(lg_c, lg_all)


def test_tiny_verify_truncate_continue(tiny_w, tiny_ref):
    """The speculative protocol: prefill, verify a drafted run with all
    logits, rewind to the accepted prefix, continue greedy decoding from
    the verifier's own prediction at the last accepted position."""
    prompt = gen_prompt(TINY.vocab_size, 20, 74)
    draft = gen_prompt(TINY.vocab_size, 6, 75)
    accept = 3
    gpu = make(TINY, tiny_w, [48])
    gpu.prefill(prompt)
    lg, am = gpu.prefill_all_logits(draft)
    assert gpu.kv_len() == 26
    gpu.truncate(len(prompt) + accept)
    assert gpu.kv_len() == 23
    tok = am[accept - 1 : accept].clone()
    toks, logits = [int(tok.item())], []
    for _ in range(5):
        lgs, ams = gpu.decode_step(token=tok)
        logits.append(lgs.cpu().numpy().copy())
        toks.append(int(ams.item()))
        tok = ams
    assert gpu.kv_len() == 28

    cache = tiny_ref.new_cache(48)
    tiny_ref.forward(prompt, cache)
    ref = tiny_ref.forward(draft, cache, all_logits=True)
    check_rows(lg.cpu().numpy(), am.cpu().numpy(), ref)
    cache.truncate(len(prompt) + accept)
    rtoks = [int(np.argmax(ref[accept - 1]))]
    rlogits = []
    for _ in range(5):
        r = tiny_ref.forward([rtoks[-1]], cache)[0]
        rlogits.append(r)
        rtoks.append(int(np.argmax(r)))
    assert toks == rtoks
    assert row_errs(np.stack(logits), np.stack(rlogits)).max() <= TOL


def test_tiny_truncate_edge_cases(tiny_w):
    from quantized_q8_dequant_amd import Qwen3Error

    prompt = gen_prompt(TINY.vocab_size, 12, 76)
    gpu = make(TINY, tiny_w, [32])
    lg0, _ = gpu.prefill(prompt)
    lg0 = lg0.cpu().numpy().copy()
    gpu.truncate(12)  # at the length: no-op
    gpu.truncate(40)  # above the length (and the capacity): no-op
    assert gpu.kv_len() == 12
    with pytest.raises(Qwen3Error) as e:
        gpu.truncate(-1)
    assert e.value.code == -1
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill_all_logits([])
    assert e.value.code == -6
    with pytest.raises(Qwen3Error) as e:
        gpu.prefill_all_logits(gen_prompt(TINY.vocab_size, 21, 77))  # 12 + 21 > 32
    assert e.value.code == -7
    assert gpu.kv_len() == 12
    # a rewind to 0 then the same prompt reproduces the first prefill exactly
    gpu.truncate(0)
    assert gpu.kv_len() == 0
    lg1, _ = gpu.prefill(prompt)
    assert np.array_equal(lg1.cpu().numpy(), lg0)
    # a partial rewind then a different continuation matches a cacheless
    # recompute over the kept prefix plus the new tokens
    gpu.truncate(5)
    tail = gen_prompt(TINY.vocab_size, 9, 78)
    lg2, _ = gpu.prefill(tail)
    ref = om.Model(TINY, tiny_w).forward_uncached(np.concatenate([prompt[:5], tail]))
    assert row_errs(lg2.cpu().numpy()[None], ref).max() <= TOL
    assert gpu.kv_len() == 14


# Long contexts on the tiny model: the attention of a block whose keys span
# several 64-key tiles is cut into runs across workgroups and merged by the
# last run; group sizes 1, 2 and 4 (head layouts of the three kernel shapes),
# f32 and bf16 caches.
LONG_SHAPES = {
    "g2": TINY,
    "g4": TINY.with_(name="tiny-g4", num_attention_heads=8, num_key_value_heads=2),
    "g1": TINY.with_(name="tiny-g1", num_attention_heads=4, num_key_value_heads=4),
    "g2-bf16kv": TINY.with_(name="tiny-bf16kv", kv_type="bf16"),
}


@pytest.mark.parametrize("name", list(LONG_SHAPES))
def test_tiny_long_context_all_logits_and_verify(name):
    shape = LONG_SHAPES[name]
    w = gen_weights(shape, 103)
    ref_model = om.Model(shape, w)
    prompt = gen_prompt(shape.vocab_size, 300, 81)  # 18 blocks of 16 + a ragged 12
    draft = gen_prompt(shape.vocab_size, 12, 82)
    gpu = make(shape, w, [340], max_batch_tokens=320)
    lg_p, am_p = gpu.prefill_all_logits(prompt)
    lg_v, am_v = gpu.prefill_all_logits(draft)
    cache = ref_model.new_cache(340)
    check_rows(lg_p.cpu().numpy(), am_p.cpu().numpy(), ref_model.forward(prompt, cache, all_logits=True))
    check_rows(lg_v.cpu().numpy(), am_v.cpu().numpy(), ref_model.forward(draft, cache, all_logits=True))
    # the same prompt in 48-row chunks: later chunks attend 64-key tiles of earlier ones
    chunked = make(shape, w, [340], max_batch_tokens=48)
    lg_c, _ = chunked.prefill(prompt)
    assert row_errs(lg_c.cpu().numpy()[None], lg_p[-1:].cpu().numpy()).max() <= TOL


TINY_BF16 = TINY.with_(name="tiny-bf16", weight_type="bf16", kv_type="bf16")


def test_tiny_bf16_all_logits_matches_oracle():
    w = gen_weights(TINY_BF16, 101)
    ref_model = om.Model(TINY_BF16, w)
    prompt = gen_prompt(TINY_BF16.vocab_size, 37, 79)
    gpu = make(TINY_BF16, w, [48], max_batch_tokens=16)
    lg, am = gpu.prefill_all_logits(prompt)
    ref = ref_model.forward(prompt, ref_model.new_cache(48), all_logits=True)
    check_rows(lg.cpu().numpy(), am.cpu().numpy(), ref)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_qwen3_0_6b_all_logits_verify_matches_oracle():
    """Qwen3-0.6B: the 512-token prompt through the all-logits step (512
    logits rows), a 16-token verify, a rewind to 5 accepted tokens and three
    decode steps, all against the oracle."""
    wl = WORKLOADS["0.6b-decode"]
    w = gen_weights(QWEN3_0_6B, wl.weight_seed)
    prompt = gen_prompt(QWEN3_0_6B.vocab_size, wl.prompt_len, wl.prompt_seed)
    draft = gen_prompt(QWEN3_0_6B.vocab_size, 16, 80)
    P, accept = len(prompt), 5
    gpu = make(QWEN3_0_6B, w, [wl.kv_capacity])
    progress("gpu all-logits prefill")
    lg_p, am_p = gpu.prefill_all_logits(prompt)
    lg_p, am_p = lg_p.cpu().numpy(), am_p.cpu().numpy()
    lg_v, am_v = gpu.prefill_all_logits(draft)
    lg_v, am_v = lg_v.cpu().numpy(), am_v.cpu().numpy()
    gpu.truncate(P + accept)
    tok = torch.tensor([int(am_v[accept - 1])], dtype=torch.int32, device="cuda:0")
    toks, logits = [int(tok.item())], []
    for _ in range(3):
        lgs, ams = gpu.decode_step(token=tok)
        logits.append(lgs.cpu().numpy().copy())
        toks.append(int(ams.item()))
        tok = ams
    gpu.close()
    del gpu
    torch.cuda.empty_cache()
    progress("oracle")
    ref_model = om.Model(QWEN3_0_6B, w)
    del w
    cache = ref_model.new_cache(wl.kv_capacity)
    check_rows(lg_p, am_p, ref_model.forward(prompt, cache, all_logits=True))
    ref_v = ref_model.forward(draft, cache, all_logits=True)
    check_rows(lg_v, am_v, ref_v)
    cache.truncate(P + accept)
    rtoks, rlogits = [int(np.argmax(ref_v[accept - 1]))], []
    for _ in range(3):
        r = ref_model.forward([rtoks[-1]], cache)[0]
        rlogits.append(r)
        rtoks.append(int(np.argmax(r)))
    assert toks == rtoks
    assert row_errs(np.stack(logits), np.stack(rlogits)).max() <= TOL
