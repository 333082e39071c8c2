"""The device sampling pipeline against the oracle's ("A transformer from
scratch", section 12.6; "The LLM stack (fucina_llm)", section 13.6).

Penalised logits must equal the oracle's bitwise (f64 arithmetic, one f32
rounding).  Tokens are index results and must be equal, except where the
oracle's draw or top-p cut lies within 1e-9 of a cumulative boundary (the
two sides sum their probabilities in different orders): such rows are
checked for validity only.  The exact nucleus's window grows four-fold up to
the whole vocabulary, as the page says ("no tail is silently clipped"):
windows past 4096 candidates (16384, 65536, all 151,936) are checked the
same way.
"""

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import model as om
from oracle import sampler as sp
from synthetic import TINY, gen_prompt, gen_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_sample(logits, cfg, u, history=None, hlen=None):
    from quantized_q8_dequant_amd import sample

    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    uni = torch.from_numpy(np.asarray(u, np.float32)).to(DEV) if u is not None else None
    h = torch.from_numpy(np.asarray(history, np.int32)).to(DEV) if history is not None else None
    hl = torch.from_numpy(np.asarray(hlen, np.int32)).to(DEV) if hlen is not None else None
    tok = sample(
        lg, uni, cfg.temperature, cfg.top_k, cfg.top_p, cfg.min_p, cfg.repeat_penalty, cfg.freq_penalty,
        cfg.presence_penalty, cfg.repeat_last_n, h, hl,
    )
    return tok.cpu().numpy(), lg.cpu().numpy()


def near_boundary(info, top_p):
    if "cum" not in info:
        return False
    cum = info["cum"]
    r = info["r"]
    if np.min(np.abs(cum - r)) <= 1e-9 * max(cum[-1], 1e-300):
        return True
    if top_p < 1.0:
        full = np.cumsum(info["p"])
        if np.min(np.abs(full - top_p)) <= 1e-9:
            return True
    return False


def test_greedy_example_from_the_pages():
    rows = {r[0]: r[1:] for r in read_golden("greedy_sampler.txt")}
    logits = np.array([[float(x) for x in rows["logits"]]], np.float32)
    tok, _ = gpu_sample(logits, sp.SamplerConfig(), None)
    assert tok[0] == int(rows["argmax"][0])


def test_penalties_bitwise():
    rng = np.random.default_rng(5)
    n, V, stride = 6, 5000, 80
    logits = (rng.standard_normal((n, V)) * 3).astype(np.float32)
    hist = rng.integers(0, 60, size=(n, stride)).astype(np.int32)  # many repeats
    hlen = np.array([0, 1, 17, 64, 70, 80], np.int32)
    cfg = sp.SamplerConfig(temperature=0.0, repeat_penalty=1.3, freq_penalty=0.4, presence_penalty=0.7, repeat_last_n=64)
    tok, pen = gpu_sample(logits, cfg, None, hist, hlen)
    for r in range(n):
        ref = sp.apply_penalties(logits[r], hist[r, : hlen[r]], cfg)
        assert np.array_equal(pen[r], ref), r
        assert tok[r] == int(np.argmax(ref))


CONFIGS = [
    (4.0, sp.SamplerConfig(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)),
    (4.0, sp.SamplerConfig(temperature=1.3, top_k=256)),
    (4.0, sp.SamplerConfig(temperature=1.0, top_p=0.9)),  # window 256 -> 1024
    (3.0, sp.SamplerConfig(temperature=0.8, top_p=0.95)),  # window -> 4096
    (2.0, sp.SamplerConfig(temperature=1.0, top_p=0.5)),  # window -> 4096
    (4.0, sp.SamplerConfig(temperature=0.5, min_p=0.1)),  # the 256 work window, min-p
    (4.0, sp.SamplerConfig(temperature=0.9, top_k=5, repeat_penalty=1.5, presence_penalty=0.5)),
]


@pytest.mark.parametrize("ci", range(len(CONFIGS)))
def test_tokens_match_the_oracle(ci):
    sigma, cfg = CONFIGS[ci]
    rng = np.random.default_rng(100 + ci)
    n, V = 8, 151936
    logits = (rng.standard_normal((n, V)) * sigma).astype(np.float32)
    u = rng.random(n).astype(np.float32)
    hist = rng.integers(0, V, size=(n, 32)).astype(np.int32)
    hist[:, 16:] = np.argsort(-logits, axis=1)[:, :16]  # penalise some of the best tokens
    hlen = np.full(n, 32, np.int32)
    tok, _ = gpu_sample(logits, cfg, u, hist, hlen)
    checked = 0
    for r in range(n):
        want, info = sp.sample(logits[r], hist[r], cfg, float(u[r]))
        if near_boundary(info, cfg.top_p):
            assert tok[r] in info["cand"]
            continue
        assert tok[r] == want, (r, tok[r], want)
        checked += 1
    assert checked >= n - 3


def _rows(kind, n, V, seed):
    rng = np.random.default_rng(seed)
    if kind == "best_in_one_slice":  # every top logit in ids [0, 4096)
        x = rng.standard_normal((n, V)) * 3.0
        x[:, :4096] += 12.0
    elif kind == "integer_logits":  # heavy ties at every cut
        x = np.round(rng.standard_normal((n, V)) * 1.5)
    else:  # "clipped": about 31% of the row tied at the maximum
        x = np.minimum(rng.standard_normal((n, V)), 0.5)
    return x.astype(np.float32)


SPECIAL = [
    # the window passes what the slices' lists are sure to hold: the whole row
    ("best_in_one_slice", sp.SamplerConfig(temperature=1.0, top_k=256)),
    ("best_in_one_slice", sp.SamplerConfig(temperature=1.0, top_k=200)),  # exactly what the lists hold
    ("best_in_one_slice", sp.SamplerConfig(temperature=1.0, top_p=0.9)),
    # the union overflows its LDS copy; ties at the cut, kept in id order
    ("integer_logits", sp.SamplerConfig(temperature=1.0, top_k=256)),
    ("integer_logits", sp.SamplerConfig(temperature=1.0, top_p=0.05)),
    ("integer_logits", sp.SamplerConfig(temperature=0.8, top_k=30, min_p=0.2)),
    # more equal keys than the window: gathered from the row in id order
    ("clipped", sp.SamplerConfig(temperature=1.0, top_k=256)),
    ("clipped", sp.SamplerConfig(temperature=1.0, top_p=0.01)),
]


@pytest.mark.parametrize("ci", range(len(SPECIAL)))
def test_tokens_match_the_oracle_on_skewed_and_tied_rows(ci):
    kind, cfg = SPECIAL[ci]
    n, V = 6, 151936
    logits = _rows(kind, n, V, 300 + ci)
    u = np.random.default_rng(400 + ci).random(n).astype(np.float32)
    tok, _ = gpu_sample(logits, cfg, u)
    checked = 0
    for r in range(n):
        want, info = sp.sample(logits[r], [], cfg, float(u[r]))
        assert len(info["cand"]) <= 4096
        if near_boundary(info, cfg.top_p):
            assert tok[r] in info["cand"]
            continue
        assert tok[r] == want, (r, tok[r], want)
        checked += 1
    assert checked >= n - 2


WIDE = [
    # (logit sigma, config, the oracle's final window)
    (3.0, sp.SamplerConfig(temperature=1.0, top_p=0.9), 16384),
    (2.0, sp.SamplerConfig(temperature=1.0, top_p=0.9), 65536),
    (1.0, sp.SamplerConfig(temperature=1.0, top_p=0.9), 151936),
    (0.2, sp.SamplerConfig(temperature=1.0, top_p=0.999, min_p=0.5), 151936),
]


@pytest.mark.parametrize("ci", range(len(WIDE)))
def test_wide_exact_nucleus_matches_the_oracle(ci):
    """Nuclei that need more than 4096 candidates: the window grows to 16384,
    65536 or the whole vocabulary, and the token is the oracle's."""
    sigma, cfg, window = WIDE[ci]
    rng = np.random.default_rng(700 + ci)
    n, V = 4, 151936
    logits = (rng.standard_normal((n, V)) * sigma).astype(np.float32)
    u = rng.random(n).astype(np.float32)
    tok, _ = gpu_sample(logits, cfg, u)
    checked = 0
    for r in range(n):
        want, info = sp.sample(logits[r], [], cfg, float(u[r]))
        assert len(info["cand"]) == window
        if near_boundary(info, cfg.top_p):
            assert tok[r] in info["cand"]
            continue
        assert tok[r] == want, (r, tok[r], want)
        checked += 1
    assert checked >= n - 1


def test_wide_nucleus_keeps_ties_in_id_order():
    """A wide window over rows of few distinct logits (steps of 0.25): the
    65536-candidate window ends inside a run of about 14,000 equal logits,
    which are taken lowest id first, and every kept run is in id order, so
    each draw lands on the oracle's token."""
    rng = np.random.default_rng(710)
    n, V = 6, 151936
    logits = (np.round(rng.standard_normal((n, V)) * 4.0) / 4.0).astype(np.float32)
    cfg = sp.SamplerConfig(temperature=1.5, top_p=0.6)
    u = rng.random(n).astype(np.float32)
    tok, _ = gpu_sample(logits, cfg, u)
    checked = 0
    for r in range(n):
        want, info = sp.sample(logits[r], [], cfg, float(u[r]))
        assert len(info["cand"]) == 65536
        if near_boundary(info, cfg.top_p):
            assert tok[r] in info["cand"]
            continue
        assert tok[r] == want, (r, tok[r], want)
        checked += 1
    assert checked >= n - 1


def test_draw_frequencies_follow_p():
    logits = np.array([1.0, 0.2, 0.7, -0.3, 0.1], np.float32)
    cfg = sp.SamplerConfig(temperature=0.7, top_k=5)
    N = 4096
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    tok, _ = gpu_sample(np.tile(logits, (N, 1)), cfg, u)
    want = np.array([sp.sample(logits, [], cfg, float(x))[0] for x in u])
    assert np.array_equal(tok, want)


def test_sampling_model_logits_with_a_history():
    w = gen_weights(TINY, 101)
    ref = om.Model(TINY, w)
    prompt = gen_prompt(TINY.vocab_size, 24, 61)
    logits = ref.forward(prompt, ref.new_cache(32))  # [1, V]
    cfg = sp.SamplerConfig(temperature=0.8, top_k=40, top_p=0.9, repeat_penalty=1.1, freq_penalty=0.2, repeat_last_n=16)
    u = np.array([0.123], np.float32)
    tok, pen = gpu_sample(logits, cfg, u, prompt[None].astype(np.int32), np.array([24], np.int32))
    want, info = sp.sample(logits[0], prompt, cfg, 0.123)
    assert np.array_equal(pen[0], info["row"])
    assert tok[0] == want


@pytest.mark.parametrize("V", [1, 7, 255, 4097, 8195])
@pytest.mark.parametrize("cfg", [
    sp.SamplerConfig(temperature=1.0, top_p=0.9),
    sp.SamplerConfig(temperature=0.8, top_k=300),  # more than the 256 cap, more than some rows
    sp.SamplerConfig(temperature=0.6, top_k=40, min_p=0.05, top_p=0.8),
    sp.SamplerConfig(temperature=0.0),
], ids=["nucleus", "top_k300", "mixed", "greedy"])
def test_odd_vocabulary_sizes(V, cfg):
    """Rows shorter than a slice, one logit past a slice (a one-element
    slice), lengths that are not multiples of four (scalar row passes)."""
    rng = np.random.default_rng(V)
    n = 5
    logits = (rng.standard_normal((n, V)) * 2.0).astype(np.float32)
    u = rng.random(n).astype(np.float32)
    tok, _ = gpu_sample(logits, cfg, u)
    for r in range(n):
        want, info = sp.sample(logits[r], [], cfg, float(u[r]))
        if near_boundary(info, cfg.top_p):
            assert tok[r] in info["cand"]
            continue
        assert tok[r] == want, (r, tok[r], want)
