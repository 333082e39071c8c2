"""Pins of the oracle's sampling pipeline ("A transformer from scratch",
section 12.6; "The LLM stack (fucina_llm)", section 13.6).  Each pin fixes
one stage against a value the pages or arithmetic give: the pages' greedy
example, the limit every knob reduces to, the penalty rule on a row worked
by hand, and the draw's frequencies against the probabilities."""

import numpy as np
import pytest

from conftest import read_golden
from oracle import sampler as sp


def test_greedy_example_from_the_pages():
    rows = {r[0]: r[1:] for r in read_golden("greedy_sampler.txt")}
    logits = np.array([float(x) for x in rows["logits"]], np.float32)
    assert sp.sample(logits, [], sp.SamplerConfig(), 0.5)[0] == int(rows["argmax"][0])


def _row(V=300, seed=1, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(V) * scale).astype(np.float32)


@pytest.mark.parametrize("u", [0.0, 0.3, 0.999])
def test_limits_reduce_to_the_argmax(u):
    row = _row()
    best = int(np.argmax(row))
    assert sp.sample(row, [], sp.SamplerConfig(temperature=0.8, top_k=1), u)[0] == best
    assert sp.sample(row, [], sp.SamplerConfig(temperature=0.8, top_p=1e-6), u)[0] == best
    assert sp.sample(row, [], sp.SamplerConfig(temperature=0.8, min_p=1.0), u)[0] == best
    assert sp.sample(row, [], sp.SamplerConfig(temperature=1e-4), u)[0] == best


def test_penalty_rule_on_a_hand_worked_row():
    logits = np.array([2.0, -1.0, 0.5, 3.0], np.float32)
    cfg = sp.SamplerConfig(repeat_penalty=2.0, freq_penalty=0.5, presence_penalty=0.25)
    out = sp.apply_penalties(logits, [0, 1, 0, 3], cfg)
    # token 0 seen twice: 2/2 - (2*0.5 + 0.25); token 1 once: -1*2 - 0.75;
    # token 3 once: 3/2 - 0.75; token 2 not in the window
    assert np.array_equal(out, np.array([-0.25, -2.75, 0.5, 0.75], np.float32))
    # only the last two tokens count with repeat_last_n = 2
    out2 = sp.apply_penalties(logits, [0, 1, 0, 3], sp.SamplerConfig(2.0, 0, 1.0, 0.0, 2.0, 0.5, 0.25, 2))
    assert np.array_equal(out2, np.array([0.25, -1.0, 0.5, 0.75], np.float32))
    # a penalty of 1 and no subtraction leave the row alone
    assert np.array_equal(sp.apply_penalties(logits, [0, 1, 3], sp.SamplerConfig()), logits)
    # greedy runs on the penalised row: token 3 (3.0) drops below token 2
    assert sp.sample(logits, [0, 1, 0, 3], cfg, 0.5)[0] == 3
    assert sp.sample(logits, [3, 3, 3, 3], sp.SamplerConfig(repeat_penalty=10.0), 0.5)[0] == 0


def test_draw_frequencies_follow_p():
    logits = np.array([1.0, 0.2, 0.7, -0.3, 0.1], np.float32)
    cfg = sp.SamplerConfig(temperature=0.7, top_k=5)
    e = np.exp((logits.astype(np.float64) - 1.0) / np.float64(np.float32(0.7)))
    p = e / e.sum()
    N = 20000
    picks = np.array([sp.sample(logits, [], cfg, (i + 0.5) / N)[0] for i in range(N)])
    freq = np.bincount(picks, minlength=5) / N
    assert np.allclose(freq, p, atol=2.0 / N)
    # the inverse CDF runs in descending order: u near 0 picks the best token
    assert picks[0] == 0 and picks[-1] == 3


def test_exact_nucleus_grows_its_window():
    """top_k = 0: probabilities over the whole vocab; the window grows past
    256 candidates when the top_p mass needs it."""
    V = 3000
    row = np.zeros(V, np.float32)
    row[:10] = 0.5
    cfg = sp.SamplerConfig(temperature=1.0, top_p=0.5)
    tok, info = sp.sample(row, [], cfg, 0.99999)
    keep = info["keep"]
    assert 256 < keep < V
    assert info["p"][:keep].sum() >= 0.5 > info["p"][: keep - 1].sum()
    e = np.ones(V)
    e[:10] = np.exp(0.5)
    assert np.allclose(info["p"], (e / e.sum())[info["cand"]], rtol=1e-12)
    # kept candidates are the ten raised tokens, then ties by ascending id
    assert list(info["cand"][:12]) == list(range(12))
    assert tok == info["cand"][keep - 1]  # u near 1 takes the last kept one
    # top_p = 1 keeps the 256-candidate work window
    _, info1 = sp.sample(row, [], sp.SamplerConfig(temperature=1.0), 0.5)
    assert info1["keep"] == 256


def test_top_k_renormalises_over_the_kept_set():
    row = _row(seed=4)
    cfg = sp.SamplerConfig(temperature=0.9, top_k=20, top_p=0.8, min_p=0.05)
    tok, info = sp.sample(row, [], cfg, 0.37)
    assert len(info["cand"]) == 20 and abs(info["p"].sum() - 1.0) < 1e-12
    assert info["keep"] <= 20 and tok in info["cand"][: info["keep"]]
    assert np.all(np.diff(row[info["cand"]]) <= 0)
