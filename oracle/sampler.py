"""The sampling pipeline over one row of logits (oracle; test infrastructure).

"A transformer from scratch", section 12.6, and "The LLM stack
(fucina_llm)", section 13.6: in this fixed order,

  penalties   for every distinct token t among the last repeat_last_n tokens
              of the history, seen c times there: a positive logit is
              divided by repeat_penalty, a negative one multiplied by it,
              then c * freq_penalty + presence_penalty is subtracted;
  greedy      temperature <= 0: the argmax of the penalised logits;
  top-k       top_k > 0: the min(top_k, 256) best candidates, in descending
              order; top_k == 0: a window of 256 candidates that grows
              four-fold until it holds the top_p mass (or the whole vocab);
  softmax     p_i = exp((l_i - l_max) / temperature) / Z, Z over the kept
              top-k set when top_k > 0, over the whole vocabulary when
              top_k == 0 (the exact nucleus);
  top-p       keep the shortest descending prefix whose cumulative p reaches
              top_p (top_p < 1);
  min-p       keep p_i >= min_p * p_0 (min_p > 0);
  draw        one uniform u in [0, 1): the first kept candidate whose
              cumulative p exceeds u times the kept cumulative total.

Readings (the pages leave these open): candidates are ordered by logit,
ties by lower token id; the penalty, the softmax and every sum are taken in
f64 and the penalised logit is rounded back to f32 once; the draw's uniform
is an input (the pages' generator is a seeded PRNG, one draw per token).
Parity: pinned (the pages' greedy example, limits of every knob, the
penalty rule on a hand-made row, the draw's frequencies against p).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MAX_CANDIDATES = 256


@dataclass(frozen=True)
class SamplerConfig:
    temperature: float = 0.0
    top_k: int = 0
    top_p: float = 1.0
    min_p: float = 0.0
    repeat_penalty: float = 1.0
    freq_penalty: float = 0.0
    presence_penalty: float = 0.0
    repeat_last_n: int = 64


def apply_penalties(logits: np.ndarray, history, cfg: SamplerConfig) -> np.ndarray:
    """Penalised copy of an f32 logits row (the pages mutate in place)."""
    out = np.array(logits, dtype=np.float32, copy=True)
    n = cfg.repeat_last_n
    window = list(history)[-n:] if n > 0 else []
    if not window:
        return out
    toks, counts = np.unique(np.asarray(window, dtype=np.int64), return_counts=True)
    rp = float(np.float32(cfg.repeat_penalty))
    fp = float(np.float32(cfg.freq_penalty))
    pp = float(np.float32(cfg.presence_penalty))
    for t, c in zip(toks, counts):
        v = float(out[t])
        v = v / rp if v > 0 else v * rp
        v = v - (float(c) * fp + pp)
        out[t] = np.float32(v)
    return out


def order(logits: np.ndarray) -> np.ndarray:
    """Token ids by descending logit, ties by ascending id."""
    ids = np.arange(logits.shape[0])
    return np.lexsort((ids, -np.asarray(logits, dtype=np.float64)))


def sample(logits: np.ndarray, history, cfg: SamplerConfig, u: float):
    """One token from a row of f32 logits.  Returns (token, info) where info
    holds the penalised row, the candidates, their p and the kept count."""
    row = apply_penalties(logits, history, cfg)
    if cfg.temperature <= 0:
        return int(np.argmax(row)), {"row": row}
    V = row.shape[0]
    srt = order(row)
    lmax = float(row[srt[0]])
    T = float(np.float32(cfg.temperature))
    top_p = float(np.float32(cfg.top_p))
    if cfg.top_k > 0:
        k = min(cfg.top_k, MAX_CANDIDATES, V)
        cand = srt[:k]
        e = np.exp((row[cand].astype(np.float64) - lmax) / T)
        p = e / np.sum(e)
    else:
        z = np.sum(np.exp((row.astype(np.float64) - lmax) / T))
        W = min(MAX_CANDIDATES, V)
        while True:
            cand = srt[:W]
            p = np.exp((row[cand].astype(np.float64) - lmax) / T) / z
            if top_p >= 1.0 or W == V or np.sum(p) >= top_p:
                break
            W = min(4 * W, V)
    keep = len(cand)
    if top_p < 1.0:
        cum = np.cumsum(p)
        hit = np.nonzero(cum >= top_p)[0]
        if hit.size:
            keep = int(hit[0]) + 1
    min_p = float(np.float32(cfg.min_p))
    if min_p > 0:
        keep = min(keep, int(np.sum(p[:keep] >= min_p * p[0])))
    kept = p[:keep]
    cum = np.cumsum(kept)
    r = float(np.float32(u)) * cum[-1]
    pick = int(np.searchsorted(cum, r, side="right"))
    pick = min(pick, keep - 1)
    return int(cand[pick]), {"row": row, "cand": cand, "p": p, "keep": keep, "r": r, "cum": cum}
