"""Elementwise / reduction operators of the forward pass (oracle).

TEST INFRASTRUCTURE ONLY.  Inputs and outputs are f32; every reduction runs
in f64 and is rounded to f32 once.
"""

from __future__ import annotations

import numpy as np


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis.

    ("A transformer from scratch", section 12.3.2; the same form serves the
    per-head Q/K norm over head_dim, minfer "Qwen3 Support Plan" section 2.2.)
    eps is a config field read from the model file's metadata (section
    12.1), whose float keys are read as f32 ("The LLM stack (fucina_llm)",
    section 13.3), so its f32 value is used.  Parity: pinned (mean(y^2) closed form, grouping equivalence).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    return (x64 * r * np.asarray(w, dtype=np.float32).astype(np.float64)).astype(np.float32)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """angle(p, i) = p / theta^(2i/head_dim), i < head_dim/2, in f64 -> [P, hd/2].

    ("A transformer from scratch", section 12.3.4.)
    """
    p = np.asarray(positions, dtype=np.float64)[:, None]
    i = np.arange(head_dim // 2, dtype=np.float64)[None, :]
    return p * np.power(float(theta), -2.0 * i / head_dim)


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """NeoX ("half") rotary embedding of x [T, heads, hd] at positions [T].

    Channel i pairs with channel i + hd/2 and the pair is rotated by
    angle(p, i) ("A transformer from scratch", section 12.3.4; minfer plan
    section 2.1: the full head is rotated).  Parity: pinned (position 0 is
    the identity, position 1 turns pair 0 by one radian, norm preservation,
    relative-position invariance incl. the course's worked values).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    hd = x64.shape[-1]
    half = hd // 2
    ang = rope_angles(positions, hd, theta)[:, None, :]  # [T, 1, half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x64[..., :half], x64[..., half:]
    out = np.empty_like(x64)
    out[..., :half] = a * c - b * s
    out[..., half:] = a * s + b * c
    return out.astype(np.float32)


def kv_head_for_head(num_heads: int, num_kv_heads: int) -> np.ndarray:
    """GQA map: consecutive query heads share a KV head, kv = h / (nh / nkv).

    ("A transformer from scratch", section 12.3.5.)
    """
    per = num_heads // num_kv_heads
    return np.arange(num_heads) // per


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos, k_pos=None) -> np.ndarray:
    """Causal grouped-query attention.

    q [T, nh, hd]; k, v [S, nkv, hd] (post-RoPE keys, raw values);
    q_pos [T] absolute positions of the queries; k_pos [S] positions of the
    keys (default 0..S-1).  Query head h reads KV head h / (nh/nkv); score
    s_j = q.k_j / sqrt(hd) for k_pos_j <= q_pos (causal, self included);
    softmax; o = sum_j p_j v_j.  ("A transformer from scratch", section
    12.3.5.)  Returns f32 [T, nh * hd].  Parity: pinned (single position
    returns v, equal keys average V, GQA == MHA with repeated heads, scale).
    """
    q64 = np.asarray(q, dtype=np.float32).astype(np.float64)
    k64 = np.asarray(k, dtype=np.float32).astype(np.float64)
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    T, nh, hd = q64.shape
    S, nkv, _ = k64.shape
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(S, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    allowed = k_pos[None, :] <= q_pos[:, None]  # [T, S]
    scale = 1.0 / np.sqrt(float(hd))
    kvh = kv_head_for_head(nh, nkv)
    out = np.empty((T, nh, hd), dtype=np.float64)
    for h in range(nh):
        g = kvh[h]
        s = (q64[:, h, :] @ k64[:, g, :].T) * scale  # [T, S]
        s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / np.sum(e, axis=1, keepdims=True)
        out[:, h, :] = p @ v64[:, g, :]
    return out.reshape(T, nh * hd).astype(np.float32)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)) in f64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up, rounded to f32 ("A transformer from scratch",
    section 12.3.6: the gate pathway carries the nonlinearity)."""
    return (silu(g) * np.asarray(u, dtype=np.float32).astype(np.float64)).astype(np.float32)


def add(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Residual-stream add in f32 (section 12.3.7)."""
    return (np.asarray(x, dtype=np.float32) + np.asarray(y, dtype=np.float32)).astype(np.float32)


def argmax_lowest(logits: np.ndarray) -> int:
    """Greedy pick: the lowest index among the maxima (reading: the pages
    keep the first maximum in their strict-greater scans)."""
    return int(np.argmax(np.asarray(logits)))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (round half to even on the 16 dropped bits),
    returned as the f32 value of that bf16.  Finite inputs only."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_linear(x: np.ndarray, w_bf16_as_f32: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """y = x @ W^T with f32 activations and bf16 weights (exactly widened),
    summed in f64, rounded once to f32 (reading of the bf16 weight arm of
    "The LLM stack (fucina_llm)", section 13.2.1: a mixed f32 x bf16 kernel
    with exact in-register widening, no activation rounding).  Every product
    of an f32 and a bf16 value is exact in f64.  Parity: pinned (the exact
    rational sum rounded once, a cancellation an f32 running sum loses,
    unit columns returning activations and weights unrounded)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    N = w_bf16_as_f32.shape[0]
    out = np.empty((x64.shape[0], N), dtype=np.float32)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        wt = np.asarray(w_bf16_as_f32[n0:n1], dtype=np.float64)  # no copy if already f64
        out[:, n0:n1] = (x64 @ wt.T).astype(np.float32)
    return out
