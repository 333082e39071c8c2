"""Pins of the oracle's operators (CPU only): RMSNorm, RoPE, attention,
SwiGLU, greedy argmax, bf16 rounding."""

import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from conftest import read_golden
from oracle import ops
from synthetic import gen_normal_rows


# -- RMSNorm ("A transformer from scratch", 12.3.2) ------------------------
def test_rmsnorm_mean_square_closed_form():
    x = gen_normal_rows((6, 1024), seed=1, scale=0.3)
    eps = 1e-6
    y = ops.rmsnorm(x, np.ones(1024, np.float32), eps).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-6, atol=0)


def test_rmsnorm_eps_guards_zero_and_weight_scales():
    y = ops.rmsnorm(np.zeros((1, 64), np.float32), np.ones(64, np.float32), 1e-6)
    assert np.all(y == 0)
    x = gen_normal_rows((3, 64), seed=2)
    w = gen_normal_rows((64,), seed=3)
    ones = ops.rmsnorm(x, np.ones(64, np.float32), 1e-6)
    assert np.allclose(ops.rmsnorm(x, w, 1e-6), ones * w, rtol=2e-7, atol=0)


def test_per_head_norm_is_plain_norm_over_head_rows():
    # per-head Q/K RMSNorm == the ordinary kernel over rows of length hd
    # (minfer "Qwen3 Support Plan", 2.2: d = hd, n = tokens * heads)
    q = gen_normal_rows((5, 16, 128), seed=4)
    w = gen_normal_rows((128,), seed=5)
    a = ops.rmsnorm(q, w, 1e-6)
    b = np.stack([ops.rmsnorm(q[t, h][None, :], w, 1e-6)[0] for t in range(5) for h in range(16)])
    assert np.array_equal(a.reshape(-1, 128), b)


# -- RoPE ("A transformer from scratch", 12.3.4) ---------------------------
def test_rope_position_zero_is_identity():
    x = gen_normal_rows((1, 3, 128), seed=6)
    assert np.array_equal(ops.rope(x, [0], 1e6), x)


def test_rope_position_one_turns_pair_zero_by_one_radian():
    x = gen_normal_rows((1, 1, 128), seed=7)
    y = ops.rope(x, [1], 1e6)[0, 0].astype(np.float64)
    a, b = float(x[0, 0, 0]), float(x[0, 0, 64])
    assert y[0] == pytest.approx(a * math.cos(1.0) - b * math.sin(1.0), rel=1e-6)
    assert y[64] == pytest.approx(a * math.sin(1.0) + b * math.cos(1.0), rel=1e-6)
    # the slowest pair (i = 63) turns by theta^(-126/128) at position 1
    ang = 1e6 ** (-126 / 128)
    a, b = float(x[0, 0, 63]), float(x[0, 0, 127])
    assert y[63] == pytest.approx(a * math.cos(ang) - b * math.sin(ang), rel=1e-6, abs=1e-9)


def test_rope_preserves_pair_norms():
    x = gen_normal_rows((9, 4, 64), seed=8)
    pos = [0, 1, 2, 100, 513, 4095, 16383, 32767, 40000]
    y = ops.rope(x, pos, 1e6).astype(np.float64)
    x64 = x.astype(np.float64)
    n0 = x64[..., :32] ** 2 + x64[..., 32:] ** 2
    n1 = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(n0, n1, rtol=1e-6)


def test_rope_course_worked_example():
    rows = read_golden("rope_course.txt")
    q = np.array([float(v) for v in rows[0][1:]], np.float32)
    k = np.array([float(v) for v in rows[1][1:]], np.float32)

    def score(pq, pk):
        a = ops.rope(q[None, None, :], [pq], 1e6)[0, 0]
        b = ops.rope(k[None, None, :], [pk], 1e6)[0, 0]
        return float(np.dot(a.astype(np.float64), b.astype(np.float64)))

    for r in rows[2:]:
        kind, p1, p2, p3, p4, tol = r[0], *map(int, r[1:5]), float(r[5])
        diff = abs(score(p1, p2) - score(p3, p4))
        if kind == "equal":
            assert diff <= tol
        else:
            assert diff > tol


def test_rope_relative_position_full_head():
    q = gen_normal_rows((1, 1, 128), seed=9)
    k = gen_normal_rows((1, 1, 128), seed=10)

    def score(pq, pk):
        a = ops.rope(q, [pq], 1e6)[0, 0].astype(np.float64)
        b = ops.rope(k, [pk], 1e6)[0, 0].astype(np.float64)
        return float(a @ b)

    base = score(7, 3)
    for s in (1, 50, 1000, 20000):
        assert abs(score(7 + s, 3 + s) - base) <= 2e-5 * (1 + abs(base))
    assert abs(score(7, 2) - base) > 1e-3


# -- attention ("A transformer from scratch", 12.3.5) ----------------------
def test_single_cached_position_returns_v():
    q = gen_normal_rows((1, 4, 64), seed=11)
    k = gen_normal_rows((1, 2, 64), seed=12)
    v = gen_normal_rows((1, 2, 64), seed=13)
    o = ops.attention(q, k, v, [0]).reshape(4, 64)
    for h in range(4):
        assert np.array_equal(o[h], v[0, h // 2])


def test_identical_keys_average_values():
    q = gen_normal_rows((1, 2, 32), seed=14)
    k = np.repeat(gen_normal_rows((1, 1, 32), seed=15), 6, axis=0)
    v = gen_normal_rows((6, 1, 32), seed=16)
    o = ops.attention(q, k, v, [5]).reshape(2, 32)
    mean = v[:, 0, :].astype(np.float64).mean(axis=0)
    assert np.allclose(o[0], mean, rtol=1e-6, atol=1e-7)
    assert np.allclose(o[1], mean, rtol=1e-6, atol=1e-7)


def test_softmax_weights_sum_to_one():
    q = gen_normal_rows((3, 4, 64), seed=17)
    k = gen_normal_rows((9, 2, 64), seed=18)
    v = np.ones((9, 2, 64), np.float32)
    o = ops.attention(q, k, v, [6, 7, 8])
    assert np.allclose(o, 1.0, rtol=0, atol=1e-6)


def test_gqa_equals_mha_with_repeated_kv_heads():
    q = gen_normal_rows((4, 16, 128), seed=19)
    k = gen_normal_rows((10, 8, 128), seed=20)
    v = gen_normal_rows((10, 8, 128), seed=21)
    pos = [6, 7, 8, 9]
    gqa = ops.attention(q, k, v, pos)
    mha = ops.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), pos)
    assert np.array_equal(gqa, mha)
    assert list(ops.kv_head_for_head(16, 8)) == [h // 2 for h in range(16)]


def test_score_scale_is_inverse_sqrt_head_dim():
    facts = {r[0]: r[1] for r in read_golden("model_facts.txt")}
    hd = int(facts["qk_scale_head_dim"])
    # two keys whose raw dot products with q differ by delta
    q = np.zeros((1, 1, hd), np.float32)
    q[0, 0, 0] = 4.0
    k = np.zeros((2, 1, hd), np.float32)
    k[0, 0, 0] = 1.0  # q.k0 = 4
    k[1, 0, 0] = -0.5  # q.k1 = -2
    v = np.zeros((2, 1, hd), np.float32)
    v[0, 0, 0] = 1.0
    v[1, 0, 1] = 1.0
    o = ops.attention(q, k, v, [1])[0].astype(np.float64)
    ratio = o[0] / o[1]  # = p0 / p1 = exp(6 / sqrt(hd))
    assert ratio == pytest.approx(math.exp(6.0 / math.sqrt(128.0)), rel=1e-6)


def test_causal_mask_ignores_later_keys():
    q = gen_normal_rows((1, 2, 32), seed=22)
    k = gen_normal_rows((8, 1, 32), seed=23)
    v = gen_normal_rows((8, 1, 32), seed=24)
    a = ops.attention(q, k, v, [3])
    k2, v2 = k.copy(), v.copy()
    k2[4:] = 9.0
    v2[4:] = -9.0
    assert np.array_equal(a, ops.attention(q, k2, v2, [3]))


# -- SwiGLU ("A transformer from scratch", 12.3.6) -------------------------
def test_silu_matches_logistic_form():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(ops.silu(z), z * expit(z), rtol=1e-12, atol=1e-300)
    assert ops.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_gates_with_the_gate_operand():
    g = np.array([[2.0, -1.0]], np.float32)
    u = np.array([[3.0, 5.0]], np.float32)
    h = ops.swiglu(g, u)
    assert h[0, 0] == np.float32(2.0 * expit(2.0) * 3.0)
    assert h[0, 1] == np.float32(-1.0 * expit(-1.0) * 5.0)


# -- greedy ("The LLM stack", 13.6) ----------------------------------------
def test_greedy_golden():
    rows = {r[0]: r[1:] for r in read_golden("greedy_sampler.txt")}
    logits = np.array([float(v) for v in rows["logits"]], np.float32)
    assert ops.argmax_lowest(logits) == int(rows["argmax"][0])


def test_greedy_ties_pick_lowest_index():
    assert ops.argmax_lowest(np.array([0.0, 3.0, 1.0, 3.0], np.float32)) == 1


# -- bf16 storage -------------------------------------------------------------
def test_bf16_round_matches_torch():
    x = gen_normal_rows((20000,), seed=25, scale=5.0)
    # exact ties: the 16 dropped bits are 0x8000
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    for arr in (x, ties, -ties):
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(ops.bf16_round(arr), ref)


# -- bf16-weight linear ("The LLM stack (fucina_llm)", section 13.2.1: bf16
# weights widened exactly in registers, activations kept in f32) -------------
def _round_f32(fr):
    """The f32 nearest to the rational fr (ties to even), by exact compare."""
    from fractions import Fraction

    f = np.float32(float(fr))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0] or (d == best[0] and (c.view(np.uint32) & 1) == 0):
            best = (d, c)
    return best[1]


def test_bf16_linear_is_the_exact_sum_rounded_once():
    from fractions import Fraction

    x = gen_normal_rows((3, 96), seed=41)
    w = ops.bf16_round(gen_normal_rows((8, 96), seed=42, scale=0.02))
    y = ops.bf16_linear(x, w)
    assert y.dtype == np.float32 and y.shape == (3, 8)
    exact = np.empty((3, 8), np.float32)
    for t in range(3):
        for n in range(8):
            acc = sum((Fraction(float(x[t, k])) * Fraction(float(w[n, k])) for k in range(96)), Fraction(0))
            exact[t, n] = _round_f32(acc)
    assert np.array_equal(y, exact)


def test_bf16_linear_keeps_what_an_f32_sum_loses():
    # x . w with w = 1: 2^24 + 1 - 2^24 is 0 in an f32 running sum, 1 exactly
    x = np.zeros((2, 32), np.float32)
    x[0, :3] = [2.0**24, 1.0, -(2.0**24)]
    x[1, :4] = [1.0, 2.0**-30, 2.0**-30, -1.0]
    w = np.ones((1, 32), np.float32)
    y = ops.bf16_linear(x, w)
    assert y[0, 0] == 1.0
    assert y[1, 0] == np.float32(2.0**-29)


def test_bf16_linear_activations_are_not_rounded():
    # a unit weight column picks out the activation itself, all 24 bits of it
    x = gen_normal_rows((4, 64), seed=43)
    w = np.zeros((64, 64), np.float32)
    w[np.arange(64), np.arange(64)] = 1.0
    assert np.array_equal(ops.bf16_linear(x, w), x)
    # and a weight row is used as the bf16 value it holds (no re-rounding)
    wb = ops.bf16_round(gen_normal_rows((5, 64), seed=44, scale=0.02))
    e = np.zeros((64, 64), np.float32)
    e[np.arange(64), np.arange(64)] = 1.0
    assert np.array_equal(ops.bf16_linear(e, wb), wb.T)
