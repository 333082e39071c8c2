"""Pins of the oracle's Q8_0 codec and quantised linear (CPU only).

Each check is tied to something the pages or arithmetic fix, not to the
oracle's own formula:
  * round trip within half a step (+ the f16 scale error), and "within
    0.05" on values in [-2, 2] ("Model files and quantization", 11.7);
  * special blocks whose codes are known in closed form;
  * constructed exact ties (round half to even, the production rounding of
    section 11.10);
  * the 34-byte wire layout and 8.5 bits per weight (section 11.7);
  * integer block dots against brute force, and their bound 32 * 127^2;
  * the linear against exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
from oracle import q8_0
from synthetic import gen_normal_rows


def test_round_trip_bound_random():
    x = gen_normal_rows((257, 128), seed=11, scale=0.7)
    qs, d = q8_0.encode(x)
    back = q8_0.decode(qs, d)
    blocks = x.reshape(-1, 32)
    d32 = (np.max(np.abs(blocks), axis=1) / np.float32(127)).astype(np.float64)
    dh = d.reshape(-1).astype(np.float64)
    bound = d32 / 2 + 127 * np.abs(d32 - dh) + 4 * np.spacing(np.abs(blocks).max(axis=1)).astype(np.float64)
    err = np.abs(blocks.astype(np.float64) - back.reshape(-1, 32).astype(np.float64)).max(axis=1)
    assert np.all(err <= bound)


def test_round_trip_within_005_on_uniform_values():
    # the public encode/decode seam round trip is verified "within 0.05"
    rng = np.random.Generator(np.random.PCG64(7))
    x = (rng.random((64, 32), dtype=np.float32) * 4.0 - 2.0).astype(np.float32)
    back = q8_0.decode(*q8_0.encode(x))
    assert np.max(np.abs(back - x)) <= 0.05


def test_zero_block():
    qs, d = q8_0.encode(np.zeros((1, 64), np.float32))
    assert np.all(qs == 0)
    assert np.all(d == 0)
    assert np.all(q8_0.decode(qs, d) == 0)


@pytest.mark.parametrize("spike", [3.0, -0.0123, 1e-3])
def test_single_spike_block(spike):
    x = np.zeros((1, 32), np.float32)
    x[0, 17] = spike
    qs, d = q8_0.encode(x)
    assert qs[0, 17] == (127 if spike > 0 else -127)
    assert np.count_nonzero(qs) == 1
    assert d[0, 0] == np.float16(np.float32(abs(spike)) / np.float32(127))


def test_amax_element_maps_to_127():
    x = gen_normal_rows((50, 32), seed=3)
    qs, _ = q8_0.encode(x)
    i = np.argmax(np.abs(x), axis=1)
    sgn = np.sign(x[np.arange(50), i])
    assert np.all(qs[np.arange(50), i] == (127 * sgn).astype(np.int8))
    assert np.abs(qs.astype(np.int32)).max() <= 127


def test_exact_ties_round_half_to_even():
    # amax = 127 gives d = 1 and inv = 1 exactly, so v * inv = v.
    x = np.zeros((1, 32), np.float32)
    vals = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, -1.5, 126.5, -126.5]
    x[0, : len(vals)] = vals
    qs, d = q8_0.encode(x)
    assert d[0, 0] == np.float16(1.0)
    assert list(qs[0, : len(vals)]) == [127, 2, 4, -2, -4, 0, 2, 0, -2, 126, -126]


def test_wire_layout_34_bytes():
    facts = {r[0]: r[1] for r in read_golden("model_facts.txt")}
    assert int(facts["q8_0_block_bytes"]) == q8_0.BLOCK_BYTES == 34
    assert float(facts["q8_0_bits_per_weight"]) == q8_0.BLOCK_BYTES * 8 / q8_0.QK
    x = np.zeros((2, 64), np.float32)
    x[0, 0] = 127.0  # d = 1.0 -> f16 bits 0x3C00, little endian 00 3C
    x[1, 33] = -254.0  # second block of row 1: d = 2.0 -> 0x4000, q = -127
    raw = q8_0.to_gguf(*q8_0.encode(x))
    assert raw.shape == (2, 68)
    assert list(raw[0, :3]) == [0x00, 0x3C, 127]
    assert list(raw[0, 34:36]) == [0, 0]
    assert list(raw[1, 34:37]) == [0x00, 0x40, 0]
    assert raw[1, 37] == np.uint8(np.int8(-127).view(np.uint8))
    qs, d = q8_0.from_gguf(raw, 64)
    qs2, d2 = q8_0.encode(x)
    assert np.array_equal(qs, qs2) and np.array_equal(d, d2)


def test_non_finite_rejected():
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        q8_0.encode(x)


def test_requantisation_is_idempotent():
    # quantising an already dequantised row reproduces the same codes/scales
    x = gen_normal_rows((40, 96), seed=5, scale=3.0)
    qs, d = q8_0.encode(x)
    qs2, d2 = q8_0.encode(q8_0.decode(qs, d))
    assert np.array_equal(qs, qs2) and np.array_equal(d, d2)


def test_block_dots_brute_force_and_bound():
    rng = np.random.Generator(np.random.PCG64(9))
    qa = rng.integers(-127, 128, size=(3, 64), dtype=np.int64).astype(np.int8)
    qw = rng.integers(-127, 128, size=(5, 64), dtype=np.int64).astype(np.int8)
    S = q8_0.block_dots(qa, qw)
    for t in range(3):
        for n in range(5):
            for b in range(2):
                ref = 0
                for i in range(32):
                    ref += int(qa[t, 32 * b + i]) * int(qw[n, 32 * b + i])
                assert S[t, n, b] == ref
    worst = q8_0.block_dots(np.full((1, 32), -127, np.int8), np.full((1, 32), -127, np.int8))
    assert worst[0, 0, 0] == 32 * 127 * 127 == 516128 < 2**24


def _exact_linear(x, w_qs, w_d):
    """Exact rational value of the Q8_0 linear for small inputs."""
    qa, da = q8_0.encode(x)
    T, K = qa.shape
    N = w_qs.shape[0]
    out = np.empty((T, N), dtype=np.float64)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 32):
                s = sum(int(qa[t, 32 * b + i]) * int(w_qs[n, 32 * b + i]) for i in range(32))
                acc += Fraction(float(w_d[n, b])) * Fraction(float(da[t, b])) * s
            out[t, n] = float(acc)
    return out


def test_linear_matches_exact_rational():
    x = gen_normal_rows((3, 96), seed=21)
    w = q8_0.Q8Weight(gen_normal_rows((4, 96), seed=22, scale=0.02))
    y = q8_0.linear(x, w)
    exact = _exact_linear(x, w.qs, w.d)
    # f32 result is the exact value rounded once (allow the f64 sum's own
    # rounding: one f32 ulp)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= np.spacing(np.abs(exact).astype(np.float32)))
    # and it equals the block-scaled form sum_b d_w d_a S_b
    qa, da = q8_0.encode(x)
    S = q8_0.block_dots(qa, w.qs).astype(np.float64)
    blockform = np.einsum("tnb,nb,tb->tn", S, w.d.astype(np.float64), da.astype(np.float64))
    assert np.array_equal(y, blockform.astype(np.float32))


def test_linear_quantises_activations():
    # the linear sees Q8_0 activations: feeding the dequantised activation
    # row gives the identical result, while the raw f32 product differs
    x = gen_normal_rows((2, 128), seed=31)
    w = q8_0.Q8Weight(gen_normal_rows((8, 128), seed=32, scale=0.02))
    y = q8_0.linear(x, w)
    xq = q8_0.decode(*q8_0.encode(x))
    assert np.array_equal(y, q8_0.linear(xq, w))
    raw = (x.astype(np.float64) @ w.deq.astype(np.float64).T).astype(np.float32)
    assert not np.array_equal(y, raw)
