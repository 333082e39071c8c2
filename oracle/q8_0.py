"""Q8_0 block codec and the quantised linear (oracle; test infrastructure).

Q8_0 ("Model files and quantization", section 11.7): 32 consecutive values
share one scale.  The block is 34 bytes on the wire: the f16 bits of the
scale d, then 32 signed bytes.  Encoding one block:

  amax = max |v_i|                      (f32)
  d    = amax / 127                     (f32 division)
  inv  = 0 if d == 0 else 1 / d         (f32 division, from the f32 d)
  q_i  = clamp(round(v_i * inv), -127, 127)
  store f16(d)

Readings where the page leaves a step open:
  * rounding of v*inv is round-half-to-even (the production encoders round
    through the 1.5 * 2^23 magic constant, section 11.10, which is RNE; the
    course's toy uses round-half-away, which only differs on exact ties);
  * the integers use inv computed from the unrounded f32 d, while the stored
    and dequantisation scale is f16(d) (the encoder computes inv_d from d
    before converting d to f16 bits);
  * an all-zero block gives d = 0, inv = 0, all q = 0.

The quantised linear ("Model files and quantization", section 11.9): the
activation row is quantised on the fly to Q8_0 as well, each 32-block pair
gives an exact integer dot S, rescaled by d_w * d_a, and the block terms are
summed.  Because f16(d_w) * f16(d_a) * S is exact in f64 and equals
sum_k dequant(w)_k * dequant(a)_k over the block, the oracle evaluates the
plain definition  y = sum_k dequant(w)_k * dequant(a)_k  in f64 and rounds to
f32 once (the GPU may sum the block terms in any f32 order).
"""

from __future__ import annotations

import numpy as np

QK = 32  # values per block
BLOCK_BYTES = 34  # 2 (f16 scale) + 32 (int8)


def f16_round(x) -> np.ndarray:
    """Round f32 to the nearest f16 (IEEE round-half-even), as f16."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def encode(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise the last axis of f32 `x` (length a multiple of 32) to Q8_0.

    Returns (qs int8 [..., K], d f16 [..., K/32]).  Parity: pinned (round
    trip bound, special blocks, constructed ties, 34-byte layout).
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    if K % QK:
        raise ValueError(f"row length {K} is not a whole number of 32-blocks")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in Q8_0 encoder input")
    blocks = x.reshape(x.shape[:-1] + (K // QK, QK))
    amax = np.max(np.abs(blocks), axis=-1)  # exact in f32
    d = (amax / np.float32(127.0)).astype(np.float32)  # f32 division
    with np.errstate(divide="ignore"):
        inv = np.where(d == 0, np.float32(0.0), np.float32(1.0) / d).astype(np.float32)
    prod = (blocks * inv[..., None]).astype(np.float32)  # f32 product
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)  # RNE
    return q.reshape(x.shape), f16_round(d)


def decode(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Dequantise: value = f32(f16 d) * q (exact in f32: 11 x 8 bit)."""
    qs = np.asarray(qs, dtype=np.int8)
    K = qs.shape[-1]
    blocks = qs.reshape(qs.shape[:-1] + (K // QK, QK)).astype(np.float32)
    out = blocks * np.asarray(d, dtype=np.float16).astype(np.float32)[..., None]
    return out.reshape(qs.shape)


def to_gguf(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Serialise to the 34-byte AoS wire format: per block, f16 bits of d
    (little endian) then 32 int8.  Returns uint8 [..., K/32 * 34]."""
    qs = np.asarray(qs, dtype=np.int8)
    K = qs.shape[-1]
    nb = K // QK
    lead = qs.shape[:-1]
    out = np.empty(lead + (nb, BLOCK_BYTES), dtype=np.uint8)
    out[..., 0:2] = np.asarray(d, dtype="<f2").reshape(lead + (nb, 1)).view(np.uint8)
    out[..., 2:] = qs.reshape(lead + (nb, QK)).view(np.uint8)
    return out.reshape(lead + (nb * BLOCK_BYTES,))


def from_gguf(raw: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of to_gguf."""
    raw = np.asarray(raw, dtype=np.uint8)
    nb = K // QK
    lead = raw.shape[:-1]
    b = raw.reshape(lead + (nb, BLOCK_BYTES))
    d = np.ascontiguousarray(b[..., 0:2]).view("<f2").reshape(lead + (nb,)).astype(np.float16)
    qs = np.ascontiguousarray(b[..., 2:]).view(np.int8).reshape(lead + (K,))
    return qs, d


def block_dots(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """Integer block dots S[t, n, b] = sum_{i<32} qa[t, 32b+i] * qw[n, 32b+i].

    ("Model files and quantization", section 11.9, the per-block integer dot.)
    qa int8 [T, K], qw int8 [N, K] -> int64 [T, N, K/32].  Evaluated exactly
    with an int64 contraction.  Parity: pinned (brute force).
    """
    qa = np.asarray(qa, dtype=np.int64)
    qw = np.asarray(qw, dtype=np.int64)
    T, K = qa.shape
    N = qw.shape[0]
    a = qa.reshape(T, K // QK, QK)
    w = qw.reshape(N, K // QK, QK)
    return np.einsum("tbi,nbi->tnb", a, w)


class Q8Weight:
    """A Q8_0 weight matrix [N, K] (logical [out, in], `in` contiguous).

    Block row r is output r ("Model files and quantization", section 11.9).
    Keeps the codes, the f16 scales and an exact f32 dequantised copy.
    """

    def __init__(self, w_f32: np.ndarray):
        self.qs, self.d = encode(w_f32)
        self.N, self.K = self.qs.shape
        self.deq = decode(self.qs, self.d)

    @classmethod
    def from_codes(cls, qs, d):
        obj = cls.__new__(cls)
        obj.qs = np.asarray(qs, dtype=np.int8)
        obj.d = np.asarray(d, dtype=np.float16)
        obj.N, obj.K = obj.qs.shape
        obj.deq = decode(obj.qs, obj.d)
        return obj

    def keep_f64(self) -> None:
        """Keep an f64 copy of the dequantised values (exact widening), so
        that repeated linears do not widen the matrix on every call.  Same
        values, same products and sums: a speed option only."""
        self.deq64 = self.deq.astype(np.float64)

    def rows(self, ids) -> np.ndarray:
        """Dequantised rows (the embedding gather; exact in f32)."""
        return self.deq[np.asarray(ids)]


def linear(x: np.ndarray, w: Q8Weight, chunk: int = 16384) -> np.ndarray:
    """y = Q8_0 linear of f32 rows x [T, K] against w [N, K] -> f32 [T, N].

    The activations are quantised per 32-block (encode); the result is the
    exact sum of dequantised products, rounded once to f32.  Parity: pinned
    against exact rational arithmetic and against the block-dot form.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    qa, da = encode(x)
    a = decode(qa, da).astype(np.float64)
    out = np.empty((x.shape[0], w.N), dtype=np.float32)
    wide = getattr(w, "deq64", None)  # the same values already widened, if kept
    for n0 in range(0, w.N, chunk):
        n1 = min(w.N, n0 + chunk)
        wt = wide[n0:n1] if wide is not None else w.deq[n0:n1].astype(np.float64)
        out[:, n0:n1] = (a @ wt.T).astype(np.float32)
    return out
