"""Seeded generators (NumPy PCG64) for weights, prompts and lengths.

Every tensor has its own stream, derived from (workload seed, canonical
index), so any tensor can be regenerated alone and tensors can be drawn in
parallel threads (NumPy releases the GIL inside the fill).

Distributions: projection and embedding weights are 0.02 * N(0, 1) in f32;
every norm weight (attn_norm, ffn_norm, output_norm, q_norm, k_norm) is
1 + 0.1 * N(0, 1) in f32.  Prompts are uniform ids in [0, vocab).
"""

from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

from .configs import ModelShape

LAYER_TENSORS = (
    "attn_norm",
    "attn_q",
    "attn_k",
    "attn_v",
    "attn_output",
    "attn_q_norm",
    "attn_k_norm",
    "ffn_norm",
    "ffn_gate",
    "ffn_up",
    "ffn_down",
)

NORM_TENSORS = frozenset({"attn_norm", "attn_q_norm", "attn_k_norm", "ffn_norm", "output_norm"})


def layer_tensor_names(layer: int) -> list[str]:
    return [f"blk.{layer}.{t}" for t in LAYER_TENSORS]


def _layer_shape(shape: ModelShape, t: str) -> tuple[int, ...]:
    H, F, hd = shape.hidden_size, shape.intermediate_size, shape.head_dim
    return {
        "attn_norm": (H,),
        "attn_q": (shape.q_width, H),
        "attn_k": (shape.kv_width, H),
        "attn_v": (shape.kv_width, H),
        "attn_output": (H, shape.q_width),
        "attn_q_norm": (hd,),
        "attn_k_norm": (hd,),
        "ffn_norm": (H,),
        "ffn_gate": (F, H),
        "ffn_up": (F, H),
        "ffn_down": (H, F),
    }[t]


def tensor_specs(shape: ModelShape) -> list[tuple[str, tuple[int, ...]]]:
    """Canonical tensor order: token_embd, per layer LAYER_TENSORS, output_norm.

    Shapes are logical [out, in] (row-major, `in` contiguous).  There is no
    output.weight: the lm_head is tied to token_embd.
    """
    specs = [("token_embd", (shape.vocab_size, shape.hidden_size))]
    for layer in range(shape.num_layers):
        for t in LAYER_TENSORS:
            specs.append((f"blk.{layer}.{t}", _layer_shape(shape, t)))
    specs.append(("output_norm", (shape.hidden_size,)))
    return specs


def _kind(name: str) -> str:
    return "norm" if name.split(".")[-1] in NORM_TENSORS else "proj"


def _stream(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(index,))))


def gen_tensor(shape: ModelShape, seed: int, name: str) -> np.ndarray:
    """Draw one named tensor (f32) of the canonical list."""
    specs = tensor_specs(shape)
    for index, (n, shp) in enumerate(specs):
        if n == name:
            return _draw(seed, index, n, shp)
    raise KeyError(name)


def _draw(seed: int, index: int, name: str, shp: tuple[int, ...]) -> np.ndarray:
    out = np.empty(shp, dtype=np.float32)
    _stream(seed, index).standard_normal(out=out, dtype=np.float32)
    if _kind(name) == "norm":
        out *= np.float32(0.1)
        out += np.float32(1.0)
    else:
        out *= np.float32(0.02)
    return out


def gen_weights(shape: ModelShape, seed: int, threads: int | None = None) -> dict[str, np.ndarray]:
    """All tensors of a model, drawn in parallel; dict name -> f32 array."""
    specs = tensor_specs(shape)
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {n: ex.submit(_draw, seed, i, n, s) for i, (n, s) in enumerate(specs)}
        return {n: f.result() for n, f in futs.items()}


def iter_weights(shape: ModelShape, seed: int):
    """Yield (name, f32 array) one tensor at a time (bounded host memory)."""
    for index, (n, s) in enumerate(tensor_specs(shape)):
        yield n, _draw(seed, index, n, s)


def gen_prompt(vocab_size: int, n: int, seed: int) -> np.ndarray:
    """n uniform token ids in [0, vocab_size), int32."""
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab_size, size=n, dtype=np.int32)


def gen_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """n lengths uniform in {lo, ..., hi} (inclusive), int32."""
    return np.random.Generator(np.random.PCG64(seed)).integers(lo, hi + 1, size=n, dtype=np.int32)


def gen_normal_rows(shp: tuple[int, ...], seed: int, scale: float = 1.0) -> np.ndarray:
    """Generic f32 scale * N(0, 1) array for op-level tests."""
    out = np.empty(shp, dtype=np.float32)
    np.random.Generator(np.random.PCG64(seed)).standard_normal(out=out, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def gen_prompts(vocab: int, lengths, seed: int) -> list[np.ndarray]:
    """One uniform-random prompt per length, each from its own child stream
    of SeedSequence(seed) (the ragged batch of independent sequences)."""
    kids = np.random.SeedSequence(seed).spawn(len(lengths))
    return [
        np.random.Generator(np.random.PCG64(k)).integers(0, vocab, size=int(n), dtype=np.int32)
        for k, n in zip(kids, lengths)
    ]
