"""Model shapes and workloads.

The shape fields are the nine integers/constants the Fucina course uses to
describe Qwen3-0.6B ("A transformer from scratch", section 12.1), plus the
weight and KV-cache element types of each workload.  Qwen3 decouples
head_dim from hidden/heads (minfer "Qwen3 Support Plan", section 2.1), so
head_dim is its own field.
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelShape:
    name: str
    vocab_size: int
    hidden_size: int
    intermediate_size: int
    num_layers: int
    num_attention_heads: int
    num_key_value_heads: int
    head_dim: int
    rms_norm_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_type: str = "q8_0"  # "q8_0" or "bf16"
    kv_type: str = "f32"  # "f32", "bf16" or "q8_0"

    @property
    def q_width(self) -> int:
        return self.num_attention_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.num_key_value_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.num_attention_heads // self.num_key_value_heads

    def with_(self, **kw) -> "ModelShape":
        return replace(self, **kw)


TINY = ModelShape(
    name="tiny",
    vocab_size=4096,
    hidden_size=256,
    intermediate_size=768,
    num_layers=2,
    num_attention_heads=4,
    num_key_value_heads=2,
    head_dim=64,
)

QWEN3_0_6B = ModelShape(
    name="qwen3-0.6b",
    vocab_size=151_936,
    hidden_size=1024,
    intermediate_size=3072,
    num_layers=28,
    num_attention_heads=16,
    num_key_value_heads=8,
    head_dim=128,
)

QWEN3_0_6B_BF16 = QWEN3_0_6B.with_(name="qwen3-0.6b-bf16", weight_type="bf16", kv_type="bf16")

QWEN3_8B = ModelShape(
    name="qwen3-8b",
    vocab_size=151_936,
    hidden_size=4096,
    intermediate_size=12_288,
    num_layers=36,
    num_attention_heads=32,
    num_key_value_heads=8,
    head_dim=128,
    kv_type="bf16",
)


@dataclass(frozen=True)
class Workload:
    """One benchmark/parity workload: a model, its seeds, and the protocol.

    protocol: "prompt then N greedy decode steps" = one prefill of
    `prompt_len` tokens (its argmax is generated token 1) followed by
    `decode_steps` decode calls, each fed the previous argmax.
    """

    name: str
    shape: ModelShape
    weight_seed: int
    prompt_seed: int
    prompt_len: int
    decode_steps: int
    kv_capacity: int
    n_seqs: int = 1
    length_seed: int = 0
    min_len: int = 0
    max_len: int = 0
    decode_contexts: tuple = ()


WORKLOADS = {
    "tiny": Workload("tiny", TINY, 101, 102, prompt_len=32, decode_steps=16, kv_capacity=64),
    "0.6b-decode": Workload(
        "0.6b-decode", QWEN3_0_6B, 201, 202, prompt_len=512, decode_steps=256, kv_capacity=768
    ),
    "0.6b-prefill4096": Workload(
        "0.6b-prefill4096", QWEN3_0_6B, 201, 302, prompt_len=4096, decode_steps=32, kv_capacity=4128
    ),
    "8b-longctx": Workload(
        "8b-longctx",
        QWEN3_8B,
        401,
        402,
        prompt_len=2048,
        decode_steps=4,
        kv_capacity=32_776,
        decode_contexts=(2048, 16_384, 32_768),
    ),
    "0.6b-bf16-batch64": Workload(
        "0.6b-bf16-batch64",
        QWEN3_0_6B_BF16,
        501,
        502,
        prompt_len=0,
        decode_steps=128,
        kv_capacity=0,
        n_seqs=64,
        length_seed=503,
        min_len=1024,
        max_len=16_384,
    ),
}
