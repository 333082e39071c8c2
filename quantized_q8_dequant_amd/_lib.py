"""ctypes declarations of the C ABI in include/qwen3_q8.h.

Loads the in-tree libqwen3q8.so (built by quantized_q8_dequant_amd.build).
There is no fallback: if the library is missing the import of this module's
`lib()` raises, so nothing can silently run another implementation.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwen3q8.so")

QWEN3_OK = 0
ERRORS = {
    -1: "QWEN3_E_INVALID_ARGUMENT",
    -2: "QWEN3_E_INVALID_CONFIG",
    -3: "QWEN3_E_INVALID_WEIGHT_SHAPE",
    -4: "QWEN3_E_UNSUPPORTED_WEIGHT_TYPE",
    -5: "QWEN3_E_WORKSPACE_TOO_SMALL",
    -6: "QWEN3_E_INVALID_SEQUENCE_LENGTH",
    -7: "QWEN3_E_KV_CACHE_OVERFLOW",
    -8: "QWEN3_E_TOKEN_OUT_OF_RANGE",
    -9: "QWEN3_E_DEVICE",
}
W_Q8_0, W_BF16 = 0, 1
KV_F32, KV_BF16, KV_Q8_0 = 0, 1, 2

EXPORTS = (
    "qwen3_workspace_bytes",
    "qwen3_create",
    "qwen3_destroy",
    "qwen3_prefill",
    "qwen3_prefill_all_logits",
    "qwen3_truncate",
    "qwen3_sample_work_bytes",
    "qwen3_sample",
    "qwen3_decode_step",
    "qwen3_decode_greedy",
    "qwen3_decode_batch",
    "qwen3_reset",
    "qwen3_step_status",
    "qwen3_inject_step_error",
    "qwen3_kv_len",
    "qwen3_last_error",
    "qwen3_q8_0_encode",
    "qwen3_bf16_encode",
    "qwen3_q8_0_repack",
    "qwen3_linear_work_bytes",
    "qwen3_q8_0_linear",
    "qwen3_q8_0_linear_noalloc",
    "qwen3_q8_0_block_dots",
    "qwen3_kv_export",
    "qwen3_replay_kernel",
    "qwen3_bf16_linear",
    "qwen3_decode_launches",
    "qwen3_peak_copy",
    "qwen3_peak_read",
    "qwen3_peak_read_partials",
    "qwen3_peak_mfma_i8",
    "qwen3_peak_mfma_i8_ops",
)


class Qwen3Error(RuntimeError):
    def __init__(self, code: int, message: str):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        super().__init__(f"{self.name}: {message}")


class Config(C.Structure):
    _fields_ = [
        ("vocab_size", C.c_int32),
        ("hidden_size", C.c_int32),
        ("intermediate_size", C.c_int32),
        ("num_layers", C.c_int32),
        ("num_attention_heads", C.c_int32),
        ("num_key_value_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("rms_norm_eps", C.c_float),
        ("rope_theta", C.c_float),
        ("weight_type", C.c_int32),
        ("kv_type", C.c_int32),
        ("max_seqs", C.c_int32),
        ("h_seq_capacity", C.POINTER(C.c_int32)),
        ("max_batch_tokens", C.c_int32),
    ]


LAYER_FIELDS = (
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


class SamplerConfig(C.Structure):
    """qwen3_sampler_config."""

    _fields_ = [
        ("temperature", C.c_float),
        ("top_k", C.c_int32),
        ("top_p", C.c_float),
        ("min_p", C.c_float),
        ("repeat_penalty", C.c_float),
        ("freq_penalty", C.c_float),
        ("presence_penalty", C.c_float),
        ("repeat_last_n", C.c_int32),
    ]


class LayerWeights(C.Structure):
    _fields_ = [(f, C.c_void_p) for f in LAYER_FIELDS]


class Weights(C.Structure):
    _fields_ = [
        ("token_embd", C.c_void_p),
        ("output_norm", C.c_void_p),
        ("layers", C.POINTER(LayerWeights)),
    ]


_LIB = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_q8_dequant_amd.build` "
            "(there is no fallback implementation)"
        )
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    p_i32 = C.POINTER(C.c_int32)
    sig = {
        "qwen3_workspace_bytes": (sz, [C.POINTER(Config)]),
        "qwen3_create": (C.c_int, [C.POINTER(Config), C.POINTER(Weights), vp, sz, vp, C.POINTER(vp)]),
        "qwen3_destroy": (None, [vp]),
        "qwen3_prefill": (C.c_int, [vp, i32, p_i32, i32, vp, vp, vp]),
        "qwen3_prefill_all_logits": (C.c_int, [vp, i32, p_i32, i32, vp, vp, vp]),
        "qwen3_truncate": (C.c_int, [vp, i32, i32, vp]),
        "qwen3_sample_work_bytes": (C.c_size_t, [i32, i32]),
        "qwen3_sample": (C.c_int, [vp, i32, i32, C.POINTER(SamplerConfig), vp, i32, vp, vp, vp, vp, vp]),
        "qwen3_decode_step": (C.c_int, [vp, i32, vp, vp, vp, vp]),
        "qwen3_decode_greedy": (C.c_int, [vp, i32, i32, vp, vp, vp, vp]),
        "qwen3_decode_batch": (C.c_int, [vp, p_i32, i32, vp, vp, vp, vp]),
        "qwen3_reset": (C.c_int, [vp, i32, vp]),
        "qwen3_step_status": (C.c_int, [vp, vp]),
        "qwen3_inject_step_error": (C.c_int, [vp, vp]),
        "qwen3_kv_len": (C.c_int, [vp, i32, p_i32]),
        "qwen3_last_error": (C.c_char_p, []),
        "qwen3_q8_0_encode": (C.c_int, [vp, i64, vp, vp]),
        "qwen3_bf16_encode": (C.c_int, [vp, i64, vp, vp]),
        "qwen3_q8_0_repack": (C.c_int, [vp, i64, i64, vp, vp, vp]),
        "qwen3_linear_work_bytes": (sz, [i64, i64]),
        "qwen3_q8_0_linear": (C.c_int, [vp, i64, i64, vp, vp, i64, vp, vp, vp]),
        "qwen3_q8_0_linear_noalloc": (C.c_int, [vp, i64, i64, vp, vp, i64, vp, vp]),
        "qwen3_q8_0_block_dots": (C.c_int, [vp, i64, i64, vp, i64, vp, vp, vp, vp]),
        "qwen3_kv_export": (C.c_int, [vp, i32, i32, vp, vp, vp]),
        "qwen3_replay_kernel": (C.c_int, [vp, i32, i32, i32, i32, vp]),
        "qwen3_bf16_linear": (C.c_int, [vp, i64, i64, vp, i64, vp, vp]),
        "qwen3_decode_launches": (i32, [vp]),
        "qwen3_peak_copy": (C.c_int, [vp, vp, sz, vp]),
        "qwen3_peak_read": (C.c_int, [vp, sz, vp, vp]),
        "qwen3_peak_read_partials": (i32, []),
        "qwen3_peak_mfma_i8": (C.c_int, [vp, i32, i32, i32, vp]),
        "qwen3_peak_mfma_i8_ops": (C.c_double, [i32, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = L
    return L


def last_error() -> str:
    return lib().qwen3_last_error().decode()


def check(rc: int) -> None:
    if rc != QWEN3_OK:
        raise Qwen3Error(rc, last_error())
