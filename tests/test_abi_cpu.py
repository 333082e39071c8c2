"""The C-ABI library on the CPU: it loads, exports every declared symbol,
sizes workspaces, and rejects bad arguments on the host before any launch.
No compute call is made (there is no GPU here)."""

import ctypes as C
import os
import re

import pytest

from conftest import ROOT
from quantized_q8_dequant_amd import _lib
from quantized_q8_dequant_amd.model import Qwen3Config, workspace_bytes
from synthetic import QWEN3_0_6B, QWEN3_8B, TINY

HEADER = os.path.join(ROOT, "include", "qwen3_q8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwen3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = _lib.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def _cfg(shape, **kw):
    c = Qwen3Config.from_shape(shape)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes_cover_weights_and_cache():
    s = QWEN3_0_6B
    n = workspace_bytes(_cfg(s), [768])
    per_layer = (s.q_width + 2 * s.kv_width) * s.hidden_size + s.hidden_size * s.q_width
    per_layer += 3 * s.intermediate_size * s.hidden_size
    q8 = (per_layer * s.num_layers + s.vocab_size * s.hidden_size) * 34 // 32
    kv = 768 * s.num_layers * 2 * s.kv_width * 4
    assert n >= q8 + kv
    assert n < (q8 + kv) * 1.5
    # a bf16 cache halves the KV part
    n2 = workspace_bytes(_cfg(s, kv_type="bf16"), [768])
    assert n - n2 >= kv // 2 - 1024 * 1024
    # bf16 weights take two bytes per weight
    nb = workspace_bytes(_cfg(s, weight_type="bf16", kv_type="bf16"), [768])
    bf = (per_layer * s.num_layers + s.vocab_size * s.hidden_size) * 2
    assert nb >= bf + kv // 2
    assert nb < (bf + kv // 2) * 1.5
    # 8B at 32k context fits easily in 288 GB
    assert workspace_bytes(_cfg(QWEN3_8B), [32776]) < 20e9


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(num_key_value_heads=3), -2),
        (dict(head_dim=65), -2),
        (dict(head_dim=96), -2),
        (dict(hidden_size=0), -2),
        (dict(intermediate_size=700), -2),
        (dict(rms_norm_eps=0.0), -2),
        (dict(rope_theta=1.0), -2),
        (dict(weight_type="q4_k"), -4),
        (dict(kv_type="f16"), -4),
    ],
)
def test_invalid_configs_rejected(kw, code):
    c, keep = _cfg(TINY, **kw).to_c([64], 0)
    assert _lib.lib().qwen3_workspace_bytes(C.byref(c)) == 0
    assert _lib.last_error()
    h = C.c_void_p()
    w = _lib.Weights(None, None, None)
    rc = _lib.lib().qwen3_create(C.byref(c), C.byref(w), None, 0, None, C.byref(h))
    assert rc == code, _lib.last_error()
    assert not h.value


def test_bad_capacity_rejected():
    c, keep = _cfg(TINY).to_c([64, 0], 0)
    assert _lib.lib().qwen3_workspace_bytes(C.byref(c)) == 0


def _fake_weights(L):
    layers = (_lib.LayerWeights * L)()
    for i in range(L):
        for f in _lib.LAYER_FIELDS:
            setattr(layers[i], f, 0x1000)
    return _lib.Weights(0x1000, 0x1000, layers), layers


def test_create_argument_errors_before_any_launch():
    lib = _lib.lib()
    c, keep = _cfg(TINY).to_c([64], 0)
    w, layers = _fake_weights(TINY.num_layers)
    h = C.c_void_p()
    need = lib.qwen3_workspace_bytes(C.byref(c))
    # null workspace
    assert lib.qwen3_create(C.byref(c), C.byref(w), None, need, None, C.byref(h)) == -1
    # misaligned workspace
    assert lib.qwen3_create(C.byref(c), C.byref(w), 0x100010, need, None, C.byref(h)) == -1
    # too small
    assert lib.qwen3_create(C.byref(c), C.byref(w), 0x100000, need - 1, None, C.byref(h)) == -5
    assert "needs" in _lib.last_error()
    # a null layer pointer
    layers[1].ffn_up = None
    assert lib.qwen3_create(C.byref(c), C.byref(w), 0x100000, need, None, C.byref(h)) == -1
    assert "layer 1" in _lib.last_error()
    assert not h.value


def test_null_handle_and_op_argument_errors():
    lib = _lib.lib()
    toks = (C.c_int32 * 2)(1, 2)
    assert lib.qwen3_prefill(None, 0, toks, 2, None, None, None) == -1
    assert lib.qwen3_decode_step(None, 0, None, None, None, None) == -1
    assert lib.qwen3_decode_greedy(None, 0, 1, None, None, None, None) == -1
    assert lib.qwen3_reset(None, 0, None) == -1
    assert lib.qwen3_step_status(None, None) == -1
    assert lib.qwen3_inject_step_error(None, None) == -1
    out = C.c_int32()
    assert lib.qwen3_kv_len(None, 0, C.byref(out)) == -1
    assert lib.qwen3_q8_0_encode(0x1000, 33, 0x2000, None) == -1
    assert lib.qwen3_q8_0_repack(0x1000, 4, 48, 0x2000, 0x3000, None) == -1
    assert lib.qwen3_q8_0_linear(0x1000, 1, 100, 0x2000, 0x3000, 8, 0x4000, None, None) == -1
    assert lib.qwen3_q8_0_linear(0x1000, 2, 1024, 0x2000, 0x3000, 8, 0x4000, None, None) == -1
    assert lib.qwen3_q8_0_block_dots(0x1000, 1, 48, 0x2000, 4, 0x3000, 0x4000, 0x5000, None) == -1
    assert lib.qwen3_linear_work_bytes(4, 1024) >= 4 * 1024 + 4 * 32 * 4
    assert lib.qwen3_bf16_linear(0x1000, 2, 48, 0x2000, 8, 0x3000, None) == -1  # k % 32
    assert lib.qwen3_bf16_linear(0x1000, 0, 64, 0x2000, 8, 0x3000, None) == -1
    assert lib.qwen3_bf16_linear(None, 2, 64, 0x2000, 8, 0x3000, None) == -1
    assert lib.qwen3_decode_launches(None) == -1
    # the allocation-free linear refuses an over-limit m x k on the host,
    # before resolving any device address
    assert lib.qwen3_q8_0_linear_noalloc(0x1000, 8192, 2048, 0x2000, 0x3000, 64, 0x4000, None) == -1
    assert "scratch" in _lib.last_error()
    assert lib.qwen3_q8_0_linear_noalloc(0x1000, 1 << 40, 2048, 0x2000, 0x3000, 64, 0x4000, None) == -1
    # encoding zero values enqueues nothing
    assert lib.qwen3_q8_0_encode(None, 0, None, None) == 0


def test_peak_probes_validate_on_the_host():
    L = _lib.lib()
    assert L.qwen3_peak_copy(C.c_void_p(16), C.c_void_p(4096), 24, None) == -1  # not a multiple of 16
    assert L.qwen3_peak_copy(None, None, 32, None) == -1
    assert L.qwen3_peak_copy(None, None, 0, None) == 0  # nothing to copy, no launch
    assert L.qwen3_peak_read(C.c_void_p(16), 40, C.c_void_p(4096), None) == -1
    assert L.qwen3_peak_read(None, 32, None, None) == -1
    assert L.qwen3_peak_read_partials() == 8192 * 4
    assert L.qwen3_peak_mfma_i8(None, 1, 1, 1, None) == -1
    assert L.qwen3_peak_mfma_i8(C.c_void_p(4096), 0, 1, 1, None) == -1
    assert L.qwen3_peak_mfma_i8(C.c_void_p(4096), 1, 0, 1, None) == -1
    # four wavefronts x four 32x32x32 MFMAs (65,536 int8 ops each) per round
    assert L.qwen3_peak_mfma_i8_ops(2048, 4000) == 2048 * 4 * 4 * 4000 * 65536.0
    assert L.qwen3_peak_mfma_i8_ops(0, 5) == 0.0


def test_sample_arguments_validated_on_the_host():
    """qwen3_sample rejects bad arguments before any launch (the pointers
    here are never dereferenced)."""
    L = _lib.lib()
    good = dict(temperature=0.7, top_k=20, top_p=0.9, min_p=0.0, repeat_penalty=1.1, freq_penalty=0.0,
                presence_penalty=0.0, repeat_last_n=64)
    dev, work = C.c_void_p(1 << 20), C.c_void_p(1 << 24)  # aligned stand-ins

    def call(cfg=None, n=2, vocab=1000, logits=dev, hist=None, stride=0, hlen=None, uni=dev, toks=dev, wk=work):
        c = _lib.SamplerConfig(**{**good, **(cfg or {})})
        return L.qwen3_sample(logits, n, vocab, C.byref(c), hist, stride, hlen, uni, toks, wk, None)

    assert call(logits=None) == -1
    assert call(toks=None) == -1
    assert call(wk=None) == -1
    assert call(wk=C.c_void_p((1 << 24) + 8)) == -1  # scratch not 256-byte aligned
    assert call(n=0) == -1 and call(vocab=0) == -1
    assert call(cfg=dict(top_k=-1)) == -1
    assert call(cfg=dict(top_p=0.0)) == -1 and call(cfg=dict(top_p=1.5)) == -1
    assert call(cfg=dict(min_p=-0.1)) == -1 and call(cfg=dict(min_p=1.1)) == -1
    assert call(cfg=dict(repeat_penalty=0.0)) == -1
    assert call(cfg=dict(freq_penalty=float("inf"))) == -1
    assert call(cfg=dict(temperature=float("nan"))) == -1
    assert call(cfg=dict(repeat_last_n=-1)) == -1 and call(cfg=dict(repeat_last_n=4097)) == -1
    assert call(hist=dev, stride=64, hlen=None) == -1  # a history needs its lengths
    assert call(hist=dev, stride=0, hlen=dev) == -1
    assert call(uni=None) == -1  # sampling needs the uniforms
    assert _lib.last_error()


def test_sample_work_bytes():
    """The scratch holds each (row, 4096-logit slice) list and its stats,
    and per row one more vocabulary of 8-byte slots (a wide exact-nucleus
    window is sorted between the row's list slots and these)."""
    L = _lib.lib()
    for n, V in ((1, 151936), (64, 151936), (3, 4097), (1, 1)):
        S = (V + 4095) // 4096
        assert L.qwen3_sample_work_bytes(n, V) >= n * S * 4096 * 8 + n * V * 8
        assert L.qwen3_sample_work_bytes(n, V) <= n * S * (4096 * 8 + 64) + n * V * 8 + 4096
