"""Thin Python binding over the C ABI: argument marshalling only.

PyTorch supplies device memory (the workspace and I/O tensors) and the
stream; every step of the forward pass runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import KV_BF16, KV_F32, KV_Q8_0, W_BF16, W_Q8_0, check, lib


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


@dataclass
class Qwen3Config:
    """Geometry of a Qwen3 dense decoder (mirrors qwen3_config)."""

    vocab_size: int
    hidden_size: int
    intermediate_size: int
    num_layers: int
    num_attention_heads: int
    num_key_value_heads: int
    head_dim: int
    rms_norm_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_type: str = "q8_0"
    kv_type: str = "f32"

    @classmethod
    def from_shape(cls, s) -> "Qwen3Config":
        return cls(
            s.vocab_size,
            s.hidden_size,
            s.intermediate_size,
            s.num_layers,
            s.num_attention_heads,
            s.num_key_value_heads,
            s.head_dim,
            s.rms_norm_eps,
            s.rope_theta,
            s.weight_type,
            s.kv_type,
        )

    def to_c(self, capacities, max_batch_tokens: int):
        caps = (C.c_int32 * len(capacities))(*[int(c) for c in capacities])
        c = _lib.Config(
            self.vocab_size,
            self.hidden_size,
            self.intermediate_size,
            self.num_layers,
            self.num_attention_heads,
            self.num_key_value_heads,
            self.head_dim,
            float(self.rms_norm_eps),
            float(self.rope_theta),
            W_Q8_0 if self.weight_type == "q8_0" else W_BF16 if self.weight_type == "bf16" else 99,
            {"f32": KV_F32, "bf16": KV_BF16, "q8_0": KV_Q8_0}.get(self.kv_type, 99),
            len(capacities),
            caps,
            int(max_batch_tokens),
        )
        return c, caps


def workspace_bytes(cfg: Qwen3Config, capacities, max_batch_tokens: int = 0) -> int:
    c, _keep = cfg.to_c(capacities, max_batch_tokens)
    n = lib().qwen3_workspace_bytes(C.byref(c))
    if n == 0:
        raise _lib.Qwen3Error(-2, _lib.last_error())
    return n


# ---- op-level wrappers --------------------------------------------------------------


def encode_q8_0(x: torch.Tensor) -> torch.Tensor:
    """f32 device tensor [..., K] -> uint8 wire blocks [..., K/32*34]."""
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
    K = x.shape[-1]
    out = torch.empty(x.shape[:-1] + (K // 32 * 34,), dtype=torch.uint8, device=x.device)
    check(lib().qwen3_q8_0_encode(x.data_ptr(), x.numel(), out.data_ptr(), _stream()))
    return out


def encode_bf16(x: torch.Tensor) -> torch.Tensor:
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    check(lib().qwen3_bf16_encode(x.data_ptr(), x.numel(), out.data_ptr(), _stream()))
    return out


def repack_q8_0(blocks: torch.Tensor, rows: int, k: int):
    """Wire blocks -> (codes int8 [rows, k], scales f16 bits as int16 [rows, k/32])."""
    qs = torch.empty((rows, k), dtype=torch.int8, device=blocks.device)
    sc = torch.empty((rows, k // 32), dtype=torch.int16, device=blocks.device)
    check(lib().qwen3_q8_0_repack(blocks.data_ptr(), rows, k, qs.data_ptr(), sc.data_ptr(), _stream()))
    return qs, sc


def q8_0_linear(x: torch.Tensor, qs: torch.Tensor, sc: torch.Tensor) -> torch.Tensor:
    m, k = x.shape
    n = qs.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    wb = lib().qwen3_linear_work_bytes(m, k)
    work = torch.empty(max(wb, 1), dtype=torch.uint8, device=x.device)
    check(lib().qwen3_q8_0_linear(x.data_ptr(), m, k, qs.data_ptr(), sc.data_ptr(), n, y.data_ptr(), work.data_ptr(), _stream()))
    return y


def sample(
    logits: torch.Tensor,
    uniform: torch.Tensor | None,
    temperature: float = 0.0,
    top_k: int = 0,
    top_p: float = 1.0,
    min_p: float = 0.0,
    repeat_penalty: float = 1.0,
    freq_penalty: float = 0.0,
    presence_penalty: float = 0.0,
    repeat_last_n: int = 64,
    history: torch.Tensor | None = None,
    history_len: torch.Tensor | None = None,
) -> torch.Tensor:
    """One token per row of f32 logits [n, V] (penalised in place); uniform
    f32 [n] in [0, 1); history int32 [n, stride] with history_len int32 [n]."""
    from ._lib import SamplerConfig

    n, V = logits.shape
    cfg = SamplerConfig(temperature, top_k, top_p, min_p, repeat_penalty, freq_penalty, presence_penalty, repeat_last_n)
    out = torch.empty(n, dtype=torch.int32, device=logits.device)
    work = torch.empty(lib().qwen3_sample_work_bytes(n, V), dtype=torch.uint8, device=logits.device)
    check(
        lib().qwen3_sample(
            logits.data_ptr(),
            n,
            V,
            C.byref(cfg),
            _ptr(history),
            int(history.shape[1]) if history is not None else 0,
            _ptr(history_len),
            _ptr(uniform),
            out.data_ptr(),
            work.data_ptr(),
            _stream(),
        )
    )
    return out


def bf16_linear(x: torch.Tensor, w_bits: torch.Tensor) -> torch.Tensor:
    """x f32 [m, k] times bf16 weights (int16 bits [n, k]) transposed -> f32 [m, n]."""
    m, k = x.shape
    n = w_bits.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    check(lib().qwen3_bf16_linear(x.data_ptr(), m, k, w_bits.data_ptr(), n, y.data_ptr(), _stream()))
    return y


def q8_0_block_dots(x: torch.Tensor, qs: torch.Tensor):
    """(qa int8 [m, k], da f16 bits int16 [m, k/32], S int32 [m, n, k/32])."""
    m, k = x.shape
    n = qs.shape[0]
    qa = torch.empty((m, k), dtype=torch.int8, device=x.device)
    da = torch.empty((m, k // 32), dtype=torch.int16, device=x.device)
    S = torch.empty((m, n, k // 32), dtype=torch.int32, device=x.device)
    check(
        lib().qwen3_q8_0_block_dots(x.data_ptr(), m, k, qs.data_ptr(), n, qa.data_ptr(), da.data_ptr(), S.data_ptr(), _stream())
    )
    return qa, da, S


def peak_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Enqueue the library's streaming copy of src into dst (same byte size,
    a multiple of 16, no overlap) on the current stream."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    check(lib().qwen3_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream()))


def peak_read(src: torch.Tensor, partials: torch.Tensor) -> None:
    """Enqueue the library's streaming read of src (a multiple of 16 bytes)
    on the current stream; partials (int32, peak_read_partials() entries)
    receive per-wavefront wrapping sums of its 32-bit words."""
    if partials.dtype != torch.int32 or partials.numel() < lib().qwen3_peak_read_partials():
        raise ValueError("partials must be int32 with qwen3_peak_read_partials() elements")
    check(lib().qwen3_peak_read(src.data_ptr(), src.numel() * src.element_size(), partials.data_ptr(), _stream()))


def peak_read_partials() -> int:
    return int(lib().qwen3_peak_read_partials())


def peak_mfma_i8(out: torch.Tensor, workgroups: int, iters: int, fill: int = 1) -> float:
    """Enqueue the int8 MFMA loop on the current stream; out is int32 with
    256 * workgroups elements.  Returns the launch's int8 operation count."""
    if out.dtype != torch.int32 or out.numel() < 256 * workgroups:
        raise ValueError("out must be int32 with 256 * workgroups elements")
    check(lib().qwen3_peak_mfma_i8(out.data_ptr(), workgroups, iters, fill, _stream()))
    return float(lib().qwen3_peak_mfma_i8_ops(workgroups, iters))


# ---- the model ------------------------------------------------------------------------


class Qwen3Model:
    """A handle over the C ABI.

    weights: dict GGUF-name -> f32 array (numpy or torch, host or device),
    in the canonical [out, in] layout.  Projections and the embedding are
    encoded on the device by the library's own encoder (Q8_0 or bf16), handed
    to qwen3_create, and the temporaries are freed afterwards.
    """

    def __init__(self, cfg: Qwen3Config, weights, capacities, max_batch_tokens: int = 0, device: str = "cuda:0"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.capacities = [int(c) for c in capacities]
        self.handle = C.c_void_p()
        c, caps = cfg.to_c(self.capacities, max_batch_tokens)
        nbytes = lib().qwen3_workspace_bytes(C.byref(c))
        if nbytes == 0:
            raise _lib.Qwen3Error(-2, _lib.last_error())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        enc = {}

        def dev(name):
            a = weights[name]
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
            return t.to(device=self.device, dtype=torch.float32).contiguous()

        def put(name):
            t = dev(name)
            if t.ndim == 1:
                enc[name] = t
            elif cfg.weight_type == "q8_0":
                enc[name] = encode_q8_0(t)
            else:
                enc[name] = encode_bf16(t)

        for name in weights:
            put(name)
        layers = (_lib.LayerWeights * cfg.num_layers)()
        for i in range(cfg.num_layers):
            for f in _lib.LAYER_FIELDS:
                setattr(layers[i], f, _ptr(enc[f"blk.{i}.{f}"]))
        w = _lib.Weights(_ptr(enc["token_embd"]), _ptr(enc["output_norm"]), layers)
        check(lib().qwen3_create(C.byref(c), C.byref(w), self.workspace.data_ptr(), nbytes, _stream(), C.byref(self.handle)))
        del enc, caps
        torch.cuda.synchronize(self.device)
        V = cfg.vocab_size
        self._io = {}  # per-sequence decode buffers (stable addresses -> graph reuse)
        self._v = V

    def close(self):
        if self.handle:
            lib().qwen3_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def io(self, seq: int):
        if seq not in self._io:
            self._io[seq] = (
                torch.empty(self._v, dtype=torch.float32, device=self.device),
                torch.zeros(1, dtype=torch.int32, device=self.device),
            )
        return self._io[seq]

    def prefill(self, tokens, seq: int = 0, logits: bool = True):
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        lg, am = self.io(seq)
        check(
            lib().qwen3_prefill(
                self.handle,
                seq,
                toks.ctypes.data_as(C.POINTER(C.c_int32)),
                int(toks.shape[0]),
                lg.data_ptr() if logits else None,
                am.data_ptr(),
                _stream(),
            )
        )
        return lg, am

    def prefill_all_logits(self, tokens, seq: int = 0, argmax: bool = True):
        """Append `tokens` to `seq` and return (logits [n, V] f32, argmax [n]
        int32 or None) for every appended position (the verify pass)."""
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = int(toks.shape[0])
        lg = torch.empty((max(n, 1), self.cfg.vocab_size), dtype=torch.float32, device=self.device)
        am = torch.empty((max(n, 1),), dtype=torch.int32, device=self.device) if argmax else None
        check(
            lib().qwen3_prefill_all_logits(
                self.handle,
                seq,
                toks.ctypes.data_as(C.POINTER(C.c_int32)),
                n,
                lg.data_ptr(),
                am.data_ptr() if argmax else None,
                _stream(),
            )
        )
        return lg[:n], (am[:n] if argmax else None)

    def truncate(self, keep_len: int, seq: int = 0):
        """Rewind `seq` to its first keep_len positions (no-op at or above its length)."""
        check(lib().qwen3_truncate(self.handle, seq, int(keep_len), _stream()))

    def decode_step(self, seq: int = 0, token: torch.Tensor | None = None, logits: bool = True):
        """One decode step fed `token` (device int32 [1]); defaults to the
        sequence's own previous argmax buffer (a device-resident greedy loop)."""
        lg, am = self.io(seq)
        tok = am if token is None else token
        check(lib().qwen3_decode_step(self.handle, seq, tok.data_ptr(), lg.data_ptr() if logits else None, am.data_ptr(), _stream()))
        return lg, am

    def decode_greedy(self, n: int, seq: int = 0, token: torch.Tensor | None = None, logits: bool = True,
                      out: torch.Tensor | None = None):
        """n greedy decode steps in one call: step 0 is fed `token` (device
        int32 [1]; default: the sequence's previous argmax), each later step
        the token the step before chose.  Returns (tokens int32 [n], the last
        step's logits); the last token is also left in the sequence's argmax
        buffer, so decode_step can continue from it."""
        lg, am = self.io(seq)
        tok = am if token is None else token
        toks = out if out is not None else torch.empty(n, dtype=torch.int32, device=self.device)
        check(lib().qwen3_decode_greedy(self.handle, seq, n, tok.data_ptr(), toks.data_ptr(),
                                         lg.data_ptr() if logits else None, _stream()))
        am.copy_(toks[n - 1 : n])
        return toks, lg

    def decode_batch(self, seqs, tokens: torch.Tensor, logits: torch.Tensor | None, argmax: torch.Tensor):
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        check(
            lib().qwen3_decode_batch(
                self.handle,
                s.ctypes.data_as(C.POINTER(C.c_int32)),
                int(s.shape[0]),
                tokens.data_ptr(),
                _ptr(logits),
                argmax.data_ptr(),
                _stream(),
            )
        )

    def reset(self, seq: int = 0):
        check(lib().qwen3_reset(self.handle, seq, _stream()))

    def step_status(self) -> None:
        """Wait for the stream and raise Qwen3Error (QWEN3_E_DEVICE) if a
        one-launch decode step failed since the last check; the host lengths
        are then those of the device again."""
        check(lib().qwen3_step_status(self.handle, _stream()))

    def inject_step_error(self) -> None:
        """Test hook: set the one-launch step's error word from the host."""
        check(lib().qwen3_inject_step_error(self.handle, _stream()))

    def kv_export(self, seq: int, layer: int):
        """(K, V) of one layer as f32 tensors [kv_heads, len, head_dim]."""
        n = self.kv_len(seq)
        shape = (self.cfg.num_key_value_heads, n, self.cfg.head_dim)
        k = torch.empty(shape, dtype=torch.float32, device=self.device)
        v = torch.empty(shape, dtype=torch.float32, device=self.device)
        check(lib().qwen3_kv_export(self.handle, seq, layer, k.data_ptr(), v.data_ptr(), _stream()))
        return k, v

    def replay_kernel(self, kind: int, layer: int = 0, reps: int = 1, seq: int = 0):
        """Enqueue `reps` launches of one decode-step kernel (benchmark hook)."""
        check(lib().qwen3_replay_kernel(self.handle, seq, kind, layer, reps, _stream()))

    def decode_launches(self) -> int:
        """Kernel launches per decode step (1: the one-launch step)."""
        return int(lib().qwen3_decode_launches(self.handle))

    def kv_len(self, seq: int = 0) -> int:
        out = C.c_int32()
        check(lib().qwen3_kv_len(self.handle, seq, C.byref(out)))
        return out.value
