"""MI355X (gfx950) forward pass of a Qwen3 dense decoder over Q8_0 weights.

The compute lives in the HIP library libqwen3q8.so behind the C ABI of
include/qwen3_q8.h; this package is its ctypes binding.
"""

from ._lib import Qwen3Error, lib  # noqa: F401
from .model import (  # noqa: F401
    Qwen3Config,
    Qwen3Model,
    bf16_linear,
    encode_bf16,
    encode_q8_0,
    peak_copy,
    peak_mfma_i8,
    peak_read,
    peak_read_partials,
    q8_0_block_dots,
    q8_0_linear,
    repack_q8_0,
    sample,
    workspace_bytes,
)
