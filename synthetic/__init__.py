"""Seeded synthetic workloads for the Qwen3 dense decoder over Q8_0 weights.

This package only draws random numbers and describes shapes.  It holds none
of the method's arithmetic: no quantisation, no normalisation, no attention.
Both the GPU library's tests/bench and the CPU oracle take their inputs from
here, so the two sides start from the same bytes and share nothing else.
"""

from .configs import (  # noqa: F401
    ModelShape,
    Workload,
    TINY,
    QWEN3_0_6B,
    QWEN3_0_6B_BF16,
    QWEN3_8B,
    WORKLOADS,
)
from .gen import (  # noqa: F401
    tensor_specs,
    layer_tensor_names,
    gen_tensor,
    gen_weights,
    iter_weights,
    gen_prompt,
    gen_lengths,
    gen_prompts,
    gen_normal_rows,
)
