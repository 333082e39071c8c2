"""CPU oracle for the Qwen3 dense decoder over Q8_0 weights.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy implementation of what the forward pass computes.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it;
the GPU library never does, and the two share no code.  The only common
dependency is the seeded input generator (`synthetic`), which holds none of
the method's arithmetic.

Floating point: the model state is f32 (the method's storage type); every
reduction (dot products, sums of squares, softmax) runs in f64 and is rounded
to f32 once per operation.  f16 and bf16 rounding happen exactly where the
method stores f16 / bf16 values.

Sources (web pages, cited by title and section):
  * Fucina course, "A transformer from scratch" (Chapter 12): forward pass,
    RMSNorm, RoPE, GQA, SwiGLU, KV cache, greedy loop.
  * Fucina course, "Model files and quantization" (Chapter 11): the Q8_0
    block format, its encoder and the integer block dot.
  * Fucina reference, "The LLM stack (fucina_llm)" (section 13): KV-cache
    contract, sampler contract.
  * minfer, "Qwen3 Support Plan": tensor inventory, decoupled head_dim,
    per-head Q/K RMSNorm.

Parity status of each function is stated in its docstring; every function
here is pinned by a CPU test (tests/test_oracle_*.py) except where a
docstring says "parity unpinned".
"""

from . import q8_0, ops, model  # noqa: F401
