"""CPU oracle for the Qwen3-0.6B-shaped decoder forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library: the only module both sides use
is `q3synth`, which generates seeded inputs and holds no arithmetic of the
method.

The implementation is plain numpy in float64, written from "Dentro de un LLM:
Inferencia en Python puro para Qwen3-0.6B en MLX" (reactapp.top, the Spanish
edition of "How Modern LLMs Actually Generate Text: A Pure Python
Walkthrough").  Each function names the step of that page it follows.

Parity pins (tests/test_oracle_pins.py) tie every function to something other
than itself; none is "parity unpinned" except the behaviour of trained weights
(the page's top-5 probability table), which needs a checkpoint that is not
available.
"""
from .qwen3 import (  # noqa: F401
    OracleModel, KVCache, rms_norm, rope_cos_sin, rope_rotate, attention_rows,
    silu, swiglu, greedy_pick, sample_top_p, to_bf16, quantize_affine, dequantize_affine,
    quantized_weights,
)
