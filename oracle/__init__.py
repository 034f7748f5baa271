"""CPU oracle for the W4A16 paged greedy-decode step — TEST INFRASTRUCTURE ONLY.

Plain, slow, NumPy float64 code that states what the decode step computes, so
that the HIP path can be checked against it. Only the tests, the smoke check
and the bench's CPU-baseline leg may import it; the library never does, and
the oracle imports nothing from the library (they share no code).

Sources (web pages on hand-building a decode-only INT4 runtime for a
Qwen2.5-Coder-7B-class model):

* "How to build your own LLM runtime from scratch" (spokes-wiki summary of a
  Towards Data Science build-log), section "What it actually builds":
  symmetric group-wise INT4 weights with group size 128, a paged KV cache of
  16 tokens per 4 KiB page, fused GEMVs for Q/K/V/O and gate/up/down,
  greedy-only sampling.
* "How To Build Your Own LLM Runtime From Scratch" (daily.dev), Summary and
  FAQ: 28 layers, FP16 activations with INT4 weights, partial KV tail pages.
* "How To Build Your Own LLM Runtime From Scratch" (daily.dev), FAQ on
  INT8-activation dp4a against FP16-activation INT4 unpack: the INT8
  activation variant (``a8.py``).
* "Inference Zero To Hero" (preface), the stable softmax shown under "How
  each chapter works": subtract the max, exponentiate, divide by the sum.
* "Build Crude Implementations for Learning", section "nanoGPT level":
  scores q.k^T / sqrt(d), causal mask, softmax, weighted sum of v.

Where the pages are silent the plainest reading is taken (Qwen2 conventions:
rotate-half RoPE, SwiGLU, QKV bias, consecutive GQA grouping); each such
reading is marked READING in the function that takes it.

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` (closed forms, invariants, brute force); none is
"parity unpinned".
"""
from .quant import quantize_w4, dequantize_w4, GROUP
from .a8 import quantize_a8, dequantize_a8, gemv_w4a8
from .model import (
    softmax, rmsnorm, rope, attend, attend_splitk, swiglu, argmax_lowest,
    ContiguousKV, PagedKVEmu, OracleModel, layer_causal, causal_forward,
    decode_step, generate, gemv_w4a16, paged_attention,
)

__all__ = [
    "quantize_w4", "dequantize_w4", "GROUP", "quantize_a8", "dequantize_a8", "gemv_w4a8", "softmax", "rmsnorm", "rope",
    "attend", "attend_splitk", "swiglu", "argmax_lowest", "ContiguousKV",
    "PagedKVEmu", "OracleModel", "layer_causal", "causal_forward",
    "decode_step", "generate", "gemv_w4a16", "paged_attention",
]
