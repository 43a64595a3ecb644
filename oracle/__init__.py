"""Plain CPU oracle for the batch-one token-to-logits decode path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  The
HIP library never calls it, and the two share no code: the only common
module is ``synth`` (seeded input generation, no method arithmetic).

What it computes follows the pages:

* the forward pass of a Qwen3-0.6B-shaped decoder -- token embedding, per
  layer RMSNorm, Q/K/V projections, per-head Q/K RMSNorm, RoPE, grouped-
  query attention with the KV-cache update, output projection and residual,
  RMSNorm, gate/up projections, SwiGLU, down projection and residual, then
  final RMSNorm and the tied vocabulary projection (Megakernels, "What runs
  in the DSL");
* the eight ordered stages per layer and their stored intermediates, and
  greedy selection by GPU argmax with ties going to the lowest token id
  (Megakernels, "GPU-wide end-to-end generation");
* chunked prefill, where every prompt row attends to its whole causal
  prefix (Megakernels, "Chunked prefill for long prompts"), which the
  oracle evaluates as one causal row block per layer -- the same per-row
  arithmetic as tokenwise prefill;
* the matrix-vector products of the weight-streaming GEMV family, including
  4-bit grouped weights (Our Kernel Benchmark Was Measuring the System
  Cache, "Summary" and "Why it mattered").

Precision: every value the pages store between stages (weights, KV cache,
logits, stage outputs) is rounded to the model's storage dtype (FP32 or
FP16); every reduction -- dot products, sums of squares, softmax sums -- is
carried out in float64 and rounded once, so the oracle's own error is far
below the rtol=atol=1e-3 FP32 comparison the pages use (Benchmark
methodology, "Long-document chunked prefill").

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, invariants, textbook special cases, hand-written golden words
(``tests/golden/``) and brute force on tiny inputs.  Greedy tokens of the
random-weight models have no printed example on the pages: beyond the
oracle itself their parity is unpinned (the whole-model invariants pin the
composition; see the model tests).
"""
from .prims import (argmax_lowest, gqa_attention, rms_norm, rope_apply,
                    rope_angles, silu, store)
from .gemv import dequant_q4g64, gemv, gemv_q4g64, unpack_int4
from .model import OracleModel

__all__ = [
    "argmax_lowest", "gqa_attention", "rms_norm", "rope_apply", "rope_angles", "silu", "store",
    "dequant_q4g64", "gemv", "gemv_q4g64", "unpack_int4", "OracleModel",
]
