"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module draws numbers and lays out data; it holds none of the decode
method's arithmetic (no norms, projections, attention or argmax).  Both the
CPU oracle and the HIP path receive exactly the arrays produced here.

The pages measure a real Qwen3-0.6B checkpoint on document prompts
(Benchmark methodology, "Long-document chunked prefill"); neither is
available, so random-init weights of the same architecture and
uniform-random token ids of the same lengths stand in for them.

Recipe (fixed, so every consumer sees identical inputs):

* weights: ``numpy.random.Generator(PCG64(seed))``; every matrix is
  ``standard_normal(shape, float32) * float32(0.02)``, drawn in the order
  E, then per layer Wq, Wk, Wv, Wo, Wg, Wu, Wd.  Matrices are row-major
  ``[out, in]``.  All RMSNorm gains are 1.0.  With this order a 2-layer
  model is exactly the first two layers of the 28-layer model.
* prompts: ``integers(0, vocab, n)`` from their own seed.
* GEMV sweep: ``W ~ N(0, 0.02)``, ``x ~ N(0, 1)``.
* int4 GEMV: ``q`` uniform integers in [-8, 7], scales ``|N(0, 0.01)|``
  rounded to FP16, activations ``N(0, 1)`` rounded to FP16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

__all__ = [
    "ModelShape", "QWEN3_0_6B", "MINI", "model_weights", "model_weights_bf16", "bf16_representable", "prompt_ids",
    "gemv_inputs", "q4g64_inputs", "pack_int4_rows", "model_weights_q4", "GEMV_SHAPES", "Q4_SHAPES",
    "PROMPT_SEEDS", "WEIGHT_SEED",
]


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Decoder geometry (Megakernels, "What runs in the DSL")."""

    n_layers: int
    hidden: int
    intermediate: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_layers(self, n: int) -> "ModelShape":
        return dataclasses.replace(self, n_layers=n)

    def weight_bytes_per_token(self, elem_bytes: int = 4) -> int:
        """Bytes of projection weights one decode token streams (layers + tied head)."""
        h, i, q, kv = self.hidden, self.intermediate, self.q_width, self.kv_width
        per_layer = (q + 2 * kv) * h + h * q + 2 * i * h + h * i
        return elem_bytes * (self.n_layers * per_layer + self.vocab * h)


# Qwen3-0.6B geometry; 28 layers.  The 2-layer model is .with_layers(2).
QWEN3_0_6B = ModelShape(n_layers=28, hidden=1024, intermediate=3072, n_q_heads=16,
                        n_kv_heads=8, head_dim=128, vocab=151936)

# A small geometry with ragged sizes (vocab not a multiple of any tile), used
# by fast CPU and GPU tests.  head_dim stays 128, as in the real model.
MINI = ModelShape(n_layers=2, hidden=512, intermediate=1024, n_q_heads=4,
                  n_kv_heads=2, head_dim=128, vocab=1000)

WEIGHT_SEED = 0
# prompt seeds: tiny-model prompt, short-generation prompts, chunk-selection
# prompt, held-out long prompt
PROMPT_SEEDS = {"tiny": 1, "short": 2, "tuning": 3, "heldout": 4}

_STD = np.float32(0.02)


def _normal(rng: np.random.Generator, shape, dtype) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= _STD
    if dtype != np.float32:
        a = a.astype(dtype)
    return a


def model_weights(shape: ModelShape, seed: int = WEIGHT_SEED, dtype=np.float32) -> Dict[str, object]:
    """Random-init weights of ``shape``.

    Returns ``{"embed": E[V,H], "final_norm": g[H], "layers": [dict, ...]}``
    where each layer dict holds ``wq[Q,H] wk[KV,H] wv[KV,H] wo[H,Q]
    wg[I,H] wu[I,H] wd[H,I]`` and gains ``in_norm[H] post_norm[H]
    q_norm[D] k_norm[D]``.  ``dtype`` float16 rounds each FP32 draw to the
    nearest FP16 (round-to-nearest-even, subnormals kept).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    h, i, q, kv, d = shape.hidden, shape.intermediate, shape.q_width, shape.kv_width, shape.head_dim
    out: Dict[str, object] = {"embed": _normal(rng, (shape.vocab, h), dtype),
                              "final_norm": np.ones(h, dtype)}
    layers: List[Dict[str, np.ndarray]] = []
    for _ in range(shape.n_layers):
        lw = {}
        for name, shp in (("wq", (q, h)), ("wk", (kv, h)), ("wv", (kv, h)), ("wo", (h, q)),
                          ("wg", (i, h)), ("wu", (i, h)), ("wd", (h, i))):
            lw[name] = _normal(rng, shp, dtype)
        lw["in_norm"] = np.ones(h, dtype)
        lw["post_norm"] = np.ones(h, dtype)
        lw["q_norm"] = np.ones(d, dtype)
        lw["k_norm"] = np.ones(d, dtype)
        layers.append(lw)
    out["layers"] = layers
    return out


def bf16_representable(a: np.ndarray) -> np.ndarray:
    """FP32 copy of ``a`` rounded to the nearest BF16 value (round-to-nearest-even on the
    high 16 bits): every result has zero low 16 bits.  Finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def model_weights_bf16(shape: ModelShape, seed: int = WEIGHT_SEED) -> Dict[str, object]:
    """``model_weights`` with every matrix rounded to BF16-representable FP32 values (the
    weights of a checkpoint converted from BF16); gains stay 1."""
    w = model_weights(shape, seed)
    w["embed"] = bf16_representable(w["embed"])
    for lw in w["layers"]:
        for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            lw[name] = bf16_representable(lw[name])
    return w


def model_weights_q4(shape: ModelShape, seed: int = WEIGHT_SEED, scale_std: float = 0.01) -> Dict[str, object]:
    """Int4 group-64 weights of ``shape``, drawn as in the int4 GEMV workload: per
    matrix ``q`` uniform in [-8, 7] and FP16 scales ``|N(0, scale_std)|`` per group
    of 64 along K.  Returns the layout of ``model_weights`` with ``format`` =
    "q4g64" and each matrix a pair ``(words uint32[rows, k/8], scales f16[rows, k/64])``
    (``pack_int4_rows`` word format); norm gains are FP16 ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    h, i, q, kv, d = shape.hidden, shape.intermediate, shape.q_width, shape.kv_width, shape.head_dim

    def mat(rows, k):
        qv = rng.integers(-8, 8, (rows, k)).astype(np.int8)
        sc = np.abs(rng.normal(0.0, scale_std, (rows, k // 64))).astype(np.float16)
        return pack_int4_rows(qv), sc

    one = np.float16
    out: Dict[str, object] = {"format": "q4g64", "embed": mat(shape.vocab, h), "final_norm": np.ones(h, one)}
    layers: List[Dict[str, object]] = []
    for _ in range(shape.n_layers):
        lw: Dict[str, object] = {}
        for name, (rows, k) in (("wq", (q, h)), ("wk", (kv, h)), ("wv", (kv, h)), ("wo", (h, q)),
                                ("wg", (i, h)), ("wu", (i, h)), ("wd", (h, i))):
            lw[name] = mat(rows, k)
        lw["in_norm"] = np.ones(h, one)
        lw["post_norm"] = np.ones(h, one)
        lw["q_norm"] = np.ones(d, one)
        lw["k_norm"] = np.ones(d, one)
        layers.append(lw)
    out["layers"] = layers
    return out


def prompt_ids(seed: int, n: int, vocab: int) -> np.ndarray:
    """``n`` uniform-random token ids in [0, vocab) as int32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, n).astype(np.int32)


# GEMV sweep shapes [M, K] of the decode projections (fused QKV, O, fused
# gate/up, down, tied vocabulary head).
GEMV_SHAPES = [(4096, 1024), (1024, 2048), (6144, 1024), (1024, 3072), (151936, 1024)]
# int4 sweep shapes [M, K].
Q4_SHAPES = [(4096, 4096), (14336, 4096), (4096, 14336)]


def gemv_inputs(m: int, k: int, t: int, seed: int, copy: int = 0, dtype=np.float32):
    """One weight matrix ``W[m,k] ~ N(0,0.02)`` and activations ``X[t,k] ~ N(0,1)``.

    ``seed`` selects the activation stream; ``copy`` selects a distinct
    weight matrix (seed ``1000*seed + copy``).  ``dtype`` float16 rounds
    both W and X to FP16.
    """
    rw = np.random.Generator(np.random.PCG64(1000 * seed + copy))
    w = rw.standard_normal((m, k), dtype=np.float32)
    w *= _STD
    rx = np.random.Generator(np.random.PCG64(seed))
    x = rx.standard_normal((t, k), dtype=np.float32)
    if dtype != np.float32:
        w = w.astype(dtype)
        x = x.astype(dtype)
    return w, x


def pack_int4_rows(q: np.ndarray) -> np.ndarray:
    """Pack signed 4-bit values ``q[m,k]`` (k % 8 == 0) into ``uint32[m, k/8]``.

    Storage format: nibble j (bits 4j..4j+3) of word w holds element
    k = 8w + j as a two's-complement 4-bit value.
    """
    m, k = q.shape
    assert k % 8 == 0
    nib = (q.astype(np.int64) & 0xF).astype(np.uint32).reshape(m, k // 8, 8)
    words = np.zeros((m, k // 8), dtype=np.uint32)
    for j in range(8):
        words |= nib[:, :, j] << np.uint32(4 * j)
    return words


def q4g64_inputs(m: int, k: int, t: int, seed: int, copy: int = 0):
    """Symmetric int4 weights, group 64 along K, one FP16 scale per group.

    Returns ``(q int8[m,k] in [-8,7], words uint32[m,k/8], scales f16[m,k/64],
    X f16[t,k])``.
    """
    assert k % 64 == 0
    rw = np.random.Generator(np.random.PCG64(1000 * seed + copy))
    q = rw.integers(-8, 8, (m, k)).astype(np.int8)
    scales = np.abs(rw.normal(0.0, 0.01, (m, k // 64))).astype(np.float16)
    rx = np.random.Generator(np.random.PCG64(seed))
    x = rx.standard_normal((t, k), dtype=np.float32).astype(np.float16)
    return q, pack_int4_rows(q), scales, x
