"""Primitive operations of the decode path, written from their definitions.

Test infrastructure (see the package docstring).  Inputs may be FP32 or
FP16 arrays; all arithmetic is float64; ``store`` rounds to the storage
dtype (round-to-nearest-even, numpy's cast).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def store(a, dtype) -> np.ndarray:
    """Round a float64 result to the storage dtype (one rounding)."""
    return np.asarray(a, dtype=F64).astype(dtype)


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm along the last axis, float64 result (not yet stored).

    y = x * (mean(x**2) + eps) ** -1/2 * gain.  The pages describe the norm
    as a reduction, a normalisation and a multiplication by the weight
    (Benchmark methodology, "Compiler comparison rules"), with a precise
    reciprocal square root (Megakernels, "Chunked prefill for long
    prompts"); eps sits inside the root and the gain multiplies directly.
    """
    x64 = np.asarray(x, dtype=F64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    return x64 / np.sqrt(ms + eps) * np.asarray(gain, dtype=F64)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """Rotation angles ``[len(positions), head_dim/2]`` in float64.

    Pair i (i < head_dim/2) turns by position * theta**(-2i/head_dim): the
    rotary constants the host precomputes once (Megakernels, "What runs in
    the DSL").  The pages fix no pairing or base; the Qwen3 convention is
    used: base theta (1e6 for these models) and half-split pairs.
    """
    half = head_dim // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=F64) / head_dim)
    return np.asarray(positions, dtype=F64)[:, None] * inv_freq[None, :]


def rope_apply(u, angles) -> np.ndarray:
    """Rotate half-split pairs (i, i + D/2) of ``u[..., D]`` by ``angles[..., D/2]``.

    u'[i]       = u[i] cos a_i - u[i+D/2] sin a_i
    u'[i+D/2]   = u[i+D/2] cos a_i + u[i] sin a_i
    Works in float64; ``angles`` broadcasts against the leading axes of u.
    """
    u64 = np.asarray(u, dtype=F64)
    half = u64.shape[-1] // 2
    lo, hi = u64[..., :half], u64[..., half:]
    c, s = np.cos(angles), np.sin(angles)
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def silu(z) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z)), float64 (SwiGLU gate)."""
    z64 = np.asarray(z, dtype=F64)
    return z64 / (1.0 + np.exp(-z64))


def gqa_attention(q, k_cache, v_cache, positions) -> np.ndarray:
    """Grouped-query causal attention, float64 result ``[n, Hq, D]``.

    ``q[n, Hq, D]`` holds the normalised, rotated queries of n rows;
    ``k_cache[Hkv, P, D]`` and ``v_cache[Hkv, P, D]`` hold the cached keys
    and values; row r attends to keys 0..positions[r] inclusive (its own,
    current key included: Megakernels, "Single-threadgroup execution" and
    "Chunked prefill for long prompts").  Query head h reads KV head
    h // (Hq/Hkv) (contiguous groups; the pages leave the mapping open).
    Scores are scaled by 1/sqrt(D) after the QK product (Megakernels,
    "Matrix-tiled attention"), then an exact softmax.
    """
    q64 = np.asarray(q, dtype=F64)
    n, hq, d = q64.shape
    hkv = k_cache.shape[0]
    group = hq // hkv
    positions = np.asarray(positions, dtype=np.int64)
    n_keys = int(positions.max()) + 1
    key_idx = np.arange(n_keys)[None, :]
    future = key_idx > positions[:, None]            # [n, n_keys]
    out = np.empty((n, hq, d), dtype=F64)
    scale = 1.0 / np.sqrt(d)
    for h in range(hq):
        j = h // group
        k64 = np.asarray(k_cache[j, :n_keys], dtype=F64)
        v64 = np.asarray(v_cache[j, :n_keys], dtype=F64)
        s = (q64[:, h, :] @ k64.T) * scale           # [n, n_keys]
        s[future] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v64
    return out


def argmax_lowest(logits) -> int:
    """Greedy token: the lowest index among the maximal logits.

    Ties go to the lowest token id (Megakernels, "GPU-wide end-to-end
    generation").  Logits must be finite: a NaN or inf is a validation
    failure, never a tie-break.  -0.0 and +0.0 compare equal (a tie).
    """
    v = np.asarray(logits)
    if v.ndim != 1 or v.size == 0:
        raise ValueError("argmax_lowest expects a non-empty vector")
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite logits")
    best = v.max()
    return int(np.flatnonzero(v == best)[0])
