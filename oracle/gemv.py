"""Matrix-vector products of the weight-streaming GEMV family.

Test infrastructure (see the package docstring).  ``Y[t, m] = sum_k
W[m, k] X[t, k]`` for one or two input vectors (the two-token variant of Our
Kernel Benchmark Was Measuring the System Cache, "Why it mattered"), with
float64 sums and an FP32 result.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def gemv(w, x) -> np.ndarray:
    """``W[M,K]`` (FP32 or FP16) times ``X[T,K]`` -> ``Y[T,M]`` FP32 (float64 sums)."""
    w64 = np.asarray(w, dtype=F64)
    x64 = np.atleast_2d(np.asarray(x, dtype=F64))
    return (x64 @ w64.T).astype(np.float32)


def unpack_int4(words, k: int) -> np.ndarray:
    """Decode ``uint32[M, k/8]`` into signed 4-bit values ``int8[M, k]``.

    Storage format (the pages do not state one): nibble j of word w is
    element 8w + j, two's complement, so raw nibbles 8..15 are -8..-1.
    """
    words = np.asarray(words, dtype=np.uint32)
    m = words.shape[0]
    out = np.empty((m, k), dtype=np.int8)
    for j in range(8):
        nib = ((words >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.int16)
        out[:, j::8] = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return out


def dequant_q4g64(words, scales, k: int) -> np.ndarray:
    """Weights ``q[m,k] * s[m, k // 64]`` as FP32 (each product is exact in FP32)."""
    q = unpack_int4(words, k).astype(F64)
    s = np.asarray(scales, dtype=F64)
    return (q * np.repeat(s, 64, axis=1)).astype(np.float32)


def gemv_q4g64(words, scales, x, k: int) -> np.ndarray:
    """int4 group-64 GEMV: dequantise on the CPU, then the plain product."""
    return gemv(dequant_q4g64(words, scales, k), x)
