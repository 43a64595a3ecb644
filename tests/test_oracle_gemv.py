"""Pins of the oracle's GEMV family: exact cases, rounding bounds, int4 golden words."""
import json
import math
import os

import numpy as np
import pytest

from oracle import dequant_q4g64, gemv, gemv_q4g64, unpack_int4
from synth import pack_int4_rows, q4g64_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_gemv_one_hot_returns_column_exactly():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((37, 300)).astype(np.float32)
    for k in (0, 5, 299):
        x = np.zeros((1, 300), np.float32)
        x[0, k] = 1.0
        assert np.array_equal(gemv(w, x)[0], w[:, k])


def test_gemv_integer_exact_against_python_ints():
    rng = np.random.default_rng(1)
    w = rng.integers(-50, 50, (9, 64))
    x = rng.integers(-20, 20, (2, 64))
    y = gemv(w.astype(np.float32), x.astype(np.float32))
    for t in range(2):
        for m in range(9):
            assert y[t, m] == sum(int(a) * int(b) for a, b in zip(w[m], x[t]))


def test_gemv_two_tokens_are_independent_rows():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((16, 64)).astype(np.float32)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    y = gemv(w, x)
    assert np.array_equal(y[0], gemv(w, x[:1])[0])
    assert np.array_equal(y[1], gemv(w, x[1:])[0])


def test_gemv_within_one_ulp_of_correctly_rounded():
    # FP32 products are exact in float64; math.fsum rounds the exact sum once.
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 1024)) * 0.02).astype(np.float32)
    x = rng.standard_normal((1, 1024)).astype(np.float32)
    y = gemv(w, x)[0]
    for m in range(8):
        exact = np.float32(math.fsum(float(a) * float(b) for a, b in zip(w[m], x[0])))
        assert abs(int(y[m].view(np.int32)) - int(exact.view(np.int32))) <= 1


def test_gemv_fp16_weights_products_exact():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((4, 512)) * 0.02).astype(np.float16)
    x = rng.standard_normal((1, 512)).astype(np.float16)
    y = gemv(w, x)[0]
    for m in range(4):
        exact = np.float32(math.fsum(float(a) * float(b) for a, b in zip(w[m], x[0])))
        assert abs(int(y[m].view(np.int32)) - int(exact.view(np.int32))) <= 1


def test_int4_golden_words():
    with open(os.path.join(GOLDEN, "int4_words.json")) as f:
        cases = json.load(f)["cases"]
    words = np.array([[int(c["word"], 16) for c in cases]], dtype=np.uint32)
    vals = unpack_int4(words, 8 * len(cases))[0]
    for i, c in enumerate(cases):
        assert list(vals[8 * i:8 * i + 8]) == c["values"], c["word"]


def test_int4_pack_unpack_roundtrip():
    rng = np.random.default_rng(5)
    q = rng.integers(-8, 8, (7, 128)).astype(np.int8)
    assert np.array_equal(unpack_int4(pack_int4_rows(q), 128), q)


def test_q4_group_boundaries():
    # q = 1 everywhere, distinct scale per group: dequantised row = repeated scales
    m, k = 3, 256
    q = np.ones((m, k), np.int8)
    s = (np.arange(m * k // 64, dtype=np.float32).reshape(m, k // 64) + 1).astype(np.float16)
    wq = dequant_q4g64(pack_int4_rows(q), s, k)
    for r in range(m):
        for g in range(k // 64):
            assert np.all(wq[r, 64 * g:64 * g + 64] == np.float32(s[r, g]))
    # with x one-hot at the first element of each group, y = that group's scale
    for g in range(k // 64):
        x = np.zeros((1, k), np.float16)
        x[0, 64 * g] = 1
        assert np.array_equal(gemv_q4g64(pack_int4_rows(q), s, x, k)[0], s[:, g].astype(np.float32))


def test_q4_negative_values_and_dequant_exact():
    q, words, s, x = q4g64_inputs(16, 128, 2, seed=7)
    wq = dequant_q4g64(words, s, 128)
    assert np.array_equal(wq, q.astype(np.float32) * np.repeat(s.astype(np.float32), 64, axis=1))
    assert q.min() == -8 and q.max() == 7
