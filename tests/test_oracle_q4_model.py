"""Pins of the oracle's int4 decoder path (weights given as int4 words and FP16
group scales; Our Kernel Benchmark Was Measuring the System Cache, "Summary").

The expected values are built here from the drawn int4 values themselves,
not from the oracle's unpacking: with power-of-two scales every weight
q * s is an FP16 value, so the int4 model must equal the dense FP16 model
holding those values bit for bit; with general scales the embedding rows the
model gathers must be q * s rounded once to FP16.
"""
import numpy as np

from oracle import OracleModel, argmax_lowest
from synth import MINI, model_weights_q4, pack_int4_rows, prompt_ids


def _q4_and_dense(shape, seed, pow2):
    rng = np.random.default_rng(seed)

    def mat(rows, k):
        q = rng.integers(-8, 8, (rows, k)).astype(np.int8)
        if pow2:
            s = np.ldexp(1.0, rng.integers(-9, -4, (rows, k // 64))).astype(np.float16)
        else:
            s = np.abs(rng.normal(0.0, 0.01, (rows, k // 64))).astype(np.float16)
        dense = q.astype(np.float64) * np.repeat(s.astype(np.float64), 64, axis=1)
        return (pack_int4_rows(q), s), dense

    h, i, qw, kv, d = shape.hidden, shape.intermediate, shape.q_width, shape.kv_width, shape.head_dim
    wq4 = {"format": "q4g64", "final_norm": np.ones(h, np.float16), "layers": []}
    wd = {"final_norm": np.ones(h, np.float16), "layers": []}
    wq4["embed"], e = mat(shape.vocab, h)
    wd["embed"] = e
    for _ in range(shape.n_layers):
        a, b = {}, {}
        for name, (rows, k) in (("wq", (qw, h)), ("wk", (kv, h)), ("wv", (kv, h)), ("wo", (h, qw)),
                                ("wg", (i, h)), ("wu", (i, h)), ("wd", (h, i))):
            a[name], b[name] = mat(rows, k)
        for name, n in (("in_norm", h), ("post_norm", h), ("q_norm", d), ("k_norm", d)):
            a[name] = b[name] = np.ones(n, np.float16)
        wq4["layers"].append(a)
        wd["layers"].append(b)
    return wq4, wd


def test_q4_model_with_pow2_scales_equals_dense_fp16():
    wq4, wd = _q4_and_dense(MINI, 3, pow2=True)
    # every weight q * 2^e is an FP16 value: the dense model holds it exactly
    for name in ("embed",):
        assert np.array_equal(wd[name].astype(np.float16).astype(np.float64), wd[name])
    dense16 = {"embed": wd["embed"].astype(np.float16), "final_norm": wd["final_norm"],
               "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in wd["layers"]]}
    ids = prompt_ids(5, 7, MINI.vocab)
    a = OracleModel(MINI, wq4, 16)
    b = OracleModel(MINI, dense16, 16)
    la, lb = a.forward_rows(ids), b.forward_rows(ids)
    assert la.dtype == np.float16 and np.array_equal(la, lb)
    for _ in range(3):
        t = argmax_lowest(la)
        la, lb = a.forward_rows([t]), b.forward_rows([t])
        assert np.array_equal(la, lb)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.v_cache, b.v_cache)


def test_q4_embedding_rows_are_rounded_products():
    wq4, wd = _q4_and_dense(MINI, 4, pow2=False)
    m = OracleModel(MINI, wq4, 4)
    assert m.dtype == np.float16
    assert np.array_equal(m.E64, wd["embed"])                       # exact q * s
    assert np.array_equal(m.E, wd["embed"].astype(np.float16))      # one rounding for the gather
    # some products are not FP16 values, so the gather really rounds
    assert np.any(m.E.astype(np.float64) != m.E64)
    for l, lw in enumerate(wd["layers"]):
        for k in ("wq", "wo", "wd"):
            assert np.array_equal(m.layers[l][k], lw[k])


def test_synth_q4_weights_shape_and_ranges():
    w = model_weights_q4(MINI, seed=1)
    words, scales = w["embed"]
    assert words.shape == (MINI.vocab, MINI.hidden // 8) and words.dtype == np.uint32
    assert scales.shape == (MINI.vocab, MINI.hidden // 64) and scales.dtype == np.float16
    assert np.all(scales >= 0)
    lw = w["layers"][0]
    assert lw["wd"][0].shape == (MINI.hidden, MINI.intermediate // 8)
    assert lw["in_norm"].dtype == np.float16
