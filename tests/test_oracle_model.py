"""Pins of the oracle's whole-model composition.

No worked numeric example exists for random weights, so the composition is
pinned by invariants that a slip would break: the 0-layer echo, exact
residual pass-through, KV-head permutation symmetry, the RoPE position
stamped into the cache, chunk invariance, the KV bookkeeping the pages
print, and a pure-Python brute force of a tiny model.
"""
import copy
import json
import math
import os

import numpy as np
import pytest

from oracle import OracleModel, argmax_lowest
from synth import MINI, QWEN3_0_6B, ModelShape, model_weights, prompt_ids

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = ModelShape(n_layers=2, hidden=8, intermediate=12, n_q_heads=4, n_kv_heads=2,
                  head_dim=4, vocab=11)


def _zero_layers(w, keys):
    w = copy.deepcopy(w)
    for lw in w["layers"]:
        for k in keys:
            lw[k] = np.zeros_like(lw[k])
    return w


def test_zero_layer_model_echoes_token():
    sh = MINI.with_layers(0)
    w = model_weights(sh, seed=0)
    m = OracleModel(sh, w, max_context=4)
    for t in prompt_ids(3, 20, sh.vocab):
        m.reset()
        assert argmax_lowest(m.forward_rows([t])) == t


def test_zero_output_projections_pass_residual_through():
    w = model_weights(MINI, seed=0)
    wz = _zero_layers(w, ["wo", "wd"])
    w0 = {"embed": w["embed"], "final_norm": w["final_norm"], "layers": []}
    ids = prompt_ids(1, 6, MINI.vocab)
    a = OracleModel(MINI, wz, 8).forward_rows(ids)
    b = OracleModel(MINI.with_layers(0), w0, 8).forward_rows(ids)
    assert np.array_equal(a, b)


def test_zero_output_projection_hides_attention_weights():
    w = _zero_layers(model_weights(MINI, seed=0), ["wo"])
    w2 = copy.deepcopy(w)
    rng = np.random.default_rng(4)
    for lw in w2["layers"]:
        for k in ("wq", "wk", "wv"):
            lw[k] = rng.standard_normal(lw[k].shape).astype(np.float32)
    ids = prompt_ids(1, 5, MINI.vocab)
    assert np.array_equal(OracleModel(MINI, w, 8).forward_rows(ids),
                          OracleModel(MINI, w2, 8).forward_rows(ids))


def test_kv_head_permutation_symmetry():
    """Swap KV heads 0 and 1 together with their query groups: same logits."""
    sh = MINI  # 4 query heads, 2 KV heads, group 2
    w = model_weights(sh, seed=0)
    d = sh.head_dim
    wp = copy.deepcopy(w)
    qperm = [2, 3, 0, 1]          # query heads of group 1 first
    kperm = [1, 0]
    for lw, lp in zip(w["layers"], wp["layers"]):
        lp["wq"] = np.concatenate([lw["wq"][h * d:(h + 1) * d] for h in qperm])
        lp["wk"] = np.concatenate([lw["wk"][j * d:(j + 1) * d] for j in kperm])
        lp["wv"] = np.concatenate([lw["wv"][j * d:(j + 1) * d] for j in kperm])
        lp["wo"] = np.concatenate([lw["wo"][:, h * d:(h + 1) * d] for h in qperm], axis=1)
    ids = prompt_ids(1, 7, sh.vocab)
    a = OracleModel(sh, w, 8).forward_rows(ids)
    b = OracleModel(sh, wp, 8).forward_rows(ids)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-6)


def test_cache_keys_unit_rms_and_rotated_by_position():
    sh = MINI
    w = model_weights(sh, seed=0)
    m = OracleModel(sh, w, 16)
    tok = 123
    m.forward_rows([tok, 5, tok, 9, 11, tok])     # same token at positions 0, 2, 5
    k = m.k_cache[0].astype(np.float64)            # layer 0: depends only on the token
    v = m.v_cache[0]
    d = sh.head_dim
    # normalised keys (gain 1) keep unit RMS through the rotation
    assert np.allclose(np.sqrt(np.mean(k[:, :6] ** 2, axis=-1)), 1.0, rtol=1e-5)
    # values at layer 0 do not depend on position
    assert np.array_equal(v[:, 0], v[:, 2]) and np.array_equal(v[:, 0], v[:, 5])
    # keys at positions 5 and 0 differ by a rotation of 5 * base^(-2i/D) per pair
    for j in range(sh.n_kv_heads):
        z0 = k[j, 0, :d // 2] + 1j * k[j, 0, d // 2:]
        z5 = k[j, 5, :d // 2] + 1j * k[j, 5, d // 2:]
        freq = sh.rope_theta ** (-2.0 * np.arange(d // 2) / d)
        assert np.allclose(z5, z0 * np.exp(1j * 5 * freq), atol=2e-6)


def test_chunk_invariance_rows_vs_tokenwise():
    sh = MINI
    w = model_weights(sh, seed=0)
    ids = prompt_ids(1, 9, sh.vocab)
    a = OracleModel(sh, w, 16)
    la = a.forward_rows(ids)
    b = OracleModel(sh, w, 16)
    for t in ids[:-1]:
        b.forward_rows([t], want_logits=False)
    lb = b.forward_rows(ids[-1:])
    c = OracleModel(sh, w, 16)
    c.forward_rows(ids[:4], want_logits=False)
    lc = c.forward_rows(ids[4:])
    for other, lo in ((b, lb), (c, lc)):
        assert np.allclose(la, lo, rtol=1e-6, atol=1e-7)
        assert np.allclose(a.k_cache[:, :, :9], other.k_cache[:, :, :9], rtol=1e-6, atol=1e-7)
        assert np.allclose(a.v_cache[:, :, :9], other.v_cache[:, :, :9], rtol=1e-6, atol=1e-7)


def test_generation_bookkeeping_matches_pages():
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        fact = json.load(f)["valid_kv_after_generation"]
    # same rule at a small size: valid entries = prompt + outputs - 1
    n_p, n_o = 7, 5
    assert fact["valid_entries"] == fact["prompt_tokens"] + fact["output_tokens"] - 1
    m = OracleModel(MINI, model_weights(MINI, seed=0), 16)
    out = m.generate(prompt_ids(1, n_p, MINI.vocab), n_o)
    assert len(out) == n_o and m.pos == n_p + n_o - 1


def test_shape_and_weight_bytes_match_pages():
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        s = json.load(f)["qwen3_0_6b_shape"]
    sh = QWEN3_0_6B
    assert (sh.n_layers, sh.hidden, sh.intermediate, sh.n_q_heads, sh.n_kv_heads, sh.head_dim,
            sh.vocab, sh.q_width) == (s["n_layers"], s["hidden"], s["intermediate"], s["n_q_heads"],
                                      s["n_kv_heads"], s["head_dim"], s["vocab"], s["q_width"])
    assert sh.weight_bytes_per_token(4) == 2_383_937_536
    assert sh.with_layers(2).weight_bytes_per_token(4) == 748_158_976


def test_fp16_storage_dtype_and_closeness():
    w16 = model_weights(MINI, seed=0, dtype=np.float16)
    ids = prompt_ids(1, 5, MINI.vocab)
    m16 = OracleModel(MINI, w16, 8)
    l16 = m16.forward_rows(ids)
    assert l16.dtype == np.float16 and m16.k_cache.dtype == np.float16
    w32 = {"embed": w16["embed"].astype(np.float32), "final_norm": w16["final_norm"].astype(np.float32),
           "layers": [{k: v.astype(np.float32) for k, v in lw.items()} for lw in w16["layers"]]}
    l32 = OracleModel(MINI, w32, 8).forward_rows(ids)
    assert np.allclose(l16.astype(np.float32), l32, rtol=2e-2, atol=2e-2)


def test_rejects_bad_ids_and_capacity():
    m = OracleModel(MINI, model_weights(MINI, seed=0), 4)
    with pytest.raises(ValueError):
        m.forward_rows([MINI.vocab])
    with pytest.raises(ValueError):
        m.forward_rows([1, 2, 3, 4, 5])


# ---------------------------------------------------------------- brute force
def _rms(v, g, eps):
    # float(): a NumPy scalar gain would pull the product down to its own precision
    ms = math.fsum(float(a) * float(a) for a in v) / len(v)
    r = 1.0 / math.sqrt(ms + eps)
    return [float(a) * r * float(b) for a, b in zip(v, g)]


def _mv(wm, v):
    return [math.fsum(float(a) * b for a, b in zip(row, v)) for row in wm]


def _f32(v):
    return [float(np.float32(a)) for a in v]


def _f16(v):
    return [float(np.float16(a)) for a in v]


# Stored values of the brute force, by stage: the embedding gather, the eight
# stage outputs of a layer (Megakernels, "GPU-wide end-to-end generation"),
# the final norm and the logits.
BRUTE_STAGES = ("gather", "norm_in", "qkv", "qk_rope", "attn", "o_res", "norm_post", "act", "down_res",
                "norm_final", "logits")


def brute_generate(sh, w, prompt, n_out, store=_f32, skip=None):
    """Token-at-a-time forward written with Python lists and math.fsum.

    ``store`` rounds a stored vector to the storage dtype (``_f32`` or ``_f16``);
    ``skip`` names one entry of ``BRUTE_STAGES`` whose rounding is left out (a
    planted slip, to show that the comparison sees that stage's rounding)."""
    d, hq, hkv, eps = sh.head_dim, sh.n_q_heads, sh.n_kv_heads, sh.rms_eps
    K = [[[] for _ in range(hkv)] for _ in range(sh.n_layers)]
    V = [[[] for _ in range(hkv)] for _ in range(sh.n_layers)]

    def rd(stage, v):
        return list(v) if stage == skip else store(v)

    def rot(u, p):
        half = d // 2
        out = [0.0] * d
        for i in range(half):
            a = p * sh.rope_theta ** (-2.0 * i / d)
            out[i] = u[i] * math.cos(a) - u[i + half] * math.sin(a)
            out[i + half] = u[i + half] * math.cos(a) + u[i] * math.sin(a)
        return out

    def step(tok, p):
        x = rd("gather", [float(a) for a in w["embed"][tok]])
        for l, lw in enumerate(w["layers"]):
            a = rd("norm_in", _rms(x, lw["in_norm"], eps))
            q, k, v = rd("qkv", _mv(lw["wq"], a)), rd("qkv", _mv(lw["wk"], a)), rd("qkv", _mv(lw["wv"], a))
            qs = [rd("qk_rope", rot(_rms(q[h * d:(h + 1) * d], lw["q_norm"], eps), p)) for h in range(hq)]
            for j in range(hkv):
                K[l][j].append(rd("qk_rope", rot(_rms(k[j * d:(j + 1) * d], lw["k_norm"], eps), p)))
                V[l][j].append(v[j * d:(j + 1) * d])
            o = []
            for h in range(hq):
                j = h // (hq // hkv)
                s = [math.fsum(a * b for a, b in zip(qs[h], kk)) / math.sqrt(d) for kk in K[l][j]]
                mx = max(s)
                e = [math.exp(t - mx) for t in s]
                den = math.fsum(e)
                o += [math.fsum(e[i] * V[l][j][i][c] for i in range(len(e))) / den for c in range(d)]
            o = rd("attn", o)
            x = rd("o_res", [a + b for a, b in zip(x, _mv(lw["wo"], o))])
            b = rd("norm_post", _rms(x, lw["post_norm"], eps))
            g, u = _mv(lw["wg"], b), _mv(lw["wu"], b)
            act = rd("act", [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
            x = rd("down_res", [a + c for a, c in zip(x, _mv(lw["wd"], act))])
        hvec = rd("norm_final", _rms(x, w["final_norm"], eps))
        return rd("logits", _mv(w["embed"], hvec))

    out, logits = [], None
    for p, t in enumerate(prompt):
        logits = step(int(t), p)
    for s in range(n_out):
        lg = np.array(logits)
        out.append(int(np.flatnonzero(lg == lg.max())[0]))
        if s + 1 < n_out:
            logits = step(out[-1], len(prompt) + s)
    return out, logits


def test_tiny_model_brute_force():
    w = model_weights(TINY, seed=0)
    # larger weights so attention and the MLP matter at this tiny width
    for lw in w["layers"]:
        for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            lw[k] = lw[k] * np.float32(25.0)
    # non-unit gains, so the order of norm, gain and rotation matters
    rng = np.random.default_rng(8)
    for lw in w["layers"]:
        for k in ("in_norm", "post_norm", "q_norm", "k_norm"):
            lw[k] = rng.uniform(0.5, 1.5, lw[k].shape).astype(np.float32)
    w["final_norm"] = rng.uniform(0.5, 1.5, w["final_norm"].shape).astype(np.float32)
    prompt = prompt_ids(1, 4, TINY.vocab)
    bt, bl = brute_generate(TINY, w, prompt, 4)
    m = OracleModel(TINY, w, 8)
    ot, orec = m.generate(prompt, 4, record=True)
    assert ot == bt
    assert np.allclose(orec[-1], np.array(bl, np.float32), rtol=1e-6, atol=1e-6)


def _tiny_weights(dtype):
    """TINY weights scaled so attention and the MLP matter at this width, with
    non-unit gains so the order of norm, gain and rotation matters; stored in
    ``dtype``."""
    w = model_weights(TINY, seed=0)
    for lw in w["layers"]:
        for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            lw[k] = (lw[k] * np.float32(25.0)).astype(dtype)
    rng = np.random.default_rng(8)
    for lw in w["layers"]:
        for k in ("in_norm", "post_norm", "q_norm", "k_norm"):
            lw[k] = rng.uniform(0.5, 1.5, lw[k].shape).astype(dtype)
    w["final_norm"] = rng.uniform(0.5, 1.5, w["final_norm"].shape).astype(dtype)
    w["embed"] = w["embed"].astype(dtype)
    return w


def _fp16_ulps(a, b):
    """Largest distance between two FP16 vectors in units of FP16 spacing at b."""
    a = np.asarray(a, dtype=np.float16).astype(np.float64)
    b = np.asarray(b, dtype=np.float16)
    return float(np.max(np.abs(a - b.astype(np.float64)) / np.spacing(np.abs(b)).astype(np.float64)))


def test_tiny_model_brute_force_fp16_storage():
    """FP16 storage mode: every stored value (each of the eight stage outputs per layer,
    the final norm and the logits) rounded to FP16, every reduction exact (math.fsum).
    The oracle in FP16 mode gives the same greedy tokens and the same FP16 logits, bit
    for bit.  (Float64 BLAS sums and math.fsum could round a value that sits on an FP16
    rounding boundary to neighbouring FP16 values; no value of this input does, so the
    comparison is exact rather than one ulp wide.)"""
    w = _tiny_weights(np.float16)
    prompt = prompt_ids(1, 4, TINY.vocab)
    bt, bl = brute_generate(TINY, w, prompt, 4, store=_f16)
    m = OracleModel(TINY, w, 8)
    assert m.dtype == np.float16
    ot, orec = m.generate(prompt, 4, record=True)
    assert orec[-1].dtype == np.float16
    assert ot == bt
    assert _fp16_ulps(bl, orec[-1]) == 0.0


# The gathered embedding row of a dense FP16 model is a stored value already, so its
# rounding is the identity here; the gather rounding of int4 models (q * s rounded once)
# is pinned in test_oracle_q4_model.py.
@pytest.mark.parametrize("stage", BRUTE_STAGES[1:])
def test_fp16_brute_force_sees_each_stage_rounding(stage):
    """The FP16 comparison above has teeth: leaving out the FP16 rounding of any one
    stored stage in the brute force changes its tokens or logits against the oracle's
    (so a dropped storage rounding in the oracle would fail that comparison too)."""
    w = _tiny_weights(np.float16)
    prompt = prompt_ids(1, 4, TINY.vocab)
    m = OracleModel(TINY, w, 8)
    ot, orec = m.generate(prompt, 4, record=True)
    bt, bl = brute_generate(TINY, w, prompt, 4, store=_f16, skip=stage)
    if stage == "logits":
        # unrounded logits: compare before any rounding
        dist = float(np.max(np.abs(np.asarray(bl) - orec[-1].astype(np.float64))))
        assert dist > 0.0
    else:
        assert bt != ot or _fp16_ulps(bl, orec[-1]) > 0.0, f"skipping the {stage} rounding went unnoticed"
