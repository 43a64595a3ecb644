"""The full 28-layer Qwen3-0.6B-shaped model on the GPU vs the oracle, in the launch
configuration bench.py times (default shapes, captured graphs).

Per step: full-vocabulary logits within rtol=atol=1e-3 (FP32), the exact greedy
token, and the new K/V slot of every layer; the whole valid K/V prefix at the end
(Benchmark methodology, "Long-document chunked prefill": the tolerance and the
cache check).  Also at full size: two-token steps, the int4 decoder (FP16
tolerance, teacher-forced) and a chunk-1024 prefill that crosses a chunk boundary.
"""
import numpy as np
import pytest

from gpu_util import _np, announce, close_rel, gpu_available, lockstep
import oracle
from synth import PROMPT_SEEDS, QWEN3_0_6B, model_weights, model_weights_q4, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def full_w():
    return model_weights(QWEN3_0_6B, seed=0)


@pytest.fixture(scope="module")
def full_orc_factory(full_w):
    cache = {}

    def make(cap):
        if cap not in cache:
            cache.clear()
            cache[cap] = oracle.OracleModel(QWEN3_0_6B, full_w, cap)
        return cache[cap]
    return make


def test_full_model_generation(full_w, full_orc_factory):
    """The 8-id short prompt, 8 greedy tokens, every step in lockstep."""
    import weight_streaming_gemv_amd as wsg
    cap = 48
    m = wsg.Model(QWEN3_0_6B, full_w, max_context=cap, prefill_chunk=32)
    orc = full_orc_factory(cap)
    prompt = prompt_ids(PROMPT_SEEDS["short"], 8, QWEN3_0_6B.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 8, label="qwen3 28L fp32")
    print(f"28 layers: tokens {toks}; max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_full_model_two_token_steps(full_w, full_orc_factory):
    """Two-token steps at full size: an accepted and a rejected draft."""
    import weight_streaming_gemv_amd as wsg
    cap = 48
    m = wsg.Model(QWEN3_0_6B, full_w, max_context=cap, prefill_chunk=32)
    orc = full_orc_factory(cap)
    orc.reset()
    prompt = prompt_ids(PROMPT_SEEDS["short"], 32, QWEN3_0_6B.vocab)
    tok = m.prefill(prompt)
    ref = orc.forward_rows(prompt)
    assert tok == oracle.argmax_lowest(ref)
    last = tok
    for s, accept in enumerate((True, False)):
        p = orc.pos
        ref0 = orc.forward_rows([last])
        g0 = oracle.argmax_lowest(ref0)
        draft = g0 if accept else (g0 + 1) % QWEN3_0_6B.vocab
        announce(f"28L step2 {s} p={p}")
        (t0, t1), n = m.step2(draft)
        ref1 = orc.forward_rows([draft])
        got = _np(m.logits())
        for row, r in ((0, ref0), (1, ref1)):
            ok, err, worst = close_rel(got[row], r, 1e-3, 1e-3)
            assert ok, f"step {s} row {row}: logits off by {err:.3e} at {worst}"
        for l in range(QWEN3_0_6B.n_layers):
            k, v, _ = m.kv(l)
            for g_, r_ in ((k, orc.k_cache[l]), (v, orc.v_cache[l])):
                ok, err, _ = close_rel(_np(g_[:, p:p + 2]), r_[:, p:p + 2], 1e-3, 1e-3)
                assert ok, f"step {s} layer {l}: K/V off by {err:.3e}"
        assert t0 == g0 and n == (2 if accept else 1)
        if accept:
            assert t1 == oracle.argmax_lowest(ref1)
            last = t1
        else:
            orc.pos = p + 1
            last = t0
    m.close()


def test_full_model_chunked_prefill_crosses_a_chunk(full_w):
    """A 1100-id prompt at chunk 1024 (the selected long-document chunk): two chunks,
    the second with 75 rows, then 2 outputs; every valid K/V entry checked."""
    import weight_streaming_gemv_amd as wsg
    cap = 1104
    m = wsg.Model(QWEN3_0_6B, full_w, max_context=cap, prefill_chunk=1024)
    orc = oracle.OracleModel(QWEN3_0_6B, full_w, cap)
    prompt = prompt_ids(PROMPT_SEEDS["tuning"], 1100, QWEN3_0_6B.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 2, label="qwen3 28L chunk 1024")
    print(f"chunk 1024: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_full_int4_decoder():
    """The 28-layer int4 decoder, teacher-forced at the FP16 tolerance."""
    import weight_streaming_gemv_amd as wsg
    w = model_weights_q4(QWEN3_0_6B, seed=0)
    cap = 24
    m = wsg.Model(QWEN3_0_6B, w, max_context=cap, dtype=wsg.WSG_F16)
    orc = oracle.OracleModel(QWEN3_0_6B, w, cap)
    prompt = prompt_ids(PROMPT_SEEDS["short"], 8, QWEN3_0_6B.vocab)
    _, _, ck = lockstep(m, orc, prompt, 4, rtol=2e-2, atol=2e-2, teacher=True, label="qwen3 28L int4")
    print(f"int4 28 layers: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()
