"""GPU decode path vs the oracle, through the C ABI, in lockstep.

Per step (Benchmark methodology, "Long-document chunked prefill";
Megakernels, "GPU-wide end-to-end generation"): full-vocabulary logits
within rtol=atol=1e-3 (FP32), the exact greedy token, and the newly written
K/V slot of every layer; the whole valid K/V prefix at the first output and
at the end.  FP16 storage is checked teacher-forced at rtol=atol=2e-2.
"""
import numpy as np
import pytest

from gpu_util import _np, announce, gpu_available, lockstep
import oracle
from synth import MINI, PROMPT_SEEDS, QWEN3_0_6B, model_weights, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def mini_w():
    return model_weights(MINI, seed=0)


def test_mini_fp32_generation_graph_and_direct(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=64)
    orc = oracle.OracleModel(MINI, mini_w, 64)
    prompt = prompt_ids(PROMPT_SEEDS["tiny"], 8, MINI.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 8, label="mini graph")
    logits_graph = _np(m.logits())
    m.set_option(wsg._abi.WSG_OPT_USE_GRAPH, 0)
    toks2, _, _ = lockstep(m, orc, prompt, 8, label="mini direct")
    assert toks2 == toks
    assert np.array_equal(_np(m.logits()), logits_graph)   # same kernels, same bits
    m.close()


def test_mini_reset_determinism(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=64)
    prompt = prompt_ids(7, 11, MINI.vocab)
    outs = []
    for _ in range(2):
        m.reset()
        t = [m.prefill(prompt)] + [m.step() for _ in range(5)]
        k, v, n = m.kv(1)
        outs.append((t, _np(m.logits()), _np(k[:, :n]), _np(v[:, :n])))
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)
    m.close()


@pytest.mark.parametrize("n_prompt", [63, 64, 65, 200, 300])
def test_mini_split_attention_long_prompt(mini_w, n_prompt):
    """Contexts beyond one 64-key split exercise the split-K merge across blocks."""
    import weight_streaming_gemv_amd as wsg
    cap = 320
    m = wsg.Model(MINI, mini_w, max_context=cap)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(9, n_prompt, MINI.vocab)
    lockstep(m, orc, prompt, 6, label=f"mini split n={n_prompt}")
    m.close()


def test_mini_error_paths(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=8)
    with pytest.raises(wsg.WsgError, match="STATE"):
        m.step()
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.prefill([1, MINI.vocab])
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.prefill(list(range(9)))
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        m.prefill([])
    assert m.position == 0
    m.prefill([1, 2, 3, 4, 5, 6, 7])
    m.step()
    assert m.position == 8
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step()
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step(MINI.vocab)
    m.reset()
    assert m.position == 0
    m.close()


@pytest.fixture(scope="module")
def c1_w():
    return model_weights(QWEN3_0_6B.with_layers(2), seed=0)


def test_tiny_qwen3_fp32_generation(c1_w):
    """2-layer Qwen3-0.6B shape, FP32: 8 prompt ids then 8 greedy tokens."""
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    m = wsg.Model(sh, c1_w, max_context=16)
    orc = oracle.OracleModel(sh, c1_w, 16)
    prompt = prompt_ids(PROMPT_SEEDS["tiny"], 8, sh.vocab)
    toks, rtoks, ck = lockstep(m, orc, prompt, 8, label="qwen3x2 fp32")
    print(f"tokens {toks}; max |dlogit| {ck.max_logit_err:.2e}; max |dkv| {ck.max_kv_err:.2e}")
    assert orc.pos == 15
    m.close()


def test_tiny_qwen3_fp16_teacher_forced(c1_w):
    """FP16 storage at the 2-layer shape, teacher-forced, rtol=atol=2e-2."""
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    w16 = {"embed": c1_w["embed"].astype(np.float16), "final_norm": c1_w["final_norm"].astype(np.float16),
           "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in c1_w["layers"]]}
    m = wsg.Model(sh, w16, max_context=16, dtype=wsg.WSG_F16)
    orc = oracle.OracleModel(sh, w16, 16)
    prompt = prompt_ids(PROMPT_SEEDS["tiny"], 8, sh.vocab)
    _, _, ck = lockstep(m, orc, prompt, 8, rtol=2e-2, atol=2e-2, teacher=True, label="qwen3x2 fp16")
    print(f"fp16 max |dlogit| {ck.max_logit_err:.2e}; max |dkv| {ck.max_kv_err:.2e}")
    m.close()
