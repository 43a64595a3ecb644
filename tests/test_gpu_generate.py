"""wsg_generate (n greedy steps enqueued back to back, one wait) against the oracle and
against the step-by-step loop (Megakernels, "GPU-wide end-to-end generation": the token
is chosen on the GPU and the device keeps the history, so no step waits for the host).

The oracle generates greedily on the CPU; the GPU tokens must equal its tokens exactly,
the last step's logits and the whole K/V prefix must sit within rtol = atol = 1e-3
(FP32), and the same model run through ``step()`` must return the same tokens and the
same logits bit for bit (the same kernels run in the same order).
"""
import numpy as np
import pytest

from gpu_util import Checker, _np, announce, gpu_available
import oracle
from synth import MINI, PROMPT_SEEDS, QWEN3_0_6B, model_weights, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def mini_w():
    return model_weights(MINI, seed=0)


def _oracle_greedy(orc, prompt, n):
    """Prompt, then n greedy steps: (tokens after the prompt and each step, last logits)."""
    orc.reset()
    ref = orc.forward_rows(prompt)
    toks = [oracle.argmax_lowest(ref)]
    for _ in range(n):
        ref = orc.forward_rows([toks[-1]])
        toks.append(oracle.argmax_lowest(ref))
    return toks, ref


def _check_generation(m, orc, prompt, n, label):
    announce(f"{label}: prefill {len(prompt)} + generate {n}")
    ref_toks, ref_logits = _oracle_greedy(orc, prompt, n)
    m.reset()
    first = m.prefill(prompt)
    assert first == ref_toks[0], (label, first, ref_toks[0])
    got = m.generate(n)
    assert got == ref_toks[1:], f"{label}: generate {got} != oracle {ref_toks[1:]}"
    assert m.position == len(prompt) + n
    ck = Checker(m, orc, 1e-3, 1e-3, label)
    ck.logits(ref_logits, n)
    ck.kv(0, orc.pos, n)
    lg = _np(m.logits()).copy()
    # the step loop on the same model: same tokens, same logits bit for bit
    announce(f"{label}: step loop")
    m.reset()
    assert m.prefill(prompt) == first
    steps = [m.step() for _ in range(n)]
    assert steps == got, (label, steps, got)
    assert np.array_equal(_np(m.logits()), lg)
    return got


@pytest.mark.parametrize("graph", [1, 0])
def test_mini_generate_crosses_attention_modes(mini_w, graph):
    """From 100 keys to 160: the fused attention launch up to 128 keys, then split-K
    attention with the merge fused into the output projection; graphs for the new
    split counts are captured while earlier steps are still queued."""
    import weight_streaming_gemv_amd as wsg
    cap = 192
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_option(wsg._abi.WSG_OPT_USE_GRAPH, graph)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    _check_generation(m, orc, prompt_ids(31, 100, MINI.vocab), 60, f"mini graph={graph}")
    m.close()


def test_mini_generate_short(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=64)
    orc = oracle.OracleModel(MINI, mini_w, 64)
    _check_generation(m, orc, prompt_ids(PROMPT_SEEDS["tiny"], 8, MINI.vocab), 15, "mini short")
    m.close()


def test_qwen3_2layer_generate():
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    w = model_weights(sh, seed=5)
    m = wsg.Model(sh, w, max_context=96)
    orc = oracle.OracleModel(sh, w, 96)
    _check_generation(m, orc, prompt_ids(PROMPT_SEEDS["tiny"], 32, sh.vocab), 16, "qwen3 2L")
    m.close()


def test_generate_continues_step_and_step2(mini_w):
    """generate, step, generate, step2 and step interleaved give the step loop's tokens."""
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=64)
    prompt = prompt_ids(7, 12, MINI.vocab)
    announce("mini interleaved: step loop")
    ref = [m.prefill(prompt)] + [m.step() for _ in range(14)]
    announce("mini interleaved: generate / step / step2")
    m.reset()
    got = [m.prefill(prompt)]
    got += m.generate(4)
    got.append(m.step())
    got += m.generate(3)
    (t0, t1), n = m.step2(ref[len(got) + 1])     # a draft that is the greedy token: accepted
    assert n == 2 and (t0, t1) == (ref[len(got)], ref[len(got) + 1])
    got += [t0, t1]
    (t0, _), n = m.step2((ref[len(got) + 1] + 1) % MINI.vocab)   # rejected
    assert n == 1 and t0 == ref[len(got)]
    got.append(t0)
    got += m.generate(14 + 1 - len(got))
    assert got == ref
    assert m.position == len(prompt) + 14
    m.close()


def test_generate_error_paths(mini_w):
    import weight_streaming_gemv_amd as wsg
    abi = wsg._abi
    m = wsg.Model(MINI, mini_w, max_context=32)
    with pytest.raises(wsg.WsgError) as e:
        m.generate(3)                               # nothing generated yet
    assert e.value.status == abi.WSG_ERR_STATE
    prompt = prompt_ids(3, 20, MINI.vocab)
    announce("mini generate errors")
    m.prefill(prompt)
    assert m.generate(0) == [] and m.position == 20
    with pytest.raises(wsg.WsgError) as e:
        m.generate(-1)
    assert e.value.status == abi.WSG_ERR_INVALID_ARG
    with pytest.raises(wsg.WsgError) as e:
        m.generate(13)                              # 20 + 13 > 32
    assert e.value.status == abi.WSG_ERR_OUT_OF_RANGE and m.position == 20
    m.set_option(abi.WSG_OPT_TIMED_STAGE, 4)
    with pytest.raises(wsg.WsgError) as e:
        m.generate(2)
    assert e.value.status == abi.WSG_ERR_STATE and m.position == 20
    m.set_option(abi.WSG_OPT_TIMED_STAGE, -1)
    toks = m.generate(12)                           # exactly to capacity
    assert len(toks) == 12 and m.position == 32
    m.reset()
    m.prefill(prompt)
    assert [m.step() for _ in range(12)] == toks
    m.close()
