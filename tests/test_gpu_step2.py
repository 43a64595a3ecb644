"""Two-token step (the verify pass of greedy speculative decoding) vs the oracle.

Row 0 of a step consumes the last token at position p, row 1 a draft at
p + 1; each weight matrix is streamed once for both rows ("Our Kernel
Benchmark Was Measuring the System Cache", "Why it mattered, concretely").
The oracle runs the two rows as two single-row forwards, which the pages'
row-by-row recipe makes the same computation (Megakernels, "GPU-wide
end-to-end generation").  Checked per step: both rows' full-vocabulary
logits (rtol=atol=1e-3 FP32, 2e-2 FP16), the exact greedy tokens (FP32), the
acceptance rule, and both new K/V slots of every layer; the emitted stream
equals plain greedy generation.
"""
import numpy as np
import pytest

from gpu_util import Checker, _np, announce, close_rel, gpu_available
import oracle
from synth import MINI, QWEN3_0_6B, ModelShape, model_weights, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# accept (1) / reject (0) schedule of the drafts; starting anywhere, the
# rejections make every position p the first row of some step
SCHEDULE = [0, 0, 1, 0, 1, 1, 0, 0, 1, 0, 0, 1]


def _f16(w):
    return {"embed": w["embed"].astype(np.float16), "final_norm": w["final_norm"].astype(np.float16),
            "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in w["layers"]]}


def _kv_slots(m, orc, lo, hi, ck, label):
    """Cache slots [lo, hi) of every layer (a rejected draft's slot included)."""
    for l in range(orc.shape.n_layers):
        k, v, _ = m.kv(l)
        for got, ref, nm in ((k, orc.k_cache[l], "K"), (v, orc.v_cache[l], "V")):
            ok, err, worst = close_rel(_np(got[:, lo:hi]), ref[:, lo:hi], ck.rtol, ck.atol)
            ck.max_kv_err = max(ck.max_kv_err, err)
            assert ok, f"{label}: layer {l} {nm}[{lo}:{hi}] off by {err:.3e}"


def spec_lockstep(m, orc, prompt, schedule, rtol=1e-3, atol=1e-3, exact=True, label=""):
    """Prefill, then one two-token step per schedule entry, the draft being the
    oracle's greedy token of row 0 (accept) or another id (reject).  Returns
    the emitted GPU tokens and the first-row positions visited."""
    V = orc.shape.vocab
    ck = Checker(m, orc, rtol, atol, label)
    m.reset()
    orc.reset()
    announce(f"{label}: prefill {len(prompt)} rows")
    tok = m.prefill(prompt)
    ref = orc.forward_rows(prompt)
    ck.logits(ref, 0)
    if exact:
        assert tok == oracle.argmax_lowest(ref), f"{label}: first token"
    emitted, visited = [tok], []
    for s, acc in enumerate(schedule, 1):
        p = orc.pos
        assert m.position == p
        visited.append(p)
        in0 = emitted[-1]
        ref0 = orc.forward_rows([in0])
        g0 = oracle.argmax_lowest(ref0)
        draft = g0 if acc else (g0 + 1 + s) % V
        announce(f"{label}: step {s} p={p} draft={'accept' if acc else 'reject'}")
        (t0, t1), n = m.step2(draft)                    # row 0 takes the last output
        ref1 = orc.forward_rows([draft])
        g1 = oracle.argmax_lowest(ref1)
        got = _np(m.logits())
        assert got.shape == (2, V)
        for row, r in ((0, ref0), (1, ref1)):
            ok, err, worst = close_rel(got[row], r, rtol, atol)
            ck.max_logit_err = max(ck.max_logit_err, err)
            assert ok, f"{label} step {s} row {row}: logits off by {err:.3e} at {worst}"
        _kv_slots(m, orc, p, p + 2, ck, f"{label} step {s}")
        if exact:
            assert t0 == g0, f"{label} step {s}: row 0 token {t0} != {g0} (margin {orc.logits_margin(ref0):.3e})"
            assert t1 == g1, f"{label} step {s}: row 1 token {t1} != {g1} (margin {orc.logits_margin(ref1):.3e})"
        assert n == (2 if t0 == draft else 1)
        if n == 2:
            emitted += [t0, t1]
        else:
            emitted.append(t0)
            orc.pos = p + 1          # the rejected draft's slot is rewritten next
        assert m.position == orc.pos
    return emitted, visited, ck


@pytest.fixture(scope="module")
def mini_w():
    return model_weights(MINI, seed=0)


@pytest.mark.parametrize("fuse,n_prompt", [(1, 9), (0, 9), (0, 58), (1, 58), (1, 120), (1, 187), (0, 187)])
def test_mini_step2_lockstep(mini_w, fuse, n_prompt):
    """Fused attention + output projection (contexts up to 128 keys) and the
    split-K launches; prompts of 58 and 187 ids make some step's rows straddle a
    64-key split boundary (first row at 63 or 191), 120 crosses the fused limit."""
    import weight_streaming_gemv_amd as wsg
    cap = 224
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_option(wsg._abi.WSG_OPT_FUSE_ATTN_O, fuse)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(40 + n_prompt, n_prompt, MINI.vocab)
    emitted, visited, ck = spec_lockstep(m, orc, prompt, SCHEDULE, label=f"mini step2 fuse={fuse} n={n_prompt}")
    if n_prompt == 58:
        assert 63 in visited
    if n_prompt == 187:
        assert 191 in visited
    ck.kv(0, orc.pos, len(SCHEDULE) + 1)
    print(f"fuse={fuse} n={n_prompt}: {len(emitted)} tokens, max |dlogit| {ck.max_logit_err:.2e}")
    m.close()


def test_qwen3x2_step2_lockstep():
    """The Qwen3-0.6B layer widths (2 layers): 8 KV heads, so the gate/up prologue
    sums 2 x 8 partial vectors."""
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    w = model_weights(sh, seed=0)
    cap = 48
    m = wsg.Model(sh, w, max_context=cap, prefill_chunk=16)
    orc = oracle.OracleModel(sh, w, cap)
    prompt = prompt_ids(41, 13, sh.vocab)
    emitted, _, ck = spec_lockstep(m, orc, prompt, SCHEDULE, label="qwen3x2 step2")
    print(f"qwen3x2: {len(emitted)} tokens, max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


VARIANTS = {
    "g1_h512": ModelShape(n_layers=2, hidden=512, intermediate=1024, n_q_heads=4, n_kv_heads=4,
                          head_dim=128, vocab=777),
    "g4_h1024": ModelShape(n_layers=2, hidden=1024, intermediate=2048, n_q_heads=8, n_kv_heads=2,
                           head_dim=128, vocab=1500),
    # two partial vectors per thread per row: 4 KV heads still fuse, 16 do not
    "g1_h2048": ModelShape(n_layers=1, hidden=2048, intermediate=1024, n_q_heads=16, n_kv_heads=16,
                           head_dim=128, vocab=640),
    "g4_h2048": ModelShape(n_layers=1, hidden=2048, intermediate=1024, n_q_heads=16, n_kv_heads=4,
                           head_dim=128, vocab=640),
    "g4_h3072": ModelShape(n_layers=1, hidden=3072, intermediate=3072, n_q_heads=24, n_kv_heads=6,
                           head_dim=128, vocab=999),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_step2_shape_variants(name, dtype):
    import weight_streaming_gemv_amd as wsg
    sh = VARIANTS[name]
    w = model_weights(sh, seed=6)
    if dtype == "f16":
        w = _f16(w)
    cap = 96
    m = wsg.Model(sh, w, max_context=cap, dtype=wsg.WSG_F32 if dtype == "f32" else wsg.WSG_F16)
    orc = oracle.OracleModel(sh, w, cap)
    tol = 1e-3 if dtype == "f32" else 2e-2
    prompt = prompt_ids(42, 60, sh.vocab)
    _, _, ck = spec_lockstep(m, orc, prompt, SCHEDULE[:8], rtol=tol, atol=tol, exact=(dtype == "f32"),
                             label=f"{name} {dtype} step2")
    print(f"{name} {dtype}: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_speculative_stream_equals_greedy(mini_w):
    """Speculative decoding with any drafts emits exactly the greedy stream: drafts
    taken from a previous greedy run with every third one corrupted."""
    import weight_streaming_gemv_amd as wsg
    cap = 96
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=32)
    prompt = prompt_ids(43, 21, MINI.vocab)
    n_out = 40
    greedy = [m.prefill(prompt)] + [m.step() for _ in range(n_out - 1)]
    m.reset()
    out = [m.prefill(prompt)]
    k = 0
    while len(out) < n_out:
        i = len(out)                     # index of the draft in the greedy stream
        draft = greedy[i] if k % 3 else (greedy[i] + 7) % MINI.vocab
        k += 1
        (t0, t1), n = m.step2(draft)
        out += [t0, t1][:n]
    assert out[:n_out] == greedy
    orc = oracle.OracleModel(MINI, mini_w, cap)
    assert greedy == orc.generate(prompt, n_out)
    m.close()


def test_step2_then_step_and_teacher_forced_input(mini_w):
    """An explicit row-0 input overrides the last output; a plain step continues
    from the last emitted token after either outcome."""
    import weight_streaming_gemv_amd as wsg
    cap = 48
    m = wsg.Model(MINI, mini_w, max_context=cap)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(44, 7, MINI.vocab)
    m.prefill(prompt)
    orc.forward_rows(prompt)
    forced = 123
    ref0 = orc.forward_rows([forced])
    g0 = oracle.argmax_lowest(ref0)
    (t0, _), n = m.step2((g0 + 1) % MINI.vocab, in_token=forced)   # rejected
    assert (t0, n) == (g0, 1)
    ok, err, _ = close_rel(_np(m.logits())[0], ref0, 1e-3, 1e-3)
    assert ok, err
    tok = m.step()                                   # consumes t0 at slot 8
    ref = orc.forward_rows([t0])
    assert tok == oracle.argmax_lowest(ref)
    ok, err, _ = close_rel(_np(m.logits()), ref, 1e-3, 1e-3)
    assert ok, err
    assert m.position == orc.pos == 9
    m.close()


def test_step2_error_paths(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=10)
    with pytest.raises(wsg.WsgError, match="STATE"):
        m.step2(5)
    m.prefill([1, 2, 3, 4, 5, 6, 7, 8])
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step2(MINI.vocab)
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step2(-1)
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step2(3, in_token=MINI.vocab)
    assert m.position == 8
    m.step2(3)                                       # slots 8 and 9: the last two
    m.rewind(9)
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step2(3)                                   # would need slot 10
    m.close()


def _two(opts):
    import weight_streaming_gemv_amd as wsg
    a = wsg._abi
    names = {"head_rows": a.WSG_OPT_ROWS["head"], "head_waves": a.WSG_OPT_HEAD_WAVES, "qkv_rows": a.WSG_OPT_ROWS["qkv"],
             "gu_rows": a.WSG_OPT_ROWS["gateup"], "down_rows": a.WSG_OPT_ROWS["down"], "o_rows": a.WSG_OPT_ROWS["o"],
             "head_grid": a.WSG_OPT_GRID["head"], "gu_grid": a.WSG_OPT_GRID["gateup"],
             "attn_o_rows": a.WSG_OPT_ROWS_ATTN_O, "fuse": a.WSG_OPT_FUSE_ATTN_O}
    return [(a.WSG_OPT_FOR_TWO_TOKEN | names[k], v) for k, v in opts.items()]


@pytest.mark.parametrize("opts", [
    {"head_rows": 1}, {"head_rows": 2, "head_waves": 8}, {"head_waves": 16, "head_rows": 1},
    {"qkv_rows": 4, "gu_rows": 2, "down_rows": 4}, {"head_grid": 64, "gu_grid": 40},
    {"attn_o_rows": 4}, {"fuse": 0, "o_rows": 2}])
def test_step2_launch_shapes(mini_w, opts):
    """Two-token launch shapes (set with WSG_OPT_FOR_TWO_TOKEN) all match the oracle;
    single-token steps keep their own shape (bit-identical before and after)."""
    import weight_streaming_gemv_amd as wsg
    cap = 96
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=32)
    prompt = prompt_ids(45, 30, MINI.vocab)
    m.prefill(prompt)
    m.step()
    before = _np(m.logits())
    for k, v in _two(opts):
        m.set_option(k, v)
    m.rewind(30)
    m.step()
    assert np.array_equal(_np(m.logits()), before)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    spec_lockstep(m, orc, prompt, SCHEDULE[:6], label=f"mini step2 {opts}")
    m.close()


def test_two_token_option_checks(mini_w):
    import weight_streaming_gemv_amd as wsg
    a = wsg._abi
    m = wsg.Model(MINI, mini_w, max_context=8)
    for opt, bad in ((a.WSG_OPT_ROWS["head"], 3), (a.WSG_OPT_HEAD_WAVES, 2), (a.WSG_OPT_FUSE_ATTN_O, 2),
                     (a.WSG_OPT_GRID["qkv"], -1)):
        with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
            m.set_option(a.WSG_OPT_FOR_TWO_TOKEN | opt, bad)
    for opt in (a.WSG_OPT_USE_GRAPH, a.WSG_OPT_TIMED_STAGE, 99):   # model-wide or unknown
        with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
            m.set_option(a.WSG_OPT_FOR_TWO_TOKEN | opt, 0)
    m.close()
