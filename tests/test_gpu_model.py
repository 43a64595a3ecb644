"""GPU decode path vs the oracle, through the C ABI, in lockstep.

Per step (Benchmark methodology, "Long-document chunked prefill";
Megakernels, "GPU-wide end-to-end generation"): full-vocabulary logits
within rtol=atol=1e-3 (FP32), the exact greedy token, and the newly written
K/V slot of every layer; the whole valid K/V prefix at the first output and
at the end.  FP16 storage is checked teacher-forced at rtol=atol=2e-2.
"""
import numpy as np
import pytest

from gpu_util import _np, announce, close_rel, gpu_available, lockstep
import oracle
from synth import MINI, PROMPT_SEEDS, QWEN3_0_6B, ModelShape, model_weights, model_weights_bf16, prompt_ids

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


@pytest.mark.parametrize("fuse,rows", [(0, 8), (1, 8), (1, 4)])
def test_mini_fused_attention_output(mini_w, fuse, rows):
    """Attention fused with the output projection (KV-head partials summed by
    the gate/up launch) and the separate launches both match the oracle, and
    give the same tokens; contexts cross one attention split (64 keys) and the
    fused limit (128 keys)."""
    import weight_streaming_gemv_amd as wsg
    cap = 160
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_option(wsg._abi.WSG_OPT_FUSE_ATTN_O, fuse)
    m.set_option(wsg._abi.WSG_OPT_ROWS_ATTN_O, rows)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(21, 58, MINI.vocab)
    lockstep(m, orc, prompt, 12, label=f"mini fuse={fuse} rows={rows} short")
    prompt = prompt_ids(21, 120, MINI.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 12, label=f"mini fuse={fuse} rows={rows}")
    print(f"fuse={fuse} rows={rows}: max |dlogit| {ck.max_logit_err:.2e}")
    m.close()


@pytest.mark.parametrize("split", [2, 4])
@pytest.mark.parametrize("graph", [1, 0])
def test_mini_split_down(mini_w, split, graph):
    """The down projection in K slices summed by the next layer's QKV launch: lockstep
    against the oracle (contexts within and past the fused attention limit), and the same
    tokens as the whole projection."""
    import weight_streaming_gemv_amd as wsg
    cap = 160
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_option(wsg._abi.WSG_OPT_USE_GRAPH, graph)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(23, 120, MINI.vocab)
    ref_toks, _, _ = lockstep(m, orc, prompt, 12, label="mini split=1")
    m.set_option(wsg._abi.WSG_OPT_SPLIT_DOWN, split)
    assert m.describe()["one_token"]["down_k_slices"] == split
    toks, _, ck = lockstep(m, orc, prompt, 12, label=f"mini split={split} graph={graph}")
    assert toks == ref_toks
    m.close()


@pytest.mark.parametrize("split", [2, 4])
def test_qwen3_2layer_split_down(split):
    """The Qwen3-shaped down projection (K = 3072) in 2 and 4 slices: one- and two-token
    steps in lockstep."""
    import weight_streaming_gemv_amd as wsg
    from gpu_util import Checker
    sh = QWEN3_0_6B.with_layers(2)
    w = model_weights(sh, seed=0)
    cap = 64
    m = wsg.Model(sh, w, max_context=cap, prefill_chunk=32)
    for opt in (wsg._abi.WSG_OPT_SPLIT_DOWN, wsg._abi.WSG_OPT_SPLIT_DOWN | wsg._abi.WSG_OPT_FOR_TWO_TOKEN):
        m.set_option(opt, split)
    orc = oracle.OracleModel(sh, w, cap)
    prompt = prompt_ids(PROMPT_SEEDS["short"], 32, sh.vocab)
    toks, _, _ = lockstep(m, orc, prompt, 6, label=f"qwen3-2L split={split}")
    ck = Checker(m, orc, 1e-3, 1e-3, f"qwen3-2L split={split} step2")
    last = toks[-1]
    for s_, accept in enumerate((True, False)):
        p = orc.pos
        ref0 = orc.forward_rows([last])
        g0 = oracle.argmax_lowest(ref0)
        draft = g0 if accept else (g0 + 1) % sh.vocab
        announce(f"qwen3-2L split={split} step2 {s_}")
        (t0, t1), n = m.step2(draft)
        ref1 = orc.forward_rows([draft])
        got = _np(m.logits())
        for row, r in ((0, ref0), (1, ref1)):
            ok, err, worst = close_rel(got[row], r, 1e-3, 1e-3)
            assert ok, f"step2 {s_} row {row}: logits off by {err:.3e}"
        assert t0 == g0 and n == (2 if accept else 1)
        if accept:
            assert t1 == oracle.argmax_lowest(ref1)
            ck.kv(p, p + 2, s_)
            last = t1
        else:
            orc.pos = p + 1
            ck.kv(p, p + 1, s_)
            last = t0
    m.close()


@pytest.mark.parametrize("shape_name", ["mini", "qwen3-2L"])
def test_fp16_split_down(shape_name, mini_w):
    """FP16 storage with the down projection in 2 slices: teacher-forced within the FP16
    tolerance (4 slices do not hold whole 512-element FP16 lane vectors at these widths,
    so the projection then runs whole)."""
    import weight_streaming_gemv_amd as wsg
    sh = MINI if shape_name == "mini" else QWEN3_0_6B.with_layers(2)
    w = mini_w if shape_name == "mini" else model_weights(sh, seed=0)
    w16 = {"embed": w["embed"].astype(np.float16), "final_norm": w["final_norm"].astype(np.float16),
           "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in w["layers"]]}
    m = wsg.Model(sh, w16, max_context=32, dtype=wsg.WSG_F16)
    m.set_option(wsg._abi.WSG_OPT_SPLIT_DOWN, 2)
    assert m.describe()["one_token"]["down_k_slices"] == 2
    orc = oracle.OracleModel(sh, w16, 32)
    lockstep(m, orc, prompt_ids(PROMPT_SEEDS["tiny"], 8, sh.vocab), 6, rtol=2e-2, atol=2e-2, teacher=True,
             label=f"{shape_name} fp16 split=2")
    m.set_option(wsg._abi.WSG_OPT_SPLIT_DOWN, 4)
    assert m.describe()["one_token"]["down_k_slices"] == 1
    m.close()


def test_fused_option_checks(mini_w):
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=8)
    for opt, bad in ((wsg._abi.WSG_OPT_FUSE_ATTN_O, 2), (wsg._abi.WSG_OPT_ROWS_ATTN_O, 2),
                     (wsg._abi.WSG_OPT_ROWS_ATTN_O, 16), (wsg._abi.WSG_OPT_SPLIT_DOWN, 3)):
        with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
            m.set_option(opt, bad)
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


@pytest.mark.parametrize("n_prompt", [600, 1000])
def test_mini_many_splits(mini_w, n_prompt):
    """Many attention splits (16 and 16 to 17 per KV head at 64 keys each),
    reached through chunked prefill."""
    import weight_streaming_gemv_amd as wsg
    cap = 1100
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=128)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(10, n_prompt, MINI.vocab)
    lockstep(m, orc, prompt, 5, label=f"mini splits n={n_prompt}")
    m.close()


# Eight KV heads (one query head each) on a narrow residual: the attention
# split size grows with the context once 24 splits per KV head would not
# cover it (more than 1536 keys), at a cost the oracle finishes in seconds.
WIDE_KV = ModelShape(n_layers=1, hidden=256, intermediate=512, n_q_heads=8, n_kv_heads=8, head_dim=128, vocab=500)


def _split_keys(n_keys, n_kv, cap):
    """Keys per split-K attention block the runtime picks for a context of n_keys (its
    documented rule: about 256 blocks over all KV heads, at least 64 keys and enough that
    the capacity needs at most 128 splits, rounded up a ladder of four sizes per doubling),
    so each case below states which block size it reaches."""
    least = max(64, (-(-cap // 128) + 15) // 16 * 16)
    need = max(least, -(-n_keys // max(1, 256 // n_kv)))
    c, e = 64, 0
    while c < need:
        base = 64 << (e // 4)
        c = base + (base // 4) * (e % 4 + 1)
        e += 1
    return c


def _split_lockstep(sh, w, cap, chunk, n_prompt, label):
    """Greedy steps in lockstep after a chunked prefill, then two two-token steps (an
    accepted and a rejected draft), each row's logits and both new K/V slots of every
    layer against the oracle."""
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(sh, w, max_context=cap, prefill_chunk=chunk)
    orc = oracle.OracleModel(sh, w, cap)
    prompt = prompt_ids(11, n_prompt, sh.vocab)
    toks, _, _ = lockstep(m, orc, prompt, 4, label=label)
    last = toks[-1]
    for s, accept in enumerate((True, False)):
        p = orc.pos
        ref0 = orc.forward_rows([last])
        g0 = oracle.argmax_lowest(ref0)
        draft = g0 if accept else (g0 + 1) % sh.vocab
        announce(f"{label} step2 {s} p={p}")
        (t0, t1), n = m.step2(draft)
        ref1 = orc.forward_rows([draft])
        got = _np(m.logits())
        for row, r in ((0, ref0), (1, ref1)):
            ok, err, worst = close_rel(got[row], r, 1e-3, 1e-3)
            assert ok, f"{label} step2 {s} row {row}: logits off by {err:.3e} at {worst}"
        for l in range(sh.n_layers):
            k, v, _ = m.kv(l)
            for g_, r_ in ((k, orc.k_cache[l]), (v, orc.v_cache[l])):
                ok, err, _ = close_rel(_np(g_[:, p:p + 2]), r_[:, p:p + 2], 1e-3, 1e-3)
                assert ok, f"{label} step2 {s}: layer {l} K/V off by {err:.3e}"
        assert t0 == g0 and n == (2 if accept else 1)
        if accept:
            assert t1 == oracle.argmax_lowest(ref1)
            last = t1
        else:
            orc.pos = p + 1
            last = t0
    m.close()


@pytest.mark.parametrize("n_prompt,keys", [(2100, 80), (3300, 112), (3600, 128), (4700, 160), (5100, 160)])
def test_long_context_split_sizes(n_prompt, keys):
    """Contexts whose split-K attention blocks take 80 keys (2100: each key-row
    folds a whole group of four keys, then a partial one), 112 keys (3300: a
    whole group and three keys), 128 keys (3600: two whole groups) and 160 keys
    (4700 and 5100, the size of the long-document generation past 4096 keys: two
    whole groups and a partial one; 5100 keys take 32 splits per head, 256
    blocks); greedy steps in lockstep, then two-token steps (an accepted and a
    rejected draft) at the same context."""
    cap = 5120
    assert _split_keys(n_prompt + 1, WIDE_KV.n_kv_heads, cap) == keys
    assert _split_keys(n_prompt + 7, WIDE_KV.n_kv_heads, cap) == keys
    _split_lockstep(WIDE_KV, model_weights(WIDE_KV, seed=3), cap, 512, n_prompt, f"wide-kv n={n_prompt}")


def test_stage_timing_inside_graphs(mini_w):
    """A per-layer stage timed in graph mode: step graphs carry event-record nodes around
    that stage's launches (one pair per layer), the accumulated time covers one launch per
    layer and step, and the results are the untimed graphs' bit for bit."""
    import weight_streaming_gemv_amd as wsg
    A = wsg._abi
    m = wsg.Model(MINI, mini_w, max_context=64, prefill_chunk=16)
    prompt = prompt_ids(41, 10, MINI.vocab)
    ref = [m.prefill(prompt)] + [m.step() for _ in range(5)]
    ref_logits = _np(m.logits()).copy()
    for stage in (A.WSG_STAGE_QKV, A.WSG_STAGE_ATTN, A.WSG_STAGE_GATEUP, A.WSG_STAGE_DOWN):
        m.set_option(A.WSG_OPT_TIMED_STAGE, stage)
        m.reset()
        toks = [m.prefill(prompt)] + [m.step() for _ in range(5)]
        ms, n, b = m.stage_time()
        assert toks == ref and np.array_equal(_np(m.logits()), ref_logits)
        assert n == 5 * MINI.n_layers and ms > 0 and b > 0, (stage, ms, n, b)
        assert 0.5 < ms * 1e3 / n < 1000, (stage, ms, n)       # microseconds per launch
    m.set_option(A.WSG_OPT_TIMED_STAGE, -1)
    m.close()


@pytest.mark.parametrize("n_prompt", [10, 150])
def test_time_stage_leaves_the_sequence_alone(mini_w, n_prompt):
    """wsg_time_stage between steps: positive times and weight bytes for every per-layer
    stage at the next step's context (fused attention at 11 keys, split attention with a
    merging output projection at 151), and the generation continues bit for bit as if no
    stage had been timed."""
    import weight_streaming_gemv_amd as wsg
    A = wsg._abi
    m = wsg.Model(MINI, mini_w, max_context=192, prefill_chunk=64)
    with pytest.raises(wsg.WsgError, match="STATE"):
        m.time_stage(A.WSG_STAGE_GATEUP)
    prompt = prompt_ids(42, n_prompt, MINI.vocab)
    ref = [m.prefill(prompt)] + [m.step() for _ in range(4)]
    ref_logits = _np(m.logits()).copy()
    m.reset()
    toks = [m.prefill(prompt)]
    for stage in (A.WSG_STAGE_QKV, A.WSG_STAGE_ATTN, A.WSG_STAGE_GATEUP, A.WSG_STAGE_DOWN):
        # a difference of whole replays: a few-microsecond stage of a 2-layer model is
        # within the replay noise, so only its magnitude is checked
        us, b = m.time_stage(stage, reps=5)
        assert np.isfinite(us) and abs(us) < 1000 and b > 0, (stage, us, b)
    if n_prompt < 128:
        with pytest.raises(wsg.WsgError, match="UNSUPPORTED"):   # fused into the attention launch
            m.time_stage(A.WSG_STAGE_O)
    else:
        us, b = m.time_stage(A.WSG_STAGE_O, reps=3)
        assert b == MINI.hidden * MINI.q_width * 4
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        m.time_stage(A.WSG_STAGE_HEAD)
    toks += [m.step() for _ in range(4)]
    assert toks == ref and np.array_equal(_np(m.logits()), ref_logits)
    m.close()


def test_describe_reports_launch_shapes(mini_w):
    """wsg_describe: the launch shapes a report records, consistent with the split rule the
    long-context tests rely on."""
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(WIDE_KV, model_weights(WIDE_KV, seed=3), max_context=5120, prefill_chunk=512)
    d = m.describe()
    assert d["one_token"]["rows_per_wave"]["head"] == 2 and d["two_token"]["rows_per_wave"]["head"] == 4
    assert d["prefill_chunk"] == 512 and d["graphs"] is True
    for e in d["attention"]["at_keys"]:
        assert e["mode"] == ("fused" if e["keys"] <= 128 else "split+merge_o"), e
        if e["keys"] > 128:
            assert e["keys_per_split"] == _split_keys(e["keys"], WIDE_KV.n_kv_heads, 5120), e
            assert e["splits"] == -(-e["keys"] // e["keys_per_split"]), e
    m.close()


def test_long_context_160_key_splits_qwen3_2layer():
    """The real head geometry (16 query heads on 8 KV heads, two query heads per split
    block) at 4.7k keys, where the attention blocks take 160 keys (30 splits per head),
    through a chunk-1024 prefill (five chunks, the last one partial)."""
    sh = QWEN3_0_6B.with_layers(2)
    cap, n_prompt = 4736, 4700
    assert _split_keys(n_prompt + 1, sh.n_kv_heads, cap) == 160
    _split_lockstep(sh, model_weights(sh, seed=0), cap, 1024, n_prompt, "qwen3-2L n=4700")


def test_graph_cache_eviction(mini_w):
    """More step graphs than the cache keeps (64): 68 positions whose contexts need
    68 different split counts; steps replayed after their graphs were evicted and
    captured again return the same bits."""
    import weight_streaming_gemv_amd as wsg
    cap = 4608
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=512)
    prompt = prompt_ids(12, 4500, MINI.vocab)
    m.prefill(prompt)
    # rewinding only goes back: visit from the longest context down (70 .. 3
    # splits of 64 keys); each step reads prefill-written keys below its slot
    positions = [130 + 64 * i for i in range(67, -1, -1)]
    first = {}
    for p in positions:
        m.rewind(p)
        m.step()
        first[p] = _np(m.logits()).copy()
    # the first four graphs were evicted; the last two are still cached
    m.reset()
    m.prefill(prompt)
    for p in positions[:4] + positions[-2:]:
        m.rewind(p)
        m.step()
        assert np.array_equal(_np(m.logits()), first[p]), f"position {p}"
    m.close()


def test_rewind_repeats_a_forward(mini_w):
    """Rewinding to slot p and stepping re-processes the recorded token at p: the same
    bits every time (the fixed-slot repeat of the fixed-context harness); rewinding
    further back matches the oracle's forward of the shorter prefix."""
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=64, prefill_chunk=16)
    prompt = prompt_ids(35, 10, MINI.vocab)
    toks = [m.prefill(prompt), m.step()]
    t2 = m.step()
    ref_logits = _np(m.logits())
    k, v, _ = m.kv(1)
    ref_k, ref_v = _np(k[:, 11]), _np(v[:, 11])
    for _ in range(3):
        m.rewind(11)
        assert m.position == 11
        assert m.step() == t2
        assert np.array_equal(_np(m.logits()), ref_logits)
        k, v, _ = m.kv(1)
        assert np.array_equal(_np(k[:, 11]), ref_k) and np.array_equal(_np(v[:, 11]), ref_v)
    m.rewind(5)
    m.step()
    orc = oracle.OracleModel(MINI, mini_w, 64)
    ref = orc.forward_rows(prompt[:6])
    ok, err, _ = close_rel(_np(m.logits()), ref, 1e-3, 1e-3)
    assert ok, err
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        m.rewind(-1)
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.rewind(7)
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


@pytest.mark.parametrize("fuse", [1, 0])
def test_fills_cache_to_capacity(mini_w, fuse):
    """A ragged chunked prefill (33 = 16 + 16 + 1 rows), then steps until the
    last one writes and attends over the final slot (cap - 1): logits, tokens
    and every K/V slot match the oracle; the next step is refused and leaves
    the position and the logits as they were.  Fused attention + output
    projection and the split-K launches."""
    import weight_streaming_gemv_amd as wsg
    cap, n_prompt = 40, 33
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=16)
    m.set_option(wsg._abi.WSG_OPT_FUSE_ATTN_O, fuse)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(77, n_prompt, MINI.vocab)
    lockstep(m, orc, prompt, cap - n_prompt + 1, label=f"mini to capacity fuse={fuse}")
    assert m.position == cap
    logits = _np(m.logits()).copy()
    with pytest.raises(wsg.WsgError, match="OUT_OF_RANGE"):
        m.step()
    assert m.position == cap
    assert np.array_equal(_np(m.logits()), logits)
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


# Query-group sizes 1, 2 and 4 and other widths (each fused row-slice
# reduction shape: 16, 32, 64 and 128 lanes per output row).
VARIANTS = {
    "g1_h512": ModelShape(n_layers=2, hidden=512, intermediate=1024, n_q_heads=4, n_kv_heads=4,
                          head_dim=128, vocab=777),
    "g4_h1024": ModelShape(n_layers=2, hidden=1024, intermediate=2048, n_q_heads=8, n_kv_heads=2,
                           head_dim=128, vocab=1500),
    "g1_h2048": ModelShape(n_layers=1, hidden=2048, intermediate=1024, n_q_heads=16, n_kv_heads=16,
                           head_dim=128, vocab=640),
    "g4_h3072": ModelShape(n_layers=1, hidden=3072, intermediate=3072, n_q_heads=24, n_kv_heads=6,
                           head_dim=128, vocab=999),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_shape_variants(name, dtype):
    import weight_streaming_gemv_amd as wsg
    sh = VARIANTS[name]
    w = model_weights(sh, seed=5)
    if dtype == "f16":
        w = {"embed": w["embed"].astype(np.float16), "final_norm": w["final_norm"].astype(np.float16),
             "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in w["layers"]]}
    cap = 80
    m = wsg.Model(sh, w, max_context=cap, dtype=wsg.WSG_F32 if dtype == "f32" else wsg.WSG_F16)
    orc = oracle.OracleModel(sh, w, cap)
    prompt = prompt_ids(31, 60, sh.vocab)
    tol = 1e-3 if dtype == "f32" else 2e-2
    _, _, ck = lockstep(m, orc, prompt, 8, rtol=tol, atol=tol, teacher=(dtype == "f16"),
                        label=f"{name} {dtype}")
    print(f"{name} {dtype}: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


@pytest.mark.parametrize("name,n_prompt", [("mini", 20), ("mini", 90), ("qwen3x2", 30)])
def test_lossless_packed_decode(name, n_prompt):
    """Packed decode weights (two exact FP32 values per 32-bit word) give bit-identical
    logits, K/V and tokens to the unpacked model, and match the oracle (Megakernels,
    "Lossless decode-weight storage").  90-id prompts reach the split-attention path,
    whose output projection is its own launch."""
    import weight_streaming_gemv_amd as wsg
    sh = MINI if name == "mini" else QWEN3_0_6B.with_layers(2)
    w = model_weights_bf16(sh, seed=0)
    cap = 128
    a = wsg.Model(sh, w, max_context=cap, prefill_chunk=32, lossless_pack=True)
    b = wsg.Model(sh, w, max_context=cap, prefill_chunk=32)
    sa, sb = a.storage(), b.storage()
    assert sa["packed_matrices"] == sa["decode_matrices"] == 1 + 4 * sh.n_layers
    assert sb["packed_matrices"] == 0
    assert sa["decode_weight_bytes"] * 2 == sb["decode_weight_bytes"] == sh.weight_bytes_per_token(4)
    prompt = prompt_ids(33, n_prompt, sh.vocab)
    ta, tb = [a.prefill(prompt)], [b.prefill(prompt)]
    assert np.array_equal(_np(a.logits()), _np(b.logits()))
    for _ in range(6):
        ta.append(a.step())
        tb.append(b.step())
        assert np.array_equal(_np(a.logits()), _np(b.logits()))
    assert ta == tb
    for l in range(sh.n_layers):
        ka, va, na = a.kv(l)
        kb, vb, nb = b.kv(l)
        assert na == nb == n_prompt + 6
        assert np.array_equal(_np(ka[:, :na]), _np(kb[:, :nb])) and np.array_equal(_np(va[:, :na]), _np(vb[:, :nb]))
    b.close()
    orc = oracle.OracleModel(sh, w, cap)
    lockstep(a, orc, prompt, 4, label=f"{name} packed n={n_prompt}")
    a.close()


def test_lossless_pack_ineligible_weights_decode_unpacked(mini_w):
    """lossless_pack on plain FP32 weights: nothing qualifies, the model runs unpacked."""
    import weight_streaming_gemv_amd as wsg
    m = wsg.Model(MINI, mini_w, max_context=32, lossless_pack=True)
    st = m.storage()
    assert st["packed_matrices"] == 0 and st["decode_weight_bytes"] == MINI.weight_bytes_per_token(4)
    orc = oracle.OracleModel(MINI, mini_w, 32)
    lockstep(m, orc, prompt_ids(34, 9, MINI.vocab), 3, label="mini pack-ineligible")
    m.close()
