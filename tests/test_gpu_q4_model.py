"""Int4 (group-64) decoder on the GPU vs the oracle, through the C ABI.

Every decode matrix and the tied embedding are int4 with FP16 group scales
("Our Kernel Benchmark Was Measuring the System Cache", "Summary": 4-bit
decode matrix-vector products); activations, KV cache and logits are FP16
with FP32 accumulation.  The oracle dequantises the same words on the CPU.
Checked per step, teacher-forced: full-vocabulary logits and the new K/V
slot of every layer within rtol=atol=2e-2 (the FP16 tolerance), the whole
valid K/V prefix at the end; single- and two-token steps; contexts past one
attention split.
"""
import numpy as np
import pytest

from gpu_util import _np, announce, close_rel, gpu_available, lockstep
import oracle
from synth import QWEN3_0_6B, ModelShape, model_weights_q4, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = 2e-2
# widths must be multiples of 1024 for int4 rows
Q4MINI = ModelShape(n_layers=2, hidden=1024, intermediate=2048, n_q_heads=8, n_kv_heads=4, head_dim=128,
                    vocab=1000)


@pytest.fixture(scope="module")
def q4mini_w():
    return model_weights_q4(Q4MINI, seed=0)


def _model(wsg, sh, w, cap):
    return wsg.Model(sh, w, max_context=cap, dtype=wsg.WSG_F16)


@pytest.mark.parametrize("n_prompt", [9, 70])
def test_q4_mini_teacher_forced(q4mini_w, n_prompt):
    """70 ids: the context passes one 64-key attention split (split-K + merge)."""
    import weight_streaming_gemv_amd as wsg
    cap = 96
    m = _model(wsg, Q4MINI, q4mini_w, cap)
    st = m.storage()
    assert st["decode_weight_bytes"] == (Q4MINI.vocab * 1024 + 2 * (2048 * 1024 + 1024 * 1024 + 4096 * 1024
                                         + 1024 * 2048)) * (1 / 2 + 1 / 32)
    orc = oracle.OracleModel(Q4MINI, q4mini_w, cap)
    _, _, ck = lockstep(m, orc, prompt_ids(50 + n_prompt, n_prompt, Q4MINI.vocab), 8, rtol=TOL, atol=TOL,
                        teacher=True, label=f"q4 mini n={n_prompt}")
    print(f"q4 mini n={n_prompt}: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_q4_qwen3x2_teacher_forced():
    """The Qwen3-0.6B layer widths (2 layers) with the full 151936-row int4 head."""
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    w = model_weights_q4(sh, seed=0)
    cap = 32
    m = _model(wsg, sh, w, cap)
    orc = oracle.OracleModel(sh, w, cap)
    _, _, ck = lockstep(m, orc, prompt_ids(51, 8, sh.vocab), 8, rtol=TOL, atol=TOL, teacher=True,
                        label="q4 qwen3x2")
    print(f"q4 qwen3x2: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


@pytest.mark.parametrize("opts", [{}, {"rows": 2}, {"rows": 4, "head_waves": 8}, {"grid": 24}])
def test_q4_launch_shapes(q4mini_w, opts):
    """Rows per wave and looping grids of the int4 GEMVs."""
    import weight_streaming_gemv_amd as wsg
    a = wsg._abi
    cap = 32
    m = _model(wsg, Q4MINI, q4mini_w, cap)
    for stage in ("qkv", "o", "gateup", "down", "head"):
        if "rows" in opts:
            m.set_option(a.WSG_OPT_ROWS[stage], opts["rows"])
        if "grid" in opts:
            m.set_option(a.WSG_OPT_GRID[stage], opts["grid"])
    if "head_waves" in opts:
        m.set_option(a.WSG_OPT_HEAD_WAVES, opts["head_waves"])
    orc = oracle.OracleModel(Q4MINI, q4mini_w, cap)
    lockstep(m, orc, prompt_ids(52, 10, Q4MINI.vocab), 5, rtol=TOL, atol=TOL, teacher=True,
             label=f"q4 mini {opts}")
    m.close()


def test_q4_two_token_step(q4mini_w):
    """Two-token steps on int4 weights: both rows' logits and K/V slots vs the oracle."""
    import weight_streaming_gemv_amd as wsg
    cap = 64
    m = _model(wsg, Q4MINI, q4mini_w, cap)
    orc = oracle.OracleModel(Q4MINI, q4mini_w, cap)
    prompt = prompt_ids(53, 11, Q4MINI.vocab)
    tok = m.prefill(prompt)
    ref = orc.forward_rows(prompt)
    ok, err, _ = close_rel(_np(m.logits()), ref, TOL, TOL)
    assert ok, err
    last = tok
    for s in range(6):
        p = orc.pos
        ref0 = orc.forward_rows([last])
        draft = oracle.argmax_lowest(ref0) if s % 2 == 0 else (oracle.argmax_lowest(ref0) + 3) % Q4MINI.vocab
        announce(f"q4 step2 {s} p={p}")
        (t0, t1), n = m.step2(draft)
        ref1 = orc.forward_rows([draft])
        got = _np(m.logits())
        for row, r in ((0, ref0), (1, ref1)):
            ok, err, worst = close_rel(got[row], r, TOL, TOL)
            assert ok, f"step {s} row {row}: logits off by {err:.3e} at {worst}"
        for l in range(Q4MINI.n_layers):
            k, v, _ = m.kv(l)
            for g_, r_ in ((k, orc.k_cache[l]), (v, orc.v_cache[l])):
                ok, err, _ = close_rel(_np(g_[:, p:p + 2]), r_[:, p:p + 2], TOL, TOL)
                assert ok, f"step {s} layer {l}: K/V off by {err:.3e}"
        assert n == (2 if t0 == draft else 1)
        if n == 1:
            orc.pos = p + 1
        last = t1 if n == 2 else t0
    m.close()


Q4_VARIANTS = {
    "g1_h1024": ModelShape(n_layers=2, hidden=1024, intermediate=1024, n_q_heads=8, n_kv_heads=8, head_dim=128,
                           vocab=700),
    "g4_h2048": ModelShape(n_layers=1, hidden=2048, intermediate=3072, n_q_heads=16, n_kv_heads=4, head_dim=128,
                           vocab=900),
}


@pytest.mark.parametrize("name", sorted(Q4_VARIANTS))
@pytest.mark.parametrize("fuse,rows", [(1, 8), (1, 4), (0, 8)])
def test_q4_variants_fused_and_split(name, fuse, rows):
    """Query groups 1 and 4 with the fused attention + int4 output slice (8 or 4 rows
    per wave; group 1 with 4 rows runs the separate launches) and without it; a
    140-id prompt passes the fused limit of 128 keys."""
    import weight_streaming_gemv_amd as wsg
    sh = Q4_VARIANTS[name]
    w = model_weights_q4(sh, seed=7)
    cap = 160
    m = _model(wsg, sh, w, cap)
    m.set_option(wsg._abi.WSG_OPT_FUSE_ATTN_O, fuse)
    m.set_option(wsg._abi.WSG_OPT_ROWS_ATTN_O, rows)
    orc = oracle.OracleModel(sh, w, cap)
    for n_p in (20, 140):
        _, _, ck = lockstep(m, orc, prompt_ids(54 + n_p, n_p, sh.vocab), 6, rtol=TOL, atol=TOL, teacher=True,
                            label=f"q4 {name} fuse={fuse} rows={rows} n={n_p}")
    m.close()


def test_q4_config_errors(q4mini_w):
    import weight_streaming_gemv_amd as wsg
    with pytest.raises(wsg.WsgError, match="UNSUPPORTED"):
        wsg.Model(Q4MINI, q4mini_w, max_context=8, dtype=wsg.WSG_F32)
    with pytest.raises(wsg.WsgError, match="UNSUPPORTED"):
        wsg.Model(Q4MINI, q4mini_w, max_context=8, dtype=wsg.WSG_F16, prefill_chunk=16)
