"""Greedy selection with ties broken by the lowest token id, on the GPU.

The pages choose the next token on the GPU and break ties by the lowest token id
(Megakernels, "GPU-wide end-to-end generation").  Random logits never tie, so the
ties here are planted:

* in logit vectors given to the stand-alone argmax (``wsg_argmax``): at index 0,
  at the last index, inside one wave, across the 4096-logit spans of its first
  launch, an all-equal vector, and signed zeros (-0.0 ties with +0.0);
* in the decode model, through the tied embedding: the head's logit of row i is
  E[i] . h, and the head sums every row in the same order, so rows copied from
  another row give bit-identical logits (copies scaled by 2 give exactly twice
  the logit, which makes them the maximum).  Planted rows are never prompt
  tokens, so the hidden state is unchanged; the oracle, run on the same planted
  weights, confirms that the tie is real and gives the expected token.  Ties sit
  at index 0, at the last vocabulary row, inside one wave's row pair, across a
  head workgroup boundary, inside one pair of block keys of the final argmax
  launch and across its threads, iterations and waves -- for one-token steps,
  both rows of a two-token step, and FP16 storage.
"""
import numpy as np
import pytest

from gpu_util import _np, announce, gpu_available
import oracle
from synth import MINI, QWEN3_0_6B, model_weights, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


# ------------------------------------------------------------ stand-alone argmax
def _gpu_argmax(vecs, dtype):
    import torch
    import weight_streaming_gemv_amd as wsg
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(vecs, dtype=dtype))).to("cuda")
    out = wsg.argmax(t)
    torch.cuda.synchronize()
    return out.cpu().numpy().tolist()


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
@pytest.mark.parametrize("n", [1, 2, 63, 4095, 4096, 4097, 151936, 1_000_003])
def test_argmax_random_rows(dtype, n):
    rng = np.random.default_rng(n)
    rows = rng.standard_normal((3, n)).astype(dtype)
    announce(f"argmax random {np.dtype(dtype).name} n={n}")
    got = _gpu_argmax(rows, dtype)
    assert got == [oracle.argmax_lowest(r) for r in rows]


def _planted_cases(n):
    """(label, vector, expected index) with exact ties at the maximum."""
    rng = np.random.default_rng(7)
    base = lambda: rng.uniform(-4.0, 4.0, n)   # noqa: E731
    cases = []

    def tie(label, idx, value=10.0):
        v = base()
        v[list(idx)] = value
        cases.append((label, v, min(idx)))

    tie("index 0 and the last index", [0, n - 1])
    tie("same wave (lanes 5 and 37)", [37, 5])
    tie("span boundary", [4096, 4095])
    tie("three spans", [2 * 4096 + 17, 4096 + 3, n - 2])
    tie("far apart", [n - 1, 123_457])
    v = base()
    v[n - 1] = 10.0
    cases.append(("unique maximum at the last index", v, n - 1))
    cases.append(("all equal", np.full(n, 0.5), 0))
    v = -np.abs(base()) - 1.0
    v[9000], v[70_000] = -0.0, 0.0
    cases.append(("-0.0 before +0.0", v, 9000))
    v = -np.abs(base()) - 1.0
    v[9000], v[70_000] = 0.0, -0.0
    cases.append(("+0.0 before -0.0", v, 9000))
    v = -np.abs(base()) - 1.0
    v[4097] = -0.0
    cases.append(("only -0.0", v, 4097))
    v = np.full(n, -60000.0)
    v[55_555] = -59968.0
    cases.append(("large negative values, one a step above", v, 55_555))
    return cases


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_argmax_planted_ties(dtype):
    n = 151936
    cases = _planted_cases(n)
    vecs = np.stack([np.asarray(c[1], dtype=dtype) for c in cases])
    for (label, v, want), row in zip(cases, vecs):
        assert oracle.argmax_lowest(row) == want, label            # the cases themselves
    announce(f"argmax planted ties {np.dtype(dtype).name}: {len(cases)} rows")
    got = _gpu_argmax(vecs, dtype)
    for (label, _, want), g in zip(cases, got):
        assert g == want, f"{label}: got {g}, want {want}"


def test_argmax_rejects_bad_arguments():
    import torch
    import weight_streaming_gemv_amd as wsg
    from weight_streaming_gemv_amd import _abi
    L = _abi.lib()
    lg = torch.zeros(8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(64, dtype=torch.uint8, device="cuda")
    assert L.wsg_argmax(0, 1, 8, lg.data_ptr(), out.data_ptr(), ws.data_ptr(), 4, None) == _abi.WSG_ERR_INVALID_ARG
    assert b"workspace" in L.wsg_last_error()
    assert L.wsg_argmax(0, 1, 8, lg.data_ptr() + 2, out.data_ptr(), ws.data_ptr(), 64, None) == _abi.WSG_ERR_INVALID_ARG
    assert L.wsg_argmax(0, 1, 8, lg.data_ptr(), out.data_ptr(), ws.data_ptr() + 4, 64, None) == _abi.WSG_ERR_INVALID_ARG
    assert wsg.argmax(lg).cpu().tolist() == [0]


# ------------------------------------------------------------- decode model
def _planted_weights(w, rows, src, factor):
    """Weights whose embedding rows `rows` are factor * E[src] (exact: factor 1 or 2)."""
    E = w["embed"].copy()
    E[list(rows)] = E[src] * E.dtype.type(factor)
    return {**w, "embed": E}


def _expect_tie(orc_logits, rows, want):
    """The planted rows are exactly the maximal logits (bit-identical; a single planted row
    is the unique maximum), and the lowest of them is `want`."""
    v = np.asarray(orc_logits)
    top = np.flatnonzero(v == v.max())
    assert set(rows) == set(top.tolist()), (top[:8], rows)
    assert oracle.argmax_lowest(v) == want


def _head_cases(V):
    """(label, planted rows, factor).  The head runs two rows per wave and four waves per
    workgroup (eight rows per block of 256 threads, one-shot grid); the final argmax
    launch reads the block keys in pairs (blocks 2i, 2i+1), pair i + 1024 k on thread i."""
    return [
        ("index 0 (copy of the winner)", [0], 1),
        ("unique maximum at the last row (doubled winner)", [V - 1], 2),
        ("one wave's row pair", [V // 2 + 1, V // 2], 2),
        ("across a head workgroup boundary", [8 * 125 + 8, 8 * 125 + 7], 2),
        ("two blocks of one key pair", [8 * 101 + 5, 8 * 100 + 3], 2),
        ("key pairs on one thread (two iterations), another thread, another wave",
         [16 * 1031 + 1, 16 * 71 + 4, 16 * 7 + 2, 16 * 8 + 1], 2),
        ("first and last blocks", [V - 2, 5], 2),
    ] if V > 20000 else [
        ("index 0 (copy of the winner)", [0], 1),
        ("unique maximum at the last row (doubled winner)", [V - 1], 2),
        ("one wave's row pair", [501, 500], 2),
        ("across a head workgroup boundary", [16, 15], 2),
        ("two blocks of one key pair", [13, 3], 2),
        ("first and last blocks", [V - 2, 5], 2),
    ]


def _run_head_ties(shape, w, prompt, dtype_flag, label):
    import weight_streaming_gemv_amd as wsg
    V = shape.vocab
    base = oracle.OracleModel(shape, w, 16)
    t0 = oracle.argmax_lowest(base.forward_rows(prompt))
    for name, rows, factor in _head_cases(V):
        assert not set(rows) & set(int(t) for t in prompt), name
        wp = _planted_weights(w, rows, t0, factor)
        orc = oracle.OracleModel(shape, wp, 16)
        ref = orc.forward_rows(prompt)
        want = min(rows) if factor == 2 else min(rows + [t0])
        _expect_tie(ref, rows + ([t0] if factor == 1 else []), want)
        announce(f"{label}: {name}")
        m = wsg.Model(shape, wp, max_context=16, dtype=dtype_flag)
        tok = m.prefill(prompt)
        lg = _np(m.logits())
        assert tok == want, f"{label} {name}: token {tok}, want {want}"
        # the planted logits are bit-identical on the GPU too
        tied = rows + ([t0] if factor == 1 else [])
        assert len({lg[i].tobytes() for i in tied}) == 1, f"{label} {name}: planted logits differ"
        # and (FP32: exact tokens) the next step runs from the tie-broken token in lockstep
        nxt = m.step()
        if dtype_flag == 0:
            assert nxt == oracle.argmax_lowest(orc.forward_rows([want])), f"{label} {name}: next token"
        m.close()


@pytest.fixture(scope="module")
def qwen2_w():
    return model_weights(QWEN3_0_6B.with_layers(2), seed=0)


def test_head_ties_mini():
    w = model_weights(MINI, seed=0)
    _run_head_ties(MINI, w, prompt_ids(1, 8, MINI.vocab), 0, "mini")


def test_head_ties_qwen3_2layer(qwen2_w):
    _run_head_ties(QWEN3_0_6B.with_layers(2), qwen2_w, prompt_ids(1, 8, QWEN3_0_6B.vocab), 0, "qwen3-2L")


def test_head_ties_qwen3_2layer_fp16(qwen2_w):
    import weight_streaming_gemv_amd as wsg
    w16 = {"embed": qwen2_w["embed"].astype(np.float16), "final_norm": qwen2_w["final_norm"].astype(np.float16),
           "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in qwen2_w["layers"]]}
    _run_head_ties(QWEN3_0_6B.with_layers(2), w16, prompt_ids(1, 8, QWEN3_0_6B.vocab), wsg.WSG_F16, "qwen3-2L fp16")


def _step2_plan(shape, w, prompt, x0):
    """Rows to plant for a two-token step after the prompt whose row 0 consumes x0 (given
    as in_token) and whose row 1 consumes the draft: each row's winner gets a copy at a
    lower id that no row consumes, so the hidden states stay those of the unplanted model
    (with the echo of random weights the two winners may coincide; then both copies tie
    in both rows).  The draft is row 0's tie-broken token, so it is accepted.  Returns
    (planted weights, row-0 token, row-1 token)."""
    base = oracle.OracleModel(shape, w, 16)
    base.forward_rows(prompt, want_logits=False)
    r0 = oracle.argmax_lowest(base.forward_rows([x0]))
    r1 = oracle.argmax_lowest(base.forward_rows([r0]))   # a copy of E[r0] is fed like r0
    used = set(int(t) for t in prompt) | {x0, r0, r1}
    free = [i for i in range(64) if i not in used]
    a, b = free[0], free[1]
    assert a < r0 and b < r1
    wp = _planted_weights(_planted_weights(w, [a], r0, 1), [b], r1, 1)
    orc = oracle.OracleModel(shape, wp, 16)
    orc.forward_rows(prompt, want_logits=False)
    ref0 = orc.forward_rows([x0])
    tie0 = [a, r0] + ([b] if r1 == r0 else [])
    t0 = min(tie0)
    _expect_tie(ref0, tie0, t0)
    ref1 = orc.forward_rows([t0])
    tie1 = [b, r1] + ([a] if r1 == r0 else [])
    t1 = min(tie1)
    _expect_tie(ref1, tie1, t1)
    return wp, t0, t1


@pytest.mark.parametrize("shape_name", ["mini", "qwen3-2L"])
def test_two_token_step_ties(shape_name, qwen2_w):
    """Both rows of a two-token step break planted ties to the lower id; the draft (row 0's
    tie-broken token) is accepted, so both tokens are emitted."""
    import weight_streaming_gemv_amd as wsg
    if shape_name == "mini":
        shape, w, x0 = MINI, model_weights(MINI, seed=0), 777
    else:
        shape, w, x0 = QWEN3_0_6B.with_layers(2), qwen2_w, 4242
    prompt = prompt_ids(1, 8, shape.vocab)
    wp, t0, t1 = _step2_plan(shape, w, prompt, x0)
    announce(f"two-token ties {shape_name}: tokens {t0}, {t1}")
    m = wsg.Model(shape, wp, max_context=16)
    m.prefill(prompt)
    (g0, g1), n = m.step2(t0, in_token=x0)
    assert (g0, g1, n) == (t0, t1, 2), (g0, g1, n, t0, t1)
    m.close()
