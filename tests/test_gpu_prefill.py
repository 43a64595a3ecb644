"""Chunked prefill vs the oracle, through the C ABI.

The projection GEMM (FP32 MFMA) is checked on its own against the oracle's
float64 product with a rigorous summation bound, then the chunked prefill of
whole models in lockstep: every valid K/V entry of every layer after the
prompt (Benchmark methodology, "Long-document chunked prefill": the whole
prefix is checked at chunk boundaries), the first token and its logits, then
decode steps.  Chunk sizes include 1, ragged tails and chunks larger than the
prompt; a second prefill call must continue the same sequence.
"""
import numpy as np
import pytest

from gpu_util import U32, _np, announce, close_rel, gemv_bound, gpu_available, lockstep
import oracle
from synth import MINI, PROMPT_SEEDS, QWEN3_0_6B, model_weights, prompt_ids

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


# Tiled path: M > 32 or K outside {256, 512, 1024, 2048, 3072}; 128x192,
# 128x128 and 64x64 tiles with 64- or 32-wide K tiles.  Small-M
# path (M <= 32): one and two 16-row tiles, ragged M, every compiled K and
# 4, 8 and 16 waves per block.
@pytest.mark.parametrize("M,N,K", [(1, 64, 32), (37, 128, 64), (65, 192, 96), (130, 4096, 1024),
                                   (1024, 4096, 1024), (500, 1024, 2048), (257, 6144, 1024),
                                   (1024, 1024, 3072), (2048, 4096, 1024), (1024, 6144, 1024), (300, 768, 192),
                                   (256, 384, 160),
                                   (1, 1024, 1024), (7, 4096, 1024), (16, 2048, 2048), (17, 64, 256),
                                   (31, 6144, 1024), (32, 1024, 3072), (31, 1024, 2048), (8, 512, 512),
                                   (3, 128, 3072)])
@pytest.mark.parametrize("acc", [0, 1])
def test_gemm_nt_f32(M, N, K, acc):
    import torch
    import weight_streaming_gemv_amd as wsg
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    announce(f"gemm_nt M={M} N={N} K={K} acc={acc}")
    Cd = torch.from_numpy(C0.copy()).cuda()
    wsg.gemm_nt(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), Cd, accumulate=bool(acc))
    torch.cuda.synchronize()
    got = Cd.cpu().numpy().astype(np.float64)
    prod = oracle.gemv(B, A).astype(np.float64)          # A @ B^T
    bound = gemv_bound(oracle.gemv(np.abs(B), np.abs(A)).astype(np.float64), K)
    ref = prod + (C0 if acc else 0.0)
    bound = bound + (U32 * np.abs(ref) if acc else 0.0) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


# SwiGLU in the product's epilogue: small-M kernel (M <= 32), 64x64 tiles
# with 32- and 64-wide K tiles, 128x192 tiles (the gate/up shape at 1024
# rows), and 128x192 picked for a K that needs 32-wide K tiles (1056), where
# the up sums do not fit the LDS B tile and 64x64 tiles take over.
@pytest.mark.parametrize("M,I,K", [(5, 96, 256), (32, 3072, 1024), (40, 96, 96), (97, 64, 128), (300, 3072, 1024),
                                   (1024, 3072, 1024), (1024, 384, 160), (1024, 3072, 1056)])
def test_gemm_swiglu_f32(M, I, K):
    """ACT = silu(A Wg^T) * (A Wu^T) against the oracle in float64: each of the
    two products within its FP32 summation bound, carried through the SwiGLU
    (|silu'| <= 1.1), plus a few float ulps for exp, divide and multiply."""
    import torch
    import weight_streaming_gemv_amd as wsg
    rng = np.random.default_rng(M * 31 + I + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    Wgu = (rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32)
    announce(f"gemm_swiglu M={M} I={I} K={K}")
    got = _np(wsg.gemm_swiglu(torch.from_numpy(A).cuda(), torch.from_numpy(Wgu).cuda())).astype(np.float64)
    assert got.shape == (M, I)
    gu = oracle.gemv(Wgu, A).astype(np.float64)             # A @ Wgu^T, [M, 2I]
    b = gemv_bound(oracle.gemv(np.abs(Wgu), np.abs(A)).astype(np.float64), K)
    g, u, bg, bu = gu[:, :I], gu[:, I:], b[:, :I], b[:, I:]
    ref = oracle.silu(g) * u
    sg = np.abs(oracle.silu(g))
    bound = 1.1 * bg * (np.abs(u) + bu) + (sg + 1.1 * bg) * bu + 8 * U32 * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


def test_gemm_swiglu_rejects_bad_shapes():
    import torch
    import weight_streaming_gemv_amd as wsg
    a = torch.zeros((4, 64), device="cuda")
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        wsg.gemm_swiglu(a, torch.zeros((2 * 48, 64), device="cuda"))     # I % 32 != 0
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        wsg.gemm_swiglu(torch.zeros((4, 48), device="cuda"), torch.zeros((64, 48), device="cuda"))   # K % 32


def test_gemm_rejects_bad_shapes():
    import torch
    import weight_streaming_gemv_amd as wsg
    a = torch.zeros((4, 48), device="cuda")
    b = torch.zeros((64, 48), device="cuda")
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        wsg.gemm_nt(a, b)          # K % 32 != 0
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        wsg.gemm_nt(torch.zeros((4, 64), device="cuda"), torch.zeros((48, 64), device="cuda"))


@pytest.fixture(scope="module")
def mini_w():
    return model_weights(MINI, seed=0)


@pytest.mark.parametrize("n_prompt,chunk", [(2, 1), (17, 16), (64, 16), (65, 64), (130, 32), (300, 64),
                                            (300, 7), (20, 64)])
def test_mini_chunked_prefill(mini_w, n_prompt, chunk):
    import weight_streaming_gemv_amd as wsg
    cap = 320
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_prefill_chunk(chunk)
    orc = oracle.OracleModel(MINI, mini_w, cap)
    prompt = prompt_ids(11, n_prompt, MINI.vocab)
    lockstep(m, orc, prompt, 4, label=f"mini chunked n={n_prompt} c={chunk}")
    m.close()


@pytest.mark.parametrize("chunk", [16, 64])
def test_stale_cache_never_leaks(mini_w, chunk):
    """Cache slots past the valid length hold whatever the allocator left there: a
    masked key still enters the prefill PV product with weight 0, so it must not be
    read as a value (0 * Inf = NaN).  Every slot is poisoned with NaN first."""
    import weight_streaming_gemv_amd as wsg
    cap = 160
    m = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=64)
    m.set_prefill_chunk(chunk)
    for l in range(MINI.n_layers):
        k, v, _ = m.kv(l)
        k.fill_(float("nan"))
        v.fill_(float("inf"))
    orc = oracle.OracleModel(MINI, mini_w, cap)
    lockstep(m, orc, prompt_ids(14, 45, MINI.vocab), 3, label=f"poisoned cache c={chunk}")
    m.close()


def test_mini_chunked_matches_tokenwise_and_continues(mini_w):
    """Chunked prefill and prefill through the decode forward (rows two per forward) agree;
    a second prefill call continues the sequence."""
    import weight_streaming_gemv_amd as wsg
    cap = 200
    prompt = prompt_ids(12, 150, MINI.vocab)
    a = wsg.Model(MINI, mini_w, max_context=cap, prefill_chunk=32)
    b = wsg.Model(MINI, mini_w, max_context=cap)
    ta = a.prefill(prompt[:100])
    ta2 = a.prefill(prompt[100:])
    tb = b.prefill(prompt)
    assert ta2 == tb
    orc = oracle.OracleModel(MINI, mini_w, cap)
    lo = orc.forward_rows(prompt[:100])
    assert ta == oracle.argmax_lowest(lo)
    lo = orc.forward_rows(prompt[100:])
    ok, err, _ = close_rel(_np(a.logits()), lo, 1e-3, 1e-3)
    assert ok, err
    for l in range(MINI.n_layers):
        ka, va, na = a.kv(l)
        kb, vb, nb = b.kv(l)
        assert na == nb == 150
        for g, r in ((ka, orc.k_cache[l]), (va, orc.v_cache[l]), (kb, orc.k_cache[l]), (vb, orc.v_cache[l])):
            ok, err, _ = close_rel(_np(g[:, :150]), r[:, :150], 1e-3, 1e-3)
            assert ok, err
    a.close()
    b.close()


@pytest.fixture(scope="module")
def c1_w():
    return model_weights(QWEN3_0_6B.with_layers(2), seed=0)


@pytest.mark.parametrize("n_prompt,chunk", [(8, 8), (32, 8), (32, 32), (200, 64), (200, 128)])
def test_tiny_qwen3_chunked_prefill(c1_w, n_prompt, chunk):
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    cap = 256
    m = wsg.Model(sh, c1_w, max_context=cap, prefill_chunk=128)
    m.set_prefill_chunk(chunk)
    orc = oracle.OracleModel(sh, c1_w, cap)
    prompt = prompt_ids(PROMPT_SEEDS["short"] if n_prompt <= 32 else 13, n_prompt, sh.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 4, label=f"qwen3x2 chunked n={n_prompt} c={chunk}")
    print(f"n={n_prompt} c={chunk}: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_qwen3x2_chunk_2048_crosses_a_chunk(c1_w):
    """A 2100-id prompt at 2048-row chunks (Qwen3 layer widths, 2 layers): the
    residual projections of the full chunk take 128 x 128 tiles with K split
    8 ways, the gate/up product its SwiGLU epilogue on 128 x 192 tiles, and a
    52-row second chunk attends across the boundary; every K/V entry, the
    first token and its logits, then decode steps, against the oracle."""
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    cap = 2112
    m = wsg.Model(sh, c1_w, max_context=cap, prefill_chunk=2048)
    orc = oracle.OracleModel(sh, c1_w, cap)
    prompt = prompt_ids(PROMPT_SEEDS["heldout"], 2100, sh.vocab)
    toks, _, ck = lockstep(m, orc, prompt, 3, label="qwen3x2 chunk 2048")
    print(f"chunk 2048: max |dlogit| {ck.max_logit_err:.2e} max |dkv| {ck.max_kv_err:.2e}")
    m.close()


def test_chunked_prefill_config_checks(c1_w):
    import weight_streaming_gemv_amd as wsg
    sh = QWEN3_0_6B.with_layers(2)
    m = wsg.Model(sh, c1_w, max_context=16, prefill_chunk=8)
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        m.set_prefill_chunk(9)
    with pytest.raises(wsg.WsgError, match="INVALID_ARG"):
        m.set_prefill_chunk(0)
    m.close()
    w16 = {"embed": c1_w["embed"].astype(np.float16), "final_norm": c1_w["final_norm"].astype(np.float16),
           "layers": [{k: v.astype(np.float16) for k, v in lw.items()} for lw in c1_w["layers"]]}
    with pytest.raises(wsg.WsgError, match="UNSUPPORTED"):
        wsg.Model(sh, w16, max_context=16, dtype=wsg.WSG_F16, prefill_chunk=8)
