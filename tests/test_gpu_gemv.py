"""GPU parity of the GEMV family against the oracle, through the C ABI.

Bound: a rigorous FP32 summation bound gamma_n * sum_k |W x| (n = K + 2,
doubled for the dot2 and dequant roundings), so any summation order passes
and a wrong row, column, scale or nibble fails.
"""
import numpy as np
import pytest

from gpu_util import announce, gemv_bound, gpu_available
import oracle
from synth import GEMV_SHAPES, Q4_SHAPES, gemv_inputs, q4g64_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dense_case(M, K, T, dtype, seed):
    npdt = np.float16 if dtype == "f16" else np.float32
    w, x = gemv_inputs(M, K, T, seed=seed, dtype=npdt)
    ref = oracle.gemv(w, x)
    bound = gemv_bound(oracle.gemv(np.abs(w.astype(np.float32)), np.abs(x.astype(np.float32))), K)
    return w, x, ref, bound


def _run_dense(M, K, T, Rs, dtype, seed=11, grid=0, flags=0):
    import torch
    import weight_streaming_gemv_amd as wsg
    w, x, ref, bound = _dense_case(M, K, T, dtype, seed)
    Wd = torch.from_numpy(w).cuda()
    Xd = torch.from_numpy(x).cuda()
    for R in Rs:
        announce(f"gemv {dtype} M={M} K={K} T={T} R={R} grid={grid} flags={flags}")
        y = wsg.gemv(Wd, Xd, rows_per_wave=R, grid_blocks=grid, flags=flags)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert got.shape == (T, M)
        assert np.all(err <= bound), f"R={R}: max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("T", [1, 2])
def test_gemv_model_shapes(shape, dtype, T):
    M, K = shape
    _run_dense(M, K, T, (1, 2, 4, 8), dtype)


@pytest.mark.parametrize("M,K,dtype", [(1000, 1000, "f32"), (777, 1001, "f32"), (13, 3, "f32"),
                                       (1000, 520, "f16"), (65, 1023, "f16"), (1, 1024, "f32"),
                                       (3, 2048, "f16"), (4097, 3072, "f32")])
@pytest.mark.parametrize("T", [1, 2])
def test_gemv_ragged(M, K, dtype, T):
    _run_dense(M, K, T, (1, 4), dtype, seed=12)


@pytest.mark.parametrize("M,K", [(1024, 3072), (1024, 2048), (4096, 1024), (1001, 3072), (7, 2048), (1, 1024)])
@pytest.mark.parametrize("T", [1, 2])
def test_gemv_f32_two_waves_per_row(M, K, T):
    """FP32 rows split over two waves (WSG_GEMV_SPLIT2): one workgroup per row pair, odd row
    counts (the last pair's second row is read clamped and not written), and grid-stride loops
    over one and three workgroups (their LDS half sums are reused pair after pair)."""
    import weight_streaming_gemv_amd as wsg
    split = wsg.WSG_GEMV_SPLIT2
    _run_dense(M, K, T, (1,), "f32", seed=14, flags=split | wsg.WSG_GEMV_NONTEMPORAL)
    _run_dense(M, K, T, (1,), "f32", seed=14, grid=3, flags=split)
    _run_dense(M, K, T, (1,), "f32", seed=14, grid=1, flags=split)
    if K == 3072:   # the default launch shape of FP32 rows of 3072 is this form
        _run_dense(M, K, T, (0,), "f32", seed=14)


@pytest.mark.parametrize("grid,flags", [(1, 0), (7, 1), (256, 0), (512, 1)])
def test_gemv_launch_shapes(grid, flags):
    _run_dense(6144, 1024, 2, (2,), "f32", grid=grid, flags=flags)
    _run_dense(4096, 1024, 1, (4,), "f16", grid=grid, flags=flags)


def _run_q4(M, K, T, Rs, seed=21, grid=0, flags=0):
    import torch
    import weight_streaming_gemv_amd as wsg
    q, words, s, x = q4g64_inputs(M, K, T, seed=seed)
    ref = oracle.gemv_q4g64(words, s, x, K)
    wabs = np.abs(oracle.dequant_q4g64(words, s, K))
    bound = gemv_bound(oracle.gemv(wabs, np.abs(x.astype(np.float32))), K, factor=3.0)
    Wq, S, X = (torch.from_numpy(words.view(np.int32)).cuda(), torch.from_numpy(s).cuda(),
                torch.from_numpy(x).cuda())
    for R in Rs:
        announce(f"gemv_q4g64 M={M} K={K} T={T} R={R} grid={grid} flags={flags}")
        y = wsg.gemv_q4g64(Wq, S, X, rows_per_wave=R, grid_blocks=grid, flags=flags)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert np.all(err <= bound), f"R={R}: max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


@pytest.mark.parametrize("shape", Q4_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("T", [1, 2])
def test_q4_model_shapes(shape, T):
    M, K = shape
    _run_q4(M, K, T, (1, 2, 4, 8))


@pytest.mark.parametrize("M,K", [(300, 192), (33, 64), (1001, 4160)])
@pytest.mark.parametrize("T", [1, 2])
def test_q4_ragged(M, K, T):
    _run_q4(M, K, T, (1, 8), seed=22)
    _run_q4(M, K, T, (2,), seed=22, grid=3, flags=1)


@pytest.mark.parametrize("M,K", [(1000, 14336), (999, 4096)])
@pytest.mark.parametrize("T", [1, 2])
def test_q4_fixed_k_ragged_and_looping(M, K, T):
    """The fixed-K int4 kernels (16 / R-wave workgroups at K = 14336, some with a
    partial last round of activation staging, 4-wave ones at K = 4096) on a ragged row
    count: one-shot grids, and grid-stride loops over three workgroups (at
    K = 4096 one row per wave issues each next row before reducing the
    current one; waves past the last row read it and discard it)."""
    _run_q4(M, K, T, (1, 4), seed=23)
    _run_q4(M, K, T, (2,), seed=23, grid=3, flags=1)
    _run_q4(M, K, T, (1,), seed=23, grid=3)


def test_gemv_determinism():
    import torch
    import weight_streaming_gemv_amd as wsg
    w, x = gemv_inputs(6144, 1024, 2, seed=5)
    Wd, Xd = torch.from_numpy(w).cuda(), torch.from_numpy(x).cuda()
    a = wsg.gemv(Wd, Xd, 2).cpu().numpy()
    b = wsg.gemv(Wd, Xd, 2, grid_blocks=64).cpu().numpy()
    assert np.array_equal(a, b)   # fixed per-row summation order, independent of launch shape
