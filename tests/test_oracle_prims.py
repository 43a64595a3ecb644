"""Pins of the oracle's primitives against closed forms, invariants and brute force.

Each check is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign or index, a swapped pairing, a transposed operand)
fails at least one of them.
"""
import cmath
import math

import numpy as np
import pytest

from oracle import argmax_lowest, gqa_attention, rms_norm, rope_angles, rope_apply, silu

EPS = 1e-6


# ---------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("c", [0.5, -3.0, 1e-2, 7.25])
def test_rms_constant_vector(c):
    n = 1024
    y = rms_norm(np.full(n, c), np.ones(n), EPS)
    assert np.allclose(y, c / math.sqrt(c * c + EPS), rtol=1e-15, atol=0)


def test_rms_one_hot():
    n, i, c = 256, 17, 2.5
    x = np.zeros(n)
    x[i] = c
    y = rms_norm(x, np.ones(n), EPS)
    expect = c / math.sqrt(c * c / n + EPS)
    assert y[i] == pytest.approx(expect, rel=1e-15)
    assert np.count_nonzero(y) == 1


def test_rms_gain_multiplies_and_eps_inside_root():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(128)
    g = rng.uniform(0.5, 2.0, 128)
    y1 = rms_norm(x, np.ones(128), EPS)
    assert np.allclose(rms_norm(x, g, EPS), y1 * g, rtol=1e-14)
    # eps inside the root: a zero vector stays zero, tiny vectors are damped
    assert np.all(rms_norm(np.zeros(8), np.ones(8), EPS) == 0)
    tiny = np.full(4, 1e-4)
    assert rms_norm(tiny, np.ones(4), EPS)[0] == pytest.approx(1e-4 / math.sqrt(1e-8 + EPS))


def test_rms_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 1024))
    y = rms_norm(x, np.ones(1024), EPS)
    assert np.allclose(rms_norm(-4.0 * x, np.ones(1024), EPS), -y, rtol=1e-5)
    # output RMS is ~1 when mean(x^2) >> eps
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-5)
    # rows are independent
    assert np.allclose(rms_norm(x[1], np.ones(1024), EPS), y[1], rtol=0, atol=0)


# ---------------------------------------------------------------- RoPE
D = 128


def test_rope_position_zero_is_identity():
    u = np.random.default_rng(1).standard_normal(D)
    assert np.array_equal(rope_apply(u, rope_angles([0], D, 1e6)[0]), u)


def test_rope_pairs_are_half_split():
    # a one-hot at dim i only ever mixes with dim i + D/2
    for i in (0, 5, 63):
        u = np.zeros(D)
        u[i] = 1.0
        y = rope_apply(u, rope_angles([37], D, 1e6)[0])
        nz = set(np.flatnonzero(np.abs(y) > 1e-300))
        assert nz <= {i, i + D // 2}
        assert (i + D // 2) in nz


def test_rope_matches_complex_rotation():
    # textbook form: (u_i + j u_{i+D/2}) * exp(j * p * base^(-2i/D))
    rng = np.random.default_rng(2)
    u = rng.standard_normal(D)
    for p in (1, 9, 4095, 5118):
        y = rope_apply(u, rope_angles([p], D, 1e6)[0])
        for i in (0, 1, 31, 63):
            z = complex(u[i], u[i + D // 2]) * cmath.exp(1j * p * 1e6 ** (-2.0 * i / D))
            assert y[i] == pytest.approx(z.real, abs=1e-12)
            assert y[i + D // 2] == pytest.approx(z.imag, abs=1e-12)


def test_rope_first_pair_turns_by_position_radians():
    u = np.zeros(D)
    u[0] = 1.0
    for p in (1, 2, 3):
        y = rope_apply(u, rope_angles([p], D, 1e6)[0])
        assert math.atan2(y[D // 2], y[0]) == pytest.approx(p if p <= math.pi else p - 2 * math.pi, abs=1e-12)


def test_rope_frequencies_geometric():
    # at p=1 pair i turns by base^(-2i/D); successive ratio base^(-2/D)
    u = np.zeros(D)
    u[:D // 2] = 1.0
    y = rope_apply(u, rope_angles([1], D, 1e6)[0])
    ang = np.arctan2(y[D // 2:], y[:D // 2])
    ratio = ang[1:] / ang[:-1]
    assert np.allclose(ratio, 1e6 ** (-2.0 / D), rtol=1e-9)
    assert ang[0] == pytest.approx(1.0, abs=1e-12)


def test_rope_preserves_pair_norms_and_relative_positions():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    m, n = 300, 123
    rq = rope_apply(q, rope_angles([m], D, 1e6)[0])
    rk = rope_apply(k, rope_angles([n], D, 1e6)[0])
    pn = lambda v: v[:D // 2] ** 2 + v[D // 2:] ** 2
    assert np.allclose(pn(rq), pn(q), rtol=1e-12)
    lhs = float(rq @ rk)
    rhs = float(rope_apply(q, rope_angles([m - n], D, 1e6)[0]) @ k)
    assert lhs == pytest.approx(rhs, rel=1e-10, abs=1e-10)


# ---------------------------------------------------------------- SiLU
def test_silu_special_values():
    assert silu(0.0) == 0.0
    assert float(silu(1.0)) == pytest.approx(0.7310585786300049, rel=1e-15)  # 1/(1+e^-1)
    assert float(silu(40.0)) == pytest.approx(40.0, rel=1e-15)
    assert abs(float(silu(-40.0))) < 1e-15
    z = np.linspace(-6, 6, 101)
    assert np.allclose(silu(-z), silu(z) - z, atol=1e-14)   # sigma(-z) = 1 - sigma(z)


# ---------------------------------------------------------------- attention
def brute_attention(q, kc, vc, pos):
    """Pure-Python causal GQA attention with math.fsum (tiny dims only)."""
    n, hq, d = q.shape
    hkv = kc.shape[0]
    out = np.zeros((n, hq, d))
    for r in range(n):
        for h in range(hq):
            j = h // (hq // hkv)
            s = [math.fsum(q[r, h, t] * kc[j, i, t] for t in range(d)) / math.sqrt(d)
                 for i in range(pos[r] + 1)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            den = math.fsum(e)
            for t in range(d):
                out[r, h, t] = math.fsum(e[i] * vc[j, i, t] for i in range(len(e))) / den
    return out


@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 1), (2, 2)])
def test_attention_brute_force(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    d, P = 4, 7
    kc = rng.standard_normal((hkv, P, d))
    vc = rng.standard_normal((hkv, P, d))
    pos = np.array([2, 3, 6])
    q = rng.standard_normal((3, hq, d))
    assert np.allclose(gqa_attention(q, kc, vc, pos), brute_attention(q, kc, vc, pos), rtol=1e-12, atol=1e-13)


def test_attention_single_key_returns_value_and_gqa_mapping():
    rng = np.random.default_rng(9)
    hq, hkv, d = 16, 8, 128
    kc = rng.standard_normal((hkv, 1, d))
    vc = rng.standard_normal((hkv, 1, d))
    q = rng.standard_normal((1, hq, d))
    o = gqa_attention(q, kc, vc, [0])
    for h in range(hq):
        assert np.array_equal(o[0, h], vc[h // 2, 0])


def test_attention_equal_keys_is_mean_of_values():
    rng = np.random.default_rng(10)
    kc = np.repeat(rng.standard_normal((1, 1, 8)), 5, axis=1)
    vc = rng.standard_normal((1, 5, 8))
    o = gqa_attention(rng.standard_normal((1, 2, 8)), kc, vc, [4])
    assert np.allclose(o[0, 0], vc[0].mean(axis=0), rtol=1e-13)
    assert np.allclose(o[0, 1], vc[0].mean(axis=0), rtol=1e-13)


def test_attention_scale_is_inverse_sqrt_d():
    # two keys whose dot products with q differ by delta*sqrt(d): weights ratio e^delta
    d, delta = 16, 0.7
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    kc = np.zeros((1, 2, d))
    kc[0, 0, 0] = delta * math.sqrt(d)
    vc = np.zeros((1, 2, d))
    vc[0, 0, 0] = 1.0                      # o[0] = weight of key 0
    w0 = gqa_attention(q, kc, vc, [1])[0, 0, 0]
    assert w0 / (1 - w0) == pytest.approx(math.exp(delta), rel=1e-12)


def test_attention_is_causal():
    rng = np.random.default_rng(11)
    kc = rng.standard_normal((2, 6, 4))
    vc = rng.standard_normal((2, 6, 4))
    q = rng.standard_normal((1, 4, 4))
    a = gqa_attention(q, kc, vc, [3])
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, 4:] = 99.0
    vc2[:, 4:] = -99.0
    assert np.array_equal(a, gqa_attention(q, kc2, vc2, [3]))


# ---------------------------------------------------------------- argmax
def test_argmax_ties_go_to_lowest_id():
    rng = np.random.default_rng(12)
    v = rng.standard_normal(151936).astype(np.float32)
    top = np.float32(v.max() + 1)
    for idxs in ([5, 9], [0, 151935], [1023, 1024, 4096], [151934, 151935], [18991, 18992]):
        w = v.copy()
        w[idxs] = top
        assert argmax_lowest(w) == min(idxs)
    assert argmax_lowest(np.zeros(151936, np.float32)) == 0
    w = v.copy()
    w[-1] = top
    assert argmax_lowest(w) == 151935


def test_argmax_signed_zero_tie_and_nonfinite():
    v = np.array([-1.0, -0.0, 0.0, -2.0], np.float32)
    assert argmax_lowest(v) == 1
    with pytest.raises(ValueError):
        argmax_lowest(np.array([0.0, np.nan], np.float32))
    with pytest.raises(ValueError):
        argmax_lowest(np.array([0.0, np.inf], np.float32))
