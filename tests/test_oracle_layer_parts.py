"""Pins of the oracle's RMSNorm, RoPE and attention: closed forms and scipy."""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_rmsnorm_constant_vector():
    n, c, eps = 64, -3.0, 1e-5
    g = (1.0 + 0.1 * np.arange(n) / n).astype(np.float32)
    out = oracle.rmsnorm(np.full(n, c), g, eps)
    expect = c / math.sqrt(c * c + eps) * g.astype(np.float64)
    assert np.allclose(out, expect, rtol=1e-15)


def test_rmsnorm_scale_invariant_without_eps():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100)
    g = np.ones(100, np.float32)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(7.25 * x, g, 0.0)
    assert np.allclose(a, b, rtol=1e-14)
    assert np.sqrt(np.mean(a * a)) == pytest.approx(1.0, rel=1e-14)


def test_rope_identity_at_zero_and_norm_preserved():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(4 * 16)
    assert np.array_equal(oracle.rope(v, 4, 16, 0, 1e4), v)
    r = oracle.rope(v, 4, 16, 1234, 5e5)
    pairs_in = v.reshape(-1, 2)
    pairs_out = r.reshape(-1, 2)
    assert np.allclose(np.hypot(*pairs_out.T), np.hypot(*pairs_in.T), rtol=1e-14)


def test_rope_composes_additively():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(2 * 128)
    ab = oracle.rope(oracle.rope(v, 2, 128, 300, 5e5), 2, 128, 211, 5e5)
    assert np.allclose(ab, oracle.rope(v, 2, 128, 511, 5e5), rtol=1e-10, atol=1e-12)


def test_rope_frequencies_adjacent_pairs():
    # head_dim 128, theta 5e5: pair 0 turns by pos radians, pair 32 by pos/sqrt(5e5),
    # pair 63 by pos * 5e5^(-126/128); the pair is (2i, 2i+1) of the head.
    hd, pos = 128, 3
    for i, rate in [(0, 1.0), (32, 1.0 / math.sqrt(5e5)), (63, 5e5 ** (-126 / 128))]:
        v = np.zeros(hd)
        v[2 * i] = 1.0
        r = oracle.rope(v, 1, hd, pos, 5e5)
        ang = pos * rate
        assert r[2 * i] == pytest.approx(math.cos(ang), abs=1e-14)
        assert r[2 * i + 1] == pytest.approx(math.sin(ang), abs=1e-14)
        assert np.count_nonzero(r) <= 2


def _cache(rng, n_kv, ctx, hd, n_pos):
    k = np.zeros((n_kv, ctx, hd), np.uint16)
    v = np.zeros((n_kv, ctx, hd), np.uint16)
    k[:, :n_pos] = rng.standard_normal((n_kv, n_pos, hd)).astype(np.float16).view(np.uint16)
    v[:, :n_pos] = rng.standard_normal((n_kv, n_pos, hd)).astype(np.float16).view(np.uint16)
    return k, v


def test_attention_matches_scipy_softmax():
    rng = np.random.default_rng(6)
    n_head, n_kv, hd, ctx, n_pos = 8, 2, 16, 40, 29
    k, v = _cache(rng, n_kv, ctx, hd, n_pos)
    q = rng.standard_normal(n_head * hd) * 2.0
    o = oracle.attention(q, k, v, n_head, n_kv, hd, ctx, n_pos)
    kf = k.view(np.float16).astype(np.float64)
    vf = v.view(np.float16).astype(np.float64)
    for h in range(n_head):
        g = h // (n_head // n_kv)
        p = softmax(kf[g, :n_pos] @ q[h * hd:(h + 1) * hd] / math.sqrt(hd))
        assert np.allclose(o[h * hd:(h + 1) * hd], p @ vf[g, :n_pos], rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    n_head, n_kv, hd, ctx = 4, 2, 8, 10
    k, v = _cache(rng, n_kv, ctx, hd, 6)
    vf = v.view(np.float16).astype(np.float64)
    q = rng.standard_normal(n_head * hd)
    # one position: o = v[0] of the head's group
    o = oracle.attention(q, k, v, n_head, n_kv, hd, ctx, 1)
    for h in range(n_head):
        assert np.array_equal(o[h * hd:(h + 1) * hd], vf[h // 2, 0])
    # identical keys: o = mean of the values
    k2 = k.copy()
    k2[:, :6] = k2[:, :1]
    o = oracle.attention(q, k2, v, n_head, n_kv, hd, ctx, 6)
    for h in range(n_head):
        assert np.allclose(o[h * hd:(h + 1) * hd], vf[h // 2, :6].mean(axis=0), rtol=1e-13)
    # one dominant score selects that position's value row
    k3 = np.zeros_like(k)
    k3[:, 4, 0] = np.float16(60.0).view(np.uint16)
    q3 = np.zeros(n_head * hd)
    q3[0::hd] = 50.0
    o = oracle.attention(q3, k3, v, n_head, n_kv, hd, ctx, 6)
    for h in range(n_head):
        assert np.allclose(o[h * hd:(h + 1) * hd], vf[h // 2, 4], rtol=1e-12)
