"""Pins of the oracle's block decoders.

Each format is checked by encoding chosen fields with the encoders in
tests/blocks.py (written from the byte layouts, as the inverse of decoding)
and requiring the decoder to return exactly the weights those fields define,
and by constant-q blocks whose GEMV has a closed form.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests import blocks

RNG = np.random.default_rng(1234)
H = blocks.f16_bits


def _f16(bits):
    return float(np.uint16(bits).view(np.float16))


def test_block_sizes_match_formats():
    assert [oracle.block_elems(f) for f in range(7)] == [32, 32, 256, 256, 256, 1, 1]
    assert [oracle.block_bytes(f) for f in range(7)] == [34, 18, 144, 210, 176, 2, 4]


@pytest.mark.parametrize("trial", range(4))
def test_q8_0_roundtrip(trial):
    d = H(RNG.uniform(1e-3, 1e-2))
    q = RNG.integers(-128, 128, 32)
    w = oracle.dequant(oracle.Q8_0, np.frombuffer(blocks.enc_q8_0(d, q), np.uint8), 1, 32)[0]
    assert np.array_equal(w, _f16(d) * q.astype(np.float64))


@pytest.mark.parametrize("trial", range(4))
def test_q4_0_roundtrip(trial):
    d = H(RNG.uniform(1e-3, 1e-2))
    q = RNG.integers(0, 16, 32)
    w = oracle.dequant(oracle.Q4_0, np.frombuffer(blocks.enc_q4_0(d, q), np.uint8), 1, 32)[0]
    assert np.array_equal(w, _f16(d) * (q - 8).astype(np.float64))


def test_q4_0_element_order_distinct_values():
    # element j carries value j % 16: an order mistake shows up as a permutation
    q = np.arange(32) % 16
    q[16:] = 15 - q[16:]
    w = oracle.dequant(oracle.Q4_0, np.frombuffer(blocks.enc_q4_0(H(1.0), q), np.uint8), 1, 32)[0]
    assert np.array_equal(w, (q - 8).astype(np.float64))


@pytest.mark.parametrize("trial", range(4))
def test_q4_k_roundtrip(trial):
    d, dmin = H(RNG.uniform(1e-3, 1e-2)), H(RNG.uniform(1e-3, 1e-2))
    sc = RNG.integers(0, 64, 8)
    mn = RNG.integers(0, 64, 8)
    q = RNG.integers(0, 16, 256)
    raw = np.frombuffer(blocks.enc_q4_k(d, dmin, sc, mn, q), np.uint8)
    w = oracle.dequant(oracle.Q4_K, raw, 1, 256)[0]
    s = np.repeat(sc, 32).astype(np.float64)
    m = np.repeat(mn, 32).astype(np.float64)
    assert np.array_equal(w, _f16(d) * s * q - _f16(dmin) * m)


def test_q4_k_scale_extremes():
    # all six bits of every scale and min set: exercises the split high bits
    sc = np.full(8, 63)
    mn = np.array([0, 63, 1, 62, 32, 31, 48, 15])
    q = np.arange(256) % 16
    raw = np.frombuffer(blocks.enc_q4_k(H(1.0), H(0.5), sc, mn, q), np.uint8)
    w = oracle.dequant(oracle.Q4_K, raw, 1, 256)[0]
    assert np.array_equal(w, 63.0 * q - 0.5 * np.repeat(mn, 32))


@pytest.mark.parametrize("trial", range(4))
def test_q6_k_roundtrip(trial):
    d = H(RNG.uniform(1e-3, 1e-2))
    sc = RNG.integers(-128, 128, 16)
    q = RNG.integers(0, 64, 256)
    raw = np.frombuffer(blocks.enc_q6_k(d, sc, q), np.uint8)
    w = oracle.dequant(oracle.Q6_K, raw, 1, 256)[0]
    assert np.array_equal(w, _f16(d) * np.repeat(sc, 16).astype(np.float64) * (q - 32))


def test_q6_k_element_order_distinct_values():
    q = np.arange(256) % 64
    raw = np.frombuffer(blocks.enc_q6_k(H(1.0), np.ones(16, np.int64), q), np.uint8)
    w = oracle.dequant(oracle.Q6_K, raw, 1, 256)[0]
    assert np.array_equal(w, (q - 32).astype(np.float64))


@pytest.mark.parametrize("trial", range(4))
def test_q5_k_roundtrip(trial):
    d, dmin = H(RNG.uniform(1e-3, 1e-2)), H(RNG.uniform(1e-3, 1e-2))
    sc = RNG.integers(0, 64, 8)
    mn = RNG.integers(0, 64, 8)
    q = RNG.integers(0, 32, 256)
    raw = np.frombuffer(blocks.enc_q5_k(d, dmin, sc, mn, q), np.uint8)
    w = oracle.dequant(oracle.Q5_K, raw, 1, 256)[0]
    s = np.repeat(sc, 32).astype(np.float64)
    m = np.repeat(mn, 32).astype(np.float64)
    assert np.array_equal(w, _f16(d) * s * q - _f16(dmin) * m)


def test_q5_k_element_order_distinct_values():
    # element e carries (e + e // 32) % 32: every sub-block sees every fifth-bit pattern
    q = (np.arange(256) + np.arange(256) // 32) % 32
    raw = np.frombuffer(blocks.enc_q5_k(H(1.0), H(0.0), np.ones(8, np.int64), np.zeros(8, np.int64), q), np.uint8)
    w = oracle.dequant(oracle.Q5_K, raw, 1, 256)[0]
    assert np.array_equal(w, q.astype(np.float64))


def test_f16_f32_rows_decode_exactly():
    v = RNG.normal(0, 1, 64)
    w16 = oracle.dequant(oracle.F16, np.frombuffer(blocks.enc_f16(v), np.uint8), 1, 64)[0]
    assert np.array_equal(w16, v.astype(np.float16).astype(np.float64))
    w32 = oracle.dequant(oracle.F32, np.frombuffer(blocks.enc_f32(v), np.uint8), 1, 64)[0]
    assert np.array_equal(w32, v.astype(np.float32).astype(np.float64))
    # special values
    sp = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 2.0 ** -24], np.float64)
    assert np.array_equal(oracle.dequant(oracle.F16, np.frombuffer(blocks.enc_f16(sp), np.uint8), 1, 6)[0], sp)


def test_f32_gemv_is_dense_matmul():
    rows, cols = 5, 96
    Wv = RNG.normal(0, 1, (rows, cols)).astype(np.float32)
    x = RNG.normal(0, 1, cols)
    y = oracle.gemv(oracle.F32, np.frombuffer(blocks.enc_f32(Wv), np.uint8), x, rows, cols)
    assert np.allclose(y, Wv.astype(np.float64) @ x, rtol=1e-13, atol=1e-13)


def _const_row(fmt, nblocks, d, qval, extra=None):
    if fmt == oracle.Q8_0:
        b = blocks.enc_q8_0(H(d), np.full(32, qval))
    elif fmt == oracle.Q4_0:
        b = blocks.enc_q4_0(H(d), np.full(32, qval))
    elif fmt == oracle.Q4_K:
        sc, mn, dmin = extra
        b = blocks.enc_q4_k(H(d), H(dmin), np.full(8, sc), np.full(8, mn), np.full(256, qval))
    elif fmt == oracle.Q5_K:
        sc, mn, dmin = extra
        b = blocks.enc_q5_k(H(d), H(dmin), np.full(8, sc), np.full(8, mn), np.full(256, qval))
    else:
        b = blocks.enc_q6_k(H(d), np.full(16, extra), np.full(256, qval))
    return np.frombuffer(b * nblocks, np.uint8)


@pytest.mark.parametrize("fmt,d,q,extra,coef", [
    (oracle.Q8_0, 0.0078125, -77, None, lambda d, q, e: d * q),
    (oracle.Q4_0, 0.0048828125, 3, None, lambda d, q, e: d * (q - 8)),
    (oracle.Q4_K, 0.001953125, 11, (37, 21, 0.00390625), lambda d, q, e: d * e[0] * q - e[2] * e[1]),
    (oracle.Q6_K, 0.0009765625, 50, -93, lambda d, q, e: d * e * (q - 32)),
    (oracle.Q5_K, 0.001953125, 27, (45, 9, 0.0078125), lambda d, q, e: d * e[0] * q - e[2] * e[1]),
])
def test_constant_block_gemv_closed_form(fmt, d, q, extra, coef):
    # every weight equal => y = w * sum(x); d chosen as powers of two (exact in f16)
    cols = 1024
    qk = oracle.block_elems(fmt)
    row = _const_row(fmt, cols // qk, d, q, extra)
    W = np.concatenate([row, row, row])
    x = wl.gen_x(cols, wl.W_TEST, 0, 99)
    y = oracle.gemv(fmt, W, x, 3, cols)
    expect = coef(d, q, extra) * float(np.sum(x.astype(np.float64)))
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_70b_q6k_layer_bytes_match_pages():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
    fig = g["q6k_70b_layer_mib"]
    shp = wl.LLAMA70B
    total = 0
    for m in wl.MATS:
        r, c = shp.mat_shape(m)
        total += r * (c // oracle.block_elems(oracle.Q6_K)) * oracle.block_bytes(oracle.Q6_K)
    assert total == 701_890_560
    assert abs(total / 2 ** 20 - fig["value"]) < fig["tolerance"]
    # the generator's layout agrees with the oracle's block sizes
    assert total == wl.layer_weight_bytes(shp, wl.ALL_Q6_K)
