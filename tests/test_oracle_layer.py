"""Pins of the oracle layer and stack with constructed weights.

Zero matrices (Q8_0 blocks with d = 0), identity and selection matrices
(Q8_0, d = 1, q = 1 on chosen entries) turn the layer into closed forms that
expose the residual wiring, the GQA head mapping, the inclusion of the new
token in attention, the f16 rounding of the cache and the SwiGLU order.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from synth import workloads as wl
from tests import blocks

ONE = blocks.f16_bits(1.0)


def q8_matrix(rows, cols, entries=(), d_bits=ONE):
    """Q8_0 matrix with q = 1 at the (r, c) entries and 0 elsewhere (d = 0 => zero matrix)."""
    q = np.zeros((rows, cols), np.int64)
    for r, c in entries:
        q[r, c] = 1
    out = bytearray()
    for r in range(rows):
        for b in range(cols // 32):
            out += blocks.enc_q8_0(d_bits, q[r, 32 * b:32 * b + 32])
    return np.frombuffer(bytes(out), np.uint8).copy()


def make_layer(shape, mats, max_ctx, n_past, wid=wl.W_TEST, layer=0):
    li = wl.gen_layer(shape, wl.ALL_Q8_0, wid, layer, max_ctx, n_past, weights=False)
    li.mats = {m: mats[m] for m in wl.MATS}
    return li


SHP = wl.LayerShape(hidden=64, n_head=4, n_kv_head=2, head_dim=16, ffn=64, rope_theta=1e4)


def zero_mats(shape):
    return {m: q8_matrix(*shape.mat_shape(m), d_bits=0) for m in wl.MATS}


def test_zero_weights_is_identity_and_appends_zero_kv():
    li = make_layer(SHP, zero_mats(SHP), 16, 5)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 1)
    out = oracle.layer(li, x, pos=5)
    assert np.array_equal(out[0], x.astype(np.float64))
    # zero values (a rotation of +0 may give -0)
    assert not li.k_cache[:, 5].view(np.float16).any() and not li.v_cache[:, 5].view(np.float16).any()


def test_attention_path_gqa_mapping_and_residual():
    # Wq = Wk = 0 => every score is 0 => o_h = mean of V[g(h)] over 0..pos (new entry included);
    # Wv passes xn[0:32] into the two kv heads; Wo = I; FFN zero => out = x + o.
    mats = zero_mats(SHP)
    mats["wv"] = q8_matrix(32, 64, [(i, i) for i in range(32)])
    mats["wo"] = q8_matrix(64, 64, [(i, i) for i in range(64)])
    pos = 6
    li = make_layer(SHP, mats, 12, pos)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 2)
    vc_before = li.v_cache.copy()
    out = oracle.layer(li, x, pos=pos)[0]
    xn = oracle.rmsnorm(x, li.attn_norm, SHP.rms_eps)
    new_v = xn[:32].astype(np.float16).view(np.uint16).reshape(2, 16)
    assert np.array_equal(li.v_cache[:, pos], new_v)
    vf = vc_before.view(np.float16).astype(np.float64)
    vf[:, pos] = new_v.view(np.float16)
    o = np.concatenate([vf[h // 2, :pos + 1].mean(axis=0) for h in range(4)])
    assert np.allclose(out, x.astype(np.float64) + o, rtol=1e-13, atol=1e-13)


def test_rope_applied_to_cached_key():
    mats = zero_mats(SHP)
    mats["wk"] = q8_matrix(32, 64, [(i, i + 5) for i in range(32)])
    pos = 9
    li = make_layer(SHP, mats, 12, pos)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 3)
    oracle.layer(li, x, pos=pos)
    xn = oracle.rmsnorm(x, li.attn_norm, SHP.rms_eps)
    k = oracle.rope(xn[5:37], 2, 16, pos, SHP.rope_theta)
    assert np.array_equal(li.k_cache[:, pos], k.astype(np.float16).view(np.uint16).reshape(2, 16))


def test_ffn_path_swiglu_closed_form():
    mats = zero_mats(SHP)
    eye = [(i, i) for i in range(64)]
    mats["wg"] = q8_matrix(64, 64, eye)
    mats["wu"] = q8_matrix(64, 64, eye)
    mats["wd"] = q8_matrix(64, 64, eye)
    li = make_layer(SHP, mats, 8, 3)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 4) * 3.0
    out = oracle.layer(li, x, pos=3)[0]
    hn = oracle.rmsnorm(x, li.ffn_norm, SHP.rms_eps)
    assert np.allclose(out, x.astype(np.float64) + hn * expit(hn) * hn, rtol=1e-13)


def test_gate_and_up_are_not_swapped():
    # gate = 2 * xn, up = xn  =>  a = silu(2 xn) * xn  (swapping gives silu(xn) * 2 xn)
    mats = zero_mats(SHP)
    mats["wg"] = q8_matrix(64, 64, [(i, i) for i in range(64)], d_bits=blocks.f16_bits(2.0))
    mats["wu"] = q8_matrix(64, 64, [(i, i) for i in range(64)])
    mats["wd"] = q8_matrix(64, 64, [(i, i) for i in range(64)])
    li = make_layer(SHP, mats, 8, 3)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 5)
    out = oracle.layer(li, x, pos=3)[0]
    hn = oracle.rmsnorm(x, li.ffn_norm, SHP.rms_eps)
    assert np.allclose(out - x, 2 * hn * expit(2 * hn) * hn, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fmts", [wl.ALL_Q4_0, wl.Q4_K_M])
def test_batched_tokens_equal_sequential(fmts):
    # verify pass over M tokens == M single-token passes at increasing positions
    shp = wl.TINY
    M, pos = 3, 7
    li_a = wl.gen_layer(shp, fmts, wl.W_TEST, 11, 16, pos)
    li_b = wl.gen_layer(shp, fmts, wl.W_TEST, 11, 16, pos)
    x = np.stack([wl.gen_x(shp.hidden, wl.W_TEST, 20 + i) for i in range(M)])
    out_a = oracle.layer(li_a, x, pos=pos, M=M)
    out_b = np.stack([oracle.layer(li_b, x[i], pos=pos + i)[0] for i in range(M)])
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(li_a.k_cache, li_b.k_cache) and np.array_equal(li_a.v_cache, li_b.v_cache)


def test_stack_with_zero_layers_follows_lm_head_permutation():
    shp = SHP
    vocab = shp.hidden
    layers = [make_layer(shp, zero_mats(shp), 8, 2, layer=l) for l in range(2)]
    emb = q8_matrix(vocab, shp.hidden, [(i, i) for i in range(vocab)])
    perm = np.random.default_rng(9).permutation(vocab)
    lm = q8_matrix(vocab, shp.hidden, [(int(perm[i]), i) for i in range(vocab)])
    g = wl.gen_gains(shp, wl.W_TEST, 0, wl.T_OUT_NORM)
    m = oracle.OracleModel(shp, layers, oracle.Q8_0, emb, oracle.Q8_0, lm, g, vocab)
    for t in [0, 5, 63]:
        nxt, margin, _, hidden = m.decode([t], pos=2, want_hidden=True)
        assert nxt[0] == perm[t]
        assert margin[0] > 0
        assert np.array_equal(hidden[0], np.eye(vocab)[t])


def test_stack_verify_equals_sequential_decode():
    shp = wl.TINY
    vocab = 96
    M, pos = 4, 5

    def model():
        layers = [wl.gen_layer(shp, wl.Q4_K_M, wl.W_TEST, 30 + l, 16, pos) for l in range(2)]
        emb = wl.gen_matrix(oracle.Q6_K, vocab, shp.hidden, wl.W_TEST, 0, wl.T_TOK_EMB)
        lm = wl.gen_matrix(oracle.Q6_K, vocab, shp.hidden, wl.W_TEST, 0, wl.T_LM_HEAD)
        g = wl.gen_gains(shp, wl.W_TEST, 0, wl.T_OUT_NORM)
        return oracle.OracleModel(shp, layers, oracle.Q6_K, emb, oracle.Q6_K, lm, g, vocab)

    toks = wl.gen_tokens(wl.W_TEST, M, vocab)
    a, _, la, _ = model().decode(toks, pos, want_logits=True)
    mb = model()
    for i in range(M):
        b, _, lb, _ = mb.decode(toks[i:i + 1], pos + i, want_logits=True)
        assert b[0] == a[i]
        assert np.array_equal(lb[0], la[i])


def test_query_rope_inside_layer_closed_form():
    # Wq = 4 I (q = 4 xn), Wk = Wv = 0 (the new key and value are zero), Wo = I,
    # FFN zero.  The cache is zero except, in kv group 0, the key at position
    # t0 is the unit vector along dimension 2i (first of pair i) and the value
    # at t0 is e_0.  Query head h of group 0 then scores t0 with
    # s_h = qr_h[2i] / sqrt(hd), where qr is q turned by pos * theta^(-2i/hd)
    # (pair (2i, 2i+1)), and every other position 0..pos scores 0; so
    # out - x at dim 0 of head h is e^s / (e^s + pos) and zero elsewhere.
    # An unrotated query, or one turned at pos +- 1, gives another value.
    mats = zero_mats(SHP)
    mats["wq"] = q8_matrix(64, 64, [(r, r) for r in range(64)], d_bits=blocks.f16_bits(4.0))
    mats["wo"] = q8_matrix(64, 64, [(r, r) for r in range(64)])
    hd, i, pos, t0 = SHP.head_dim, 1, 9, 3
    li = make_layer(SHP, mats, 12, pos)
    li.k_cache[...] = 0
    li.v_cache[...] = 0
    li.k_cache[0, t0, 2 * i] = blocks.f16_bits(1.0)
    li.v_cache[0, t0, 0] = blocks.f16_bits(1.0)
    x = wl.gen_x(SHP.hidden, wl.W_TEST, 6).astype(np.float64) * 2.0
    out = oracle.layer(li, x, pos=pos)[0]
    g = li.attn_norm.astype(np.float64)
    xn = x / math.sqrt(np.mean(x * x) + SHP.rms_eps) * g
    q = 4.0 * xn
    ang = pos * SHP.rope_theta ** (-2.0 * i / hd)
    expect = np.zeros(64)
    for h in range(2):  # the two query heads of kv group 0
        a, b = q[h * hd + 2 * i], q[h * hd + 2 * i + 1]
        s = (a * math.cos(ang) - b * math.sin(ang)) / math.sqrt(hd)
        expect[h * hd] = math.exp(s) / (math.exp(s) + pos)
    assert np.allclose(out - x, expect, rtol=1e-12, atol=1e-14)
    # the same layer with the query unrotated, or turned one position off,
    # lands measurably elsewhere (the pin separates those mistakes)
    for wrong in (0.0, (pos - 1) * SHP.rope_theta ** (-2.0 * i / hd), (pos + 1) * SHP.rope_theta ** (-2.0 * i / hd)):
        a, b = q[2 * i], q[2 * i + 1]
        s = (a * math.cos(wrong) - b * math.sin(wrong)) / math.sqrt(hd)
        assert abs(math.exp(s) / (math.exp(s) + pos) - expect[0]) > 1e-3


def test_stack_output_norm_logit_values():
    # Zero layers (the final hidden state is the embedding row), a Q8_0
    # embedding with distinct, non-unit rows and an identity LM head: the
    # logits are the output RMSNorm of the embedding row, e / sqrt(mean(e^2)
    # + eps) * g, value for value.
    shp = SHP
    vocab = shp.hidden
    layers = [make_layer(shp, zero_mats(shp), 8, 2, layer=l) for l in range(2)]
    rng = np.random.default_rng(21)
    q = rng.integers(-127, 128, size=(vocab, shp.hidden))
    d = blocks.f16_bits(1.0 / 16.0)
    emb_rows = bytearray()
    for r in range(vocab):
        for b in range(shp.hidden // 32):
            emb_rows += blocks.enc_q8_0(d, q[r, 32 * b:32 * b + 32])
    emb = np.frombuffer(bytes(emb_rows), np.uint8).copy()
    lm = q8_matrix(vocab, shp.hidden, [(i, i) for i in range(vocab)])
    g = wl.gen_gains(shp, wl.W_TEST, 0, wl.T_OUT_NORM)
    m = oracle.OracleModel(shp, layers, oracle.Q8_0, emb, oracle.Q8_0, lm, g, vocab)
    for t in [0, 17, 63]:
        nxt, margin, logits, hidden = m.decode([t], pos=2, want_logits=True, want_hidden=True)
        e = q[t].astype(np.float64) / 16.0
        assert np.array_equal(hidden[0], e)
        expect = e / math.sqrt(np.mean(e * e) + shp.rms_eps) * g.astype(np.float64)
        assert np.allclose(logits[0], expect, rtol=1e-13, atol=0)
        assert nxt[0] == int(np.argmax(expect))
        assert abs(math.sqrt(np.mean(e * e)) - 1.0) > 0.5  # the norm is far from a no-op here


def test_composed_decode_equals_plain_decode():
    # the stored conditioning estimates of the 70B stack rerun each decode
    # step composed from the oracle's parts (embedding row, layers, output
    # norm, LM head) with a perturbation in between; without it the
    # composition is the plain decode, bit for bit
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_stack70b_golden.py")
    spec = importlib.util.spec_from_file_location("make_stack70b_golden", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    from tests.stack_util import HostStack
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=3, vocab=300, max_ctx=24, n_past=9, wid=wl.W_TEST + 70)
    om_a, om_b = hs.oracle_model(), hs.oracle_model()
    _, _, lg, _ = om_a.decode([hs.first_token], 9, want_logits=True)
    lg_b = mod.perturbed_decode(om_b, hs, hs.first_token, 9, 0.0, 0)
    assert np.array_equal(lg[0], lg_b)
    for a, b in zip(om_a.layers_in, om_b.layers_in):
        assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.v_cache, b.v_cache)
    # a perturbation of the size used there moves these logits a little, not at all is wrong
    om_c = hs.oracle_model()
    lg_c = mod.perturbed_decode(om_c, hs, hs.first_token, 9, 1.5e-5, 0)
    d = np.abs(lg_c - lg[0]).max() / np.abs(lg[0]).max()
    assert 0 < d < 1e-3
