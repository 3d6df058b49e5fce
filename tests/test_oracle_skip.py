"""Pins of the oracle's layer skip: the skip mask, the per-layer cosine
similarity and the choice of layers (ntransformer pages, p1 feature list:
layers picked by cosine similarity are skipped).

 - A skipped layer is the same as a stack built without it (bitwise).
 - A layer whose output projections are zero leaves the residual stream
   unchanged, so its similarity is 1; other layers stay below 1.
 - The similarity of layer l equals the cosine (numpy) between the final
   hidden states of the stacks of the first l and the first l + 1 layers.
 - The choice of layers follows hand-worked examples of the rule.
"""
import copy

import numpy as np
import pytest

import oracle
from synth import workloads as wl
from tests.stack_util import HostStack


def stack(n_layer=4, fmts=wl.Q4_K_M, wid=wl.W_TEST + 40, n_past=6):
    return HostStack(wl.TINY, fmts, n_layer=n_layer, vocab=300, max_ctx=24, n_past=n_past, wid=wid)


def model_of(hs, keep):
    """Oracle model over copies of the chosen layers (fresh caches)."""
    layers = []
    for l in keep:
        c = copy.copy(hs.layers[l])
        c.k_cache = hs.layers[l].k_cache.copy()
        c.v_cache = hs.layers[l].v_cache.copy()
        layers.append(c)
    return oracle.OracleModel(hs.shape, layers, hs.emb_fmt, hs.tok_emb, hs.head_fmt, hs.lm_head, hs.out_norm,
                              hs.vocab)


@pytest.mark.parametrize("M", [1, 2])
def test_skip_mask_equals_stack_without_those_layers(M):
    hs = stack(n_layer=5)
    toks = wl.gen_tokens(wl.W_TEST + 41, M, hs.vocab)
    skip = np.array([0, 1, 0, 1, 0], np.uint8)
    a = model_of(hs, range(5)).decode_skip(toks, 6, skip=skip, want_logits=True)
    b = model_of(hs, [0, 2, 4]).decode(toks, 6, want_logits=True)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[2], b[2])
    # and differs from the full stack
    c = model_of(hs, range(5)).decode(toks, 6, want_logits=True)
    assert not np.array_equal(a[2], c[2])


def test_identity_layer_has_similarity_one():
    hs = stack(n_layer=4)
    for name in ("wo", "wd"):
        hs.layers[2].mats[name][:] = 0   # d = dmin = 0 in every block: a zero matrix
    _, _, _, cos = model_of(hs, range(4)).decode_skip([hs.first_token], 6, want_cosine=True)
    assert abs(cos[0, 2] - 1.0) <= 1e-14
    for l in (0, 1, 3):
        assert -1.0 < cos[0, l] < 1.0 - 1e-9, (l, cos[0, l])


def test_skipped_layer_similarity_not_written():
    hs = stack(n_layer=3)
    _, _, _, cos = model_of(hs, range(3)).decode_skip([hs.first_token], 6, skip=[0, 1, 0], want_cosine=True)
    assert np.isnan(cos[0, 1]) and not np.isnan(cos[0, 0]) and not np.isnan(cos[0, 2])


@pytest.mark.parametrize("M", [1, 2])
def test_similarity_matches_prefix_stacks(M):
    hs = stack(n_layer=3)
    toks = wl.gen_tokens(wl.W_TEST + 42, M, hs.vocab)
    _, _, _, cos = model_of(hs, range(3)).decode_skip(toks, 6, want_cosine=True)
    # residual stream entering layer 0: the embedding rows
    emb = oracle.dequant(hs.emb_fmt, hs.tok_emb, hs.vocab, hs.shape.hidden)
    states = [emb[np.asarray(toks)]]
    for l in range(1, 4):
        _, _, _, hid = model_of(hs, range(l)).decode(toks, 6, want_hidden=True)
        states.append(hid)
    for l in range(3):
        for i in range(M):
            a, b = states[l][i], states[l + 1][i]
            ref = np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b))
            assert abs(cos[i, l] - ref) <= 1e-12, (l, i, cos[i, l], ref)


def test_select_skip_hand_examples():
    s = [0.5, 0.9, 0.9, 0.1, 0.95]
    assert oracle.select_skip(s, 2).tolist() == [0, 1, 0, 0, 1]          # 0.95, then the first 0.9
    assert oracle.select_skip(s, 3).tolist() == [0, 1, 1, 0, 1]
    assert oracle.select_skip(s, 2, first=2).tolist() == [0, 0, 1, 0, 1]
    assert oracle.select_skip(s, 1, first=0, last=4).tolist() == [0, 1, 0, 0, 0]
    assert oracle.select_skip(s, 0).tolist() == [0] * 5
    assert oracle.select_skip(s, 3, first=1, last=4).tolist() == [0, 1, 1, 1, 0]
    assert oracle.select_skip([-0.2, -0.1, -0.3], 1).tolist() == [0, 1, 0]
    # NaN outside the eligible range is ignored, inside it is an error
    assert oracle.select_skip([np.nan, 0.2, 0.3], 1, first=1).tolist() == [0, 0, 1]
    with pytest.raises(ValueError):
        oracle.select_skip([np.nan, 0.2, 0.3], 1)
    with pytest.raises(ValueError):
        oracle.select_skip(s, 3, first=3)
    with pytest.raises(ValueError):
        oracle.select_skip(s, 1, first=4, last=2)
