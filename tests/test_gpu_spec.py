"""Layer skip, its calibration, and self-speculative rounds (HIP) against the oracle.

Bars: a skip mask gives bitwise the stack built without those layers (also
when the skipped layers are streamed); calibration similarities within 1e-4
of the oracle's per token; greedy tokens identical to the oracle.  A
speculative round must emit exactly the tokens of plain greedy decoding,
whatever the draft proposes.
"""
import copy

import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu

LOGIT_TOL = 5e-3
COS_TOL = 1e-4


def sub_stack(hs, keep):
    h = copy.copy(hs)
    h.layers = [hs.layers[i] for i in keep]
    h.n_layer = len(keep)
    return h


def identity_layers(hs, layers):
    """Zero output projections: the layer leaves the residual stream unchanged."""
    for l in layers:
        for name in ("wo", "wd"):
            hs.layers[l].mats[name] = np.zeros_like(hs.layers[l].mats[name])


def oracle_greedy(hs, first, pos0, steps, skip=None):
    om = hs.oracle_model()
    toks, margins, t = [], [], first
    for s in range(steps):
        nxt, margin, _, _ = om.decode_skip([t], pos0 + s, skip=skip)
        toks.append(int(nxt[0]))
        margins.append(float(margin[0]))
        t = int(nxt[0])
    return toks, margins


def gpu_decode(h, token, pos0, vocab):
    import torch
    dev = device()
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(vocab, device=dev)
    h.decode_step(torch.tensor([token], dtype=torch.int32, device=dev),
                  torch.tensor([pos0], dtype=torch.int32, device=dev), nxt, ws, logits)
    torch.cuda.synchronize()
    return int(nxt.item()), logits.cpu().numpy()


@pytest.mark.parametrize("first_streamed", [None, 2], ids=["resident", "streamed"])
def test_skip_mask_equals_stack_without_layers(first_streamed):
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=5, vocab=400, max_ctx=32, n_past=9, wid=wl.W_TEST + 50)
    skip = [0, 1, 0, 1, 0]
    say(f"skip {skip} first_streamed {first_streamed}")
    cs = torch.cuda.Stream() if first_streamed is not None else None
    h = hs.device_model(dev, first_streamed=first_streamed, copy_stream=cs)
    h.set_skip(skip)
    t_a, l_a = gpu_decode(h, hs.first_token, 9, hs.vocab)
    t_b, l_b = gpu_decode(sub_stack(hs, [0, 2, 4]).device_model(dev), hs.first_token, 9, hs.vocab)
    assert t_a == t_b and np.array_equal(l_a, l_b)
    nxt, margin, ref, _ = hs.oracle_model().decode_skip([hs.first_token], 9, skip=skip, want_logits=True)
    assert rel_inf(l_a, ref[0]) <= LOGIT_TOL
    assert t_a == int(nxt[0])


def test_calibration_matches_oracle_similarities_and_choice():
    import quantized_decode_dequant_amd as nt
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=6, vocab=400, max_ctx=40, n_past=12, wid=wl.W_TEST + 51)
    identity_layers(hs, [2])
    T = 4
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    cos = torch.zeros(hs.n_layer, dtype=torch.float32, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([12], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    g_toks, per_tok = [], []
    for s in range(T):
        before = cos.clone()
        h.calibrate_step(tok, pos, nxt, cos, ws)
        torch.cuda.synchronize()
        per_tok.append((cos - before).cpu().numpy())
        g_toks.append(int(nxt.item()))
        tok.copy_(nxt)
        pos += 1
    om = hs.oracle_model()
    o_toks, o_cos, t = [], [], hs.first_token
    for s in range(T):
        n_, _, _, c = om.decode_skip([t], 12 + s, want_cosine=True)
        o_toks.append(int(n_[0]))
        o_cos.append(c[0])
        t = int(n_[0])
    say(f"gpu cos sums {cos.cpu().numpy()} tokens {g_toks} oracle {o_toks}")
    assert g_toks == o_toks
    for s in range(T):
        assert np.max(np.abs(per_tok[s] - o_cos[s])) <= COS_TOL, s
    sums = cos.cpu().numpy()
    assert abs(sums[2] - T) <= 1e-5
    # the choice: compared where the oracle's scores are separated by more than the tolerance
    o_sum = np.sum(o_cos, axis=0)
    for k in range(1, 5):
        ref = np.sort(o_sum)[::-1]
        if ref[k - 1] - ref[k] > T * COS_TOL:
            assert np.array_equal(nt.select_skip(sums, k, 1, 5), __import__("oracle").select_skip(o_sum, k, 1, 5)), k


def run_spec(h, hs, draft_skip, K, rounds, pos0):
    import torch
    dev = device()
    ws = torch.zeros(h.spec_workspace_bytes(K), dtype=torch.uint8, device=dev)
    cur = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([pos0], dtype=torch.int32, device=dev)
    out = torch.zeros(K + 1, dtype=torch.int32, device=dev)
    n_out = torch.zeros(1, dtype=torch.int32, device=dev)
    emitted, counts = [], []
    for r in range(rounds):
        h.spec_step(draft_skip, K, cur, pos, out, n_out, ws)
        torch.cuda.synchronize()
        n = int(n_out.item())
        o = out.cpu().numpy().tolist()
        assert 1 <= n <= K + 1
        assert all(v == -1 for v in o[n:])
        emitted += o[:n]
        counts.append(n)
        assert int(cur.item()) == o[n - 1]
    assert int(pos.item()) == pos0 + len(emitted)
    return emitted, counts


@pytest.mark.parametrize("K", [3, 7])
def test_spec_random_draft_emits_greedy_tokens(K):
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=6, vocab=500, max_ctx=80, n_past=10, wid=wl.W_TEST + 52)
    draft_skip = [0, 0, 0, 1, 1, 1]
    say(f"K {K} draft_skip {draft_skip}")
    emitted, counts = run_spec(hs.device_model(dev), hs, draft_skip, K, rounds=5, pos0=10)
    ref, margins = oracle_greedy(hs, hs.first_token, 10, len(emitted))
    say(f"counts {counts} gpu {emitted} oracle {ref} min margin {min(margins):.3g}")
    assert emitted == ref


@pytest.mark.parametrize("K", [2, 5])
def test_spec_identity_draft_accepts_every_token(K):
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=6, vocab=500, max_ctx=80, n_past=10, wid=wl.W_TEST + 53)
    identity_layers(hs, [3, 4, 5])   # the draft's skipped layers change nothing
    emitted, counts = run_spec(hs.device_model(dev), hs, [0, 0, 0, 1, 1, 1], K, rounds=4, pos0=10)
    ref, margins = oracle_greedy(hs, hs.first_token, 10, len(emitted))
    say(f"counts {counts} min margin {min(margins):.3g}")
    assert emitted == ref
    if min(margins) > 1e-2:
        assert counts == [K + 1] * 4


def test_spec_streamed_layers_and_model_skip():
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.ALL_Q6_K, n_layer=6, vocab=300, max_ctx=64, n_past=7, wid=wl.W_TEST + 54)
    identity_layers(hs, [5])
    h = hs.device_model(dev, first_streamed=3, copy_stream=torch.cuda.Stream())
    h.set_skip([0, 1, 0, 0, 0, 0])                 # the full stack leaves layer 1 out
    K = 4
    emitted, counts = run_spec(h, hs, [0, 0, 0, 0, 1, 1], K, rounds=4, pos0=7)
    ref, margins = oracle_greedy(hs, hs.first_token, 7, len(emitted), skip=[0, 1, 0, 0, 0, 0])
    say(f"counts {counts} gpu {emitted} oracle {ref}")
    assert emitted == ref


def test_spec_whole_stack_draft():
    dev = device()
    hs = HostStack(wl.TINY, wl.ALL_Q4_0, n_layer=3, vocab=256, max_ctx=64, n_past=5, wid=wl.W_TEST + 55)
    emitted, counts = run_spec(hs.device_model(dev), hs, None, 3, rounds=4, pos0=5)
    ref, margins = oracle_greedy(hs, hs.first_token, 5, len(emitted))
    say(f"counts {counts} min margin {min(margins):.3g}")
    assert emitted == ref
