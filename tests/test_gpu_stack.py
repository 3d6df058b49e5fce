"""Parity of nt_decode_step / nt_verify_step (HIP) against the oracle stack.

Bars: greedy tokens identical at every step; logits within 5e-3
(||.||_inf relative); streamed layers give bitwise the resident result.
"""
import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu

LOGIT_TOL = 5e-3


def greedy_gpu(h, first, pos0, steps, vocab):
    import torch
    dev = device()
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([first], dtype=torch.int32, device=dev)
    pos = torch.tensor([pos0], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(vocab, dtype=torch.float32, device=dev)
    toks, lgs = [], []
    for s in range(steps):
        h.decode_step(tok, pos, nxt, ws, logits)
        torch.cuda.synchronize()
        toks.append(int(nxt.item()))
        lgs.append(logits.cpu().numpy().copy())
        tok.copy_(nxt)
        pos += 1
    return toks, lgs


def greedy_oracle(om, first, pos0, steps):
    toks, lgs, margins = [], [], []
    t = first
    for s in range(steps):
        nxt, margin, logits, _ = om.decode([t], pos0 + s, want_logits=True)
        toks.append(int(nxt[0]))
        lgs.append(logits[0])
        margins.append(float(margin[0]))
        t = int(nxt[0])
    return toks, lgs, margins


@pytest.mark.parametrize("fmts", [wl.Q4_K_M, wl.ALL_Q4_0], ids=["q4_k_m", "q4_0"])
def test_stack_tiny_greedy(fmts):
    hs = HostStack(wl.TINY, fmts, n_layer=4, vocab=1000, max_ctx=48, n_past=20, wid=wl.W_TEST + 1)
    steps = 6
    g_toks, g_lgs = greedy_gpu(hs.device_model(device()), hs.first_token, 20, steps, hs.vocab)
    o_toks, o_lgs, margins = greedy_oracle(hs.oracle_model(), hs.first_token, 20, steps)
    say(f"gpu {g_toks} oracle {o_toks} margins {[f'{m:.3g}' for m in margins]}")
    for s in range(steps):
        assert rel_inf(g_lgs[s], o_lgs[s]) <= LOGIT_TOL, s
    assert g_toks == o_toks


@pytest.mark.parametrize("emb_fmt,head_fmt", [(wl.F16, wl.Q5_K), (wl.F32, wl.Q8_0), (wl.Q5_K, wl.Q4_K)],
                         ids=["f16_q5k", "f32_q8", "q5k_q4k"])
def test_stack_embedding_and_head_formats(emb_fmt, head_fmt):
    hs = HostStack(wl.TINY, wl.Q5_K_M, n_layer=2, vocab=700, max_ctx=40, n_past=9, wid=wl.W_TEST + 6,
                   emb_fmt=emb_fmt, head_fmt=head_fmt)
    steps = 4
    g_toks, g_lgs = greedy_gpu(hs.device_model(device()), hs.first_token, 9, steps, hs.vocab)
    o_toks, o_lgs, margins = greedy_oracle(hs.oracle_model(), hs.first_token, 9, steps)
    say(f"gpu {g_toks} oracle {o_toks}")
    for s in range(steps):
        assert rel_inf(g_lgs[s], o_lgs[s]) <= LOGIT_TOL, s
    assert g_toks == o_toks


def test_verify_matches_oracle_and_decode():
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=3, vocab=777, max_ctx=40, n_past=11, wid=wl.W_TEST + 2)
    M = 4
    toks = wl.gen_tokens(wl.W_TEST + 2, M, hs.vocab)
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    logits = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    pos = torch.tensor([11], dtype=torch.int32, device=dev)
    h.verify_step(torch.from_numpy(toks).to(dev), M, pos, out, ws, logits)
    torch.cuda.synchronize()
    nxt, margins, ref_logits, _ = hs.oracle_model().decode(toks, 11, want_logits=True)
    g = logits.cpu().numpy().reshape(M, hs.vocab)
    for i in range(M):
        assert rel_inf(g[i], ref_logits[i]) <= LOGIT_TOL
    assert out.cpu().numpy().tolist() == nxt.tolist()
    # M = 1 verify == decode step on a fresh copy of the caches
    h1 = hs.device_model(dev)
    h2 = hs.device_model(dev)
    a = torch.zeros(1, dtype=torch.int32, device=dev)
    b = torch.zeros(1, dtype=torch.int32, device=dev)
    la = torch.zeros(hs.vocab, device=dev)
    lb = torch.zeros(hs.vocab, device=dev)
    t = torch.from_numpy(toks[:1]).to(dev)
    h1.verify_step(t, 1, pos, a, torch.zeros(h1.workspace_bytes(1), dtype=torch.uint8, device=dev), la)
    h2.decode_step(t, pos, b, torch.zeros(h2.workspace_bytes(1), dtype=torch.uint8, device=dev), lb)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("M", [1, 3])
def test_streamed_layers_bitwise_equal_resident(M):
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.ALL_Q6_K, n_layer=5, vocab=500, max_ctx=32, n_past=9, wid=wl.W_TEST + 3)
    toks = torch.from_numpy(wl.gen_tokens(wl.W_TEST + 3, M, hs.vocab)).to(dev)
    pos = torch.tensor([9], dtype=torch.int32, device=dev)
    res = []
    copy_stream = torch.cuda.Stream()
    for fs in (None, 2, 0):
        h = hs.device_model(dev, first_streamed=fs, copy_stream=copy_stream if fs is not None else None)
        ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
        out = torch.zeros(M, dtype=torch.int32, device=dev)
        logits = torch.zeros(M * hs.vocab, device=dev)
        for rep in range(2):  # second pass reuses the staging buffers
            h.verify_step(toks, M, pos, out, ws, logits)
        torch.cuda.synchronize()
        res.append((out.clone(), logits.clone(), [d.k_cache.clone() for d in h.keep["dls"]]))
    for r in res[1:]:
        assert torch.equal(r[0], res[0][0])
        assert torch.equal(r[1], res[0][1])
        for a, b in zip(r[2], res[0][2]):
            assert torch.equal(a, b)


@pytest.mark.parametrize("M,mix", [(2, "q4_0"), (2, "q4_k_m"), (3, "q4_k_m")])
def test_verify_few_tokens_equals_sequential_decode(M, mix):
    # two tokens per layer (three for the LM head) run the GEMV engine once
    # per token unless the layer is all Q4_K / Q6_K: a verify pass of M
    # tokens then equals M decode steps bitwise (Q4_0 layers); Q4_K_M layers
    # at M = 2 and every layer at M = 3 use the small-M GEMM and are held to
    # the oracle bar instead
    import torch
    dev = device()
    fmts = {"q4_0": wl.ALL_Q4_0, "q4_k_m": wl.Q4_K_M}[mix]
    hs = HostStack(wl.TINY, fmts, n_layer=3, vocab=901, max_ctx=40, n_past=13, wid=wl.W_TEST + 8)
    toks = wl.gen_tokens(wl.W_TEST + 8, M, hs.vocab)
    hv = hs.device_model(dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    logits = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    pos = torch.tensor([13], dtype=torch.int32, device=dev)
    hv.verify_step(torch.from_numpy(toks).to(dev), M, pos, out,
                   torch.zeros(hv.workspace_bytes(M), dtype=torch.uint8, device=dev), logits)
    hd = hs.device_model(dev)
    ws = torch.zeros(hd.workspace_bytes(1), dtype=torch.uint8, device=dev)
    seq_out, seq_lg, keep = [], [], []
    for i in range(M):
        b = torch.zeros(1, dtype=torch.int32, device=dev)
        lb = torch.zeros(hs.vocab, device=dev)
        t_i = torch.from_numpy(toks[i:i + 1]).to(dev)
        p_i = torch.tensor([13 + i], dtype=torch.int32, device=dev)
        hd.decode_step(t_i, p_i, b, ws, lb)
        seq_out.append(b)
        seq_lg.append(lb)
        keep += [t_i, p_i]
    torch.cuda.synchronize()
    g = logits.view(M, hs.vocab)
    if M == 2 and mix == "q4_0":
        assert torch.equal(out, torch.cat(seq_out))
        for i in range(M):
            assert torch.equal(g[i], seq_lg[i]), i
        for a, b in zip(hv.keep["dls"], hd.keep["dls"]):
            assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.v_cache, b.v_cache)
    nxt, _, ref, _ = hs.oracle_model().decode(toks, 13, want_logits=True)
    for i in range(M):
        assert rel_inf(g[i].cpu().numpy(), ref[i]) <= LOGIT_TOL
    assert out.cpu().numpy().tolist() == nxt.tolist()


@pytest.mark.parametrize("hidden,ffn", [(288, 352), (512, 416)])
def test_verify_rows_not_whole_256_blocks(hidden, ffn):
    # hidden 288: no layer hands its output on staged and the small-M LM head
    # (M = 4) stages its own input; ffn 416: only down stages its activation
    import torch
    dev = device()
    shape = wl.LayerShape(hidden=hidden, n_head=4, n_kv_head=2, head_dim=32, ffn=ffn)
    hs = HostStack(shape, wl.ALL_Q8_0, n_layer=3, vocab=611, max_ctx=40, n_past=11, wid=wl.W_TEST + 10,
                   emb_fmt=wl.Q8_0, head_fmt=wl.Q8_0)
    M = 4
    toks = wl.gen_tokens(wl.W_TEST + 10, M, hs.vocab)
    hv = hs.device_model(dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    logits = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    pos = torch.tensor([11], dtype=torch.int32, device=dev)
    hv.verify_step(torch.from_numpy(toks).to(dev), M, pos, out,
                   torch.zeros(hv.workspace_bytes(M), dtype=torch.uint8, device=dev), logits)
    torch.cuda.synchronize()
    nxt, _, ref, _ = hs.oracle_model().decode(toks, 11, want_logits=True)
    g = logits.view(M, hs.vocab)
    for i in range(M):
        assert rel_inf(g[i].cpu().numpy(), ref[i]) <= LOGIT_TOL, i
    assert out.cpu().numpy().tolist() == nxt.tolist()


@pytest.mark.parametrize("M", [1, 4])
def test_streamed_70b_shape_bitwise_equal_resident(M):
    # Llama-70B-shaped Q6_K layers (701,890,560-byte blobs), three of five
    # streamed from pinned host memory through the two staging buffers (the
    # third copy waits for the first buffer to be freed); the buffers start
    # as NaN bytes, so a layer read before its copy landed would show
    import torch
    dev = device()
    hs = HostStack(wl.LLAMA70B, wl.ALL_Q6_K, n_layer=5, vocab=2048, max_ctx=64, n_past=40, wid=wl.W_TEST + 9)
    toks = torch.from_numpy(wl.gen_tokens(wl.W_TEST + 9, M, hs.vocab)).to(dev)
    pos = torch.tensor([40], dtype=torch.int32, device=dev)
    copy_stream = torch.cuda.Stream()
    res = []
    for fs in (None, 2):
        say(f"70B-shaped stack of 5 Q6_K layers, first streamed {fs}, M={M}")
        h = hs.device_model(dev, first_streamed=fs, copy_stream=copy_stream if fs is not None else None)
        ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
        out = torch.zeros(M, dtype=torch.int32, device=dev)
        logits = torch.zeros(M * hs.vocab, device=dev)
        h.verify_step(toks, M, pos, out, ws, logits)
        torch.cuda.synchronize()
        res.append((out.clone(), logits.clone(), [d.k_cache.clone() for d in h.keep["dls"]]))
        del h, ws
        torch.cuda.empty_cache()
    assert not torch.isnan(res[0][1]).any()
    assert torch.equal(res[1][0], res[0][0])
    assert torch.equal(res[1][1], res[0][1])
    for a, b in zip(res[1][2], res[0][2]):
        assert torch.equal(a, b)
    say(f"streamed 70B-shaped stack, M={M}: tokens {res[0][0].tolist()} bitwise equal to resident")
