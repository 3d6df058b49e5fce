"""A decode step captured in a HIP graph and replayed: token and position
live on the device, so one captured step (plus the token hand-off and the
position increment) can be replayed for successive tokens.

Bar: every replay gives bitwise the token, logits and KV cache row of the
same step run eagerly (the kernels are deterministic).  Between replays the
program does its own eager work and synchronizes.
"""
import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu


def _stack():
    return HostStack(wl.TINY, wl.Q4_K_M, n_layer=3, vocab=700, max_ctx=40, n_past=12, wid=wl.W_TEST + 9)


def _eager(hs, steps):
    import torch
    dev = device()
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([hs.n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    out = []
    for _ in range(steps):
        h.decode_step(tok, pos, nxt, ws, logits)
        tok.copy_(nxt)
        pos.add_(1)
        torch.cuda.synchronize()
        kc = h.keep["dls"][-1].k_cache.cpu().numpy().copy()
        out.append((int(nxt.item()), logits.cpu().numpy().copy(), kc))
    return out


def test_decode_step_graph_replays_match_eager():
    import torch
    hs = _stack()
    steps = 5
    ref = _eager(hs, steps)
    dev = device()
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([hs.n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # warm-up outside the capture (first-call setup); it writes the KV
        # row at n_past, which the first replay rewrites with the same values
        h.decode_step(tok, pos, nxt, ws, logits)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        h.decode_step(tok, pos, nxt, ws, logits)
        tok.copy_(nxt)
        pos.add_(1)
    tok.fill_(hs.first_token)
    pos.fill_(hs.n_past)
    torch.cuda.synchronize()
    scratch = torch.arange(4096, dtype=torch.float32, device=dev)
    for s in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        got_tok = int(tok.item())
        got_lg = logits.cpu().numpy()
        got_kc = h.keep["dls"][-1].k_cache.cpu().numpy()
        say(f"replay {s}: token {got_tok} (eager {ref[s][0]})")
        assert got_tok == ref[s][0]
        assert np.array_equal(got_lg, ref[s][1])
        assert np.array_equal(got_kc, ref[s][2])
        assert int(pos.item()) == hs.n_past + s + 1
        # the program's own eager work between replays
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
