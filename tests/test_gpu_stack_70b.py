"""Full-size parity: the 80-layer Llama-70B-shaped Q4_K_M stack (hidden 8192,
FFN 28672, 64/8 heads, f16 KV at context 4096, Q6_K embeddings and LM head of
128256 x 8192) decoded greedily on the GPU and by the fp64 oracle from the
same seeded inputs.  Bar: identical greedy tokens; logits within 5e-3.

One step by default (the oracle needs ~45 s per token on 16 cores); set
NT_STACK70B_STEPS for more.  Needs ~45 GB of host memory.
"""
import os

import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_stack_70b_q4_k_m_greedy():
    import torch
    steps = int(os.environ.get("NT_STACK70B_STEPS", "1"))
    n_past = 4096
    say("generating the 80-layer 70B-shaped stack")
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=128256, max_ctx=n_past + steps, n_past=n_past,
                   wid=wl.W_STACK_70B)
    dev = device()
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    g_toks, g_lgs = [], []
    for s in range(steps):
        h.decode_step(tok, pos, nxt, ws, logits)
        torch.cuda.synchronize()
        g_toks.append(int(nxt.item()))
        g_lgs.append(logits.cpu().numpy())
        tok.copy_(nxt)
        pos += 1
    del h
    torch.cuda.empty_cache()
    om = hs.oracle_model()
    t = hs.first_token
    for s in range(steps):
        say(f"oracle step {s}")
        nxt_o, margin, lg, _ = om.decode([t], n_past + s, want_logits=True)
        err = rel_inf(g_lgs[s], lg[0])
        say(f"step {s}: gpu {g_toks[s]} oracle {int(nxt_o[0])} margin {margin[0]:.4g} logits rel err {err:.2e}")
        assert err <= 5e-3
        assert g_toks[s] == int(nxt_o[0])
        t = int(nxt_o[0])
