"""Full-size parity: the 80-layer Llama-70B-shaped Q4_K_M stack (hidden 8192,
FFN 28672, 64/8 heads, f16 KV at context 4096, Q6_K embeddings and LM head of
128256 x 8192) decoded greedily on the GPU, in the bench's launch
configuration (nt_decode_step), against the fp64 oracle on the same seeded
inputs.  Bar: identical greedy tokens; logits within 5e-3 of the largest
|logit|.

The oracle's tokens and sampled logits for the first steps are stored in
tests/golden/stack70b_q4km_greedy.json (written by make_stack70b_golden.py,
which calls only the oracle; ~45 s per token on 16 cores), so the test
checks every stored step without recomputing it.  Without that file, or with
NT_STACK70B_LIVE=1, the oracle also runs here for NT_STACK70B_STEPS steps
(default 1; needs ~45 GB of host memory).

On these random weights the residual stream grows through the 80 layers
(logits of ~3400) and attention is close to a one-position choice, so at some
steps the stack amplifies rounding: the stored file also holds, per step, how
far the oracle's own logits move when 10% of its past cache entries change by
one f16 ulp (perturbed_err).  Logits are held to the bar at the steps where
that movement stays under a tenth of the bar, where the bar is meaningful.

The decode is a trajectory: each step appends K/V entries that the GPU
rounds from fp32 and the oracle from fp64, and the amplifying steps grow
those differences.  Tokens are identical for the first TRAJECTORY_STEPS
steps; at step 16 the two trajectories part (the GPU emits 123785, the
stored oracle 83067).  The oracle run on the GPU's own caches after step 15
gives the GPU's token with logits within 8.4e-4, and the oracle's own
trajectory flips a token at step 18 under the one-ulp perturbation, so the
parting is the stack's sensitivity, not a step the GPU computes wrongly.
The later stored steps are kept as the record and not compared.
"""
import json
import os

import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "stack70b_q4km_greedy.json")
TOL = 5e-3
STABLE = TOL / 10  # oracle's own logit movement under a one-ulp cache perturbation
TRAJECTORY_STEPS = 16  # stored steps before the GPU and oracle trajectories part


def gpu_greedy(hs, n_past, steps, dev):
    import torch
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    toks, lgs = [], []
    for s in range(steps):
        h.decode_step(tok, pos, nxt, ws, logits)
        torch.cuda.synchronize()
        toks.append(int(nxt.item()))
        lgs.append(logits.cpu().numpy())
        tok.copy_(nxt)
        pos += 1
    del h
    torch.cuda.empty_cache()
    return toks, lgs


@pytest.mark.timeout(900)
def test_stack_70b_q4_k_m_greedy():
    dev = device()  # before the 45 GB of host inputs are generated
    golden = json.load(open(GOLDEN)) if os.path.exists(GOLDEN) else None
    live = golden is None or os.environ.get("NT_STACK70B_LIVE") == "1"
    n_live = int(os.environ.get("NT_STACK70B_STEPS", "1")) if live else 0
    n_gold = min(len(golden["steps"]), TRAJECTORY_STEPS) if golden else 0
    steps = max(n_live, n_gold)
    n_past = 4096
    say(f"generating the 80-layer 70B-shaped stack ({steps} steps: {n_gold} stored, {n_live} live)")
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=128256, max_ctx=n_past + steps, n_past=n_past,
                   wid=wl.W_STACK_70B)
    g_toks, g_lgs = gpu_greedy(hs, n_past, steps, dev)
    if golden:
        assert golden["first_token"] == hs.first_token and golden["n_past"] == n_past
        idx = np.asarray(golden["sample_idx"])
        n_checked = 0
        for s, st in enumerate(golden["steps"][:n_gold]):
            got = g_lgs[s]
            err = float(np.abs(got[idx] - np.asarray(st["sample_logits"])).max() / st["logit_max_abs"])
            top = np.abs(np.array([got[i] - v for i, v in st["top5"]])).max() / st["logit_max_abs"]
            moved = st.get("perturbed_err", 0.0)
            stable = moved <= STABLE
            say(f"step {s}: gpu {g_toks[s]} oracle {st['next']} margin {st['margin']:.4g} "
                f"sampled logits err {err:.2e}, top-5 err {top:.2e}; oracle under perturbation {moved:.2e}"
                f"{'' if stable else ' (amplifying step: token only)'}")
            assert st["token_in"] == (hs.first_token if s == 0 else g_toks[s - 1])
            assert g_toks[s] == st["next"]
            if stable:
                assert err <= TOL and top <= TOL
                n_checked += 1
        assert n_checked >= n_gold // 2
    if n_live:
        om = hs.oracle_model()
        t = hs.first_token
        for s in range(n_live):
            say(f"oracle step {s}")
            nxt_o, margin, lg, _ = om.decode([t], n_past + s, want_logits=True)
            err = rel_inf(g_lgs[s], lg[0])
            say(f"step {s}: gpu {g_toks[s]} oracle {int(nxt_o[0])} margin {margin[0]:.4g} logits rel err {err:.2e}")
            assert err <= TOL
            assert g_toks[s] == int(nxt_o[0])
            t = int(nxt_o[0])
