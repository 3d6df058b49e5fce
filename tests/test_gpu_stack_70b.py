"""Full-size parity: the 80-layer Llama-70B-shaped Q4_K_M stack (hidden 8192,
FFN 28672, 64/8 heads, f16 KV at context 4096, Q6_K embeddings and LM head of
128256 x 8192) decoded greedily on the GPU through nt_decode_step, the
bench's launch configuration, against the fp64 oracle on the same seeded
inputs.

Teacher forcing (the bar).  tests/golden/stack70b_q4km_teacher.{json,npz},
written by make_stack70b_golden.py from the oracle alone (~45 s per token on
16 cores), hold the oracle's own greedy decode of 64 steps from context 4096:
per step the input token, the greedy token, the full logit vector and the
f16 K/V rows the step appended to every layer.  Before GPU step s the rows
of oracle steps 0..s-1 are in the GPU caches (each step's rows are written
over the GPU's own right after it) and the input is the oracle's token, so
every step starts from the oracle's state and is compared on its own:
  - the greedy token equals the oracle's, at every step;
  - the full logit vector is within 5e-3 of the largest |logit|.
The K/V rows the GPU appended are compared with the oracle's and reported
(the largest deviation per step and the layer it is in): inside the stack a
layer's rows carry the deviation of every layer before it, and on these
random weights some layers amplify it (e.g. layers 54-56 at step 3), so the
rows are a diagnosis of where a step's deviation grows, while the bar is on
what the step outputs.
The conditioning estimate stored with each step (cond_err: how far the
oracle's own logits move when the residual stream entering every layer moves
by 1.5e-5 of its largest magnitude, the half step of the fixed point the GPU
holds activations in) says which steps are posed at the bar.  Where it
exceeds a tenth of the bar, the oracle itself cannot fix the logits to 5e-3
under deviations of the GPU's size, and the step is held to the token (its
logit deviation is reported, not asserted).

A step whose GPU token differs from the oracle's is checked for backward
stability instead: the GPU runs the step again layer by layer
(nt_decode_layer) from the embedding row, and every layer's output must be
within 1e-3 of the oracle's layer applied to the same GPU input (each GPU
layer is right on the state it was given; measured ~1e-5).  The two chains
then part only where the step itself amplifies deviations of that size: on
these random weights some attention heads choose between positions whose
scores differ by ~2e-5 of their size.  Reported beside it: the deepest layer
L whose GPU input is within 1e-3 of the oracle's own.  (The diagnosis behind
this reading, in the design notes: at step 22 the fp64 oracle continued
from the GPU's residual stream entering layer 17, 1.3e-4 from its own,
gives the GPU's token.)  Such steps are listed with their numbers in the
design notes.  A step without a stored estimate is held to both checks.

Free-running (a record, not the bar).  Without teacher forcing each step
appends K/V rows that the GPU rounds from fp32 and the oracle from fp64, and
this random-weight stack amplifies such differences at some steps, so the two
trajectories part after some steps (the stored record,
stack70b_q4km_greedy.json, shows where).  That test checks the first step,
where both start from the same state, and prints the rest.
"""
import json
import os

import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TEACHER_JSON = os.path.join(GOLDEN, "stack70b_q4km_teacher.json")
TEACHER_NPZ = os.path.join(GOLDEN, "stack70b_q4km_teacher.npz")
FREE_JSON = os.path.join(GOLDEN, "stack70b_q4km_greedy.json")
TOL = 5e-3
N_PAST = 4096


BACK_DEV = 1e-3  # per-layer accuracy required along the GPU's own chain (layer bar 5e-3; measured ~1e-5)


def backward_check(hs, om, h, kv, s, token, p, dev):
    """Step s layer by layer on the GPU (nt_decode_layer) and in the oracle,
    both from the embedding row (the oracle's caches hold its rows of steps
    < s).  Returns (the largest per-layer error of the GPU against the
    oracle's layer on the GPU's own input, its layer, L, the GPU's deviation
    from the oracle's chain entering layer L), L the deepest layer whose GPU
    input is within BACK_DEV of the oracle's."""
    import torch

    import oracle
    import quantized_decode_dequant_amd as nt
    sh = hs.shape
    for q in range(s):
        for li, r in zip(om.layers_in, kv[q]):
            li.k_cache[:, N_PAST + q, :] = r[0]
            li.v_cache[:, N_PAST + q, :] = r[1]
    rb = sh.hidden // oracle.block_elems(hs.emb_fmt) * oracle.block_bytes(hs.emb_fmt)
    xo = [oracle.dequant(hs.emb_fmt, hs.tok_emb[token * rb:(token + 1) * rb], 1, sh.hidden)]
    for li in om.layers_in:
        xo.append(oracle.layer(li, xo[-1], p))
    dls = h.keep["dls"]
    cfg = nt.layer_cfg(sh.hidden, sh.n_head, sh.n_kv_head, sh.head_dim, sh.ffn, hs.max_ctx, sh.rope_theta,
                       sh.rms_eps)
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    posd = torch.tensor([p], dtype=torch.int32, device=dev)
    x = torch.from_numpy(xo[0].astype(np.float32)).to(dev)
    xg = [xo[0]]
    local, at = 0.0, 0
    for l, d in enumerate(dls):
        nt.decode_layer(cfg, d.struct, x, 1, posd, ws)
        torch.cuda.synchronize()
        xg.append(x.cpu().numpy().astype(np.float64))
        # the oracle's layer on the GPU's input; both wrote their own K/V row at p
        e = rel_inf(xg[-1], oracle.layer(om.layers_in[l], xg[l], p))
        if e > local:
            local, at = e, l
    L = max(l for l in range(81) if rel_inf(xg[l], xo[l]) <= BACK_DEV)
    return local, at, L, rel_inf(xg[L], xo[L])


def load_teacher():
    g = json.load(open(TEACHER_JSON))
    z = np.load(TEACHER_NPZ)
    n = min(len(g["steps"]), z["kv_rows"].shape[0], z["logits"].shape[0])
    return g, z["kv_rows"][:n], z["logits"][:n], n


@pytest.mark.timeout(900)
def test_stack_70b_q4_k_m_teacher_forced():
    import torch
    dev = device()  # before the 45 GB of host inputs are generated
    g, kv, ref_logits, n = load_teacher()
    say(f"teacher-forced 70B stack: {n} stored oracle steps")
    assert n >= 1
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=128256, max_ctx=N_PAST + n, n_past=N_PAST,
                   wid=wl.W_STACK_70B)
    assert g["first_token"] == hs.first_token and g["n_past"] == N_PAST
    h = hs.device_model(dev)
    dls = h.keep["dls"]
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    token_only, backward = [], []
    worst, kv_worst = 0.0, 0.0
    om = None
    for s, st in enumerate(g["steps"][:n]):
        p = N_PAST + s
        assert st["pos"] == p and st["token_in"] == (hs.first_token if s == 0 else g["steps"][s - 1]["next"])
        tok.fill_(st["token_in"])
        pos.fill_(p)
        h.decode_step(tok, pos, nxt, ws, logits)
        torch.cuda.synchronize()
        got = logits.cpu().numpy().astype(np.float64)
        err = rel_inf(got, ref_logits[s])
        gpu_tok = int(nxt.item())
        assert np.isfinite(got).all() and gpu_tok == int(np.argmax(got)), s
        cond = st.get("cond_err")
        ill = cond is not None and cond > TOL / 10
        # the rows this step appended, against the oracle's
        kv_err, kv_at = 0.0, None
        for l, d in enumerate(dls):
            for c, cache in enumerate((d.k_cache, d.v_cache)):
                mine = cache[:, p, :].cpu().numpy().view(np.float16).astype(np.float64)
                e = rel_inf(mine, kv[s, l, c].view(np.float16).astype(np.float64))
                if e > kv_err:
                    kv_err, kv_at = e, (l, "KV"[c])
        back = None
        if gpu_tok != st["next"]:
            if om is None:
                om = hs.oracle_model()
            back = backward_check(hs, om, h, kv, s, st["token_in"], p, dev)
        # the next step starts from the oracle's state
        for l, d in enumerate(dls):
            for c, cache in enumerate((d.k_cache, d.v_cache)):
                cache[:, p, :] = torch.from_numpy(kv[s, l, c].view(np.int16)).to(dev)
        say(f"step {s}: gpu {gpu_tok} oracle {st['next']} margin {st['margin']:.4g} logits err {err:.2e} "
            f"appended K/V err {kv_err:.2e} (layer {kv_at[0]} {kv_at[1]})" + (f"; conditioning {cond:.2e}" if cond is not None else "")
            + (" (token only)" if ill and back is None else "")
            + (f" (backward check: every GPU layer within {back[0]:.2e} of the oracle's on the same input (layer "
               f"{back[1]}); the GPU's chain within {BACK_DEV} of the oracle's up to layer {back[2]} "
               f"({back[3]:.2e})" if back else ""))
        if back is not None:
            assert back[0] <= BACK_DEV, s
            backward.append((s, back[1], back[0]))
            continue
        if ill:
            token_only.append(s)
        else:
            assert err <= TOL, s
            worst = max(worst, err)
        kv_worst = max(kv_worst, kv_err)
    say(f"teacher-forced: {n} steps, the oracle's token at every step except {[b[0] for b in backward]} "
        f"(backward stability, (step, layer, largest per-layer error): {backward}); "
        f"at the {n - len(token_only) - len(backward)} steps posed at the bar, logits within {worst:.2e} of the largest |logit| "
        f"(bar {TOL}); token-only steps {token_only}; appended K/V rows within {kv_worst:.2e} of their largest "
        f"magnitude")


# verify windows (M, first step): every step of each is posed at the bar
VERIFY_WINDOWS = [(4, 0), (4, 28), (4, 36), (4, 44), (4, 52), (4, 60), (2, 0), (2, 30), (2, 50), (3, 1), (3, 33),
                  (3, 55), (8, 28), (8, 40), (8, 56)]


@pytest.mark.timeout(600)
def test_stack_70b_q4_k_m_verify_passes_teacher_forced():
    """Verify passes (M = 2, 3, 4 and 8: the engine per token, the paired /
    split small-M forms and the plain one) over windows of the stored
    trajectory.  The caches hold the oracle's rows of every step before the
    window; a pass over the window's M input tokens appends the rows of its
    own earlier tokens on the GPU, so row i starts from the oracle's state up
    to the window and from the GPU's own rows inside it.  Each row is held to
    the bar (logits within 5e-3 of the largest |logit|, the oracle's token);
    the windows are chosen among steps whose conditioning estimate poses them
    at the bar."""
    import torch
    dev = device()
    g, kv, ref_logits, n = load_teacher()
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=128256, max_ctx=N_PAST + n, n_past=N_PAST,
                   wid=wl.W_STACK_70B)
    h = hs.device_model(dev)
    dls = h.keep["dls"]

    def put_rows(s):
        for l, d in enumerate(dls):
            for c, cache in enumerate((d.k_cache, d.v_cache)):
                cache[:, N_PAST + s, :] = torch.from_numpy(kv[s, l, c].view(np.int16)).to(dev)

    for s in range(n):
        put_rows(s)
    worst = 0.0
    for M, s0 in VERIFY_WINDOWS:
        if s0 + M > n:
            continue
        steps = g["steps"][s0:s0 + M]
        assert all(st.get("cond_err") is not None and st["cond_err"] <= TOL / 10 for st in steps), (M, s0)
        ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
        toks = torch.tensor([st["token_in"] for st in steps], dtype=torch.int32, device=dev)
        pos = torch.tensor([N_PAST + s0], dtype=torch.int32, device=dev)
        out = torch.zeros(M, dtype=torch.int32, device=dev)
        lg = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
        h.verify_step(toks, M, pos, out, ws, lg)
        torch.cuda.synchronize()
        got = lg.view(M, hs.vocab).cpu().numpy().astype(np.float64)
        errs = [rel_inf(got[i], ref_logits[s0 + i]) for i in range(M)]
        say(f"verify M={M} from step {s0}: logits within {['%.2e' % e for e in errs]}, tokens "
            f"{out.cpu().numpy().tolist()} (oracle {[st['next'] for st in steps]})")
        for i, st in enumerate(steps):
            assert errs[i] <= TOL, (M, s0, i)
            assert int(out[i].item()) == st["next"], (M, s0, i)
        worst = max(worst, max(errs))
        for i in range(M):
            put_rows(s0 + i)  # the next window starts from the oracle's rows again
        del ws
    say(f"verify windows: logits within {worst:.2e} of the largest |logit| (bar {TOL}), every token the oracle's")


@pytest.mark.timeout(600)
def test_stack_70b_q4_k_m_free_running_record():
    import torch
    dev = device()
    g = json.load(open(FREE_JSON))
    steps = len(g["steps"])
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=128256, max_ctx=N_PAST + steps, n_past=N_PAST,
                   wid=wl.W_STACK_70B)
    assert g["first_token"] == hs.first_token
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([N_PAST], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.zeros(hs.vocab, dtype=torch.float32, device=dev)
    idx = np.asarray(g["sample_idx"])
    parted = None
    for s, st in enumerate(g["steps"]):
        h.decode_step(tok, pos, nxt, ws, logits)
        torch.cuda.synchronize()
        got = logits.cpu().numpy()
        err = float(np.abs(got[idx] - np.asarray(st["sample_logits"])).max() / st["logit_max_abs"])
        same = int(nxt.item()) == st["next"]
        say(f"free-running step {s}: gpu {int(nxt.item())} oracle {st['next']} sampled logits err {err:.2e}")
        if s == 0:
            # both start from the same state here
            assert same and err <= TOL
        if not same:
            parted = s
            break
        tok.copy_(nxt)
        pos += 1
    say(f"free-running trajectories " + (f"part at step {parted}" if parted is not None else
                                         f"agree over all {steps} stored steps"))
