"""Writes tests/golden/stack70b_q4km_greedy.json: the fp64 oracle's greedy
decode of the 80-layer Llama-70B-shaped Q4_K_M stack (hidden 8192, FFN 28672,
64/8 heads, f16 KV at context 4096, Q6_K embeddings and LM head of
128256 x 8192) from the seeded inputs the GPU test builds.

Calls only the oracle (and the seeded input generator).  Per step it stores
the input token and position, the greedy token, the top-1/top-2 margin, the
largest |logit|, the top five (index, logit) pairs and the logits at 256
fixed indices, so that a GPU run can be checked token by token and on sampled
logits without recomputing the oracle (~45 s per token on 16 cores).

With --perturb-seed S it instead reruns the stored steps (same input tokens)
with one f16 ulp added to or taken from a random 10% of every layer's past
K/V cache entries -- the size of the differences between the GPU's cache
entries (rounded from fp32) and the oracle's (rounded from fp64) -- and
stores, per step, how far the oracle's own sampled logits move
(perturbed_err, relative to the largest |logit|).  Steps where the stack
amplifies such a perturbation are where the GPU's logits may differ by more
than the rounding bar while the tokens still agree.

usage: python tests/golden/make_stack70b_golden.py --steps 22
       python tests/golden/make_stack70b_golden.py --perturb-seed 5
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from synth import workloads as wl  # noqa: E402
from tests.stack_util import HostStack  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stack70b_q4km_greedy.json")
N_PAST = 4096
VOCAB = 128256
N_SAMPLE = 256


def sample_indices() -> list:
    """256 distinct logit indices spread over the vocabulary (fixed, not random)."""
    return [int(i) for i in np.linspace(0, VOCAB - 1, N_SAMPLE).round().astype(np.int64)]


def perturb_past(om, n_past: int, seed: int) -> None:
    """One f16 ulp up or down in a random 10% of the finite, non-zero past
    K/V entries of every layer of the oracle's own caches."""
    rng = np.random.default_rng(seed)
    for li in om.layers_in:
        for c in (li.k_cache, li.v_cache):
            bits = c[:, :n_past, :].view(np.uint16)
            pick = rng.random(bits.shape) < 0.1
            nb = bits.astype(np.int32) + np.where(rng.random(bits.shape) < 0.5, 1, -1)
            ok = pick & ((bits & 0x7C00) != 0x7C00) & ((nb & 0x7C00) != 0x7C00) & ((bits & 0x7FFF) != 0)
            bits[ok] = nb[ok].astype(np.uint16)


def perturbed(args):
    g = json.load(open(args.out))
    steps = g["steps"]
    t0 = time.time()
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=VOCAB, max_ctx=N_PAST + len(steps), n_past=N_PAST,
                   wid=wl.W_STACK_70B)
    om = hs.oracle_model()
    perturb_past(om, N_PAST, args.perturb_seed)
    idx = np.asarray(g["sample_idx"])
    for s, st in enumerate(steps):
        nxt, margin, lg, _ = om.decode([st["token_in"]], st["pos"], want_logits=True)
        err = float(np.abs(lg[0][idx] - np.asarray(st["sample_logits"])).max() / st["logit_max_abs"])
        st["perturbed_err"] = err
        st["perturbed_next"] = int(nxt[0])
        print(f"step {s}: perturbed oracle {int(nxt[0])} (stored {st['next']}), sampled logits moved {err:.2e} "
              f"after {time.time() - t0:.0f} s", flush=True)
        g["perturb_seed"] = args.perturb_seed
        with open(args.out, "w") as f:
            json.dump(g, f)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--out", default=OUT)
    ap.add_argument("--perturb-seed", type=int, default=None)
    args = ap.parse_args()
    if args.perturb_seed is not None:
        perturbed(args)
        return
    t0 = time.time()
    print("generating the 80-layer 70B-shaped stack", flush=True)
    hs = HostStack(wl.LLAMA70B, wl.Q4_K_M, n_layer=80, vocab=VOCAB, max_ctx=N_PAST + args.steps, n_past=N_PAST,
                   wid=wl.W_STACK_70B)
    om = hs.oracle_model()
    idx = sample_indices()
    steps = []
    t = hs.first_token
    for s in range(args.steps):
        nxt, margin, lg, _ = om.decode([t], N_PAST + s, want_logits=True)
        l0 = lg[0]
        top = np.argsort(-l0, kind="stable")[:5]
        steps.append({"token_in": int(t), "pos": N_PAST + s, "next": int(nxt[0]), "margin": float(margin[0]),
                      "logit_max_abs": float(np.abs(l0).max()),
                      "top5": [[int(i), float(l0[i])] for i in top],
                      "sample_logits": [float(l0[i]) for i in idx]})
        print(f"step {s}: token {int(t)} -> {int(nxt[0])} (margin {float(margin[0]):.4g}) "
              f"after {time.time() - t0:.0f} s", flush=True)
        t = int(nxt[0])
        # written after every step, so a run cut short still leaves its steps
        with open(args.out, "w") as f:
            json.dump({"what": "fp64 oracle greedy decode of the 80-layer Llama-70B-shaped Q4_K_M stack, "
                               "context 4096, seeded inputs (synth workload W_STACK_70B)",
                       "script": "tests/golden/make_stack70b_golden.py", "first_token": hs.first_token,
                       "n_past": N_PAST, "vocab": VOCAB, "sample_idx": idx, "steps": steps}, f)
    print(f"wrote {len(steps)} steps to {args.out}", flush=True)


if __name__ == "__main__":
    main()
