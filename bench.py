#!/usr/bin/env python3
"""Benchmark: greedy batch-1 decode of an 80-layer Llama-70B-shaped Q4_K_M stack.

Workload: hidden 8192, 64 query / 8 kv heads, head_dim 128, FFN 28672; Q4_K
for Q/K/O/gate/up and Q6_K for V/down in every layer; embeddings and LM head
128256 x 8192 Q6_K; F16 KV cache holding 4096 past positions; greedy argmax.
A step is one decode token (every row of the hot path: block decode, GEMVs,
RMSNorm, RoPE, KV append, GQA attention, SwiGLU, residuals, LM head, argmax).
All inputs are seeded synthetic data of those shapes (no trained weights).

Prints one JSON line.  `value` is decode tokens/s with every input resident
in HBM; `roofline` is the dominant kernel (the fused gate/up + SwiGLU GEMV)
timed with HIP events on its launch stream inside the timed region;
`cpu_baseline` is the fp64 oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_decode_dequant_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str, launch_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    e = d.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def build_stack(n_layer: int, max_ctx: int, n_past: int, dev):
    """Seeded 70B-shaped stack, generated layer by layer on the host and copied to HBM."""
    import numpy as np
    import torch

    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    from synth import workloads as wl

    shape, fmts, wid = wl.LLAMA70B, wl.Q4_K_M, wl.W_STACK_70B
    t0 = time.time()
    layers = []
    for l in range(n_layer):
        li = wl.gen_layer(shape, fmts, wid, l, max_ctx, n_past)
        layers.append(DeviceLayer(li, dev))
        del li
        if l % 10 == 9:
            log(f"[bench] layers generated: {l + 1}/{n_layer} ({time.time() - t0:.0f} s)")
    vocab = 128256
    emb = torch.from_numpy(wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wid, 0, wl.T_TOK_EMB)).to(dev)
    head = torch.from_numpy(wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wid, 0, wl.T_LM_HEAD)).to(dev)
    norm = torch.from_numpy(wl.gen_gains(shape, wid, 0, wl.T_OUT_NORM)).to(dev)
    first = int(wl.gen_tokens(wid, 1, vocab)[0])
    cfg = cfg_of(shape, max_ctx)
    h = nt.ModelHandle(cfg, [d.struct for d in layers], vocab, emb, wl.Q6_K, head, wl.Q6_K, norm)
    h.keep = (layers, emb, head, norm)
    wbytes = sum(d.weight_bytes() for d in layers) + head.numel() + emb.numel() // vocab
    log(f"[bench] stack ready: {n_layer} layers, {wbytes / 1e9:.2f} GB weights ({time.time() - t0:.0f} s)")
    return h, first, vocab, wbytes, shape, fmts


def cpu_baseline(sample_layers: int, n_layer_full: int, n_past: int):
    """The oracle (as it stands) on one decode token through `sample_layers`
    layers of the same shapes plus the LM head, scaled to tokens/s of the
    full stack."""
    import numpy as np

    import oracle
    from synth import workloads as wl

    shape, fmts, wid = wl.LLAMA70B, wl.Q4_K_M, wl.W_STACK_70B
    max_ctx = n_past + 1
    layers = [wl.gen_layer(shape, fmts, wid, l, max_ctx, n_past) for l in range(sample_layers)]
    vocab = 128256
    emb = wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wid, 0, wl.T_TOK_EMB)
    head = wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wid, 0, wl.T_LM_HEAD)
    norm = wl.gen_gains(shape, wid, 0, wl.T_OUT_NORM)
    first = int(wl.gen_tokens(wid, 1, vocab)[0])
    m = oracle.OracleModel(shape, layers, wl.Q6_K, emb, wl.Q6_K, head, norm, vocab)
    t0 = time.time()
    x = np.zeros((1, shape.hidden))
    oracle.lib()  # load before timing
    t0 = time.time()
    m.decode([first], n_past)
    t_all = time.time() - t0
    # LM head alone, to scale only the layer part
    xn = np.ones(shape.hidden)
    t1 = time.time()
    oracle.gemv(wl.Q6_K, head, xn, vocab, shape.hidden)
    t_head = time.time() - t1
    t_layers = max(t_all - t_head, 1e-9)
    per_token = t_layers * n_layer_full / sample_layers + t_head
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return dict(value=1.0 / per_token, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"one decode token through {sample_layers} of {n_layer_full} 70B-shaped Q4_K_M layers "
                       f"(context {n_past}) plus the 128256x8192 Q6_K LM head, fp64; {t_all:.1f} s measured, "
                       f"layer time scaled x{n_layer_full / sample_layers:.0f}")


def read_ceiling(dev) -> float:
    """Achievable HBM read bandwidth: nt_read_probe over 8 x 256 MiB buffers
    in rotation (more than the 256 MB last-level cache)."""
    import torch

    import quantized_decode_dequant_amd as nt
    bufs = [torch.empty(256 << 20, dtype=torch.uint8, device=dev) for _ in range(8)]
    out = torch.zeros(4, dtype=torch.int32, device=dev)
    for i in range(4):
        nt.read_probe(bufs[i % 8], out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(32):
        nt.read_probe(bufs[i % 8], out)
    e1.record()
    torch.cuda.synchronize()
    gbs = 32 * (256 << 20) / (e0.elapsed_time(e1) / 1e3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return gbs


def summarize_profile(d: str) -> None:
    """Per-kernel table from rocprofv3 output: kernel durations (rocpd SQLite
    database of --kernel-trace) and mean counter values per dispatch (csv of --pmc)."""
    import csv
    import glob
    import sqlite3
    from collections import defaultdict

    def short(n):
        return n.replace("void ", "").replace("nt::(anonymous namespace)::", "").split("(")[0][:70]

    for db in sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True)):
        c = sqlite3.connect(db)
        rows = c.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
        print(f"{'kernel':70s} {'calls':>6s} {'total_us':>11s} {'avg_us':>9s} {'pct':>6s}")
        for name, calls, tot, avg, pct in rows:
            print(f"{short(name):70s} {calls:6d} {tot:11.1f} {avg:9.2f} {pct:6.2f}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(f)):
            agg[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, cs in agg.items():
            print(f"{k:70s} " + "  ".join(f"{n}={sum(v) / len(v):.6g} (n={len(v)})" for n, v in sorted(cs.items())))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--layers", type=int, default=80, help="stack depth (80 is the workload)")
    ap.add_argument("--cpu-sample-layers", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one device copy of 256 MiB (calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", metavar="DIR", help="print per-kernel statistics of a rocprofv3 output "
                    "directory (kernel trace or counter csv) and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profile(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the decode path is not sharded (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_decode_dequant_amd as nt

    dev = torch.device("cuda:0")
    n_past = 4096
    max_ctx = n_past + max(args.steps, args.warmup)
    h, first, vocab, wbytes, shape, fmts = build_stack(args.layers, max_ctx, n_past, dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([first], dtype=torch.int32, device=dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def run(k):
        for _ in range(k):
            h.decode_step(tok, pos, nxt, ws, None, stream)
            tok.copy_(nxt)
            pos.add_(1)

    if args.copy_probe:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE read 256 MiB each when the counters are exact
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    read_gbs = read_ceiling(dev)
    log(f"[bench] streaming-read ceiling (nt_read_probe): {read_gbs:.0f} GB/s")
    log(f"[bench] warmup {args.warmup} steps")
    run(args.warmup)
    torch.cuda.synchronize()
    # the timed steps decode from context 4096 again (the cache rows written
    # by the warmup are overwritten)
    tok.fill_(first)
    pos.fill_(n_past)
    torch.cuda.synchronize()
    nt.trace_begin(nt.TRACE_FFN_UP)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    tokens = []
    for _ in range(args.steps):
        h.decode_step(tok, pos, nxt, ws, None, stream)
        tokens.append(nxt.clone())
        tok.copy_(nxt)
        pos.add_(1)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_ffn, ffn_ms = nt.trace_end()
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / args.steps
    tok_s = args.steps / (gpu_ms / 1e3)
    toks = [int(t.item()) for t in tokens]
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/token, {tok_s:.2f} tok/s (wall {wall:.2f} s)")

    # dominant kernel: gate/up + SwiGLU, 2 x ffn x hidden Q4_K weights per launch
    q4k_row = nt.row_bytes(fmts["wg"], shape.hidden)
    ffn_bytes = 2 * shape.ffn * q4k_row + shape.hidden * 4 * 2 + shape.ffn * 4
    ffn_avg_s = ffn_ms / 1e3 / max(1, n_ffn)
    achieved = ffn_bytes / ffn_avg_s / 1e9
    traffic = counter_traffic("ffn_gate_up", ffn_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, {args.cpu_sample_layers} layers)")
        cpu = cpu_baseline(args.cpu_sample_layers, args.layers, n_past)

    out = {
        "metric": "quant GEMV effective GB/s (% HBM peak); decode tok/s for 70B-shaped Q4_K_M",
        "value": round(tok_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_k/q6_k weights, i8 dot products, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "llama70b-shaped Q4_K_M 80-layer greedy decode, f16 KV at context 4096",
            "layers": args.layers, "hidden": shape.hidden, "n_head": shape.n_head, "n_kv_head": shape.n_kv_head,
            "head_dim": shape.head_dim, "ffn": shape.ffn, "vocab": vocab, "context": n_past, "batch": 1,
            "weight_bytes_per_token": wbytes,
        },
        "weight_gbs": round(wbytes / (ms_per_step / 1e3) / 1e9, 1),
        "weight_roofline_frac": round(wbytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "read_ceiling_gbs": round(read_gbs, 1),
        "roofline": {
            "kernel": "k_qgemv<EPI_SWIGLU> (gate/up GEMV + SwiGLU, Q4_K 2x28672x8192)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "launches": n_ffn, "avg_launch_us": round(ffn_avg_s * 1e6, 2), "bytes_per_launch": ffn_bytes,
        },
        "cpu_baseline": cpu,
        "tokens_head": toks[:8],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
