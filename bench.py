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
`gemv` carries the GEMV half of the metric: the single Q8_0 4096x4096 GEMV
and the seven 70B-shaped Q4_K_M projections, each timed as HIP graph replays
over distinct weight copies (effective GB/s and fraction of 8 TB/s), with
the oracle's GB/s for the same GEMVs on this host's cores beside them.

Secondary workloads (`--workload`, one JSON line each; not the headline):
  gemv     the single Q8_0 4096x4096 GEMV and the seven 70B-shaped Q4_K_M
           projections, each rotated over distinct weight copies (more than
           the 256 MB last-level cache), timed as HIP graph replays of
           back-to-back launches: effective GB/s per GEMV.
  layer8b  one 8B-shaped Q4_0 decoder layer at position 512, over 32 distinct
           layers: GB/s per layer.
  decode8b greedy decode of a 32-layer Llama-8B-shaped Q8_0 stack from
           context 512 (the pages' one decode figure is for Llama 8B Q8_0).
  gemm_small  the verify pass's small-M GEMM on the 70B-shaped gate (Q4_K)
           and down (Q6_K) matrices for M = 1, 2, 4, 8: weight GB/s per pass.
  verify   80 Q6_K 70B-shaped layers, 36 resident and 44 streamed from
           pinned host memory through two HBM staging buffers, verify passes
           of M = 1, 2, 4, 8 tokens from context 4096: verified positions/s,
           host-to-device GB/s against a copy-only run, and the overlap of
           copies with compute against an all-resident run.
  spec     self-speculative rounds on the same stack (the 36 resident layers
           draft K = 3 or 7 tokens, one streamed verify pass checks them):
           round, draft-step and verify times, tokens emitted per round, and
           plain streamed decode with 20 calibrated layers skipped.
  tiers    nt_plan_tiers places the 80-layer Q4_K_M and Q6_K stacks within
           24 and 48 GB of device memory; greedy decode time at each
           placement.
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


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))


def cpu_baseline(sample_layers: int, n_layer_full: int, n_past: int):
    """The oracle (as it stands) on one decode token through `sample_layers`
    layers of the same shapes plus the LM head, scaled to tokens/s of the
    full stack: the layers all have the same shapes and work, so the
    80-layer time is the sampled layers' time times 80 / sample_layers."""
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
    return dict(value=1.0 / per_token, unit="tokens/s", cores=oracle_threads(), kind="oracle",
                cpu=cpu_model(),
                sample=f"one decode token through {sample_layers} of {n_layer_full} 70B-shaped Q4_K_M layers "
                       f"(context {n_past}) plus the 128256x8192 Q6_K LM head, fp64; {t_all:.1f} s measured, "
                       f"layer time scaled x{n_layer_full / sample_layers:.0f}")


def read_ceiling(dev) -> float:
    """Achievable HBM read bandwidth: nt_read_probe over one 2 GiB buffer
    (eight times the 256 MB last-level cache), 8 launches.  Each launch reads
    2 GiB, so its start and end (~2-3 us) cost under 1%; launches of 256 MiB
    read ~6% below this."""
    import torch

    import quantized_decode_dequant_amd as nt
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    out = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        nt.read_probe(buf, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(8):
        nt.read_probe(buf, out)
    e1.record()
    torch.cuda.synchronize()
    gbs = 8 * (2 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf
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


def timed(fn, n: int) -> float:
    """Mean milliseconds of fn() over n calls on the current stream (after one warm call)."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def timed_graph(fn, n: int, reps: int = 5) -> float:
    """Mean milliseconds per fn() call with n calls captured in one HIP graph
    and the graph replayed `reps` times (after one eager warm call and one
    warm replay): the launches run back to back on the device, without the
    host's per-call cost between them."""
    import torch
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * n)


def gemv_cases(extra: bool):
    """(name, format, rows, cols, workload id, tensor tag): the single Q8_0
    4096x4096 GEMV and the seven 70B-shaped Q4_K_M projections; with
    `extra`, the pages' other formats at the same kinds of shape."""
    import synth
    from synth import workloads as wl
    cases = [("q8_0_4096x4096", wl.Q8_0, 4096, 4096, wl.W_GEMV_Q8, 0)]
    for n in ["wq", "wk", "wv", "wo", "wg", "wu", "wd"]:
        r, c = wl.LLAMA70B.mat_shape(n)
        cases.append((f"70b_{n}_{synth.FMT_NAMES[wl.Q4_K_M[n]]}_{r}x{c}", wl.Q4_K_M[n], r, c, wl.W_GEMV_70B,
                      wl.MAT_TAG[n]))
    if extra:
        for n in ["wq", "wg", "wd"]:
            r, c = wl.LLAMA70B.mat_shape(n)
            cases.append((f"x70b_{n}_q5_k_{r}x{c}", wl.Q5_K, r, c, wl.W_GEMV_70B, 20 + wl.MAT_TAG[n]))
        cases.append(("xf16_4096x4096", wl.F16, 4096, 4096, wl.W_GEMV_Q8, 1))
        cases.append(("xf32_4096x4096", wl.F32, 4096, 4096, wl.W_GEMV_Q8, 2))
    return cases


def oracle_gemv_gbs(cases) -> dict:
    """The oracle's GEMV (fp64, as it stands) on the same weights and
    activation as each case: weight GB/s on this host's cores."""
    import oracle
    from synth import workloads as wl
    oracle.lib()
    out = {}
    for name, fmt, rows, cols, wid, tag in cases:
        W = wl.gen_matrix(fmt, rows, cols, wid, 0, tag)
        x = wl.gen_x(cols, wid)
        t0 = time.perf_counter()
        oracle.gemv(fmt, W, x, rows, cols)
        dt = time.perf_counter() - t0
        out[name] = round((W.nbytes + 4 * cols + 4 * rows) / dt / 1e9, 3)
    return out


def time_gemvs(dev, cases) -> dict:
    """Effective GB/s of each GEMV case, weights rotated over distinct copies
    so no launch finds them in the last-level cache; times are HIP graph
    replays of back-to-back launches (eager launches beside them)."""
    import torch

    import quantized_decode_dequant_amd as nt
    from synth import workloads as wl

    res = {}
    for name, fmt, rows, cols, wid, tag in cases:
        wbytes = rows * nt.row_bytes(fmt, cols)
        ncopy = 32 if name.startswith("q8_0") else max(2, -(-512_000_000 // wbytes))
        base = torch.from_numpy(wl.gen_matrix(fmt, rows, cols, wid, 0, tag)).to(dev)
        Ws = [base.clone() for _ in range(ncopy)]
        x = torch.from_numpy(wl.gen_x(cols, wid)).to(dev)
        y = torch.empty(rows, dtype=torch.float32, device=dev)
        it = [0]

        def one():
            nt.gemv_q(fmt, Ws[it[0] % ncopy], x, y, rows, cols)
            it[0] += 1

        n_calls = max(100, 2 * ncopy)
        ms_eager = timed(one, n_calls)
        ms = timed_graph(one, n_calls)
        alg = wbytes + 4 * cols + 4 * rows
        res[name] = dict(us=round(ms * 1e3, 2), gbs=round(alg / ms / 1e6, 1),
                         frac_peak=round(alg / ms / 1e6 / HBM_PEAK_GBS, 4), copies=ncopy, alg_bytes=alg,
                         us_eager_launches=round(ms_eager * 1e3, 2))
        log(f"[bench] {name}: {ms * 1e3:.1f} us ({ms_eager * 1e3:.1f} us launched one by one from the host), "
            f"{alg / ms / 1e6:.0f} GB/s")
        del Ws, base
        torch.cuda.empty_cache()
    return res


def seven_gemv_gbs(res: dict) -> float:
    """Effective GB/s of the seven 70B projections run one after the other."""
    b = sum(v["alg_bytes"] for k, v in res.items() if k.startswith("70b"))
    us = sum(v["us"] for k, v in res.items() if k.startswith("70b"))
    return round(b / us / 1e3, 1)


def workload_gemv(dev) -> dict:
    """The single Q8_0 4096x4096 GEMV and the 70B-shaped projections (and the
    pages' other formats): effective GB/s of each GEMV."""
    read_gbs = read_ceiling(dev)
    res = time_gemvs(dev, gemv_cases(extra=True))
    return {"metric": "quant GEMV effective GB/s (% HBM peak)", "unit": "GB/s", "n_gpus": 1,
            "value": res["q8_0_4096x4096"]["gbs"], "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "single GEMVs: Q8_0 4096x4096 and the 70B-shaped Q4_K_M projections "
                                   "(plus, prefixed x, Q5_K 70B-shaped and F16/F32 4096x4096), "
                                   "weights rotated over distinct copies; times are HIP graph replays of "
                                   "back-to-back launches"},
            "read_ceiling_gbs": round(read_gbs, 1), "gemv": res,
            "seven_gemv_layer_gbs": seven_gemv_gbs(res)}


def workload_layer8b(dev) -> dict:
    """One 8B-shaped Q4_0 layer at position 512, timed over 32
    distinct layers (3.9 GB of weights, more than the last-level cache)."""
    import torch

    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    from synth import workloads as wl

    shape, n_past, nl = wl.LLAMA8B, 512, 32
    cfg = cfg_of(shape, n_past + 1)
    li = wl.gen_layer(shape, wl.ALL_Q4_0, wl.W_LAYER_8B, 0, n_past + 1, n_past)
    dls = [DeviceLayer(li, dev) for _ in range(nl)]
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    x = torch.from_numpy(wl.gen_x(shape.hidden, wl.W_LAYER_8B)).to(dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    it = [0]

    def one():
        nt.decode_layer(cfg, dls[it[0] % nl].struct, x, 1, pos, ws)
        it[0] += 1

    ms = timed(one, 4 * nl)
    wbytes = dls[0].weight_bytes()
    kv = 2 * shape.n_kv_head * (n_past + 1) * shape.head_dim * 2
    alg = wbytes + kv + 2 * shape.n_kv_head * shape.head_dim * 2 + 4 * (3 * shape.hidden + shape.ffn)
    return {"metric": "8B-shaped Q4_0 decoder layer effective GB/s", "unit": "GB/s", "n_gpus": 1,
            "value": round(alg / ms / 1e6, 1), "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "llama8b-shaped Q4_0 layer, position 512, 32 distinct layers"},
            "us_per_layer": round(ms * 1e3, 2), "alg_bytes": alg, "frac_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}


def workload_gemm_small(dev) -> dict:
    """Small-M GEMMs of the verify pass (nt_gemm_q_small): the 70B-shaped
    Q4_K gate (28672 x 8192) and Q6_K down (8192 x 28672) matrices for M = 1,
    2, 4, 8 tokens, weights rotated over distinct copies, timed as HIP graph
    replays.  M = 1 is the GEMV engine; M >= 2 reads the weights once for all
    tokens on int8 MFMA."""
    import torch

    import quantized_decode_dequant_amd as nt
    from synth import workloads as wl

    res = {}
    for n in ("wg", "wd"):
        fmt = wl.Q4_K_M[n]
        rows, cols = wl.LLAMA70B.mat_shape(n)
        wbytes = rows * nt.row_bytes(fmt, cols)
        ncopy = max(2, -(-512_000_000 // wbytes))
        base = torch.from_numpy(wl.gen_matrix(fmt, rows, cols, wl.W_GEMV_70B, 0, wl.MAT_TAG[n])).to(dev)
        Ws = [base.clone() for _ in range(ncopy)]
        X = torch.from_numpy(wl.gen_x(8 * cols, wl.W_GEMV_70B)).to(dev).view(8, cols)
        Y = torch.empty(8, rows, dtype=torch.float32, device=dev)
        for M in (1, 2, 4, 8):
            ws_bytes = nt.gemm_q_small_workspace_bytes(M, rows, cols)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            it = [0]

            def one():
                nt.gemm_q_small(fmt, Ws[it[0] % ncopy], X, Y, M, rows, cols, ws)
                it[0] += 1

            ms = timed_graph(one, max(20, 2 * ncopy))
            alg = wbytes + 4 * M * (rows + cols)
            key = f"70b_{n}_{'q4_k' if fmt == wl.Q4_K else 'q6_k'}_{rows}x{cols}_M{M}"
            res[key] = {"us": round(ms * 1e3, 2), "weight_gbs": round(wbytes / ms / 1e6, 1),
                        "token_rows_per_us": round(M * rows / (ms * 1e3), 1), "alg_bytes": alg}
            log(f"[bench] {key}: {ms * 1e3:.1f} us, weights at {wbytes / ms / 1e6:.0f} GB/s")
        del Ws, base
    return {"metric": "small-M GEMM: weight GB/s per pass of M tokens", "unit": "GB/s", "n_gpus": 1,
            "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "70B-shaped Q4_K gate and Q6_K down matrices, M = 1, 2, 4, 8 tokens, weights "
                                   "rotated over distinct copies, HIP graph replays"},
            "gemm_small": res}


def workload_decode8b(dev, steps: int) -> dict:
    """Greedy decode of a 32-layer Llama-8B-shaped stack in Q8_0 (hidden 4096,
    32/8 heads, FFN 14336, Q8_0 embeddings and LM head of 128256 x 4096), from
    context 512: the configuration behind the only decode figure the pages
    give (Llama 8B Q8_0 on an RTX 3090; context not stated there)."""
    import torch

    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    from synth import workloads as wl

    shape, fmts, wid, n_layer, vocab, n_past = wl.LLAMA8B, wl.ALL_Q8_0, wl.W_LAYER_8B, 32, 128256, 512
    max_ctx = n_past + steps + 1
    layers = [DeviceLayer(wl.gen_layer(shape, fmts, wid, l, max_ctx, n_past), dev) for l in range(n_layer)]
    emb = torch.from_numpy(wl.gen_matrix(wl.Q8_0, vocab, shape.hidden, wid, 0, wl.T_TOK_EMB)).to(dev)
    head = torch.from_numpy(wl.gen_matrix(wl.Q8_0, vocab, shape.hidden, wid, 0, wl.T_LM_HEAD)).to(dev)
    norm = torch.from_numpy(wl.gen_gains(shape, wid, 0, wl.T_OUT_NORM)).to(dev)
    h = nt.ModelHandle(cfg_of(shape, max_ctx), [d.struct for d in layers], vocab, emb, wl.Q8_0, head, wl.Q8_0, norm)
    wbytes = sum(d.weight_bytes() for d in layers) + head.numel() + emb.numel() // vocab
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    first = int(wl.gen_tokens(wid, 1, vocab)[0])
    tok = torch.tensor([first], dtype=torch.int32, device=dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    h.decode_step(tok, pos, nxt, ws, None, stream)  # warm
    torch.cuda.synchronize()
    tok.fill_(first)
    pos.fill_(n_past)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        h.decode_step(tok, pos, nxt, ws, None, stream)
        tok.copy_(nxt)
        pos.add_(1)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    log(f"[bench] decode8b: {ms:.3f} ms per token, {1e3 / ms:.1f} tok/s, {wbytes / ms / 1e6:.0f} GB/s of weights")
    return {"metric": "decode tok/s, Llama-8B-shaped Q8_0", "unit": "tokens/s", "n_gpus": 1,
            "value": round(1e3 / ms, 2), "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "32-layer llama8b-shaped Q8_0 greedy decode (Q8_0 embeddings and LM head), "
                                   "f16 KV from context 512", "steps": steps},
            "ms_per_token": round(ms, 4), "weight_bytes_per_token": wbytes,
            "weight_gbs": round(wbytes / ms / 1e6, 1),
            "pages_figure_for_context": {"value": 48.9, "unit": "tokens/s", "hardware": "RTX 3090",
                                         "note": "Llama 8B Q8_0; context not stated on the pages"}}


class StreamedStack:
    """80 Q6_K 70B-shaped layers, the first 36 resident in HBM and the other
    44 in pinned host memory, streamed through two HBM staging buffers; every
    layer is a copy of one seeded layer (the timing does not depend on the
    weight values), with its own KV cache."""

    def __init__(self, dev, max_ctx: int, n_past: int = 4096, n_layer: int = 80, fs: int = 36, mix=None):
        import torch

        import quantized_decode_dequant_amd as nt
        from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of, pack_blob
        from synth import workloads as wl

        shape, vocab = wl.LLAMA70B, 128256
        self.n_layer, self.fs, self.vocab, self.n_past = n_layer, fs, vocab, n_past
        self.cfg = cfg = cfg_of(shape, max_ctx)
        t0 = time.time()
        self.mix = mix = wl.ALL_Q6_K if mix is None else mix
        self.li = li = wl.gen_layer(shape, mix, wl.W_VERIFY_70B, 0, max_ctx, n_past)
        blob = pack_blob(cfg, li)
        self.sb = sb = blob.size
        self.host = host = [None] * n_layer
        for l in range(fs, n_layer):
            host[l] = torch.empty(sb, dtype=torch.uint8, pin_memory=True)
            host[l].numpy()[:] = blob
        self.stage = (torch.empty(sb, dtype=torch.uint8, device=dev), torch.empty(sb, dtype=torch.uint8, device=dev)) \
            if fs < n_layer else (None, None)
        self.layers = [DeviceLayer(li, dev, weights_on_device=(l < fs)) for l in range(n_layer)]
        log(f"[bench] streamed stack ready: {fs} resident + {n_layer - fs} streamed layers of {sb / 1e6:.1f} MB "
            f"({time.time() - t0:.0f} s)")
        self.emb = torch.from_numpy(wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wl.W_VERIFY_70B, 0,
                                                  wl.T_TOK_EMB)).to(dev)
        self.head = torch.from_numpy(wl.gen_matrix(wl.Q6_K, vocab, shape.hidden, wl.W_VERIFY_70B, 0,
                                                   wl.T_LM_HEAD)).to(dev)
        self.norm = torch.from_numpy(wl.gen_gains(shape, wl.W_VERIFY_70B, 0, wl.T_OUT_NORM)).to(dev)
        self.copy_stream = torch.cuda.Stream()
        self.h = nt.ModelHandle(cfg, [d.struct for d in self.layers], vocab, self.emb, wl.Q6_K, self.head, wl.Q6_K,
                                self.norm, first_streamed=fs, host_layers=host, stage=self.stage, stage_bytes=sb,
                                copy_stream=self.copy_stream)
        self.stream_bytes = sb * (n_layer - fs)


def workload_tiers(dev) -> dict:
    """Tier placement (p1 "3-Tier Adaptive Caching"): nt_plan_tiers places the
    80-layer 70B-shaped stack (Q4_K_M and Q6_K, context 4096) within a device
    budget, and greedy decode runs at that placement: the resident layers read
    HBM, the streamed ones cross the host link once per token."""
    import torch

    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import cfg_of
    from synth import workloads as wl

    n_past, vocab = 4096, 128256
    cfg = cfg_of(wl.LLAMA70B, n_past + 16)
    res = {}
    for name, mix in (("q4_k_m", wl.Q4_K_M), ("q6_k", wl.ALL_Q6_K)):
        for budget in (24 * 10**9, 48 * 10**9):
            p = nt.plan_tiers(cfg, [mix] * 80, vocab, wl.Q6_K, wl.Q6_K, 1, budget)
            if not p["ok"]:
                res[f"{name}_{budget // 10**9}gb"] = {"plan": p}
                continue
            S = StreamedStack(dev, n_past + 16, n_past, fs=p["first_streamed"], mix=mix)
            h = S.h
            stream = torch.cuda.current_stream()
            ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
            tok = torch.tensor([int(wl.gen_tokens(wl.W_VERIFY_70B, 1, vocab)[0])], dtype=torch.int32, device=dev)
            pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
            nxt = torch.zeros(1, dtype=torch.int32, device=dev)
            used = torch.cuda.memory_allocated(dev)
            ms = timed(lambda: h.decode_step(tok, pos, nxt, ws, None, stream), 3)
            key = f"{name}_{budget // 10**9}gb"
            res[key] = {"resident_layers": p["first_streamed"], "streamed_layers": p["n_streamed"],
                        "plan_device_gb": round(p["device_bytes"] / 1e9, 3),
                        "torch_allocated_gb": round(used / 1e9, 3),
                        "host_gb_per_token": round(p["host_bytes"] / 1e9, 3),
                        "decode_ms": round(ms, 2), "tokens_per_s": round(1e3 / ms, 3),
                        "h2d_gbs": round(p["host_bytes"] / ms / 1e6, 1)}
            log(f"[bench] tiers {key}: {p['first_streamed']} resident + {p['n_streamed']} streamed, "
                f"{ms:.1f} ms per token")
            del S, h, ws
            torch.cuda.empty_cache()
    return {"metric": "decode tok/s at a planned device/pinned-host placement", "unit": "tokens/s", "n_gpus": 1,
            "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "80-layer llama70b-shaped stacks (Q4_K_M, Q6_K), context 4096, placed by "
                                   "nt_plan_tiers within 24 and 48 GB of device memory"},
            "tiers": res}


def workload_verify(dev, passes: int) -> dict:
    """Streamed verify passes (80 Q6_K 70B-shaped layers, 44 streamed) of M = 1, 2, 4, 8 tokens."""
    import numpy as np
    import torch

    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer
    from synth import workloads as wl

    n_past = 4096
    S = StreamedStack(dev, n_past + 8, n_past)
    hs, cfg, li, host, stage, sb = S.h, S.cfg, S.li, S.host, S.stage, S.sb
    n_layer, fs, vocab = S.n_layer, S.fs, S.vocab
    emb, head, norm = S.emb, S.head, S.norm
    stream = torch.cuda.current_stream()
    toks = torch.from_numpy(wl.gen_tokens(wl.W_VERIFY_70B, 8, vocab)).to(dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    out = torch.zeros(8, dtype=torch.int32, device=dev)
    stream_bytes = S.stream_bytes
    # copy-only: the 44 layer copies alone
    def copies():
        for l in range(fs, n_layer):
            stage[l & 1].copy_(host[l], non_blocking=True)
    copy_ms = timed(copies, 2)
    res = {"h2d_probe_gbs": round(stream_bytes / copy_ms / 1e6, 1), "copy_only_ms": round(copy_ms, 1)}
    for M in [1, 2, 4, 8]:
        ws = torch.zeros(hs.workspace_bytes(M), dtype=torch.uint8, device=dev)
        ms = timed(lambda: hs.verify_step(toks, M, pos, out, ws, None, stream), passes)
        res[f"M{M}"] = {"pass_ms": round(ms, 1), "verified_pos_per_s": round(M / (ms / 1e3), 2),
                        "h2d_gbs": round(stream_bytes / ms / 1e6, 1)}
        log(f"[bench] verify M={M}: {ms:.1f} ms per pass")
        del ws
    # compute-only: the same 80 layers all resident
    del hs, S
    resident = [DeviceLayer(li, dev) for _ in range(n_layer)]
    hr = nt.ModelHandle(cfg, [d.struct for d in resident], vocab, emb, wl.Q6_K, head, wl.Q6_K, norm)
    for M in [1, 2, 4, 8]:
        ws = torch.zeros(hr.workspace_bytes(M), dtype=torch.uint8, device=dev)
        ms = timed(lambda: hr.verify_step(toks, M, pos, out, ws, None, stream), max(3, passes))
        t_pipe = res[f"M{M}"]["pass_ms"]
        res[f"M{M}"]["compute_only_ms"] = round(ms, 2)
        res[f"M{M}"]["overlap_efficiency"] = round((copy_ms + ms - t_pipe) / min(copy_ms, ms), 3)
        del ws
    del resident, hr
    best = max(res[f"M{M}"]["verified_pos_per_s"] for M in [1, 2, 4, 8])
    return {"metric": "streamed verify: verified positions/s", "unit": "positions/s", "n_gpus": 1,
            "value": best, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "80 Q6_K 70B-shaped layers, 36 resident + 44 streamed from pinned host memory, "
                                   "verify passes from context 4096", "stream_bytes_per_pass": stream_bytes},
            "verify": res}


def workload_spec(dev, rounds: int) -> dict:
    """Self-speculative rounds and layer skip on the streamed 80-layer Q6_K stack: the 36
    resident layers draft, the whole stack verifies (its 44 streamed layers
    cross the host link once per round).  Reports the draft step, the verify
    pass and the round, the tokens a round emitted on these seeded weights,
    and plain streamed decode with and without 20 calibrated skipped layers.
    Emitted tokens per round depend on how often the draft agrees with the
    whole stack, which seeded random weights do not model: `break_even`
    gives the tokens per round at which rounds beat plain decode."""
    import numpy as np
    import torch

    import quantized_decode_dequant_amd as nt
    from synth import workloads as wl

    n_past = 4096
    S = StreamedStack(dev, n_past + 64, n_past)
    h, n_layer, fs, vocab = S.h, S.n_layer, S.fs, S.vocab
    stream = torch.cuda.current_stream()
    first = int(wl.gen_tokens(wl.W_VERIFY_70B, 1, vocab)[0])
    draft_skip = [1 if l >= fs else 0 for l in range(n_layer)]
    res = {}
    ws1 = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([first], dtype=torch.int32, device=dev)
    pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    # plain streamed decode (every layer; 44 layer copies per token)
    plain_ms = timed(lambda: h.decode_step(tok, pos, nxt, ws1, None, stream), 3)
    # draft step: the resident layers and the LM head
    h.set_skip(draft_skip)
    draft_ms = timed(lambda: h.decode_step(tok, pos, nxt, ws1, None, stream), 10)
    h.set_skip(None)
    res["plain_decode_ms"] = round(plain_ms, 2)
    res["draft_step_ms"] = round(draft_ms, 3)
    log(f"[bench] spec: plain streamed decode {plain_ms:.1f} ms, draft step {draft_ms:.2f} ms")
    for K in (3, 7):
        ws = torch.zeros(h.spec_workspace_bytes(K), dtype=torch.uint8, device=dev)
        cur = torch.tensor([first], dtype=torch.int32, device=dev)
        p = torch.tensor([n_past], dtype=torch.int32, device=dev)
        out = torch.zeros(K + 1, dtype=torch.int32, device=dev)
        n_out = torch.zeros(1, dtype=torch.int32, device=dev)
        h.spec_step(draft_skip, K, cur, p, out, n_out, ws, stream)   # warm
        torch.cuda.synchronize()
        emitted, t_ms = 0, 0.0
        for r in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            h.spec_step(draft_skip, K, cur, p, out, n_out, ws, stream)
            e1.record()
            torch.cuda.synchronize()
            t_ms += e0.elapsed_time(e1)
            emitted += int(n_out.item())
        round_ms = t_ms / rounds
        wsv = torch.zeros(h.workspace_bytes(K + 1), dtype=torch.uint8, device=dev)
        toks = torch.from_numpy(wl.gen_tokens(wl.W_VERIFY_70B, K + 1, vocab)).to(dev)
        av = torch.zeros(K + 1, dtype=torch.int32, device=dev)
        verify_ms = timed(lambda: h.verify_step(toks, K + 1, pos, av, wsv, None, stream), 2)
        res[f"K{K}"] = {"round_ms": round(round_ms, 1), "verify_ms": round(verify_ms, 1),
                        "tokens_per_round": round(emitted / rounds, 2),
                        "tokens_per_s": round(emitted / rounds / (round_ms / 1e3), 3),
                        "break_even_tokens_per_round": round(round_ms / plain_ms, 2)}
        log(f"[bench] spec K={K}: round {round_ms:.1f} ms, {emitted / rounds:.2f} tokens per round")
        del ws, wsv
    # layer skip: calibrate on 4 tokens, skip the 20 most similar of layers 1..78
    cos = torch.zeros(n_layer, dtype=torch.float32, device=dev)
    t, p = tok.clone(), pos.clone()
    for _ in range(4):
        h.calibrate_step(t, p, nxt, cos, ws1, stream)
        t.copy_(nxt)
        p.add_(1)
    torch.cuda.synchronize()
    mask = nt.select_skip(cos.cpu().numpy(), 20, 1, n_layer - 1)
    h.set_skip(mask)
    skip_ms = timed(lambda: h.decode_step(tok, pos, nxt, ws1, None, stream), 3)
    h.set_skip(None)
    n_stream_skipped = int(mask[fs:].sum())
    res["skip20"] = {"decode_ms": round(skip_ms, 2), "skipped_layers": np.nonzero(mask)[0].tolist(),
                     "streamed_layers_skipped": n_stream_skipped,
                     "tokens_per_s": round(1e3 / skip_ms, 3)}
    log(f"[bench] skip20: {skip_ms:.1f} ms per token ({n_stream_skipped} of the skipped layers streamed)")
    best = max(res[f"K{K}"]["tokens_per_s"] for K in (3, 7))
    return {"metric": "self-speculative decode: emitted tokens/s (seeded random weights)", "unit": "tokens/s",
            "n_gpus": 1, "value": best, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "80 Q6_K 70B-shaped layers, 36 resident (the draft) + 44 streamed from pinned "
                                   "host memory, K = 3 and 7 drafted tokens per round, context 4096",
                       "stream_bytes_per_pass": S.stream_bytes},
            "spec": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--layers", type=int, default=80, help="stack depth (80 is the workload)")
    ap.add_argument("--cpu-sample-layers", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-every", type=int, default=41,
                    help="decode: time one gate/up launch in this many with kernel-stamped HIP events "
                         "(prime to the 80 layers, so every layer is sampled)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one device copy of 256 MiB (calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", metavar="DIR", help="print per-kernel statistics of a rocprofv3 output "
                    "directory (kernel trace or counter csv) and exit")
    ap.add_argument("--workload", choices=["decode", "decode8b", "gemv", "layer8b", "gemm_small", "verify", "spec", "tiers"], default="decode",
                    help="decode (the headline, default) or one of the secondary workloads")
    ap.add_argument("--passes", type=int, default=5, help="verify workload: timed passes per M; spec: rounds per K")
    ap.add_argument("--graph-steps", action="store_true",
                    help="decode: also time the steps as replays of one captured step (reported beside value)")
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
    if args.workload != "decode":
        fn = {"gemv": lambda: workload_gemv(dev), "layer8b": lambda: workload_layer8b(dev),
              "verify": lambda: workload_verify(dev, args.passes),
              "spec": lambda: workload_spec(dev, args.passes),
              "tiers": lambda: workload_tiers(dev), "gemm_small": lambda: workload_gemm_small(dev),
              "decode8b": lambda: workload_decode8b(dev, args.steps)}[args.workload]
        print(json.dumps(fn()), flush=True)
        return
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
    # the roofline kernel's launches are timed inside the timed region with
    # HIP events that the runtime stamps with the kernel's own start and end
    # (nt_trace_*).  One launch in --trace-every (41) is sampled: a traced
    # launch costs the host ~16 us to enqueue, and timing all of them slowed
    # the decode by 3.5%, one in ten by 0.3%; 41 is prime to the layer count,
    # so the samples cycle through every layer
    trace_every = args.trace_every
    nt.trace_begin(nt.TRACE_FFN_UP, trace_every)
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

    # dominant kernel: gate/up + SwiGLU, once per layer.  Algorithmic bytes
    # per launch: the two ffn x hidden weight matrices, x and the norm gains
    # read, the SwiGLU output written.
    ffn_bytes = 2 * shape.ffn * nt.row_bytes(fmts["wg"], shape.hidden) + shape.hidden * 4 * 2 + shape.ffn * 4
    if n_ffn == 0:
        raise RuntimeError("no gate/up launch was traced")
    ffn_avg_s = ffn_ms / 1e3 / n_ffn
    achieved = ffn_bytes / ffn_avg_s / 1e9
    traffic = counter_traffic("ffn_gate_up", ffn_bytes)

    graph_ms = None
    if args.graph_steps:
        # one decode step (with the token hand-off and the position increment)
        # captured in a HIP graph, replayed from context 4096 again
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                h.decode_step(tok, pos, nxt, ws, None, side)
                tok.copy_(nxt)
                pos.add_(1)
        stream.wait_stream(side)
        tok.fill_(first)
        pos.fill_(n_past)
        g.replay()
        torch.cuda.synchronize()
        tok.fill_(first)
        pos.fill_(n_past)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        log(f"[bench] graph replays: {graph_ms:.3f} ms/token")
        del g

    # the GEMV half of the metric: the single Q8_0 4096x4096 GEMV and the
    # seven 70B-shaped projections, alone (graph replays, rotated copies)
    cases = gemv_cases(extra=False)
    gres = time_gemvs(dev, cases)
    gemv = {"timing": "HIP graph replays of back-to-back launches, weights rotated over distinct copies "
                      "larger than the 256 MB last-level cache",
            "q8_0_4096x4096": gres["q8_0_4096x4096"],
            "llama70b_q4_k_m": {k: v for k, v in gres.items() if k.startswith("70b")},
            "llama70b_seven_gemvs_gbs": seven_gemv_gbs(gres)}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] oracle GEMVs")
        gemv["cpu_oracle"] = {"gbs": oracle_gemv_gbs(cases), "cores": oracle_threads(), "cpu": cpu_model(),
                              "kind": "oracle", "what": "the oracle's fp64 GEMV on the same weights, one call each"}
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
        "dtype": "q4_k/q6_k weights; activations as 16-bit fixed point per 32-block, split into two int8 "
                 "planes for i8 dot products; f32 accumulate",
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
            "kernel": "k_qgemv<EPI_SWIGLU> (RMSNorm + gate/up GEMV + SwiGLU, Q4_K 2x28672x8192)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "launches": n_ffn, "launches_sampled_every": trace_every, "avg_launch_us": round(ffn_avg_s * 1e6, 2),
            "bytes_per_launch": ffn_bytes,
        },
        "cpu_baseline": cpu,
        "gemv": gemv,
        "tokens_head": toks[:8],
        **({"ms_per_step_graph_replay": round(graph_ms, 4)} if graph_ms is not None else {}),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
