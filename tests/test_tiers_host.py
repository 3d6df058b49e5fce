"""Host logic of the device/pinned-host tier placement (nt_plan_tiers; no GPU
needed).  The plan is checked against a brute-force search written here over
every first_streamed, with the byte accounting rebuilt from the block sizes of
the formats: the largest prefix of resident layers whose device footprint
(fixed part + resident weights + two staging buffers) fits the budget and whose
streamed bytes fit the host budget."""
import numpy as np
import pytest

from synth import workloads as wl

# bytes per block and weights per block of each format (the GGUF layouts)
BLOCK = {wl.Q8_0: (34, 32), wl.Q4_0: (18, 32), wl.Q4_K: (144, 256), wl.Q6_K: (210, 256), wl.Q5_K: (176, 256)}
NAMES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
U64 = (1 << 64) - 1


def up256(v):
    return (v + 255) // 256 * 256


def mat_bytes(fmt, rows, cols):
    b, qk = BLOCK[fmt]
    return rows * (cols // qk) * b


def layer_bytes(shape, fmts):
    nq, nkv = shape.n_head * shape.head_dim, shape.n_kv_head * shape.head_dim
    dims = dict(wq=(nq, shape.hidden), wk=(nkv, shape.hidden), wv=(nkv, shape.hidden), wo=(shape.hidden, nq),
                wg=(shape.ffn, shape.hidden), wu=(shape.ffn, shape.hidden), wd=(shape.hidden, shape.ffn))
    return sum(up256(mat_bytes(fmts[n], *dims[n])) for n in NAMES)


def workspace(cfg, n_layer, vocab, emb_fmt, head_fmt, M):
    """Workspace the plan must hold: the library's own size queries on a model of this shape."""
    import ctypes
    import quantized_decode_dequant_amd as nt
    arr = (nt.Layer * max(1, n_layer))()
    m = nt.Model()
    m.cfg, m.n_layer, m.vocab = cfg, n_layer, vocab
    m.tok_emb, m.lm_head = nt.QMat(emb_fmt, None), nt.QMat(head_fmt, None)
    m.layers = ctypes.cast(arr, ctypes.POINTER(nt.Layer))
    if M == 1:
        return nt.lib().nt_step_workspace_bytes(ctypes.byref(m), 1)
    return nt.lib().nt_spec_workspace_bytes(ctypes.byref(m), M - 1)


def brute_force(shape, max_ctx, fmts_list, vocab, emb_fmt, head_fmt, M, dev_budget, host_budget):
    from quantized_decode_dequant_amd.model import cfg_of
    cfg = cfg_of(shape, max_ctx)
    n = len(fmts_list)
    blob = [layer_bytes(shape, f) for f in fmts_list]
    gains = up256(shape.hidden * 4)
    kv = up256(shape.n_kv_head * max_ctx * shape.head_dim * 2)
    fixed = (up256(mat_bytes(emb_fmt, vocab, shape.hidden)) + up256(mat_bytes(head_fmt, vocab, shape.hidden)) + gains
             + n * (2 * gains + 2 * kv) + workspace(cfg, n, vocab, emb_fmt, head_fmt, M))
    best = None
    for k in range(n + 1):
        stage = max(blob[k:], default=0)
        dev = fixed + sum(blob[:k]) + 2 * stage
        host = sum(blob[k:])
        if dev <= dev_budget and host <= host_budget:
            best = dict(first_streamed=k, n_streamed=n - k, fixed_bytes=fixed, resident_bytes=sum(blob[:k]),
                        stage_bytes=stage, device_bytes=dev, host_bytes=host, ok=True)
    return cfg, best


def plan(cfg, fmts_list, vocab, emb_fmt, head_fmt, M, dev_budget, host_budget=None):
    import quantized_decode_dequant_amd as nt
    return nt.plan_tiers(cfg, fmts_list, vocab, emb_fmt, head_fmt, M, dev_budget, host_budget)


def test_plan_matches_brute_force_on_random_mixes_and_budgets():
    rng = np.random.default_rng(11)
    fmts = list(BLOCK)
    for case in range(200):
        shape = wl.TINY if case % 2 else wl.LLAMA8B
        n = int(rng.integers(0, 12))
        mixes = [{nm: int(rng.choice(fmts)) for nm in NAMES} for _ in range(n)]
        vocab = int(rng.integers(1, 5000))
        emb, head = int(rng.choice(fmts)), int(rng.choice(fmts))
        M = int(rng.integers(1, 9))
        max_ctx = int(rng.integers(1, 3000))
        cfg, full = brute_force(shape, max_ctx, mixes, vocab, emb, head, M, U64, U64)
        # budgets around every breakpoint: nothing fits, part fits, all fits
        dev = int(rng.integers(full["fixed_bytes"] // 2, full["device_bytes"] + 2 * max([0] + [
            layer_bytes(shape, f) for f in mixes]) + 1))
        host = U64 if case % 3 else int(rng.integers(0, full["resident_bytes"] + 2))
        _, ref = brute_force(shape, max_ctx, mixes, vocab, emb, head, M, dev, host)
        got = plan(cfg, mixes, vocab, emb, head, M, dev, host)
        if ref is None:
            assert not got["ok"], case
            assert got["first_streamed"] == 0
        else:
            assert got == ref, (case, got, ref)


def test_plan_edges():
    from quantized_decode_dequant_amd.model import cfg_of
    shape, n, vocab = wl.TINY, 6, 1000
    mixes = [dict(wl.Q4_K_M)] * n
    cfg, full = brute_force(shape, 64, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, U64, U64)
    blob = layer_bytes(shape, mixes[0])
    # exactly everything: no staging buffers
    got = plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, full["device_bytes"])
    assert got["ok"] and got["first_streamed"] == n and got["stage_bytes"] == 0 and got["host_bytes"] == 0
    # one byte less: streaming starts, and then two staging buffers must fit beside the prefix
    got = plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, full["device_bytes"] - 1)
    assert got["ok"] and got["first_streamed"] == n - 3 and got["stage_bytes"] == blob
    assert got["device_bytes"] == full["fixed_bytes"] + (n - 3) * blob + 2 * blob
    # the fixed part plus two staging buffers is the least that works (every layer streamed)
    least = full["fixed_bytes"] + 2 * blob
    got = plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, least)
    assert got["ok"] and got["first_streamed"] == 0 and got["host_bytes"] == n * blob
    assert not plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, least - 1)["ok"]
    # a host budget below what must be streamed fails too
    assert not plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, least, host_budget=n * blob - 1)["ok"]
    # no layers
    got = plan(cfg, [], vocab, wl.Q6_K, wl.Q6_K, 1, U64)
    assert got["ok"] and got["first_streamed"] == 0 and got["n_streamed"] == 0
    # a larger workspace (more tokens per pass) never lets more layers stay resident
    for budget in range(full["fixed_bytes"], full["device_bytes"] + 1, blob // 3):
        f1 = plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 1, budget)
        f8 = plan(cfg, mixes, vocab, wl.Q6_K, wl.Q6_K, 8, budget)
        assert f8["first_streamed"] <= f1["first_streamed"] or not f8["ok"]


def test_plan_rejects_bad_arguments():
    import quantized_decode_dequant_amd as nt
    cfg = nt.layer_cfg(256, 8, 2, 32, 512, 64)
    mixes = [dict(wl.Q4_K_M)]
    for M in (0, 9):
        with pytest.raises(nt.NtError):
            nt.plan_tiers(cfg, mixes, 100, wl.Q6_K, wl.Q6_K, M, U64)
    with pytest.raises(nt.NtError):  # F16 matrices do not run in decoder layers
        nt.plan_tiers(cfg, [dict(wl.Q4_K_M, wq=wl.F16)], 100, wl.Q6_K, wl.Q6_K, 1, U64)
    with pytest.raises(nt.NtError):  # vocab must be positive
        nt.plan_tiers(cfg, mixes, 0, wl.Q6_K, wl.Q6_K, 1, U64)


def test_q4_k_m_keeps_more_70b_layers_resident_than_q6_k():
    """p1 "3-Tier Adaptive Caching": at one device budget the Q4_K_M stack keeps
    more of its 80 layers resident (fewer bytes to copy per token) than the
    larger Q6_K stack.  Budgets of 24 GB (the pages' card) and 48 GB."""
    from quantized_decode_dequant_amd.model import cfg_of
    shape, vocab = wl.LLAMA70B, 128256
    cfg = cfg_of(shape, 4160)
    q6 = dict(wq=wl.Q6_K, wk=wl.Q6_K, wv=wl.Q6_K, wo=wl.Q6_K, wg=wl.Q6_K, wu=wl.Q6_K, wd=wl.Q6_K)
    for budget in (24 * 10**9, 48 * 10**9):
        a = plan(cfg, [dict(wl.Q4_K_M)] * 80, vocab, wl.Q6_K, wl.Q6_K, 1, budget)
        b = plan(cfg, [q6] * 80, vocab, wl.Q6_K, wl.Q6_K, 1, budget)
        assert a["ok"] and b["ok"]
        assert a["first_streamed"] > b["first_streamed"]
        assert a["device_bytes"] <= budget and b["device_bytes"] <= budget
        assert a["host_bytes"] < b["host_bytes"]
    # 288 GB of HBM holds either stack whole
    assert plan(cfg, [q6] * 80, vocab, wl.Q6_K, wl.Q6_K, 8, 288 * 10**9)["first_streamed"] == 80
