"""Parity of nt_decode_layer (HIP) against the fp64 oracle layer.

Bar: ||x_out - x_oracle||_inf / ||x_oracle||_inf <= 5e-3 per token; the
appended f16 K/V rows agree within 2e-3 of their largest magnitude.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say, to_dev

pytestmark = pytest.mark.gpu

LAYER_TOL = 5e-3
KV_TOL = 2e-3


def run_layer(shape, fmts, wid, layer, max_ctx, n_past, M, x=None):
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    say(f"layer hidden={shape.hidden} fmts={[synth.FMT_NAMES[fmts[m]] for m in wl.MATS]} pos={n_past} M={M}")
    li = wl.gen_layer(shape, fmts, wid, layer, max_ctx, n_past)
    if x is None:
        x = np.stack([wl.gen_x(shape.hidden, wid, layer, 200 + i) for i in range(M)])
    dl = DeviceLayer(li, device())
    cfg = cfg_of(shape, max_ctx)
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, M), dtype=torch.uint8, device=device())
    xd = to_dev(x.astype(np.float32).reshape(-1))
    pos = torch.tensor([n_past], dtype=torch.int32, device=device())
    nt.decode_layer(cfg, dl.struct, xd, M, pos, ws)
    torch.cuda.synchronize()
    got = xd.cpu().numpy().reshape(M, shape.hidden)
    kc = dl.k_cache.cpu().numpy().view(np.uint16)
    vc = dl.v_cache.cpu().numpy().view(np.uint16)
    ref = oracle.layer(li, x, n_past, M)  # updates li's caches in place
    return got, ref, kc, vc, li


def check(got, ref, kc, vc, li, n_past, M):
    for i in range(M):
        err = rel_inf(got[i], ref[i])
        say(f"  token {i}: layer rel err {err:.2e}")
        assert err <= LAYER_TOL
    for c_gpu, c_ref in ((kc, li.k_cache), (vc, li.v_cache)):
        new_g = c_gpu[:, n_past:n_past + M].view(np.float16).astype(np.float64)
        new_r = c_ref[:, n_past:n_past + M].view(np.float16).astype(np.float64)
        assert rel_inf(new_g, new_r) <= KV_TOL
        # everything else in the cache is untouched
        assert np.array_equal(np.delete(c_gpu, range(n_past, n_past + M), axis=1),
                              np.delete(c_ref, range(n_past, n_past + M), axis=1))


@pytest.mark.parametrize("fmts", [wl.ALL_Q8_0, wl.ALL_Q4_0, wl.Q4_K_M, wl.ALL_Q6_K, wl.Q5_K_M, wl.ALL_Q5_K],
                         ids=["q8_0", "q4_0", "q4_k_m", "q6_k", "q5_k_m", "q5_k"])
@pytest.mark.parametrize("n_past,M", [(37, 1), (0, 1), (20, 3), (63, 1), (30, 2)])
def test_layer_tiny(fmts, n_past, M):
    got, ref, kc, vc, li = run_layer(wl.TINY, fmts, wl.W_TEST, 3, 64, n_past, M)
    check(got, ref, kc, vc, li, n_past, M)


# Output rows that are not whole 256-blocks: a small-M layer then stages the
# gate/up and down activations with staging launches instead of in the
# reduce launches of the projections before (hidden 288: neither; ffn 416:
# only down's)
ODD_SHAPES = {
    "h288_f352": wl.LayerShape(hidden=288, n_head=4, n_kv_head=2, head_dim=32, ffn=352),
    "h512_f416": wl.LayerShape(hidden=512, n_head=8, n_kv_head=2, head_dim=64, ffn=416),
}


@pytest.mark.parametrize("fmts", [wl.ALL_Q4_0, wl.ALL_Q8_0], ids=["q4_0", "q8_0"])
@pytest.mark.parametrize("name,M", [("h288_f352", 3), ("h288_f352", 4), ("h512_f416", 3)])
def test_layer_rows_not_whole_256_blocks(fmts, name, M):
    got, ref, kc, vc, li = run_layer(ODD_SHAPES[name], fmts, wl.W_TEST, 13, 64, 21, M)
    check(got, ref, kc, vc, li, 21, M)


# 8 query heads per kv head, head_dim 128 (the 70B group size)
GROUP8 = wl.LayerShape(hidden=2048, n_head=16, n_kv_head=2, head_dim=128, ffn=4096)


@pytest.mark.parametrize("fmts", [wl.ALL_Q8_0, wl.ALL_Q4_0, wl.Q4_K_M, wl.ALL_Q6_K, wl.Q5_K_M],
                         ids=["q8_0", "q4_0", "q4_k_m", "q6_k", "q5_k_m"])
@pytest.mark.parametrize("n_past", [0, 63, 64, 200, 1000])
def test_layer_group8_batch1(fmts, n_past):
    # 1..1001 positions: one split of one round up to many splits, ragged last round
    got, ref, kc, vc, li = run_layer(GROUP8, fmts, wl.W_TEST, 7, 1024, n_past, 1)
    check(got, ref, kc, vc, li, n_past, 1)


# head sizes and group sizes of the attention tile shapes (head_dim 32: two
# waves per output tile; 64: one; 128: two tiles per wave; 256: four), with
# 1, 2, 4 and 8 query heads per kv head
ATTN_SHAPES = {
    "hd64_g1": wl.LayerShape(hidden=512, n_head=8, n_kv_head=8, head_dim=64, ffn=1024),
    "hd64_g2": wl.LayerShape(hidden=512, n_head=8, n_kv_head=4, head_dim=64, ffn=1024),
    "hd256_g4": wl.LayerShape(hidden=1024, n_head=4, n_kv_head=1, head_dim=256, ffn=1024),
    "hd256_g8": wl.LayerShape(hidden=2048, n_head=8, n_kv_head=1, head_dim=256, ffn=1024),
    "hd32_g8": wl.LayerShape(hidden=512, n_head=16, n_kv_head=2, head_dim=32, ffn=1024),
    "hd128_g1": wl.LayerShape(hidden=512, n_head=4, n_kv_head=4, head_dim=128, ffn=1024),
}


@pytest.mark.parametrize("name", sorted(ATTN_SHAPES))
@pytest.mark.parametrize("n_past", [0, 70, 300])
def test_layer_attention_shapes(name, n_past):
    # every split holds at most 256 positions: 300 cached positions span two
    # or more splits at every head size, 70 a single ragged one
    got, ref, kc, vc, li = run_layer(ATTN_SHAPES[name], wl.ALL_Q8_0, wl.W_TEST, 11, 320, n_past, 1)
    check(got, ref, kc, vc, li, n_past, 1)


@pytest.mark.parametrize("name", ["hd64_g2", "hd256_g8"])
def test_layer_attention_shapes_verify_tokens(name):
    # three tokens in one pass: token i attends to positions 0..pos+i
    got, ref, kc, vc, li = run_layer(ATTN_SHAPES[name], wl.ALL_Q4_0, wl.W_TEST, 12, 320, 130, 3)
    check(got, ref, kc, vc, li, 130, 3)


def test_layer_group8_repeat_calls_share_workspace():
    # consecutive calls on one workspace give identical results, and a
    # workspace filled with other bytes gives the same (its contents need no
    # initialisation); with 0xFF bytes (NaN floats) the partial slots of the
    # attention splits past the position (3 of the cache's 8 here) hold NaN,
    # which the combine must mask by selection, not by weights of zero
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    shape, max_ctx, n_past = GROUP8, 512, 300
    li = wl.gen_layer(shape, wl.Q4_K_M, wl.W_TEST, 8, max_ctx, n_past)
    dl = DeviceLayer(li, device())
    cfg = cfg_of(shape, max_ctx)
    x0 = to_dev(wl.gen_x(shape.hidden, wl.W_TEST, 8, 201).astype(np.float32))
    pos = torch.tensor([n_past], dtype=torch.int32, device=device())
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, 1), dtype=torch.uint8, device=device())
    outs = []
    for i in range(5):
        xd = x0.clone()
        w = ws if i < 3 else torch.full_like(ws, 0x5A if i == 3 else 0xFF)  # contents need no initialisation
        nt.decode_layer(cfg, dl.struct, xd, 1, pos, w)
        torch.cuda.synchronize()
        outs.append(xd.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_layer_8b_q4_0_full():
    # Llama-3-8B-shaped layer, Q4_0, 512 cached positions
    got, ref, kc, vc, li = run_layer(wl.LLAMA8B, wl.ALL_Q4_0, wl.W_LAYER_8B, 0, 520, 512, 1)
    check(got, ref, kc, vc, li, 512, 1)


@pytest.mark.parametrize("M", [1, 4])
def test_layer_8b_q8_0_full(M):
    # a layer of the 8B-shaped Q8_0 stack the 8B decode workload times, from
    # its first position (512 cached), one token and a four-token verify pass
    got, ref, kc, vc, li = run_layer(wl.LLAMA8B, wl.ALL_Q8_0, wl.W_LAYER_8B, 5, 520, 512, M)
    check(got, ref, kc, vc, li, 512, M)


def test_layer_70b_q4_k_m_full():
    # Llama-70B-shaped layer in the Q4_K_M mix, 4096 cached positions
    got, ref, kc, vc, li = run_layer(wl.LLAMA70B, wl.Q4_K_M, wl.W_GEMV_70B, 0, 4104, 4096, 1)
    check(got, ref, kc, vc, li, 4096, 1)


@pytest.mark.parametrize("fmts", [wl.Q4_K_M, wl.ALL_Q6_K], ids=["q4_k_m", "q6_k"])
@pytest.mark.parametrize("M", [4, 8])
def test_layer_70b_verify_full(fmts, M):
    # the verify pass's layer at full Llama-70B shape: M drafted tokens at
    # positions 4096..4096+M-1 through one layer (small-M GEMM for every
    # projection), every output value of every token against the oracle
    got, ref, kc, vc, li = run_layer(wl.LLAMA70B, fmts, wl.W_VERIFY_70B, 1, 4104, 4096, M)
    check(got, ref, kc, vc, li, 4096, M)


@pytest.mark.parametrize("M,bad", [(1, 16), (1, 116), (1, -1), (2, 15), (3, 14), (3, -2)])
def test_layer_position_out_of_range_leaves_cache_alone(M, bad):
    # pos < 0 or pos + M > max_ctx: no token writes the cache and x comes out
    # NaN (M = 2 runs the engine per token, M = 3 the small-M GEMM); a later
    # call at a valid position on the same workspace is unaffected
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    shape, max_ctx = wl.TINY, 16
    li = wl.gen_layer(shape, wl.ALL_Q4_0, wl.W_TEST, 4, max_ctx, 10)
    dl = DeviceLayer(li, device())
    k0 = dl.k_cache.clone()
    v0 = dl.v_cache.clone()
    cfg = cfg_of(shape, max_ctx)
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, M), dtype=torch.uint8, device=device())
    x = np.stack([wl.gen_x(shape.hidden, wl.W_TEST, 4, 300 + i) for i in range(M)]).astype(np.float32)
    xd = to_dev(x.reshape(-1))
    pos = torch.tensor([bad], dtype=torch.int32, device=device())
    nt.decode_layer(cfg, dl.struct, xd, M, pos, ws)
    torch.cuda.synchronize()
    assert torch.equal(dl.k_cache, k0) and torch.equal(dl.v_cache, v0)
    assert torch.isnan(xd).all()
    # the same workspace at a valid position: the oracle's layer
    xd = to_dev(x.reshape(-1))
    pos = torch.tensor([10], dtype=torch.int32, device=device())
    nt.decode_layer(cfg, dl.struct, xd, M, pos, ws)
    torch.cuda.synchronize()
    ref = oracle.layer(li, x, 10, M)
    got = xd.cpu().numpy().reshape(M, shape.hidden)
    for i in range(M):
        assert rel_inf(got[i], ref[i]) <= LAYER_TOL


def test_layer_argument_errors():
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    li = wl.gen_layer(wl.TINY, wl.ALL_Q4_0, wl.W_TEST, 5, 16, 4)
    dl = DeviceLayer(li, device())
    cfg = cfg_of(wl.TINY, 16)
    need = nt.layer_workspace_bytes(cfg, 1)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device=device())
    xd = to_dev(np.ones(wl.TINY.hidden, np.float32))
    pos = torch.tensor([4], dtype=torch.int32, device=device())
    with pytest.raises(nt.NtError) as e:
        nt.decode_layer(cfg, dl.struct, xd, 1, pos, ws)
    assert e.value.status == -3
    with pytest.raises(nt.NtError) as e:
        nt.decode_layer(cfg, dl.struct, xd, 9, pos, torch.zeros(need, dtype=torch.uint8, device=device()))
    assert e.value.status == -1


@pytest.mark.parametrize("M", [1, 3])
def test_layer_attention_trace_one_interval_per_call(M):
    # the attention of a layer call is one split launch over all M queries
    # and one combine; the trace records one interval per call, from the
    # split's start to the combine's end, and the traced calls give the
    # untraced result
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of
    shape, max_ctx, n_past = GROUP8, 512, 300
    li = wl.gen_layer(shape, wl.Q4_K_M, wl.W_TEST, 9, max_ctx, n_past)
    dl = DeviceLayer(li, device())
    cfg = cfg_of(shape, max_ctx)
    x0 = to_dev(np.stack([wl.gen_x(shape.hidden, wl.W_TEST, 9, 400 + i) for i in range(M)]).astype(np.float32)
                .reshape(-1))
    pos = torch.tensor([n_past], dtype=torch.int32, device=device())
    ws = torch.zeros(nt.layer_workspace_bytes(cfg, M), dtype=torch.uint8, device=device())
    outs = []
    for traced in (False, True, False):
        xd = x0.clone()
        if traced:
            nt.trace_begin(nt.TRACE_ATTN)
        for _ in range(2):
            xd.copy_(x0)
            nt.decode_layer(cfg, dl.struct, xd, M, pos, ws)
        torch.cuda.synchronize()
        if traced:
            n, ms = nt.trace_end()
            say(f"  M={M}: {n} attention intervals, {ms * 1e3 / max(n, 1):.2f} us each")
            assert n == 2 and ms > 0.0
        outs.append(xd.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("name,n_past", [("hd64_g2", 120), ("hd128_g1", 56), ("hd32_g8", 248)])
def test_layer_verify_eight_tokens_fill_the_cache(name, n_past):
    # eight tokens in one pass whose last position is the cache's last
    # (pos + 7 = max_ctx - 1): one attention launch covers the eight queries,
    # each with its own causal end, and the cache's last split holds the new
    # tokens only
    max_ctx = n_past + 8
    got, ref, kc, vc, li = run_layer(ATTN_SHAPES[name], wl.ALL_Q8_0, wl.W_TEST, 13, max_ctx, n_past, 8)
    check(got, ref, kc, vc, li, n_past, 8)
