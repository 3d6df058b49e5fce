"""Error behaviour of the steps, on the GPU (every kernel still exits
normally: the conditions are forced from the host).

  - a position out of range (pos < 0 or pos + M > max_ctx), which only the
    kernels can see since the position lives in device memory: the step's
    tokens are -1, no cache entry is written, and the next call at a valid
    position on the same workspace is unaffected; a speculative round emits
    nothing and keeps its position and current token;
  - a failed copy in the middle of a streamed pass (forced by the library's
    test hook, nt_test_fail_stream_copy): the call returns NT_EHIP, no entry
    outside the pass's own positions changes, and repeating the pass at the
    same position gives bitwise the result of an uninterrupted pass.
"""
import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu


def caches(h):
    return [(d.k_cache.clone(), d.v_cache.clone()) for d in h.keep["dls"]]


def same_caches(a, b, keep_pos=None):
    """Bitwise equal caches; with keep_pos = (p0, p1) only positions outside [p0, p1) are compared."""
    for (ka, va), (kb, vb) in zip(a, b):
        if keep_pos is not None:
            p0, p1 = keep_pos
            sel = [i for i in range(ka.shape[1]) if not p0 <= i < p1]
            ka, va, kb, vb = ka[:, sel], va[:, sel], kb[:, sel], vb[:, sel]
        if not (bool((ka == kb).all()) and bool((va == vb).all())):
            return False
    return True


@pytest.mark.parametrize("M,bad", [(1, 24), (1, -3), (2, 23), (4, 21)])
def test_step_position_out_of_range(M, bad):
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=3, vocab=500, max_ctx=24, n_past=10, wid=wl.W_TEST + 40)
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
    toks = torch.from_numpy(wl.gen_tokens(wl.W_TEST + 40, M, hs.vocab)).to(dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    logits = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    before = caches(h)
    h.verify_step(toks, M, torch.tensor([bad], dtype=torch.int32, device=dev), out, ws, logits)
    torch.cuda.synchronize()
    assert out.tolist() == [-1] * M
    assert same_caches(caches(h), before)
    # the same model and workspace at a valid position: equal to a fresh model's pass
    pos = torch.tensor([10], dtype=torch.int32, device=dev)
    h.verify_step(toks, M, pos, out, ws, logits)
    h2 = hs.device_model(dev)
    out2 = torch.zeros(M, dtype=torch.int32, device=dev)
    logits2 = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    h2.verify_step(toks, M, pos, out2, torch.zeros(h2.workspace_bytes(M), dtype=torch.uint8, device=dev), logits2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(logits, logits2)
    assert min(out.tolist()) >= 0
    assert same_caches(caches(h), caches(h2))


def test_decode_step_out_of_range_token_is_minus_one():
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.ALL_Q6_K, n_layer=2, vocab=300, max_ctx=20, n_past=5, wid=wl.W_TEST + 41)
    h = hs.device_model(dev)
    ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    before = caches(h)
    for bad in (20, 21, 1000, -1):
        h.decode_step(tok, torch.tensor([bad], dtype=torch.int32, device=dev), nxt, ws)
        torch.cuda.synchronize()
        assert int(nxt.item()) == -1, bad
    assert same_caches(caches(h), before)


def test_spec_round_out_of_range_emits_nothing():
    import torch
    dev = device()
    K, max_ctx = 3, 24
    hs = HostStack(wl.TINY, wl.Q4_K_M, n_layer=2, vocab=400, max_ctx=max_ctx, n_past=10, wid=wl.W_TEST + 42)
    h = hs.device_model(dev)
    ws = torch.zeros(h.spec_workspace_bytes(K), dtype=torch.uint8, device=dev)
    p0 = max_ctx - K  # the verify pass needs positions p0 .. p0 + K
    cur = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([p0], dtype=torch.int32, device=dev)
    out = torch.zeros(K + 1, dtype=torch.int32, device=dev)
    n_out = torch.full((1,), 99, dtype=torch.int32, device=dev)
    before = caches(h)
    h.spec_step(None, K, cur, pos, out, n_out, ws)
    torch.cuda.synchronize()
    assert int(n_out.item()) == 0
    assert out.tolist() == [-1] * (K + 1)
    assert int(pos.item()) == p0 and int(cur.item()) == hs.first_token
    # the draft steps may have written their own positions (p0 and on, stale
    # past the position); nothing before p0 changed
    assert same_caches(caches(h), before, keep_pos=(p0, max_ctx))


@pytest.mark.parametrize("fail_at,M", [(0, 1), (2, 1), (3, 3)])
def test_streaming_copy_failure_then_repeat(fail_at, M):
    # six Q6_K layers, four streamed: copies 0 and 1 go out before the first
    # layer, copies 2 and 3 inside the loop after a staging buffer is freed
    import quantized_decode_dequant_amd as nt
    import torch
    dev = device()
    hs = HostStack(wl.TINY, wl.ALL_Q6_K, n_layer=6, vocab=500, max_ctx=32, n_past=9, wid=wl.W_TEST + 43)
    toks = torch.from_numpy(wl.gen_tokens(wl.W_TEST + 43, M, hs.vocab)).to(dev)
    pos = torch.tensor([9], dtype=torch.int32, device=dev)
    ref = hs.device_model(dev)
    r_out = torch.zeros(M, dtype=torch.int32, device=dev)
    r_lg = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    ref.verify_step(toks, M, pos, r_out, torch.zeros(ref.workspace_bytes(M), dtype=torch.uint8, device=dev), r_lg)
    cs = torch.cuda.Stream()
    h = hs.device_model(dev, first_streamed=2, copy_stream=cs)
    ws = torch.zeros(h.workspace_bytes(M), dtype=torch.uint8, device=dev)
    out = torch.zeros(M, dtype=torch.int32, device=dev)
    lg = torch.zeros(M * hs.vocab, dtype=torch.float32, device=dev)
    before = caches(h)
    say(f"streamed pass with the copy of streamed layer {fail_at} failing, M={M}")
    nt.test_fail_stream_copy(fail_at)
    with pytest.raises(nt.NtError) as e:
        h.verify_step(toks, M, pos, out, ws, lg)
    assert e.value.status == -4  # NT_EHIP
    torch.cuda.synchronize()
    cs.synchronize()
    assert same_caches(caches(h), before, keep_pos=(9, 9 + M))
    # the hook disarmed itself: the repeated pass runs whole
    h.verify_step(toks, M, pos, out, ws, lg)
    torch.cuda.synchronize()
    assert torch.equal(out, r_out) and torch.equal(lg, r_lg)
    assert same_caches(caches(h), caches(ref))
    nt.test_fail_stream_copy(-1)
