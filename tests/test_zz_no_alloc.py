"""nt_decode_step_noalloc (the decode step on the library's own device
array, for callers that cannot allocate) against nt_decode_step with a
caller workspace: equal tokens and logits, bit for bit, on two calls in a
row, the second with a smaller model (the array then holds the first call's
bytes), and the size and streaming limits reported as errors."""
import ctypes

import numpy as np
import pytest

from synth import workloads as wl
from tests.gpu_util import device, say
from tests.stack_util import HostStack

pytestmark = pytest.mark.gpu


def one_step(hs, noalloc):
    import torch
    dev = device()
    h = hs.device_model(dev)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([hs.n_past], dtype=torch.int32, device=dev)
    nxt = torch.full((1,), -7, dtype=torch.int32, device=dev)
    logits = torch.full((hs.vocab,), float("nan"), dtype=torch.float32, device=dev)
    if noalloc:
        h.decode_step_noalloc(tok, pos, nxt, logits)
    else:
        ws = torch.full((h.workspace_bytes(1),), 0x5A, dtype=torch.uint8, device=dev)
        h.decode_step(tok, pos, nxt, ws, logits)
    torch.cuda.synchronize()
    caches = [(d.k_cache.cpu().numpy(), d.v_cache.cpu().numpy()) for d in h.keep["dls"]]
    return int(nxt.item()), logits.cpu().numpy(), caches


def test_noalloc_step_equals_workspace_step_twice_then_smaller():
    big = HostStack(wl.TINY, wl.Q4_K_M, n_layer=3, vocab=1500, max_ctx=96, n_past=70, wid=wl.W_TEST + 60)
    small = HostStack(wl.TINY, wl.ALL_Q8_0, n_layer=2, vocab=300, max_ctx=24, n_past=5, wid=wl.W_TEST + 61)
    for hs in (big, small):
        say(f"no-alloc step: {hs.n_layer} layers, vocab {hs.vocab}, max_ctx {hs.max_ctx}")
        t_a, l_a, c_a = one_step(hs, noalloc=True)
        t_b, l_b, c_b = one_step(hs, noalloc=False)
        assert t_a == t_b and t_a >= 0
        assert np.array_equal(l_a, l_b)
        for (ka, va), (kb, vb) in zip(c_a, c_b):
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_noalloc_limits():
    import quantized_decode_dequant_amd as nt
    import torch
    dev = device()
    assert nt.lib().nt_decode_step_noalloc_max_bytes() == 32 << 20
    hs = HostStack(wl.TINY, wl.ALL_Q6_K, n_layer=3, vocab=400, max_ctx=32, n_past=9, wid=wl.W_TEST + 62)
    tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
    pos = torch.tensor([9], dtype=torch.int32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    # streamed layers are refused
    h = hs.device_model(dev, first_streamed=1, copy_stream=torch.cuda.Stream())
    with pytest.raises(nt.NtError) as e:
        h.decode_step_noalloc(tok, pos, nxt)
    assert e.value.status == -5
    # a workspace beyond the array is refused (the cache capacity sets the
    # attention partials: 1024 splits of 64 heads x 128 dims is 32 MiB)
    h = hs.device_model(dev)
    m = h.m
    saved = (m.cfg.hidden, m.cfg.n_head, m.cfg.n_kv_head, m.cfg.head_dim, m.cfg.max_ctx)
    m.cfg.hidden, m.cfg.n_head, m.cfg.n_kv_head, m.cfg.head_dim, m.cfg.max_ctx = 8192, 64, 8, 128, 65536
    assert nt.lib().nt_step_workspace_bytes(ctypes.byref(m), 1) > (32 << 20)
    with pytest.raises(nt.NtError) as e:
        h.decode_step_noalloc(tok, pos, nxt)
    assert e.value.status == -3
    m.cfg.hidden, m.cfg.n_head, m.cfg.n_kv_head, m.cfg.head_dim, m.cfg.max_ctx = saved
    h.decode_step_noalloc(tok, pos, nxt)
    torch.cuda.synchronize()
    assert int(nxt.item()) >= 0
