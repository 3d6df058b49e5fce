"""A stack placed by nt_plan_tiers runs within its device budget and decodes
bitwise like the all-resident stack (p1 "3-Tier Adaptive Caching")."""
import pytest

from synth import workloads as wl
from tests.gpu_util import device, say
from tests.stack_util import HostStack
from tests.test_tiers_host import U64

pytestmark = pytest.mark.gpu


def device_bytes(h, ws) -> int:
    """Bytes of every device tensor a model handle keeps, plus its workspace."""
    k = h.keep
    n = ws.numel()
    for d in k["dls"]:
        n += sum(t.numel() for t in d.mats.values() if t is not None)
        n += sum(t.numel() * t.element_size() for t in (d.attn_norm, d.ffn_norm, d.k_cache, d.v_cache))
    n += sum(t.numel() * t.element_size() for t in (k["emb"], k["head"], k["norm"]))
    n += sum(t.numel() for t in k["stage"] if t is not None)
    return n


@pytest.mark.parametrize("fmts", ["Q4_K_M", "ALL_Q6_K"])
def test_planned_stack_fits_budget_and_matches_resident(fmts):
    import torch
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd.model import cfg_of
    dev = device()
    mix = getattr(wl, fmts)
    n_layer, vocab, max_ctx, n_past = 6, 700, 48, 11
    hs = HostStack(wl.TINY, mix, n_layer=n_layer, vocab=vocab, max_ctx=max_ctx, n_past=n_past, wid=wl.W_TEST + 41)
    cfg = cfg_of(wl.TINY, max_ctx)
    full = nt.plan_tiers(cfg, [mix] * n_layer, vocab, wl.Q6_K, wl.Q6_K, 1, U64)
    assert full["ok"] and full["first_streamed"] == n_layer
    copy_stream = torch.cuda.Stream()
    runs = []
    # all resident, then budgets that leave 3 and 0 layers resident
    for budget in (full["device_bytes"], full["device_bytes"] - 1,
                   full["fixed_bytes"] + 2 * (full["resident_bytes"] // n_layer)):
        p = nt.plan_tiers(cfg, [mix] * n_layer, vocab, wl.Q6_K, wl.Q6_K, 1, budget)
        say(f"budget {budget}: first_streamed {p['first_streamed']}, device {p['device_bytes']}")
        assert p["ok"] and p["device_bytes"] <= budget
        fs = p["first_streamed"]
        h = hs.device_model(dev, first_streamed=fs, copy_stream=copy_stream if fs < n_layer else None)
        ws = torch.zeros(h.workspace_bytes(1), dtype=torch.uint8, device=dev)
        # what the model actually holds on the device is within the plan (the plan
        # rounds every buffer up to 256 bytes)
        assert device_bytes(h, ws) <= p["device_bytes"]
        tok = torch.tensor([hs.first_token], dtype=torch.int32, device=dev)
        pos = torch.tensor([n_past], dtype=torch.int32, device=dev)
        nxt = torch.zeros(1, dtype=torch.int32, device=dev)
        logits = torch.zeros(vocab, dtype=torch.float32, device=dev)
        toks, lgs = [], []
        for s in range(3):
            h.decode_step(tok, pos, nxt, ws, logits)
            torch.cuda.synchronize()
            toks.append(int(nxt.item()))
            lgs.append(logits.clone())
            tok.copy_(nxt)
            pos += 1
        runs.append((fs, toks, lgs))
    assert [r[0] for r in runs] == [n_layer, n_layer - 3, 0]
    for fs, toks, lgs in runs[1:]:
        assert toks == runs[0][1], fs
        for a, b in zip(lgs, runs[0][2]):
            assert torch.equal(a, b), fs
