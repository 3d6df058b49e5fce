"""Device-side holders for a decoder layer and a decoder stack.

Uploads host arrays (numpy) into PyTorch device tensors and keeps the
nt_layer / nt_model structs of the C ABI pointing at them.  No compute here:
every step of the decode runs in libnt's kernels.
"""
from __future__ import annotations

import numpy as np

from . import MAT_NAMES, LayerCfg, ModelHandle, _ptr, block_bytes, block_elems, layer_cfg, make_layer


def _dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def mat_shapes(cfg: LayerCfg) -> dict:
    nq, nkv = cfg.n_head * cfg.head_dim, cfg.n_kv_head * cfg.head_dim
    return dict(wq=(nq, cfg.hidden), wk=(nkv, cfg.hidden), wv=(nkv, cfg.hidden), wo=(cfg.hidden, nq),
                wg=(cfg.ffn, cfg.hidden), wu=(cfg.ffn, cfg.hidden), wd=(cfg.hidden, cfg.ffn))


class DeviceLayer:
    """One layer's tensors on the device.  `src` has attributes mats (name -> uint8 array),
    fmts (name -> format), attn_norm, ffn_norm, k_cache, v_cache (f16 bits)."""

    def __init__(self, src, device, weights_on_device: bool = True):
        self.fmts = dict(src.fmts)
        self.mats = {n: (_dev(src.mats[n], device) if weights_on_device else None) for n in MAT_NAMES}
        self.attn_norm = _dev(src.attn_norm, device)
        self.ffn_norm = _dev(src.ffn_norm, device)
        import torch
        self.k_cache = _dev(src.k_cache.view(np.int16), device).view(torch.int16)
        self.v_cache = _dev(src.v_cache.view(np.int16), device).view(torch.int16)
        self.struct = make_layer(self.attn_norm, self.ffn_norm, self.mats, self.fmts, self.k_cache, self.v_cache)

    def weight_bytes(self) -> int:
        return sum(int(t.numel()) for t in self.mats.values() if t is not None)


def cfg_of(shape, max_ctx: int) -> LayerCfg:
    return layer_cfg(shape.hidden, shape.n_head, shape.n_kv_head, shape.head_dim, shape.ffn, max_ctx,
                     shape.rope_theta, shape.rms_eps)


def pack_blob(cfg: LayerCfg, src, out: np.ndarray | None = None) -> np.ndarray:
    """A streamed layer's seven matrices back to back, each padded to 256 bytes."""
    shapes = mat_shapes(cfg)
    offs, o = [], 0
    for n in MAT_NAMES:
        offs.append(o)
        r, c = shapes[n]
        o += (r * (c // block_elems(src.fmts[n])) * block_bytes(src.fmts[n]) + 255) // 256 * 256
    if out is None:
        out = np.zeros(o, dtype=np.uint8)
    for n, off in zip(MAT_NAMES, offs):
        m = np.ascontiguousarray(src.mats[n]).reshape(-1)
        out[off:off + m.size] = m
    return out
