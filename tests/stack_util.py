"""Builds a seeded decoder stack for the GPU and for the oracle from the same host arrays."""
import numpy as np

import oracle
from synth import workloads as wl


class HostStack:
    def __init__(self, shape, fmts, n_layer, vocab, max_ctx, n_past, wid, emb_fmt=wl.Q6_K, head_fmt=wl.Q6_K):
        self.shape, self.fmts, self.n_layer, self.vocab = shape, fmts, n_layer, vocab
        self.max_ctx, self.n_past, self.wid = max_ctx, n_past, wid
        self.layers = [wl.gen_layer(shape, fmts, wid, l, max_ctx, n_past) for l in range(n_layer)]
        self.emb_fmt, self.head_fmt = emb_fmt, head_fmt
        self.tok_emb = wl.gen_matrix(emb_fmt, vocab, shape.hidden, wid, 0, wl.T_TOK_EMB)
        self.lm_head = wl.gen_matrix(head_fmt, vocab, shape.hidden, wid, 0, wl.T_LM_HEAD)
        self.out_norm = wl.gen_gains(shape, wid, 0, wl.T_OUT_NORM)
        self.first_token = int(wl.gen_tokens(wid, 1, vocab)[0])

    def oracle_model(self):
        """The oracle works on its own copies of the caches."""
        import copy
        layers = []
        for li in self.layers:
            c = copy.copy(li)
            c.k_cache = li.k_cache.copy()
            c.v_cache = li.v_cache.copy()
            layers.append(c)
        return oracle.OracleModel(self.shape, layers, self.emb_fmt, self.tok_emb, self.head_fmt, self.lm_head,
                                  self.out_norm, self.vocab)

    def device_model(self, device, first_streamed=None, copy_stream=None):
        import torch
        import quantized_decode_dequant_amd as nt
        from quantized_decode_dequant_amd.model import DeviceLayer, cfg_of, pack_blob
        cfg = cfg_of(self.shape, self.max_ctx)
        fs = self.n_layer if first_streamed is None else first_streamed
        dls = [DeviceLayer(li, device, weights_on_device=(l < fs)) for l, li in enumerate(self.layers)]
        host, stage, sb = [None] * self.n_layer, (None, None), 0
        if fs < self.n_layer:
            blobs = [pack_blob(cfg, li) for li in self.layers[fs:]]
            sb = blobs[0].size
            host[fs:] = [torch.from_numpy(b).pin_memory() for b in blobs]
            # staging buffers start as 0xFF bytes: f16 scales of NaN, so a
            # layer computed from a buffer before its copy landed gives NaN
            stage = (torch.full((sb,), 0xFF, dtype=torch.uint8, device=device),
                     torch.full((sb,), 0xFF, dtype=torch.uint8, device=device))
        keep = dict(
            dls=dls, host=host, stage=stage,
            emb=torch.from_numpy(self.tok_emb).to(device), head=torch.from_numpy(self.lm_head).to(device),
            norm=torch.from_numpy(self.out_norm).to(device))
        h = nt.ModelHandle(cfg, [d.struct for d in dls], self.vocab, keep["emb"], self.emb_fmt, keep["head"],
                           self.head_fmt, keep["norm"], first_streamed=fs, host_layers=host, stage=stage,
                           stage_bytes=sb, copy_stream=copy_stream)
        h.keep = keep
        return h
