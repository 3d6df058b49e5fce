"""Input recipes: shapes, formats and seeds of the synthetic workloads.

Shapes follow the models the pages run: a Llama-3-8B-shaped layer and a
Llama-3.1-70B-shaped layer/stack (ntransformer pages: p1 "About" and the
roadmap, which name Llama 8B and Llama 3.1 70B).  Everything is drawn from
`synth`; nothing here computes any part of the decode.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import BLOCK, F16, F32, Q4_0, Q4_K, Q5_K, Q6_K, Q8_0, key, matrix_bytes, normal_f16, normal_f32, quant, uint_below

# stream tags
T_WQ, T_WK, T_WV, T_WO, T_WG, T_WU, T_WD = 1, 2, 3, 4, 5, 6, 7
T_ATTN_NORM, T_FFN_NORM, T_KC, T_VC, T_X = 8, 9, 10, 11, 12
T_TOK_EMB, T_LM_HEAD, T_OUT_NORM, T_TOKEN, T_GEMV_W, T_GEMV_X = 13, 14, 15, 16, 17, 18

MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
MAT_TAG = dict(wq=T_WQ, wk=T_WK, wv=T_WV, wo=T_WO, wg=T_WG, wu=T_WU, wd=T_WD)


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_head: int
    n_kv_head: int
    head_dim: int
    ffn: int
    rope_theta: float = 5e5
    rms_eps: float = 1e-5

    def mat_shape(self, name: str) -> tuple[int, int]:
        q = self.n_head * self.head_dim
        kv = self.n_kv_head * self.head_dim
        return dict(wq=(q, self.hidden), wk=(kv, self.hidden), wv=(kv, self.hidden),
                    wo=(self.hidden, q), wg=(self.ffn, self.hidden), wu=(self.ffn, self.hidden),
                    wd=(self.hidden, self.ffn))[name]


LLAMA8B = LayerShape(hidden=4096, n_head=32, n_kv_head=8, head_dim=128, ffn=14336)
LLAMA70B = LayerShape(hidden=8192, n_head=64, n_kv_head=8, head_dim=128, ffn=28672)
TINY = LayerShape(hidden=256, n_head=8, n_kv_head=2, head_dim=32, ffn=512, rope_theta=1e4)

ALL_Q4_0 = {m: Q4_0 for m in MATS}
ALL_Q8_0 = {m: Q8_0 for m in MATS}
ALL_Q6_K = {m: Q6_K for m in MATS}
# Q4_K_M mix: Q4_K for Q/K/O/gate/up, Q6_K for V/down.
Q4_K_M = dict(wq=Q4_K, wk=Q4_K, wv=Q6_K, wo=Q4_K, wg=Q4_K, wu=Q4_K, wd=Q6_K)
# Q5_K_M mix: Q5_K for Q/K/O/gate/up, Q6_K for V/down.
Q5_K_M = dict(wq=Q5_K, wk=Q5_K, wv=Q6_K, wo=Q5_K, wg=Q5_K, wu=Q5_K, wd=Q6_K)
ALL_Q5_K = {m: Q5_K for m in MATS}

# workload ids (first key tag)
W_GEMV_Q8 = 1
W_LAYER_8B = 2
W_GEMV_70B = 3
W_STACK_70B = 4
W_VERIFY_70B = 5
W_TEST = 100


@dataclass
class LayerInputs:
    shape: LayerShape
    fmts: dict
    mats: dict                  # name -> uint8 bytes (row-major blocks)
    attn_norm: np.ndarray       # f32 [hidden]
    ffn_norm: np.ndarray        # f32 [hidden]
    k_cache: np.ndarray         # uint16 (f16 bits) [n_kv][max_ctx][head_dim]
    v_cache: np.ndarray
    max_ctx: int
    n_past: int
    extra: dict = field(default_factory=dict)

    def weight_bytes(self) -> int:
        return sum(int(v.nbytes) for v in self.mats.values())


def layer_weight_bytes(shape: LayerShape, fmts: dict) -> int:
    return sum(matrix_bytes(fmts[m], *shape.mat_shape(m)) for m in MATS)


def gen_matrix(fmt: int, rows: int, cols: int, wid: int, layer: int, tag: int, out=None):
    return quant(fmt, rows, cols, key(wid, layer, tag), out=out)


def gen_kv(shape: LayerShape, wid: int, layer: int, tag: int, max_ctx: int, n_past: int,
           out: np.ndarray | None = None) -> np.ndarray:
    """f16 cache [n_kv][max_ctx][head_dim]: positions < n_past are N(0,1), the rest zero."""
    hd = shape.head_dim
    if out is None:
        out = np.zeros((shape.n_kv_head, max_ctx, hd), dtype=np.uint16)
    else:
        out[...] = 0
    for g in range(shape.n_kv_head):
        normal_f16(key(wid, layer, tag * 64 + g), n_past * hd, out=out[g, :n_past].reshape(-1))
    return out


def gen_gains(shape: LayerShape, wid: int, layer: int, tag: int) -> np.ndarray:
    """RMSNorm gains 1 + 0.02 * N(0,1)."""
    return normal_f32(key(wid, layer, tag), shape.hidden, mean=1.0, std=0.02)


def gen_layer(shape: LayerShape, fmts: dict, wid: int, layer: int, max_ctx: int, n_past: int,
              weights: bool = True) -> LayerInputs:
    mats = {}
    if weights:
        for m in MATS:
            r, c = shape.mat_shape(m)
            mats[m] = gen_matrix(fmts[m], r, c, wid, layer, MAT_TAG[m])
    return LayerInputs(
        shape=shape, fmts=dict(fmts), mats=mats,
        attn_norm=gen_gains(shape, wid, layer, T_ATTN_NORM),
        ffn_norm=gen_gains(shape, wid, layer, T_FFN_NORM),
        k_cache=gen_kv(shape, wid, layer, T_KC, max_ctx, n_past),
        v_cache=gen_kv(shape, wid, layer, T_VC, max_ctx, n_past),
        max_ctx=max_ctx, n_past=n_past)


def gen_x(n: int, wid: int, layer: int = 0, tag: int = T_X) -> np.ndarray:
    return normal_f32(key(wid, layer, tag), n)


def gen_tokens(wid: int, n: int, vocab: int) -> np.ndarray:
    return uint_below(key(wid, 0, T_TOKEN), n, vocab)


__all__ = [n for n in dir() if not n.startswith("_")] + ["BLOCK", "Q4_0", "Q4_K", "Q6_K", "Q8_0"]
