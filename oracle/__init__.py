"""fp64 CPU oracle for quantized batch-1 Llama decode.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product
library never loads it.  The arithmetic lives in ``oracle.c`` (plain C,
double precision, sums in index order, OpenMP over independent output rows);
this module only marshals numpy arrays to it.  It shares no code with the HIP
library.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
  dequant      - encoder round trips on hand-built blocks, constant-q closed
                 forms; the GGUF compatibility of the Q4_K / Q6_K bit packing
                 is parity unpinned (no GGUF file is available).
  gemv         - dense numpy matmul over independently pinned dequant; one-hot x.
  rmsnorm/rope/attention/silu - closed forms and scipy special cases.
  layer/decode - constructed-weight invariants (zero, identity, selection
                 matrices), sequential-versus-batched invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")

Q8_0, Q4_0, Q4_K, Q6_K, Q5_K, F16, F32 = 0, 1, 2, 3, 4, 5, 6


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_kv_head", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("max_ctx", ctypes.c_int64),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double)]


class Mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("data", ctypes.c_void_p)]


class LayerW(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("ffn_norm", ctypes.c_void_p),
                ("wq", Mat), ("wk", Mat), ("wv", Mat), ("wo", Mat), ("wg", Mat), ("wu", Mat), ("wd", Mat),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("cfg", Cfg), ("n_layer", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("tok_emb", Mat), ("lm_head", Mat), ("out_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerW))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i64, dbl, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        L.or_half.restype = dbl
        L.or_half.argtypes = [ctypes.c_uint16]
        L.or_to_half.restype = ctypes.c_uint16
        L.or_to_half.argtypes = [dbl]
        L.or_block_elems.restype = i32
        L.or_block_elems.argtypes = [i32]
        L.or_block_bytes.restype = i32
        L.or_block_bytes.argtypes = [i32]
        L.or_dequant_row.restype = None
        L.or_dequant_row.argtypes = [i32, vp, i64, vp]
        L.or_gemv.restype = None
        L.or_gemv.argtypes = [i32, vp, vp, vp, i64, i64]
        L.or_gemv_f32.restype = None
        L.or_gemv_f32.argtypes = [i32, vp, vp, vp, i64, i64]
        L.or_rmsnorm.restype = None
        L.or_rmsnorm.argtypes = [vp, vp, i64, dbl, vp]
        L.or_rope.restype = None
        L.or_rope.argtypes = [vp, i32, i32, i64, dbl]
        L.or_attention.restype = None
        L.or_attention.argtypes = [vp, vp, vp, i32, i32, i32, i64, i64, vp]
        L.or_silu.restype = dbl
        L.or_silu.argtypes = [dbl]
        L.or_layer.restype = None
        L.or_layer.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(LayerW), vp, i32, i64]
        L.or_argmax.restype = i64
        L.or_argmax.argtypes = [vp, i64, vp]
        L.or_decode.restype = None
        L.or_decode.argtypes = [ctypes.POINTER(Model), vp, i32, i64, vp, vp, vp, vp]
        L.or_decode_ex.restype = None
        L.or_decode_ex.argtypes = [ctypes.POINTER(Model), vp, i32, i64, vp, vp, vp, vp, vp, vp]
        L.or_select_skip.restype = i32
        L.or_select_skip.argtypes = [vp, i32, i32, i32, i32, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data


def block_elems(fmt: int) -> int:
    return lib().or_block_elems(fmt)


def block_bytes(fmt: int) -> int:
    return lib().or_block_bytes(fmt)


def half_to_f64(bits: int) -> float:
    return lib().or_half(int(bits))


def f64_to_half(v: float) -> int:
    return int(lib().or_to_half(float(v)))


def dequant(fmt: int, data: np.ndarray, rows: int, cols: int) -> np.ndarray:
    data = np.ascontiguousarray(data, dtype=np.uint8)
    qk, bb = block_elems(fmt), block_bytes(fmt)
    assert cols % qk == 0 and data.size >= rows * cols // qk * bb
    out = np.empty((rows, cols), dtype=np.float64)
    rb = cols // qk * bb
    for r in range(rows):
        lib().or_dequant_row(fmt, data.ctypes.data + r * rb, cols, out[r].ctypes.data)
    return out


def gemv(fmt: int, W: np.ndarray, x: np.ndarray, rows: int, cols: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    y = np.empty(rows, dtype=np.float64)
    if x.dtype == np.float32:
        x = np.ascontiguousarray(x)
        lib().or_gemv_f32(fmt, _p(W), _p(x), _p(y), rows, cols)
    else:
        x = np.ascontiguousarray(x, dtype=np.float64)
        lib().or_gemv(fmt, _p(W), _p(x), _p(y), rows, cols)
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(x)
    lib().or_rmsnorm(_p(x), _p(g), x.size, eps, _p(out))
    return out


def rope(v: np.ndarray, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    v = np.array(v, dtype=np.float64, copy=True)
    lib().or_rope(_p(v), n_heads, head_dim, pos, theta)
    return v


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, n_head: int, n_kv: int,
              head_dim: int, max_ctx: int, n_pos: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    kc = np.ascontiguousarray(k_cache, dtype=np.uint16)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint16)
    o = np.empty(n_head * head_dim, dtype=np.float64)
    lib().or_attention(_p(q), _p(kc), _p(vc), n_head, n_kv, head_dim, max_ctx, n_pos, _p(o))
    return o


def silu(z: float) -> float:
    return lib().or_silu(float(z))


def argmax(v: np.ndarray) -> tuple[int, float]:
    v = np.ascontiguousarray(v, dtype=np.float64)
    m = ctypes.c_double()
    i = lib().or_argmax(_p(v), v.size, ctypes.addressof(m))
    return int(i), m.value


def make_cfg(shape, max_ctx: int) -> Cfg:
    return Cfg(shape.hidden, shape.n_head, shape.n_kv_head, shape.head_dim, shape.ffn, max_ctx,
               float(shape.rope_theta), float(shape.rms_eps))


class _Keep(list):
    """Holds references to arrays whose addresses sit in ctypes structs."""


def make_layer_w(li, keep: list) -> LayerW:
    """LayerW over the arrays of a synth.workloads.LayerInputs (caches updated in place)."""
    w = LayerW()
    for a in (li.attn_norm, li.ffn_norm, li.k_cache, li.v_cache):
        assert a.flags["C_CONTIGUOUS"]
    w.attn_norm = li.attn_norm.ctypes.data
    w.ffn_norm = li.ffn_norm.ctypes.data
    for m in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        arr = np.ascontiguousarray(li.mats[m])
        keep.append(arr)
        setattr(w, m, Mat(li.fmts[m], arr.ctypes.data))
    w.k_cache = li.k_cache.ctypes.data
    w.v_cache = li.v_cache.ctypes.data
    keep.extend([li.attn_norm, li.ffn_norm, li.k_cache, li.v_cache])
    return w


def layer(li, x: np.ndarray, pos: int, M: int = 1) -> np.ndarray:
    """Run one layer on x ([M][hidden] f32 or f64); li's caches are updated in place."""
    keep = _Keep()
    cfg = make_cfg(li.shape, li.max_ctx)
    w = make_layer_w(li, keep)
    xx = np.array(x, dtype=np.float64, copy=True).reshape(M, li.shape.hidden)
    lib().or_layer(ctypes.byref(cfg), ctypes.byref(w), _p(xx), M, pos)
    return xx


class OracleModel:
    """A decoder stack over host arrays: layers (LayerInputs), embeddings, LM head."""

    def __init__(self, shape, layers, tok_emb_fmt, tok_emb, lm_head_fmt, lm_head, out_norm, vocab):
        self.keep = _Keep()
        self.shape = shape
        self.vocab = vocab
        self.layers_in = layers
        arr = (LayerW * len(layers))()
        for i, li in enumerate(layers):
            arr[i] = make_layer_w(li, self.keep)
        self.keep.extend([arr, tok_emb, lm_head, out_norm])
        self.m = Model(make_cfg(shape, layers[0].max_ctx), len(layers), vocab,
                       Mat(tok_emb_fmt, tok_emb.ctypes.data), Mat(lm_head_fmt, lm_head.ctypes.data),
                       out_norm.ctypes.data, ctypes.cast(arr, ctypes.POINTER(LayerW)))

    def decode(self, tokens, pos: int, want_logits: bool = False, want_hidden: bool = False):
        """Returns (next tokens [M], margins [M], logits [M][vocab] or None, hidden or None)."""
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        M = tokens.size
        nxt = np.empty(M, dtype=np.int32)
        margin = np.empty(M, dtype=np.float64)
        logits = np.empty((M, self.vocab), dtype=np.float64) if want_logits else None
        hidden = np.empty((M, self.shape.hidden), dtype=np.float64) if want_hidden else None
        lib().or_decode(ctypes.byref(self.m), _p(tokens), M, pos, _p(nxt),
                        _p(logits) if logits is not None else None, _p(margin),
                        _p(hidden) if hidden is not None else None)
        return nxt, margin, logits, hidden

    def decode_skip(self, tokens, pos: int, skip=None, want_logits: bool = False, want_cosine: bool = False):
        """Pass with layer skip: skip is None or [n_layer] flags.  Returns (next [M], margins [M],
        logits [M][vocab] or None, cosine [M][n_layer] or None; NaN where a layer was skipped)."""
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        M, n = tokens.size, self.m.n_layer
        sk = None if skip is None else np.ascontiguousarray(np.asarray(skip, dtype=np.uint8).reshape(n))
        nxt = np.empty(M, dtype=np.int32)
        margin = np.empty(M, dtype=np.float64)
        logits = np.empty((M, self.vocab), dtype=np.float64) if want_logits else None
        cos = np.full((M, n), np.nan, dtype=np.float64) if want_cosine else None
        lib().or_decode_ex(ctypes.byref(self.m), _p(tokens), M, pos, _p(sk) if sk is not None else None, _p(nxt),
                           _p(logits) if logits is not None else None, _p(margin), None,
                           _p(cos) if cos is not None else None)
        return nxt, margin, logits, cos


def select_skip(score, n_skip: int, first: int = 0, last: int | None = None) -> np.ndarray:
    """or_select_skip: flags of the n_skip layers in [first, last) with the largest scores."""
    sc = np.ascontiguousarray(np.asarray(score, dtype=np.float64).reshape(-1))
    n = sc.size
    last = n if last is None else last
    mask = np.zeros(n, dtype=np.uint8)
    if lib().or_select_skip(_p(sc), n, n_skip, first, last, _p(mask)) != 0:
        raise ValueError("or_select_skip: bad arguments")
    return mask
