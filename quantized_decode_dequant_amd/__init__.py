"""Python binding of libnt (the gfx950 quantized decode library).

Argument marshalling only: every step runs in the HIP kernels of libnt.so,
called through its C ABI (include/nt.h).  PyTorch provides device memory and
streams.  There is no fallback: if libnt.so is missing or cannot be loaded,
importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnt.so")

NT_Q8_0, NT_Q4_0, NT_Q4_K, NT_Q6_K, NT_Q5_K, NT_F16, NT_F32 = 0, 1, 2, 3, 4, 5, 6
STATUS = {0: "NT_OK", -1: "NT_EINVAL", -2: "NT_EALIGN", -3: "NT_EWORKSPACE", -4: "NT_EHIP", -5: "NT_EUNSUPPORTED"}


class NtError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_head", ctypes.c_int32), ("n_kv_head", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class QMat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("data", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("ffn_norm", ctypes.c_void_p),
                ("wq", QMat), ("wk", QMat), ("wv", QMat), ("wo", QMat), ("wg", QMat), ("wu", QMat), ("wd", QMat),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("cfg", LayerCfg), ("n_layer", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("tok_emb", QMat), ("lm_head", QMat), ("out_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(Layer)), ("first_streamed", ctypes.c_int32),
                ("host_layer", ctypes.POINTER(ctypes.c_void_p)), ("stage", ctypes.c_void_p * 2),
                ("stage_bytes", ctypes.c_size_t), ("copy_stream", ctypes.c_void_p), ("skip", ctypes.c_void_p)]


class TierPlan(ctypes.Structure):
    _fields_ = [("first_streamed", ctypes.c_int32), ("n_streamed", ctypes.c_int32),
                ("fixed_bytes", ctypes.c_uint64), ("resident_bytes", ctypes.c_uint64),
                ("stage_bytes", ctypes.c_uint64), ("device_bytes", ctypes.c_uint64),
                ("host_bytes", ctypes.c_uint64)]


_lib = None

EXPORTS = {
    # name: (restype, argtypes)
    "nt_block_elems": (ctypes.c_int, [ctypes.c_int]),
    "nt_block_bytes": (ctypes.c_int, [ctypes.c_int]),
    "nt_row_bytes": (ctypes.c_int64, [ctypes.c_int, ctypes.c_int64]),
    "nt_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "nt_max_cols": (ctypes.c_int64, []),
    "nt_gemv_q": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "nt_gemm_q_small_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]),
    "nt_gemm_q_small": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]),
    "nt_layer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(LayerCfg), ctypes.c_int]),
    "nt_decode_layer": (ctypes.c_int, [ctypes.POINTER(LayerCfg), ctypes.POINTER(Layer), ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]),
    "nt_step_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Model), ctypes.c_int]),
    "nt_layer_blob_bytes": (ctypes.c_size_t, [ctypes.POINTER(LayerCfg), ctypes.POINTER(Layer)]),
    "nt_decode_step": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nt_verify_step": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]),
    "nt_calibrate_step": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "nt_select_skip": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]),
    "nt_plan_tiers": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_int, ctypes.c_size_t, ctypes.c_size_t,
                                     ctypes.POINTER(TierPlan)]),
    "nt_spec_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Model), ctypes.c_int]),
    "nt_spec_step": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "nt_trace_begin": (ctypes.c_int, [ctypes.c_int]),
    "nt_trace_begin_every": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "nt_trace_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]),
    "nt_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "nt_test_fail_stream_copy": (ctypes.c_int, [ctypes.c_int]),
    "nt_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(Model), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "nt_decode_step_noalloc_max_bytes": (ctypes.c_size_t, []),
}

TRACE_GEMV, TRACE_GEMV_RESID, TRACE_QKV, TRACE_FFN_UP, TRACE_ATTN = 0, 1, 2, 3, 4


def test_fail_stream_copy(j: int) -> None:
    """Arm the streaming pipeline's failure hook (nt_test_fail_stream_copy)."""
    _check("nt_test_fail_stream_copy", lib().nt_test_fail_stream_copy(int(j)))


def read_probe(buf, out, stream=None) -> None:
    """Streaming read of a whole uint8 device tensor (nt_read_probe)."""
    _check("nt_read_probe", lib().nt_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                                _stream(stream)))


def trace_begin(kind: int, every: int = 1) -> None:
    """Time launches 0, every, 2*every, ... of one kernel kind from now on with
    HIP events (nt_trace_begin_every)."""
    _check("nt_trace_begin_every", lib().nt_trace_begin_every(kind, every))


def trace_end() -> tuple[int, float]:
    """(launches traced, summed milliseconds) since trace_begin (nt_trace_end)."""
    n = ctypes.c_int()
    ms = ctypes.c_double()
    _check("nt_trace_end", lib().nt_trace_end(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def lib():
    """Load libnt.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run quantized_decode_dequant_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise NtError(fn, rc)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def block_elems(fmt: int) -> int:
    return lib().nt_block_elems(fmt)


def block_bytes(fmt: int) -> int:
    return lib().nt_block_bytes(fmt)


def row_bytes(fmt: int, cols: int) -> int:
    return lib().nt_row_bytes(fmt, cols)


def gemv_q(fmt: int, W, x, y, rows: int, cols: int, stream=None) -> None:
    """y = W x  (nt_gemv_q)."""
    _check("nt_gemv_q", lib().nt_gemv_q(fmt, _ptr(W), _ptr(x), _ptr(y), rows, cols, _stream(stream)))


def gemm_q_small_workspace_bytes(M: int, rows: int, cols: int) -> int:
    """Workspace bytes of nt_gemm_q_small (0 when M == 1 or the shape is unsupported)."""
    return lib().nt_gemm_q_small_workspace_bytes(M, rows, cols)


def gemm_q_small(fmt: int, W, X, Y, M: int, rows: int, cols: int, ws=None, stream=None) -> None:
    """Y[m] = W X[m] for M <= 8 tokens, weights read once  (nt_gemm_q_small)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("nt_gemm_q_small",
           lib().nt_gemm_q_small(fmt, _ptr(W), _ptr(X), _ptr(Y), M, rows, cols,
                                 None if ws is None else _ptr(ws), nbytes, _stream(stream)))


def select_skip(score, n_skip: int, first: int = 0, last: int | None = None):
    """Flags (numpy uint8 [n_layer]) of the n_skip layers in [first, last) with the largest
    scores, lower index first among equal scores  (nt_select_skip; host only)."""
    import numpy as np
    sc = np.ascontiguousarray(np.asarray(score, dtype=np.float32).reshape(-1))
    n = sc.size
    mask = np.zeros(n, dtype=np.uint8)
    _check("nt_select_skip", lib().nt_select_skip(sc.ctypes.data, n, n_skip, first, n if last is None else last,
                                                  mask.ctypes.data))
    return mask


def plan_tiers(cfg: LayerCfg, layer_fmts: list, vocab: int, emb_fmt: int, head_fmt: int, M: int,
               device_budget: int, host_budget: int | None = None) -> dict:
    """Device/pinned-host placement of a stack's layers (nt_plan_tiers; host only).
    layer_fmts: one {matrix name: format} dict per layer.  Returns the plan's fields
    and ok (False when no placement meets the limits)."""
    n = len(layer_fmts)
    arr = (Layer * max(1, n))()
    for i, f in enumerate(layer_fmts):
        for name in MAT_NAMES:
            setattr(arr[i], name, QMat(f[name], None))
    m = Model()
    m.cfg = cfg
    m.n_layer = n
    m.vocab = vocab
    m.tok_emb = QMat(emb_fmt, None)
    m.lm_head = QMat(head_fmt, None)
    m.layers = ctypes.cast(arr, ctypes.POINTER(Layer))
    m.first_streamed = n
    plan = TierPlan()
    hb = (1 << 64) - 1 if host_budget is None else host_budget
    rc = lib().nt_plan_tiers(ctypes.byref(m), M, device_budget, hb, ctypes.byref(plan))
    if rc not in (0, -5):
        _check("nt_plan_tiers", rc)
    out = {k: int(getattr(plan, k)) for k, _ in TierPlan._fields_}
    out["ok"] = rc == 0
    return out


def layer_cfg(hidden, n_head, n_kv_head, head_dim, ffn, max_ctx, rope_theta=5e5, rms_eps=1e-5) -> LayerCfg:
    return LayerCfg(hidden, n_head, n_kv_head, head_dim, ffn, max_ctx, rope_theta, rms_eps)


MAT_NAMES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def make_layer(attn_norm, ffn_norm, mats: dict, fmts: dict, k_cache, v_cache) -> Layer:
    """nt_layer over device tensors (mats: name -> uint8 tensor, fmts: name -> format id)."""
    L = Layer()
    L.attn_norm = _ptr(attn_norm)
    L.ffn_norm = _ptr(ffn_norm)
    for n in MAT_NAMES:
        setattr(L, n, QMat(fmts[n], _ptr(mats[n]) if mats.get(n) is not None else None))
    L.k_cache = _ptr(k_cache)
    L.v_cache = _ptr(v_cache)
    return L


def layer_workspace_bytes(cfg: LayerCfg, M: int = 1) -> int:
    return lib().nt_layer_workspace_bytes(ctypes.byref(cfg), M)


def decode_layer(cfg: LayerCfg, layer: Layer, x, M: int, pos_dev, ws, stream=None) -> None:
    """One decoder layer on x ([M][hidden] fp32, in place)  (nt_decode_layer)."""
    _check("nt_decode_layer", lib().nt_decode_layer(ctypes.byref(cfg), ctypes.byref(layer), _ptr(x), M,
                                                    _ptr(pos_dev), _ptr(ws), ws.numel() * ws.element_size(),
                                                    _stream(stream)))


def layer_blob_bytes(cfg: LayerCfg, layer: Layer) -> int:
    return lib().nt_layer_blob_bytes(ctypes.byref(cfg), ctypes.byref(layer))


def blob_offsets(cfg: LayerCfg, fmts: dict, shapes: dict) -> list:
    """Byte offsets of the seven matrices inside a streamed-layer blob (each padded to 256 B)."""
    offs, o = [], 0
    for n in MAT_NAMES:
        offs.append(o)
        r, c = shapes[n]
        o += (r * (c // block_elems(fmts[n])) * block_bytes(fmts[n]) + 255) // 256 * 256
    offs.append(o)
    return offs


class ModelHandle:
    """Keeps an nt_model and the ctypes arrays it points to alive."""

    def __init__(self, cfg: LayerCfg, layers: list, vocab: int, tok_emb, tok_emb_fmt: int, lm_head, lm_head_fmt: int,
                 out_norm, first_streamed: int | None = None, host_layers=None, stage=(None, None),
                 stage_bytes: int = 0, copy_stream=None, skip=None):
        self.layers_arr = (Layer * max(1, len(layers)))(*layers)
        n = len(layers)
        self.skip_arr = None
        self.first_streamed = n if first_streamed is None else first_streamed
        self.host_arr = (ctypes.c_void_p * max(1, n))()
        if host_layers is not None:
            for i, h in enumerate(host_layers):
                self.host_arr[i] = _ptr(h) if h is not None else None
        m = Model()
        m.cfg = cfg
        m.n_layer = n
        m.vocab = vocab
        m.tok_emb = QMat(tok_emb_fmt, _ptr(tok_emb))
        m.lm_head = QMat(lm_head_fmt, _ptr(lm_head))
        m.out_norm = _ptr(out_norm)
        m.layers = ctypes.cast(self.layers_arr, ctypes.POINTER(Layer))
        m.first_streamed = self.first_streamed
        m.host_layer = ctypes.cast(self.host_arr, ctypes.POINTER(ctypes.c_void_p))
        m.stage[0] = _ptr(stage[0])
        m.stage[1] = _ptr(stage[1])
        m.stage_bytes = stage_bytes
        m.copy_stream = _stream(copy_stream) if copy_stream is not None else None
        self.m = m
        self.set_skip(skip)

    def _flags(self, flags):
        if flags is None:
            return None
        arr = (ctypes.c_uint8 * max(1, self.m.n_layer))()
        vals = list(flags)
        if len(vals) != self.m.n_layer:
            raise ValueError("skip flags need one entry per layer")
        for i, v in enumerate(vals):
            arr[i] = 1 if v else 0
        return arr

    def set_skip(self, flags) -> None:
        """Layers with a true flag are not run (nt_model.skip); None runs every layer."""
        self.skip_arr = self._flags(flags)
        self.m.skip = ctypes.cast(self.skip_arr, ctypes.c_void_p).value if self.skip_arr is not None else None

    def workspace_bytes(self, M: int = 1) -> int:
        return lib().nt_step_workspace_bytes(ctypes.byref(self.m), M)

    def decode_step(self, token_dev, pos_dev, next_dev, ws, logits_dev=None, stream=None) -> None:
        """nt_decode_step."""
        _check("nt_decode_step", lib().nt_decode_step(ctypes.byref(self.m), _ptr(token_dev), _ptr(pos_dev),
                                                      _ptr(next_dev), _ptr(logits_dev), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream(stream)))

    def decode_step_noalloc(self, token_dev, pos_dev, next_dev, logits_dev=None, stream=None) -> None:
        """nt_decode_step_noalloc: the decode step on the library's own device workspace."""
        _check("nt_decode_step_noalloc", lib().nt_decode_step_noalloc(ctypes.byref(self.m), _ptr(token_dev),
                                                                      _ptr(pos_dev), _ptr(next_dev),
                                                                      _ptr(logits_dev), _stream(stream)))

    def verify_step(self, tokens_dev, M: int, pos_dev, argmax_dev, ws, logits_dev=None, stream=None) -> None:
        """nt_verify_step."""
        _check("nt_verify_step", lib().nt_verify_step(ctypes.byref(self.m), _ptr(tokens_dev), M, _ptr(pos_dev),
                                                      _ptr(argmax_dev), _ptr(logits_dev), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream(stream)))

    def calibrate_step(self, token_dev, pos_dev, next_dev, cos_dev, ws, stream=None) -> None:
        """nt_calibrate_step: a decode step that adds each layer's input/output cosine
        similarity to cos_dev (fp32 [n_layer])."""
        _check("nt_calibrate_step", lib().nt_calibrate_step(ctypes.byref(self.m), _ptr(token_dev), _ptr(pos_dev),
                                                            _ptr(next_dev), _ptr(cos_dev), _ptr(ws),
                                                            ws.numel() * ws.element_size(), _stream(stream)))

    def spec_workspace_bytes(self, K: int) -> int:
        return lib().nt_spec_workspace_bytes(ctypes.byref(self.m), K)

    def spec_step(self, draft_skip, K: int, cur_dev, pos_dev, out_dev, n_out_dev, ws, stream=None) -> None:
        """nt_spec_step: one self-speculative round (K drafted tokens, one verify pass)."""
        flags = self._flags(draft_skip)
        _check("nt_spec_step", lib().nt_spec_step(ctypes.byref(self.m),
                                                  ctypes.cast(flags, ctypes.c_void_p).value if flags is not None
                                                  else None, K, _ptr(cur_dev), _ptr(pos_dev), _ptr(out_dev),
                                                  _ptr(n_out_dev), _ptr(ws), ws.numel() * ws.element_size(),
                                                  _stream(stream)))
