"""Seeded synthetic inputs for the quantized decode path.

Test and benchmark infrastructure: the fp64 oracle and the HIP path are both
fed from these buffers.  Nothing here computes any part of the decode (no
dequantization, no dot products, no normalisation); it only draws bytes.
The C source ``synth.c`` documents the random stream and the block byte
layouts it writes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "synth.c")
_LIB = os.path.join(_DIR, "libsynth.so")

BASE_SEED = 20261202

# Format ids shared with the C ABI of the library and the oracle.
Q8_0, Q4_0, Q4_K, Q6_K, Q5_K, F16, F32 = 0, 1, 2, 3, 4, 5, 6
FMT_NAMES = {Q8_0: "q8_0", Q4_0: "q4_0", Q4_K: "q4_k", Q6_K: "q6_k", Q5_K: "q5_k", F16: "f16", F32: "f32"}
# (weights per block, bytes per block)
BLOCK = {Q8_0: (32, 34), Q4_0: (32, 18), Q4_K: (256, 144), Q6_K: (256, 210), Q5_K: (256, 176), F16: (1, 2),
         F32: (1, 4)}


def row_bytes(fmt: int, cols: int) -> int:
    qk, bb = BLOCK[fmt]
    assert cols % qk == 0, (fmt, cols)
    return cols // qk * bb


def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return rows * row_bytes(fmt, cols)


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64]
        L.synth_word.restype = u64
        L.synth_word.argtypes = [u64, u64]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [dbl]
        L.synth_quant.restype = ctypes.c_int
        L.synth_quant.argtypes = [ctypes.c_int, u64, i64, i64, dbl, dbl, vp]
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [u64, i64, i64, dbl, dbl, vp]
        L.synth_normal_f16.restype = None
        L.synth_normal_f16.argtypes = [u64, i64, i64, vp]
        L.synth_uint_below.restype = None
        L.synth_uint_below.argtypes = [u64, i64, ctypes.c_uint32, vp]
        _lib = L
    return _lib


def key(*tags: int, seed: int = BASE_SEED) -> int:
    """Key of the sub-stream named by up to three integer tags."""
    t = list(tags) + [0] * (3 - len(tags))
    assert len(t) == 3
    return lib().synth_key(seed, *[int(v) & 0xFFFFFFFFFFFFFFFF for v in t])


def _ptr(out) -> int:
    if isinstance(out, np.ndarray):
        assert out.flags["C_CONTIGUOUS"]
        return out.ctypes.data
    return int(out)  # raw host address (e.g. pinned memory)


def quant(fmt: int, rows: int, cols: int, k: int, out=None, dlo: float = 1e-3, dhi: float = 1e-2,
          row0: int = 0) -> np.ndarray | None:
    """Rows [row0, row0+rows) of a seeded quantized matrix with `cols` columns."""
    nb_row = cols // BLOCK[fmt][0]
    nbytes = matrix_bytes(fmt, rows, cols)
    ret = None
    if out is None:
        out = ret = np.empty(nbytes, dtype=np.uint8)
    rc = lib().synth_quant(fmt, k, row0 * nb_row, rows * nb_row, dlo, dhi, _ptr(out))
    assert rc == 0
    return ret


def normal_f32(k: int, n: int, mean: float = 0.0, std: float = 1.0, out=None, i0: int = 0):
    ret = None
    if out is None:
        out = ret = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(k, i0, n, mean, std, _ptr(out))
    return ret


def normal_f16(k: int, n: int, out=None, i0: int = 0):
    """f16 bit patterns (uint16) of N(0,1) draws."""
    ret = None
    if out is None:
        out = ret = np.empty(n, dtype=np.uint16)
    lib().synth_normal_f16(k, i0, n, _ptr(out))
    return ret


def uint_below(k: int, n: int, bound: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_uint_below(k, n, bound, out.ctypes.data)
    return out


def f64_to_f16_bits(v: float) -> int:
    return int(lib().synth_f64_to_f16(float(v)))
