"""Pins of the oracle GEMV: dense numpy fp64 matmul over the decoded matrix, one-hot x."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("rows,cols", [(37, 512), (5, 256), (1, 2048)])
def test_gemv_equals_dense_matmul(fmt, rows, cols):
    W = synth.quant(fmt, rows, cols, synth.key(wl.W_TEST, fmt, rows * cols))
    x = wl.gen_x(cols, wl.W_TEST, fmt, rows)
    dense = oracle.dequant(fmt, W, rows, cols)
    ref = dense @ x.astype(np.float64)
    y = oracle.gemv(fmt, W, x, rows, cols)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_one_hot_selects_column(fmt):
    rows, cols = 9, 512
    W = synth.quant(fmt, rows, cols, synth.key(wl.W_TEST, 7, fmt))
    dense = oracle.dequant(fmt, W, rows, cols)
    for k in [0, 1, 15, 16, 31, 32, 100, 255, 256, 511]:
        x = np.zeros(cols, np.float32)
        x[k] = 1.0
        assert np.array_equal(oracle.gemv(fmt, W, x, rows, cols), dense[:, k])


def test_gemv_f32_input_is_widened_exactly():
    rows, cols = 4, 256
    W = synth.quant(0, rows, cols, synth.key(wl.W_TEST, 8))
    x = wl.gen_x(cols, wl.W_TEST, 8)
    assert np.array_equal(oracle.gemv(0, W, x, rows, cols), oracle.gemv(0, W, x.astype(np.float64), rows, cols))
