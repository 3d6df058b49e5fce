"""Parity of nt_gemv_q (HIP) against the fp64 oracle, element by element.

Bar: ||y - y_oracle||_inf / ||y_oracle||_inf <= 2e-3 per output vector.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as wl
from tests.gpu_util import device, rel_inf, say, to_dev

pytestmark = pytest.mark.gpu

GEMV_TOL = 2e-3
FMTS = [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32]


def run_gemv(fmt, rows, cols, tag, guard=64):
    import torch
    import quantized_decode_dequant_amd as nt
    say(f"gemv fmt={synth.FMT_NAMES[fmt]} rows={rows} cols={cols}")
    W = synth.quant(fmt, rows, cols, synth.key(wl.W_TEST, tag, fmt))
    x = wl.gen_x(cols, wl.W_TEST, tag)
    Wd = to_dev(W)
    xd = to_dev(x)
    ybuf = torch.full((rows + 2 * guard,), float("nan"), dtype=torch.float32, device=device())
    y = ybuf[guard:guard + rows]
    nt.gemv_q(fmt, Wd, xd, y, rows, cols)
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert np.isnan(yb[:guard]).all() and np.isnan(yb[guard + rows:]).all(), "write outside y"
    return W, x, yb[guard:guard + rows]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 256), (37, 512), (300, 2048), (1000, 4096), (129, 14336)])
def test_gemv_parity_small(fmt, rows, cols):
    W, x, y = run_gemv(fmt, rows, cols, tag=rows + cols)
    ref = oracle.gemv(fmt, W, x, rows, cols)
    err = rel_inf(y, ref)
    say(f"  max rel err {err:.2e}")
    assert err <= GEMV_TOL


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_K, synth.Q6_K])
@pytest.mark.parametrize("rows", [8192, 8448])
def test_gemv_burst_boundary(fmt, rows):
    # 4096 columns (one slice) over 256 workgroups of 16 waves: 8192 rows give
    # every workgroup 32 segments (the whole share in flight at once, the burst
    # launch), 8448 give some 33 (the streaming launch)
    W, x, y = run_gemv(fmt, rows, 4096, tag=rows + fmt)
    ref = oracle.gemv(fmt, W, x, rows, 4096)
    err = rel_inf(y, ref)
    say(f"  max rel err {err:.2e}")
    assert err <= GEMV_TOL


def test_gemv_q8_0_4096_full():
    # the single-GEMV workload: Q8_0 4096 x 4096
    W, x, y = run_gemv(synth.Q8_0, 4096, 4096, tag=1)
    ref = oracle.gemv(synth.Q8_0, W, x, 4096, 4096)
    err = rel_inf(y, ref)
    say(f"  Q8_0 4096x4096 max rel err {err:.2e}")
    assert err <= GEMV_TOL


@pytest.mark.parametrize("name", ["wq", "wk", "wv", "wg", "wd"])
def test_gemv_70b_projection_shapes(name):
    # Llama-70B-shaped projections in the Q4_K_M mix, full size
    rows, cols = wl.LLAMA70B.mat_shape(name)
    fmt = wl.Q4_K_M[name]
    W, x, y = run_gemv(fmt, rows, cols, tag=100 + wl.MAT_TAG[name])
    ref = oracle.gemv(fmt, W, x, rows, cols)
    err = rel_inf(y, ref)
    say(f"  70B {name} {rows}x{cols} max rel err {err:.2e}")
    assert err <= GEMV_TOL


def test_gemv_70b_gate_q5_k_full():
    rows, cols = wl.LLAMA70B.mat_shape("wg")
    W, x, y = run_gemv(synth.Q5_K, rows, cols, tag=150)
    err = rel_inf(y, oracle.gemv(synth.Q5_K, W, x, rows, cols))
    say(f"  70B gate Q5_K {rows}x{cols} max rel err {err:.2e}")
    assert err <= GEMV_TOL


@pytest.mark.parametrize("fmt,cols", [(synth.F16, 8), (synth.F16, 1000), (synth.F16, 4104),
                                      (synth.F32, 4), (synth.F32, 1004), (synth.F32, 8196)])
@pytest.mark.parametrize("rows", [1, 3, 257])
def test_gemv_unquantized_ragged(fmt, cols, rows):
    W, x, y = run_gemv(fmt, rows, cols, tag=cols + rows)
    err = rel_inf(y, oracle.gemv(fmt, W, x, rows, cols))
    say(f"  max rel err {err:.2e}")
    assert err <= 1e-5


def test_gemv_unquantized_argument_errors():
    import torch
    import quantized_decode_dequant_amd as nt
    L = nt.lib()
    buf = torch.zeros(4096, dtype=torch.uint8, device=device())
    a = buf.data_ptr()
    assert L.nt_gemv_q(synth.F16, a, a, a, 4, 4, None) == -1     # 4 x 2 bytes: not whole 16-byte loads
    assert L.nt_gemv_q(synth.F32, a, a, a, 4, 6, None) == -1
    assert L.nt_gemv_q(synth.F32, a + 4, a, a, 4, 8, None) == -2


def test_gemv_deterministic_and_empty():
    import torch
    import quantized_decode_dequant_amd as nt
    rows, cols = 2048, 8192
    W = to_dev(synth.quant(synth.Q4_K, rows, cols, synth.key(wl.W_TEST, 77)))
    x = to_dev(wl.gen_x(cols, wl.W_TEST, 77))
    y1 = torch.empty(rows, device=device())
    y2 = torch.empty(rows, device=device())
    nt.gemv_q(synth.Q4_K, W, x, y1, rows, cols)
    nt.gemv_q(synth.Q4_K, W, x, y2, rows, cols)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    nt.gemv_q(synth.Q4_K, W, x, y1, 0, cols)  # rows == 0: no-op
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_gemv_special_inputs():
    import torch
    import quantized_decode_dequant_amd as nt
    rows, cols = 64, 1024
    for fmt in FMTS:
        W = synth.quant(fmt, rows, cols, synth.key(wl.W_TEST, 88, fmt))
        Wd = to_dev(W)
        for kind in ["zero", "onehot", "huge"]:
            x = np.zeros(cols, np.float32)
            if kind == "onehot":
                x[333] = 1.0
            elif kind == "huge":
                x = wl.gen_x(cols, wl.W_TEST, 89) * np.float32(1e30)
            y = torch.empty(rows, device=device())
            nt.gemv_q(fmt, Wd, to_dev(x), y, rows, cols)
            torch.cuda.synchronize()
            ref = oracle.gemv(fmt, W, x, rows, cols)
            got = y.cpu().numpy()
            if kind == "zero":
                assert not got.any()
            else:
                assert rel_inf(got, ref) <= GEMV_TOL, (fmt, kind)


def test_trace_times_each_launch_inside_the_stream_interval():
    # nt_trace_*: every launch of the kind (or one in `every`) is timed by
    # events stamped with the kernel's own start and end, so the summed
    # durations are positive and fit inside an event pair around all of them;
    # the traced launches still give the oracle's result
    import torch
    import quantized_decode_dequant_amd as nt
    rows, cols, n = 4096, 4096, 12
    W = synth.quant(synth.Q8_0, rows, cols, synth.key(wl.W_TEST, 91, synth.Q8_0))
    x = wl.gen_x(cols, wl.W_TEST, 91)
    Wd, xd = to_dev(W), to_dev(x)
    y = torch.empty(rows, dtype=torch.float32, device=device())
    for every, expect in ((1, n), (5, 3)):
        torch.cuda.synchronize()
        nt.trace_begin(nt.TRACE_GEMV, every)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            nt.gemv_q(synth.Q8_0, Wd, xd, y, rows, cols)
        e1.record()
        torch.cuda.synchronize()
        launches, ms = nt.trace_end()
        outer = e0.elapsed_time(e1)
        say(f"  every {every}: {launches} launches, {ms * 1e3 / max(launches, 1):.2f} us each, "
            f"{outer * 1e3 / n:.2f} us per launch between outer events")
        assert launches == expect
        assert 0.0 < ms < outer
    err = rel_inf(y.cpu().numpy(), oracle.gemv(synth.Q8_0, W, x, rows, cols))
    assert err <= GEMV_TOL
