"""Parity of nt_gemm_q_small (HIP, int8 MFMA, weights read once for M tokens)
against the fp64 oracle, token by token.

Bar: ||Y[m] - Y_oracle[m]||_inf / ||Y_oracle[m]||_inf <= 2e-3 for every token m;
for a one-row matrix, over that row's M values.
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


def run_small(fmt, M, rows, cols, tag, guard=64):
    import torch
    import quantized_decode_dequant_amd as nt
    say(f"gemm_q_small fmt={synth.FMT_NAMES[fmt]} M={M} rows={rows} cols={cols}")
    W = synth.quant(fmt, rows, cols, synth.key(wl.W_TEST, 500 + tag, fmt))
    X = np.stack([wl.gen_x(cols, wl.W_TEST, 600 + tag + m) for m in range(M)]).astype(np.float32)
    Wd = to_dev(W)
    Xd = to_dev(X)
    ybuf = torch.full((M * rows + 2 * guard,), float("nan"), dtype=torch.float32, device=device())
    Y = ybuf[guard:guard + M * rows]
    nb = nt.gemm_q_small_workspace_bytes(M, rows, cols) if M > 1 else 0
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=device()).fill_(0xA5)  # contents need no init
    nt.gemm_q_small(fmt, Wd, Xd, Y, M, rows, cols, ws if M > 1 else None)
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert np.isnan(yb[:guard]).all() and np.isnan(yb[guard + M * rows:]).all(), "write outside Y"
    return W, X, yb[guard:guard + M * rows].reshape(M, rows), (Wd, Xd, ws)


def check_tokens(fmt, W, X, Y, rows, cols, row_idx=None):
    if row_idx is None:
        Wf = oracle.dequant(fmt, W, rows, cols)
        idx = np.arange(rows)
    else:
        rb = synth.row_bytes(fmt, cols)
        Wf = np.stack([oracle.dequant(fmt, W[r * rb:(r + 1) * rb], 1, cols)[0] for r in row_idx])
        idx = np.asarray(row_idx)
    worst = 0.0
    refs = np.stack([Wf @ X[m].astype(np.float64) for m in range(X.shape[0])])
    if len(idx) == 1:
        # one row: its output vector is the M tokens' values (the max-relative
        # metric over a single value measures the cancellation of that one sum)
        worst = rel_inf(Y[:, idx[0]], refs[:, 0])
    else:
        for m in range(X.shape[0]):
            worst = max(worst, rel_inf(Y[m, idx], refs[m]))
    say(f"  max rel err over tokens {worst:.2e}")
    assert worst <= GEMV_TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [2, 3, 8])
@pytest.mark.parametrize("rows,cols", [(1, 256), (37, 512), (300, 2048), (129, 14336)])
def test_gemm_small_parity(fmt, M, rows, cols):
    W, X, Y, _ = run_small(fmt, M, rows, cols, tag=rows + cols + M)
    check_tokens(fmt, W, X, Y, rows, cols)


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0])
@pytest.mark.parametrize("cols", [32, 4128, 2080])
def test_gemm_small_ragged_columns(fmt, cols):
    # 32-weight formats: the last 256-column tile-slice holds fewer blocks
    W, X, Y, _ = run_small(fmt, 4, 50, cols, tag=cols)
    check_tokens(fmt, W, X, Y, 50, cols)


@pytest.mark.parametrize("name", ["wq", "wk", "wv", "wo", "wg", "wd"])
@pytest.mark.parametrize("M", [4, 8])
def test_gemm_small_70b_shapes(name, M):
    # Llama-70B-shaped projections in the Q4_K_M mix, every row of every
    # token against the oracle's GEMV
    rows, cols = wl.LLAMA70B.mat_shape(name)
    fmt = wl.Q4_K_M[name]
    W, X, Y, _ = run_small(fmt, M, rows, cols, tag=700 + wl.MAT_TAG[name])
    worst = 0.0
    for m in range(M):
        worst = max(worst, rel_inf(Y[m], oracle.gemv(fmt, W, X[m], rows, cols)))
    say(f"  max rel err over tokens {worst:.2e}")
    assert worst <= GEMV_TOL


def test_gemm_small_m1_is_gemv_and_deterministic():
    import torch
    import quantized_decode_dequant_amd as nt
    fmt, rows, cols = synth.Q4_K, 300, 2048
    W, X, Y, (Wd, Xd, ws) = run_small(fmt, 3, rows, cols, tag=42)
    Y2 = torch.empty(3 * rows, dtype=torch.float32, device=device())
    nt.gemm_q_small(fmt, Wd, Xd, Y2, 3, rows, cols, ws)
    torch.cuda.synchronize()
    assert np.array_equal(Y.reshape(-1), Y2.cpu().numpy()), "two runs differ"
    # M = 1 is the GEMV engine
    y1 = torch.empty(rows, dtype=torch.float32, device=device())
    yg = torch.empty(rows, dtype=torch.float32, device=device())
    nt.gemm_q_small(fmt, Wd, Xd[0], y1, 1, rows, cols)
    nt.gemv_q(fmt, Wd, Xd[0], yg, rows, cols)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy(), yg.cpu().numpy())


def test_gemm_small_argument_errors():
    import torch
    import quantized_decode_dequant_amd as nt
    dev = device()
    W = torch.zeros(4352 * 4, dtype=torch.uint8, device=dev)
    X = torch.zeros(2 * 4096, dtype=torch.float32, device=dev)
    Y = torch.zeros(2 * 4, dtype=torch.float32, device=dev)
    small = torch.zeros(256, dtype=torch.uint8, device=dev)
    with pytest.raises(nt.NtError):  # workspace too small
        nt.gemm_q_small(synth.Q8_0, W, X, Y, 2, 4, 4096, small)
    with pytest.raises(nt.NtError):  # no workspace for M > 1
        nt.gemm_q_small(synth.Q8_0, W, X, Y, 2, 4, 4096, None)
    with pytest.raises(nt.NtError):  # M out of range
        nt.gemm_q_small(synth.Q8_0, W, X, Y, 9, 4, 4096, small)
    assert nt.gemm_q_small_workspace_bytes(1, 4, 4096) == 0
    assert nt.gemm_q_small_workspace_bytes(2, 4, 4096) > 0
