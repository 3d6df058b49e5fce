"""Helpers of the GPU tests: device placement and error metrics."""
import numpy as np


def device():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, pad: int = 0, fill: int = 0):
    """Device copy of a host array, optionally inside a guard band of `pad` elements each side."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if pad == 0:
        return t.to(device())
    full = torch.full((a.size + 2 * pad,), fill, dtype=t.dtype)
    full[pad:pad + a.size] = t.reshape(-1)
    return full.to(device())[pad:pad + a.size].view(t.shape)


def rel_inf(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
