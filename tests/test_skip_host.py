"""Host logic of layer skip and speculative rounds in libnt (no GPU needed):
nt_select_skip picks the same layers as the oracle's choice on the same
scores, and the entry points reject bad arguments before enqueuing work."""
import ctypes

import numpy as np
import pytest

import oracle


def test_select_skip_matches_oracle_on_random_scores_with_ties():
    import quantized_decode_dequant_amd as nt
    rng = np.random.default_rng(7)
    for case in range(300):
        n = int(rng.integers(1, 90))
        # few distinct values so that ties are common
        sc = rng.choice(np.float32([0.1, 0.5, 0.9, 0.95, 0.99, -0.3]), size=n) if case % 2 else \
            rng.uniform(-1, 1, n).astype(np.float32)
        first = int(rng.integers(0, n + 1))
        last = int(rng.integers(first, n + 1))
        k = int(rng.integers(0, last - first + 1))
        got = nt.select_skip(sc, k, first, last)
        ref = oracle.select_skip(sc.astype(np.float64), k, first, last)
        assert np.array_equal(got, ref), (case, n, first, last, k)
        assert int(got.sum()) == k


def test_select_skip_errors():
    import quantized_decode_dequant_amd as nt
    sc = np.float32([0.5, np.nan, 0.7])
    with pytest.raises(nt.NtError):
        nt.select_skip(sc, 1)                  # NaN inside the range
    assert nt.select_skip(sc, 1, first=2).tolist() == [0, 0, 1]
    with pytest.raises(nt.NtError):
        nt.select_skip(np.float32([0.1, 0.2]), 3)
    with pytest.raises(nt.NtError):
        nt.select_skip(np.float32([0.1, 0.2]), 0, first=2, last=1)


def test_spec_and_calibrate_reject_bad_arguments_before_any_launch():
    import quantized_decode_dequant_amd as nt
    L = nt.lib()
    m = nt.Model()  # zeroed: its config is invalid
    buf = ctypes.create_string_buffer(4096)
    a = (ctypes.addressof(buf) + 255) & ~255
    assert L.nt_spec_workspace_bytes(ctypes.byref(m), 3) == 0
    for K in (0, 8):
        assert L.nt_spec_step(ctypes.byref(m), None, K, a, a, a, a, a, 1024, None) == -1
    assert L.nt_spec_step(ctypes.byref(m), None, 3, a, a, a, a, a, 1024, None) == -1   # bad config
    assert L.nt_spec_step(None, None, 3, a, a, a, a, a, 1024, None) == -1
    assert L.nt_calibrate_step(ctypes.byref(m), a, a, a, None, a, 1024, None) == -1
    assert L.nt_calibrate_step(ctypes.byref(m), a, a, a, a, a, 1024, None) == -1
