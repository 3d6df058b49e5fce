"""The C ABI library loads and exports every symbol include/nt.h declares (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "nt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nt_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for n in ["nt_gemv_q", "nt_gemm_q_small", "nt_decode_layer", "nt_decode_step", "nt_verify_step"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    import quantized_decode_dequant_amd as nt
    from quantized_decode_dequant_amd import build
    build.build(force=False)
    L = ctypes.CDLL(nt.LIB_PATH)
    missing = [n for n in declared_symbols() if not hasattr(L, n)]
    assert not missing, missing
    assert set(declared_symbols()) == set(nt.EXPORTS)


def test_metadata_calls_without_gpu():
    import quantized_decode_dequant_amd as nt
    L = nt.lib()
    assert [L.nt_block_elems(f) for f in range(7)] == [32, 32, 256, 256, 256, 1, 1]
    assert [L.nt_block_bytes(f) for f in range(7)] == [34, 18, 144, 210, 176, 2, 4]
    assert L.nt_row_bytes(nt.NT_Q5_K, 8192) == 5632
    assert L.nt_row_bytes(nt.NT_F16, 100) == 200
    assert L.nt_block_elems(9) == 0
    assert L.nt_row_bytes(nt.NT_Q4_K, 8192) == 4608
    assert L.nt_row_bytes(nt.NT_Q6_K, 28672) == 23520
    assert L.nt_row_bytes(nt.NT_Q4_K, 8191) == 0
    assert L.nt_status_str(-3) == b"workspace too small"


def test_gemv_argument_errors_return_before_any_launch():
    # every call here fails validation, so no GPU work is enqueued
    import quantized_decode_dequant_amd as nt
    L = nt.lib()
    buf = ctypes.create_string_buffer(64)
    a = (ctypes.addressof(buf) + 15) & ~15
    assert L.nt_gemv_q(7, a, a, a, 4, 256, None) == -1            # unknown format
    assert L.nt_gemv_q(nt.NT_Q4_K, a, a, a, 4, 100, None) == -1   # cols % 256
    assert L.nt_gemv_q(nt.NT_Q4_K, None, a, a, 4, 256, None) == -1
    assert L.nt_gemv_q(nt.NT_Q4_K, a + 2, a, a, 4, 256, None) == -2
    assert L.nt_gemv_q(nt.NT_Q4_K, a, a, a, 0, 256, None) == 0      # empty: no-op
    assert L.nt_gemv_q(nt.NT_Q8_0, a, a, a, 4, 1 << 20, None) == -5 # too wide
