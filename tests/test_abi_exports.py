"""The C-ABI library loads and exports every function include/qwg.h declares (no GPU calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    names = re.findall(r"\b(qwg_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("qwg_gemv", "qwg_dequantize", "qwg_repack", "qwg_decode_step", "qwg_calibrate_skip",
                 "qwg_spec_step", "qwg_model_set_tensor", "qwg_attn_decode"):
        assert must in names


def test_library_exports_every_declared_symbol():
    from quantized_weight_streaming_gemv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqwg.so not built")
    L = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_size_queries_without_gpu():
    from quantized_weight_streaming_gemv_amd import _lib, ops
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqwg.so not built")
    assert [ops.block_bytes(q) for q in (2, 8, 12, 13, 14)] == [18, 34, 144, 176, 210]
    assert ops.row_bytes(12, 8192) == 32 * 144 and ops.row_bytes(12, 100) == 0
    # packed layout keeps the payload bytes (plus < 1 KiB alignment per matrix)
    for q in (2, 8, 12, 13, 14):
        canon = 4096 * ops.row_bytes(q, 8192)
        pb = ops.packed_bytes(q, 4096, 8192)
        assert canon <= pb < canon + 1024
    with pytest.raises(_lib.QwgError):
        ops.packed_bytes(12, 10, 100)
    with pytest.raises(_lib.QwgError):
        ops.packed_bytes(7, 10, 256)


def test_model_create_validates_without_gpu():
    from quantized_weight_streaming_gemv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqwg.so not built")
    L = _lib.lib()
    d = _lib.ModelDesc(2, 512, 4, 2, 128, 1536, 1000, 64, 5e5, 1e-5, -1, 12, 12, 12, 12, 4)
    h = ctypes.c_void_p(None)
    assert L.qwg_model_create(ctypes.byref(d), ctypes.byref(h)) == 0
    assert L.qwg_model_arena_bytes(h) > 0
    L.qwg_model_destroy(h)
    bad = _lib.ModelDesc(2, 500, 4, 2, 128, 1536, 1000, 64, 5e5, 1e-5, -1, 12, 12, 12, 12, 4)
    assert L.qwg_model_create(ctypes.byref(bad), ctypes.byref(h)) == -2
    bad2 = _lib.ModelDesc(2, 512, 4, 2, 64, 1536, 1000, 64, 5e5, 1e-5, -1, 12, 12, 12, 12, 4)
    assert L.qwg_model_create(ctypes.byref(bad2), ctypes.byref(h)) == -2
    bad3 = _lib.ModelDesc(2, 512, 4, 2, 128, 1536, 1000, 64, 5e5, 1e-5, -1, 7, 12, 12, 12, 4)
    assert L.qwg_model_create(ctypes.byref(bad3), ctypes.byref(h)) == -6


def test_pointer_checks_without_gpu():
    """Misaligned or NULL device pointers are refused before anything reaches the GPU (the addresses
    below are never dereferenced)."""
    from quantized_weight_streaming_gemv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqwg.so not built")
    L = _lib.lib()
    A, M = 1 << 20, (1 << 20) + 4  # aligned / misaligned fake addresses
    gw = L.qwg_gemv_work_bytes(12, 16, 256, 1)
    assert gw > 0 and L.qwg_gemv_work_bytes(12, 16, 300, 1) == 0 and L.qwg_gemv_work_bytes(12, 16, 256, 9) == 0
    assert L.qwg_gemv(12, M, 16, 256, A, 1, A, A, gw, None) == -1
    assert L.qwg_gemv(12, A, 16, 256, M, 1, A, A, gw, None) == -1
    assert L.qwg_gemv(12, A, 16, 256, A, 1, A, M, gw, None) == -1
    assert L.qwg_gemv(12, None, 16, 256, A, 1, A, A, gw, None) == -1
    assert L.qwg_gemv(12, A, 16, 256, A, 1, A, None, gw, None) == -1
    assert L.qwg_gemv(12, A, 16, 256, A, 1, A, A, gw - 16, None) == -3
    # K-split shapes need room for the partial sums as well as the digits
    assert L.qwg_gemv_work_bytes(12, 4096, 65536, 8) > L.qwg_gemv_work_bytes(12, 4096, 4096, 8)
    aw = L.qwg_argmax_work_bytes()
    assert aw >= 8
    assert L.qwg_argmax(A, 100, A, A, aw - 1, None) == -3
    assert L.qwg_argmax(A, 100, A, None, aw, None) == -1
    assert L.qwg_argmax(A, 100, A, A + 4, aw, None) == -1
    assert L.qwg_dequantize(12, A, 16, 256, M, None) == -1
    wb = L.qwg_attn_work_bytes(100, 8, 2, 128, 1)
    assert wb > 0
    for bad in range(5):
        p = [A] * 5
        p[bad] = M
        assert L.qwg_attn_decode(p[0], p[1], p[2], 100, 8, 2, 128, 1, p[3], p[4], wb, None) == -1, bad
    assert L.qwg_attn_decode(A, A, A, 100, 8, 2, 128, 1, A, A, wb - 8, None) == -3
    # up to 64 columns (a prompt pass), at most 64 query heads per KV head
    assert L.qwg_attn_work_bytes(100, 64, 8, 128, 64) > 0 and L.qwg_attn_work_bytes(100, 64, 8, 128, 65) == 0
    assert L.qwg_attn_work_bytes(100, 65, 1, 128, 1) == 0 and L.qwg_attn_work_bytes(100, 64, 1, 128, 64) > 0
    assert L.qwg_attn_decode(A, A, A, 100, 8, 2, 128, 65, A, A, 1 << 30, None) == -2
    assert L.qwg_attn_decode(A, A, A, 100, 65, 1, 128, 1, A, A, 1 << 30, None) == -2
    assert L.qwg_rope(M, 8, 128, A, 0, None) == -1
    assert L.qwg_rope(A, 8, 128, A, -1, None) == -2
    assert L.qwg_rope(A, 8, 64, A, 0, None) == -2
