"""Kernel-level entry points of libqwg.so on torch device tensors (argument marshalling only).

PyTorch provides device memory and streams; every computation is a library kernel."""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import call, lib


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def block_bytes(qtype: int) -> int:
    return int(lib().qwg_block_bytes(qtype))


def block_weights(qtype: int) -> int:
    return int(lib().qwg_block_weights(qtype))


def row_bytes(qtype: int, k: int) -> int:
    return int(lib().qwg_row_bytes(qtype, k))


def packed_bytes(qtype: int, rows: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    call("qwg_packed_bytes", qtype, rows, k, ctypes.byref(out))
    return int(out.value)


def repack(qtype: int, canon, rows: int, k: int, out=None, stream=None):
    """canon: uint8 device tensor [rows][row_bytes] -> packed uint8 device tensor."""
    torch = _torch()
    if out is None:
        out = torch.empty(max(packed_bytes(qtype, rows, k), 1), dtype=torch.uint8, device=canon.device)
    call("qwg_repack", qtype, _ptr(canon), rows, k, _ptr(out), _stream(stream))
    return out


def dequantize(qtype: int, packed, rows: int, k: int, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((rows, k), dtype=torch.float32, device=packed.device)
    call("qwg_dequantize", qtype, _ptr(packed), rows, k, _ptr(out), _stream(stream))
    return out


def gemv_work_bytes(qtype: int, rows: int, k: int, n_cols: int) -> int:
    return int(lib().qwg_gemv_work_bytes(qtype, rows, k, n_cols))


def gemv(qtype: int, packed, rows: int, k: int, x, out=None, work=None, stream=None):
    """x: fp32 [k] or [n][k] (n <= 8) -> y fp32 [rows] or [n][rows].  work: device scratch of
    gemv_work_bytes(...) bytes (allocated here when not given)."""
    torch = _torch()
    x2 = x.reshape(-1, k)
    n = x2.shape[0]
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    if work is None:
        work = torch.empty(max(gemv_work_bytes(qtype, rows, k, n), 16), dtype=torch.uint8, device=x.device)
    call("qwg_gemv", qtype, _ptr(packed), rows, k, _ptr(x2), n, _ptr(out), _ptr(work),
         work.numel() * work.element_size(), _stream(stream))
    return out.reshape(rows) if x.dim() == 1 else out


def gemv_timed(qtype: int, packed, rows: int, k: int, x, out, work, stream=None) -> float:
    """qwg_gemv_timed: run the GEMV, wait, and return its kernel time in ms."""
    x2 = x.reshape(-1, k)
    ms = ctypes.c_float(0.0)
    call("qwg_gemv_timed", qtype, _ptr(packed), rows, k, _ptr(x2), x2.shape[0], _ptr(out), _ptr(work),
         work.numel() * work.element_size(), ctypes.byref(ms), _stream(stream))
    return float(ms.value)


NOALLOC_SCRATCH_BYTES = 16 << 20  # QWG_NOALLOC_SCRATCH_BYTES


def gemv_noalloc(qtype: int, packed, rows: int, k: int, x, out, stream=None):
    """qwg_gemv_noalloc: the GEMV with the library's static scratch (no work buffer; `out` must be given,
    so nothing is allocated here either)."""
    x2 = x.reshape(-1, k)
    call("qwg_gemv_noalloc", qtype, _ptr(packed), rows, k, _ptr(x2), x2.shape[0], _ptr(out), _stream(stream))
    return out


def set_gemv_geometry(waves_per_group: int = 0, rows_per_wave: int = 0, pipeline_depth: int = 0,
                      row_passes: int = 0) -> None:
    call("qwg_set_gemv_geometry", waves_per_group, rows_per_wave, pipeline_depth, row_passes)


def set_gemv_mfma(on: bool) -> None:
    """Several-column (2..8) Q4_K / Q5_K / Q6_K GEMVs on the matrix cores (True, the default) or on integer dot
    products."""
    call("qwg_set_gemv_mfma", 1 if on else 0)


def rmsnorm(x, g, eps: float, out=None, stream=None):
    torch = _torch()
    n = g.numel()
    x2 = x.reshape(-1, n)
    if out is None:
        out = torch.empty_like(x2)
    call("qwg_rmsnorm", _ptr(x2), _ptr(g), n, eps, x2.shape[0], _ptr(out), _stream(stream))
    return out.reshape(x.shape)


def rope_table(max_pos: int, head_dim: int, base: float) -> np.ndarray:
    t = np.empty((max_pos, head_dim // 2, 2), dtype=np.float32)
    call("qwg_rope_table", max_pos, head_dim, float(base), t.ctypes.data)
    return t


def rope(v, n_heads: int, head_dim: int, table, pos: int, stream=None):
    call("qwg_rope", _ptr(v), n_heads, head_dim, _ptr(table), pos, _stream(stream))
    return v


def attn_work_bytes(n_pos: int, n_q: int, n_kv: int, head_dim: int, n_cols: int) -> int:
    return int(lib().qwg_attn_work_bytes(n_pos, n_q, n_kv, head_dim, n_cols))


def attn_decode(q, kc, vc, n_pos: int, n_q: int, n_kv: int, head_dim: int, n_cols: int = 1, out=None, work=None,
                stream=None):
    """q fp32 [n_cols][n_q*hd]; kc, vc int16/uint16-bit fp16 tensors [ctx][n_kv][hd]."""
    torch = _torch()
    if out is None:
        out = torch.empty((n_cols, n_q * head_dim), dtype=torch.float32, device=q.device)
    wb = attn_work_bytes(n_pos, n_q, n_kv, head_dim, n_cols)
    if work is None:
        work = torch.empty(max(wb, 4), dtype=torch.uint8, device=q.device)
    call("qwg_attn_decode", _ptr(q), _ptr(kc), _ptr(vc), n_pos, n_q, n_kv, head_dim, n_cols, _ptr(out), _ptr(work),
         work.numel() * work.element_size(), _stream(stream))
    return out


def swiglu(g, u, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty_like(g)
    call("qwg_swiglu", _ptr(g), _ptr(u), g.numel(), _ptr(out), _stream(stream))
    return out


def cosine(a, b, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=a.device)
    call("qwg_cosine", _ptr(a), _ptr(b), a.numel(), _ptr(out), _stream(stream))
    return out


def argmax(x, out=None, work=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=x.device)
    if work is None:
        work = torch.empty(int(lib().qwg_argmax_work_bytes()), dtype=torch.uint8, device=x.device)
    call("qwg_argmax", _ptr(x), x.numel(), _ptr(out), _ptr(work), work.numel() * work.element_size(),
         _stream(stream))
    return out


def read_bytes(src, nbytes: Optional[int] = None, sink=None, grid: int = 0, unroll: int = 0, timed: bool = False,
               stream=None):
    """Plain streaming read of a device tensor's bytes (the achievable-bandwidth reference).  Returns the
    sink, or with timed=True the kernel's duration in ms (the call then waits for it)."""
    torch = _torch()
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if sink is None:
        sink = torch.empty(int(lib().qwg_read_sink_words()), dtype=torch.int32, device=src.device)
    ms = ctypes.c_float(0.0)
    call("qwg_read_bytes", _ptr(src), n, _ptr(sink), grid, unroll, ctypes.byref(ms) if timed else None,
         _stream(stream))
    return float(ms.value) if timed else sink
