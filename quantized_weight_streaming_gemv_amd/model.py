"""Model-level entry points of libqwg.so: a Llama decoder in a torch-allocated HBM arena.

PyTorch supplies the device arena and the streams; the library places the weights (resident
layers in the arena, streamed layers in pinned host images), runs every kernel and owns the
decode / skip / self-speculative control flow."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from ._lib import ModelDesc, call, lib


def _layer_types(layer_qtypes, n_layers):
    """A C-contiguous int32 [n_layers][4] copy of per-layer (QKV, WO, GATE|UP, DOWN) types, or None."""
    if layer_qtypes is None:
        return None
    t = np.ascontiguousarray(layer_qtypes, dtype=np.int32)
    if t.shape != (n_layers, 4):
        raise ValueError("layer_qtypes must be [n_layers][4]")
    return t


def plan_residency(*, n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_ctx, rope_theta, rms_eps, qtype_attn,
                   qtype_ffn, qtype_embed, qtype_head, max_cols=1, layer_qtypes=None, device_budget: int = 0,
                   host_budget: int = 0):
    """Automatic tier placement (qwg_plan_residency): (n_resident, arena_bytes, pinned_bytes) for the
    largest number of HBM-resident layers whose arena fits device_budget bytes (0 = free device
    memory less a reserve), the rest streamed from pinned host images within host_budget bytes
    (0 = 90% of MemAvailable).  Raises QwgError(QWG_E_NOMEM) if nothing fits."""
    lt = _layer_types(layer_qtypes, n_layers)
    desc = ModelDesc(n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_ctx, rope_theta, rms_eps, -1,
                     qtype_attn, qtype_ffn, qtype_embed, qtype_head, max_cols, None if lt is None else lt.ctypes.data)
    n, a, h = ctypes.c_int32(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    call("qwg_plan_residency", ctypes.byref(desc), int(device_budget), int(host_budget), ctypes.byref(n),
         ctypes.byref(a), ctypes.byref(h))
    return int(n.value), int(a.value), int(h.value)


class Model:
    def __init__(self, *, n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_ctx, rope_theta, rms_eps,
                 qtype_attn, qtype_ffn, qtype_embed, qtype_head, n_resident=-1, max_cols=1, layer_qtypes=None,
                 device="cuda:0"):
        import torch
        self.torch = torch
        lt = _layer_types(layer_qtypes, n_layers)  # read by qwg_model_create only (the model copies it)
        self.desc = ModelDesc(n_layers, hidden, n_q, n_kv, head_dim, ffn, vocab, max_ctx, rope_theta, rms_eps,
                              n_resident, qtype_attn, qtype_ffn, qtype_embed, qtype_head, max_cols,
                              None if lt is None else lt.ctypes.data)
        self.handle = ctypes.c_void_p(None)
        call("qwg_model_create", ctypes.byref(self.desc), ctypes.byref(self.handle))
        self.arena_bytes = int(lib().qwg_model_arena_bytes(self.handle))
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=self.device)
            self.compute_stream = torch.cuda.current_stream(self.device)
            self.copy_stream = torch.cuda.Stream(self.device)
        call("qwg_model_bind", self.handle, self.arena.data_ptr(), self.arena_bytes,
             self.compute_stream.cuda_stream, self.copy_stream.cuda_stream)
        self.vocab, self.hidden, self.n_layers = vocab, hidden, n_layers

    # ------------------------------------------------------------------ lifetime
    def close(self):
        if self.handle is not None and self.handle.value:
            lib().qwg_model_destroy(self.handle)
            self.handle = None
            self.arena = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ load
    def set_tensor(self, layer: int, tensor_id: int, qtype: int, canon: np.ndarray):
        canon = np.ascontiguousarray(canon, dtype=np.uint8)
        call("qwg_model_set_tensor", self.handle, layer, tensor_id, qtype, canon.ctypes.data, canon.nbytes)

    def set_norm(self, layer: int, which: int, g: np.ndarray):
        g = np.ascontiguousarray(g, dtype=np.float32)
        call("qwg_model_set_norm", self.handle, layer, which, g.ctypes.data, g.size)

    def set_kv(self, layer: int, k: np.ndarray, v: np.ndarray):
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        call("qwg_model_set_kv", self.handle, layer, k.ctypes.data, v.ctypes.data, k.shape[0])

    def get_kv(self, layer: int, n_pos: int):
        nkv, hd = self.desc.n_kv, self.desc.head_dim
        k = np.empty((n_pos, nkv, hd), dtype=np.uint16)
        v = np.empty_like(k)
        call("qwg_model_get_kv", self.handle, layer, k.ctypes.data, v.ctypes.data, n_pos)
        return k, v

    # ------------------------------------------------------------------ decode
    def decode_step(self, token: int, want_logits: bool = False):
        nxt = ctypes.c_int32(0)
        logits = np.empty(self.vocab, dtype=np.float32) if want_logits else None
        call("qwg_decode_step", self.handle, int(token), ctypes.byref(nxt),
             logits.ctypes.data if want_logits else None)
        return int(nxt.value), logits

    def calibrate_skip(self, tau: float, token: int):
        nxt = ctypes.c_int32(0)
        cos = np.empty(self.n_layers, dtype=np.float32)
        mask = np.empty(self.n_layers, dtype=np.uint8)
        call("qwg_calibrate_skip", self.handle, float(tau), int(token), ctypes.byref(nxt), cos.ctypes.data,
             mask.ctypes.data)
        return int(nxt.value), cos, mask

    def set_layer_skip(self, layer: int, skip: bool):
        call("qwg_set_layer_skip", self.handle, layer, int(bool(skip)))

    def get_layer_skip(self) -> np.ndarray:
        m = np.empty(self.n_layers, dtype=np.uint8)
        call("qwg_get_layer_skip", self.handle, m.ctypes.data)
        return m

    def prefill(self, tokens: Sequence[int], want_logits: bool = False):
        """Run a prompt (positions n_past ..); returns (next greedy token, its logits or None)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        nt = ctypes.c_int32(0)
        logits = np.empty(self.vocab, dtype=np.float32) if want_logits else None
        call("qwg_prefill", self.handle, t.ctypes.data, t.size, ctypes.byref(nt),
             logits.ctypes.data if want_logits else None)
        return int(nt.value), logits

    def spec_step(self, token: int, draft_layers: int, k: int):
        out = np.zeros(k + 1, dtype=np.int32)
        n_out, n_acc = ctypes.c_int32(0), ctypes.c_int32(0)
        call("qwg_spec_step", self.handle, int(token), draft_layers, k, out.ctypes.data, ctypes.byref(n_out),
             ctypes.byref(n_acc))
        return [int(t) for t in out[: n_out.value]], int(n_acc.value)

    def verify(self, tokens: Sequence[int], want_logits: bool = True):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        n = t.size
        logits = np.empty((n, self.vocab), dtype=np.float32) if want_logits else None
        am = np.empty(n, dtype=np.int32)
        call("qwg_verify", self.handle, t.ctypes.data, n, logits.ctypes.data if want_logits else None, am.ctypes.data)
        return logits, am

    # ------------------------------------------------------------------ state / debug
    @property
    def n_past(self) -> int:
        return int(lib().qwg_model_n_past(self.handle))

    def truncate(self, n_past: int):
        call("qwg_model_truncate", self.handle, n_past)

    def set_capture(self, on: bool):
        call("qwg_model_set_capture", self.handle, int(bool(on)))

    def get_hidden(self, layer: int) -> np.ndarray:
        out = np.empty(self.hidden, dtype=np.float32)
        call("qwg_model_get_hidden", self.handle, layer, out.ctypes.data)
        return out

    def set_timing(self, tensor_id: int):
        call("qwg_model_set_timing", self.handle, tensor_id)

    def get_timing(self):
        ms, n, b = ctypes.c_double(0), ctypes.c_int64(0), ctypes.c_int64(0)
        call("qwg_model_get_timing", self.handle, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(b))
        return float(ms.value), int(n.value), int(b.value)

    def set_debug(self, knob: int, value: int) -> None:
        """Test hooks: _lib.DEBUG_SPIN_US (delay each streamed layer's compute), _lib.DEBUG_FAIL_AT_LAYER."""
        call("qwg_model_set_debug", self.handle, knob, value)

    def first_nonfinite(self) -> int:
        """First layer (-1 = embedding) whose captured hidden state is non-finite; n_layers: only the logits;
        -2: none."""
        out = ctypes.c_int32(0)
        call("qwg_model_first_nonfinite", self.handle, ctypes.byref(out))
        return int(out.value)

    def get_timing_class(self, tensor_id: int):
        """(total ms, launches, total algorithmic bytes) of one timing class since set_timing."""
        ms, n, b = ctypes.c_double(0), ctypes.c_int64(0), ctypes.c_int64(0)
        call("qwg_model_get_timing_class", self.handle, tensor_id, ctypes.byref(ms), ctypes.byref(n),
             ctypes.byref(b))
        return float(ms.value), int(n.value), int(b.value)

    def spill_layer(self, layer: int, path: str) -> None:
        """Move a streamed layer's image to a file (the file-backed tier); the caller removes the file."""
        call("qwg_model_spill_layer", self.handle, layer, path.encode())

    def file_stats(self):
        b, ms = ctypes.c_int64(0), ctypes.c_double(0)
        call("qwg_model_file_stats", self.handle, ctypes.byref(b), ctypes.byref(ms))
        return int(b.value), float(ms.value)

    def stream_stats(self):
        b, ms = ctypes.c_int64(0), ctypes.c_double(0)
        call("qwg_model_stream_stats", self.handle, ctypes.byref(b), ctypes.byref(ms))
        return int(b.value), float(ms.value)

    def sync(self):
        call("qwg_sync", self.handle)
