"""ctypes binding of libqwg.so (include/qwg.h).  Argument marshalling only: every step of the
decode path runs in the library's HIP kernels.  There is no CPU fallback: if the library is
missing or cannot be loaded, every entry point raises."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwg.so")

QWG_OK = 0
ERRORS = {-1: "QWG_E_INVAL", -2: "QWG_E_SHAPE", -3: "QWG_E_NOMEM", -4: "QWG_E_HIP", -5: "QWG_E_STATE",
          -6: "QWG_E_UNSUPPORTED"}

Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 2, 8, 12, 13, 14
T_EMBED, T_HEAD, T_WQ, T_WK, T_WV, T_WO, T_WGATE, T_WUP, T_WDOWN = 0, 1, 2, 3, 4, 5, 6, 7, 8
NORM_ATTN, NORM_FFN, NORM_FINAL = 9, 10, 11
TIME_ALL_GEMV = -2
DEBUG_SPIN_US, DEBUG_FAIL_AT_LAYER = 1, 2


class QwgError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__("%s failed: %s (%s)" % (fn, msg, ERRORS.get(code, code)))
        self.code = code


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("n_resident", ctypes.c_int32), ("qtype_attn", ctypes.c_int32),
                ("qtype_ffn", ctypes.c_int32), ("qtype_embed", ctypes.c_int32), ("qtype_head", ctypes.c_int32),
                ("max_cols", ctypes.c_int32), ("layer_qtypes", ctypes.c_void_p)]


vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
f32, f64 = ctypes.c_float, ctypes.c_double
P_i32, P_i64, P_f64, P_sz = (ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_size_t))

# name -> (restype, argtypes); every name here is declared in include/qwg.h
SIGNATURES = {
    "qwg_last_error": (ctypes.c_char_p, []),
    "qwg_version": (ctypes.c_int, []),
    "qwg_block_bytes": (sz, [ctypes.c_int]),
    "qwg_block_weights": (ctypes.c_int, [ctypes.c_int]),
    "qwg_row_bytes": (sz, [ctypes.c_int, i64]),
    "qwg_packed_bytes": (ctypes.c_int, [ctypes.c_int, i64, i64, P_sz]),
    "qwg_repack": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp]),
    "qwg_dequantize": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, vp]),
    "qwg_gemv_work_bytes": (sz, [ctypes.c_int, i64, i64, ctypes.c_int]),
    "qwg_gemv": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, vp, vp, sz, vp]),
    "qwg_gemv_noalloc": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, vp, vp]),
    "qwg_gemv_timed": (ctypes.c_int, [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, vp, vp, sz,
                                      ctypes.POINTER(ctypes.c_float), vp]),
    "qwg_set_gemv_geometry": (ctypes.c_int, [ctypes.c_int] * 4),
    "qwg_set_gemv_mfma": (ctypes.c_int, [ctypes.c_int]),
    "qwg_model_spill_layer": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p]),
    "qwg_model_file_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "qwg_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "qwg_plan_residency": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "qwg_rmsnorm": (ctypes.c_int, [vp, vp, i64, f32, ctypes.c_int, vp, vp]),
    "qwg_rope_table": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, f64, vp]),
    "qwg_rope": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp]),
    "qwg_attn_work_bytes": (sz, [ctypes.c_int] * 5),
    "qwg_attn_decode": (ctypes.c_int, [vp, vp, vp] + [ctypes.c_int] * 5 + [vp, vp, sz, vp]),
    "qwg_swiglu": (ctypes.c_int, [vp, vp, i64, vp, vp]),
    "qwg_cosine": (ctypes.c_int, [vp, vp, i64, vp, vp]),
    "qwg_argmax_work_bytes": (sz, []),
    "qwg_argmax": (ctypes.c_int, [vp, i64, vp, vp, sz, vp]),
    "qwg_model_create": (ctypes.c_int, [ctypes.POINTER(ModelDesc), ctypes.POINTER(vp)]),
    "qwg_model_arena_bytes": (sz, [vp]),
    "qwg_model_bind": (ctypes.c_int, [vp, vp, sz, vp, vp]),
    "qwg_model_destroy": (None, [vp]),
    "qwg_model_set_tensor": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, sz]),
    "qwg_model_set_norm": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int]),
    "qwg_model_set_kv": (ctypes.c_int, [vp, ctypes.c_int, vp, vp, ctypes.c_int]),
    "qwg_model_get_kv": (ctypes.c_int, [vp, ctypes.c_int, vp, vp, ctypes.c_int]),
    "qwg_decode_step": (ctypes.c_int, [vp, i32, P_i32, vp]),
    "qwg_calibrate_skip": (ctypes.c_int, [vp, f32, i32, P_i32, vp, vp]),
    "qwg_set_layer_skip": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int]),
    "qwg_get_layer_skip": (ctypes.c_int, [vp, vp]),
    "qwg_spec_step": (ctypes.c_int, [vp, i32, ctypes.c_int, ctypes.c_int, vp, P_i32, P_i32]),
    "qwg_verify": (ctypes.c_int, [vp, vp, ctypes.c_int, vp, vp]),
    "qwg_model_n_past": (ctypes.c_int, [vp]),
    "qwg_model_truncate": (ctypes.c_int, [vp, ctypes.c_int]),
    "qwg_model_set_capture": (ctypes.c_int, [vp, ctypes.c_int]),
    "qwg_model_get_hidden": (ctypes.c_int, [vp, ctypes.c_int, vp]),
    "qwg_model_set_timing": (ctypes.c_int, [vp, ctypes.c_int]),
    "qwg_model_get_timing": (ctypes.c_int, [vp, P_f64, P_i64, P_i64]),
    "qwg_model_get_timing_class": (ctypes.c_int, [vp, ctypes.c_int, P_f64, P_i64, P_i64]),
    "qwg_model_set_debug": (ctypes.c_int, [vp, ctypes.c_int, i64]),
    "qwg_model_first_nonfinite": (ctypes.c_int, [vp, P_i32]),
    "qwg_model_stream_stats": (ctypes.c_int, [vp, P_i64, P_f64]),
    "qwg_sync": (ctypes.c_int, [vp]),
    "qwg_read_sink_words": (sz, []),
    "qwg_read_bytes": (ctypes.c_int, [vp, sz, vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float), vp]),
    "qwg_host_alloc": (ctypes.c_int, [sz, ctypes.POINTER(vp)]),
    "qwg_host_free": (ctypes.c_int, [vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was never built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqwg.so is not built (run __graft_entry__.build()); no fallback exists")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(rc: int, fn: str) -> None:
    if rc != QWG_OK:
        msg = lib().qwg_last_error()
        raise QwgError(rc, fn, msg.decode() if msg else "")


def call(name: str, *args) -> int:
    rc = getattr(lib(), name)(*args)
    check(rc, name)
    return rc
