"""ctypes wrapper of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU-baseline
leg of bench.py.  The GPU library never imports it and it never imports the GPU
library.  Inputs come from the seeded generator (the `synth` module) as canonical
block bytes, fp32 gains and fp16 KV rows.

Model-level control flow written out here in plain Python on top of the C step:
  * layer-skip calibration: the NTransformer pages describe a cosine-similarity test
    that marks layers whose output is nearly their input as skippable (NTransformer
    page, "Key results" and "Key features"; "RTX 3090 1枚でLlama 70B" article,
    section on the layer-skip mechanism).  Read as: one full step records
    cos(h_in, h_out) per layer; layers with cos >= tau are skipped from then on.
  * self-speculative decoding: the VRAM-resident first layers act as the draft model
    (NTransformer page, "Key features"; Show HN page, "speed-up techniques").  The plain
    definition of verification is k+1 sequential full decode steps.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile liboracle.so: plain C++17, no fast-math, no FMA contraction."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Dims(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("rms_eps", ctypes.c_double)]


class Layer(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p * 7), ("qt", ctypes.c_int32 * 7), ("g_attn", ctypes.c_void_p),
                ("g_ffn", ctypes.c_void_p), ("kc", ctypes.c_void_p), ("vc", ctypes.c_void_p)]


class Model(ctypes.Structure):
    _fields_ = [("dims", Dims), ("layers", ctypes.POINTER(Layer)), ("embed", ctypes.c_void_p),
                ("qt_embed", ctypes.c_int32), ("head", ctypes.c_void_p), ("qt_head", ctypes.c_int32),
                ("g_final", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.orc_block_weights.argtypes = [ctypes.c_int]
        L.orc_block_bytes.argtypes = [ctypes.c_int]
        L.orc_half_value.argtypes = [ctypes.c_uint16]
        L.orc_half_value.restype = dbl
        L.orc_half_from_double.argtypes = [dbl]
        L.orc_half_from_double.restype = ctypes.c_uint16
        L.orc_dequant.argtypes = [ctypes.c_int, vp, i64, i64, vp]
        L.orc_gemv.argtypes = [ctypes.c_int, vp, i64, i64, vp, ctypes.c_int, vp, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i64, dbl, vp]
        L.orc_rmsnorm.restype = None
        L.orc_rope.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, dbl]
        L.orc_rope.restype = None
        L.orc_attention.argtypes = [vp, vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.orc_attention.restype = None
        L.orc_silu.argtypes = [dbl]
        L.orc_silu.restype = dbl
        L.orc_swiglu.argtypes = [vp, vp, i64, vp]
        L.orc_swiglu.restype = None
        L.orc_cosine.argtypes = [vp, vp, i64]
        L.orc_cosine.restype = dbl
        L.orc_argmax_f32.argtypes = [vp, i64]
        L.orc_argmax_f32.restype = i64
        L.orc_layer_forward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Layer), vp, i64]
        L.orc_head.argtypes = [ctypes.POINTER(Model), vp, vp]
        L.orc_threads.argtypes = []
        L.orc_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_set_threads.restype = ctypes.c_int
        L.orc_step.argtypes = [ctypes.POINTER(Model), i32, i64, i32, vp, vp, vp, vp, ctypes.POINTER(i32)]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------------------ elementary ops

def dequant(qtype: int, canon: np.ndarray, rows: int, k: int) -> np.ndarray:
    canon = _c(canon, np.uint8)
    out = np.empty((rows, k), dtype=np.float32)
    if lib().orc_dequant(qtype, _ptr(canon), rows, k, _ptr(out)) != 0:
        raise ValueError("bad qtype/k")
    return out


def gemv(qtype: int, canon: np.ndarray, rows: int, k: int, x: np.ndarray):
    """x: [k] or [n][k] (any float dtype, converted exactly to fp64). Returns (y, a) shaped like x's columns."""
    x2 = _c(np.atleast_2d(x), np.float64)
    n = x2.shape[0]
    assert x2.shape[1] == k
    y = np.empty((n, rows), dtype=np.float64)
    a = np.empty((n, rows), dtype=np.float64)
    canon = _c(canon, np.uint8)
    if lib().orc_gemv(qtype, _ptr(canon), rows, k, _ptr(x2), n, _ptr(y), _ptr(a)) != 0:
        raise ValueError("bad qtype/k")
    if np.ndim(x) == 1:
        return y[0], a[0]
    return y, a


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = _c(x, np.float64)
    g = _c(g, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(g), x.size, eps, _ptr(out))
    return out


def rope(v: np.ndarray, n_heads: int, hd: int, pos: int, base: float) -> np.ndarray:
    v = _c(v, np.float64).copy()
    lib().orc_rope(_ptr(v), n_heads, hd, pos, base)
    return v


def attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, n_pos: int, nq: int, nkv: int, hd: int) -> np.ndarray:
    q = _c(q, np.float64)
    kc = _c(kc, np.uint16)
    vc = _c(vc, np.uint16)
    out = np.empty(nq * hd, dtype=np.float64)
    lib().orc_attention(_ptr(q), _ptr(kc), _ptr(vc), n_pos, nq, nkv, hd, _ptr(out))
    return out


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    out = np.empty_like(g)
    lib().orc_swiglu(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = _c(a, np.float64)
    b = _c(b, np.float64)
    return lib().orc_cosine(_ptr(a), _ptr(b), a.size)


def argmax_f32(x: np.ndarray) -> int:
    x = _c(x, np.float64)
    return int(lib().orc_argmax_f32(_ptr(x), x.size))


def half_value(bits: int) -> float:
    return lib().orc_half_value(bits)


def half_from_double(v: float) -> int:
    return int(lib().orc_half_from_double(float(v)))


# ------------------------------------------------------------------------------ model

def threads() -> int:
    """OpenMP threads the oracle's row loops use."""
    return int(lib().orc_threads())


def set_threads(n: int) -> int:
    """Use n threads in the row loops from now on (results do not depend on it); returns the old count."""
    return int(lib().orc_set_threads(n))


def layer_forward(wl, layer: int, weights: dict, h: np.ndarray, kc: np.ndarray, vc: np.ndarray, pos: int,
                  max_ctx: Optional[int] = None) -> np.ndarray:
    """One decoder layer on explicitly given tensors: weights {tensor_id: canonical bytes}, h [hidden]
    (any float dtype, widened exactly to fp64), KV caches [max_ctx][n_kv][hd] fp16 bits (row pos is
    written).  Returns the layer's output h in fp64."""
    import synth
    ctx = max_ctx or kc.shape[0]
    dims = Dims(wl.n_layers, wl.hidden, wl.n_q, wl.n_kv, wl.head_dim, wl.ffn, wl.vocab, ctx, wl.rope_theta,
                wl.rms_eps)
    lay = Layer()
    keep = []
    for i, t in enumerate(OracleModel.TENSORS):
        w = _c(weights[t], np.uint8)
        keep.append(w)
        lay.w[i] = w.ctypes.data
        lay.qt[i] = wl.qtype_of(t, layer)
    ga, gf = wl.gain(layer, synth.G_ATTN), wl.gain(layer, synth.G_FFN)
    keep += [ga, gf]
    lay.g_attn, lay.g_ffn = ga.ctypes.data, gf.ctypes.data
    assert kc.dtype == np.uint16 and kc.flags["C_CONTIGUOUS"] and vc.flags["C_CONTIGUOUS"]
    lay.kc, lay.vc = kc.ctypes.data, vc.ctypes.data
    out = _c(h, np.float64).copy()
    if lib().orc_layer_forward(ctypes.byref(dims), ctypes.byref(lay), _ptr(out), pos) != 0:
        raise ValueError("orc_layer_forward failed")
    return out


def head_logits(wl, head: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Final RMSNorm and output head on h (fp64 logits)."""
    import synth
    n = rmsnorm(_c(h, np.float64), wl.gain(-1, synth.G_FINAL), wl.rms_eps)
    y, _ = gemv(wl.qtype_head, head, wl.vocab, wl.hidden, n)
    return y

class OracleModel:
    """A Llama decoder held as canonical bytes (from `synth`), run by the CPU oracle.

    Weights are borrowed numpy arrays; the KV caches are owned here ([max_ctx][n_kv][hd] fp16).
    """

    TENSORS = (2, 3, 4, 5, 6, 7, 8)  # WQ WK WV WO WGATE WUP WDOWN (ids shared with synth)

    def __init__(self, wl, max_ctx: Optional[int] = None, layers: Optional[Sequence[int]] = None,
                 load_weights: bool = True):
        import synth
        self.wl = wl
        self.max_ctx = max_ctx or (wl.n_prior + 64)
        self.n_past = wl.n_prior
        L = wl.n_layers
        self._keep = []
        self.dims = Dims(L, wl.hidden, wl.n_q, wl.n_kv, wl.head_dim, wl.ffn, wl.vocab, self.max_ctx,
                         wl.rope_theta, wl.rms_eps)
        self.layers = (Layer * L)()
        self.kc: List[np.ndarray] = []
        self.vc: List[np.ndarray] = []
        for l in range(L):
            kc = np.zeros((self.max_ctx, wl.n_kv, wl.head_dim), dtype=np.uint16)
            vc = np.zeros_like(kc)
            kc[:wl.n_prior] = wl.kv_prior(l, synth.KCACHE)
            vc[:wl.n_prior] = wl.kv_prior(l, synth.VCACHE)
            self.kc.append(kc)
            self.vc.append(vc)
            lay = self.layers[l]
            if load_weights:
                for i, t in enumerate(self.TENSORS):
                    w = wl.weight(l, t)
                    self._keep.append(w)
                    lay.w[i] = w.ctypes.data
                    lay.qt[i] = wl.qtype_of(t, l)
            ga, gf = wl.gain(l, synth.G_ATTN), wl.gain(l, synth.G_FFN)
            self._keep += [ga, gf]
            lay.g_attn, lay.g_ffn = ga.ctypes.data, gf.ctypes.data
            lay.kc, lay.vc = kc.ctypes.data, vc.ctypes.data
        self.model = Model()
        self.model.dims = self.dims
        self.model.layers = ctypes.cast(self.layers, ctypes.POINTER(Layer))
        if load_weights:
            emb, head = wl.weight(-1, synth.EMBED), wl.weight(-1, synth.HEAD)
            self._keep += [emb, head]
            self.model.embed, self.model.head = emb.ctypes.data, head.ctypes.data
        self.model.qt_embed, self.model.qt_head = wl.qtype_embed, wl.qtype_head
        gfin = wl.gain(-1, synth.G_FINAL)
        self._keep.append(gfin)
        self.model.g_final = gfin.ctypes.data
        self.skip = np.zeros(L, dtype=np.uint8)

    def step(self, token: int, n_run: Optional[int] = None, pos: Optional[int] = None, want_hidden=False):
        """One greedy decode step at position n_past (or pos). Returns dict(next, logits, hidden, cos)."""
        D = self.dims
        pos = self.n_past if pos is None else pos
        n_run = D.n_layers if n_run is None else n_run
        logits = np.empty(D.vocab, dtype=np.float64)
        hidden = np.empty((D.n_layers + 1, D.hidden), dtype=np.float64) if want_hidden else None
        cos = np.empty(D.n_layers, dtype=np.float64)
        nxt = ctypes.c_int32(0)
        rc = lib().orc_step(ctypes.byref(self.model), token, pos, n_run, _ptr(self.skip), _ptr(hidden), _ptr(cos),
                            _ptr(logits), ctypes.byref(nxt))
        if rc != 0:
            raise ValueError("orc_step failed")
        return dict(next=int(nxt.value), logits=logits, hidden=hidden, cos=cos, pos=pos)

    def decode(self, token: int, **kw):
        r = self.step(token, **kw)
        self.n_past = r["pos"] + 1
        return r

    def calibrate_skip(self, tau: float, token: int):
        """Full step with every layer computed; mask = fp32(cos) >= fp32(tau), then n_past advances."""
        self.skip[:] = 0
        r = self.decode(token)
        cos32 = r["cos"].astype(np.float32)
        self.skip[:] = (cos32 >= np.float32(tau)).astype(np.uint8)
        r["mask"] = self.skip.copy()
        return r

    def spec_round(self, token: int, draft_layers: int, k: int, log=None):
        """Self-speculative round: draft k tokens with the first draft_layers layers, verify with k+1
        sequential full steps, accept the longest agreeing prefix, emit accepted drafts + one more.
        log (optional) is called with a short message after every step."""
        p = self.n_past
        drafts, draft_logits = [], []
        t = token
        for j in range(k):
            r = self.step(t, n_run=draft_layers, pos=p + j)
            t = r["next"]
            drafts.append(t)
            draft_logits.append(r["logits"])
            if log:
                log("oracle draft %d: %d" % (j, t))
        cols = [token] + drafts
        verdict, logits = [], []
        for j in range(k + 1):
            r = self.step(cols[j], pos=p + j)
            verdict.append(r["next"])
            logits.append(r["logits"])
            if log:
                log("oracle verify column %d: %d" % (j, r["next"]))
        a = 0
        while a < k and verdict[a] == drafts[a]:
            a += 1
        out = drafts[:a] + [verdict[a]]
        self.n_past = p + a + 1
        return dict(tokens=out, n_accepted=a, drafts=drafts, verdict=verdict, logits=np.stack(logits),
                    draft_logits=np.stack(draft_logits))
