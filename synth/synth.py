"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds no arithmetic of the method: it only draws counter-based random numbers
(SplitMix64, see synth.c) and writes them out as canonical GGUF-style block
bytes, fp32 vectors and fp16 KV rows.  Both consumers decode these bytes with
their own, independent code.

Workload recipes follow the Llama shapes and value distributions of the five
synthetic workloads this project measures (8B and 70B Llama decode shapes with
Q8_0 / Q4_K / Q6_K / Q5_K weights); the formats themselves are the ones in the
quantization-format table of the "Show HN ... Llama 3.1 70B" NTransformer page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

# GGUF type numbering (the pages name the GGUF model format).
F32, F16, Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 0, 1, 2, 8, 12, 13, 14
QTYPE_NAMES = {F32: "F32", F16: "F16", Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}
BLOCK_WEIGHTS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q5_K: 176, Q6_K: 210}

# tensor identifiers (also used by the C ABI of the GPU library)
EMBED, HEAD, WQ, WK, WV, WO, WGATE, WUP, WDOWN = 0, 1, 2, 3, 4, 5, 6, 7, 8
G_ATTN, G_FFN, G_FINAL, KCACHE, VCACHE, TOKEN, XVEC = 9, 10, 11, 12, 13, 14, 15


def build(force: bool = False) -> str:
    """Compile libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class QParams(ctypes.Structure):
    _fields_ = [("qtype", ctypes.c_int32), ("q_lo", ctypes.c_int32), ("q_hi", ctypes.c_int32),
                ("sc_lo", ctypes.c_int32), ("sc_hi", ctypes.c_int32), ("m_lo", ctypes.c_int32),
                ("m_hi", ctypes.c_int32), ("d_sigma", ctypes.c_double), ("dmin_sigma", ctypes.c_double),
                ("d_mult", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.syn_key.argtypes = [u64, u64]
        L.syn_key.restype = u64
        L.syn_draw.argtypes = [u64, u64]
        L.syn_draw.restype = u64
        L.syn_f16_bits.argtypes = [ctypes.c_double]
        L.syn_f16_bits.restype = ctypes.c_uint16
        L.syn_matrix.argtypes = [ctypes.POINTER(QParams), u64, i64, i64, i64, vp]
        L.syn_matrix.restype = ctypes.c_int
        L.syn_normal_f32.argtypes = [u64, i64, i64, ctypes.c_double, ctypes.c_double, vp]
        L.syn_normal_f32.restype = None
        L.syn_normal_f16.argtypes = [u64, i64, i64, ctypes.c_double, ctypes.c_double, vp]
        L.syn_normal_f16.restype = None
        L.syn_uniform_int.argtypes = [u64, i64, i64, i64]
        L.syn_uniform_int.restype = i64
        L.syn_block_fields.argtypes = [ctypes.POINTER(QParams), u64, i64, i64, i64, vp, vp, vp, vp, vp]
        L.syn_block_fields.restype = ctypes.c_int
        _lib = L
    return _lib


@dataclass(frozen=True)
class QDist:
    """Value distribution of one quantized tensor."""
    qtype: int
    q: tuple
    sc: tuple = (0, 0)
    m: tuple = (0, 0)
    d_sigma: float = 0.0
    dmin_sigma: float = 0.0
    d_mult: float = 1.0

    def params(self) -> QParams:
        return QParams(self.qtype, self.q[0], self.q[1], self.sc[0], self.sc[1], self.m[0], self.m[1],
                       self.d_sigma, self.dmin_sigma, self.d_mult)


# Default distributions per format: Q8_0 q~U[-127,127], d=|N|*0.02; Q4_K q~U[0,15],
# sc,m~U[0,63], d,dmin=|N|*0.01; Q6_K q~U[0,63], sc~U[-64,63], d=|N|*0.01;
# Q5_K q~U[0,31], sc,m~U[0,63], d,dmin=|N|*0.01; Q4_0 q~U[0,15], d=|N|*0.02.
DEFAULT_DIST = {
    Q8_0: QDist(Q8_0, (-127, 127), d_sigma=0.02),
    Q4_0: QDist(Q4_0, (0, 15), d_sigma=0.02),
    Q4_K: QDist(Q4_K, (0, 15), (0, 63), (0, 63), 0.01, 0.01),
    Q5_K: QDist(Q5_K, (0, 31), (0, 63), (0, 63), 0.01, 0.01),
    Q6_K: QDist(Q6_K, (0, 63), (-64, 63), d_sigma=0.01),
}


def key(seed: int, stream: int) -> int:
    return int(lib().syn_key(seed & (2**64 - 1), stream & (2**64 - 1)))


def stream_id(workload: int, layer: int, tensor: int) -> int:
    """Stream identifier of one tensor: (workload, layer or -1 for global, tensor id)."""
    return (workload << 40) | ((layer + 1) << 16) | tensor


def row_bytes(qtype: int, k: int) -> int:
    return (k // BLOCK_WEIGHTS[qtype]) * BLOCK_BYTES[qtype]


def matrix(dist: QDist, k_: int, rows: int, r0: int = 0, nr: Optional[int] = None, *, tkey: int,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    """Canonical block bytes of rows [r0, r0+nr) of a rows x k_ matrix, shape (nr, row_bytes)."""
    if nr is None:
        nr = rows - r0
    if r0 < 0 or nr < 0 or r0 + nr > rows:
        raise ValueError("row range out of bounds")
    rb = row_bytes(dist.qtype, k_)
    if out is None:
        out = np.empty((nr, rb), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags["C_CONTIGUOUS"] and out.size >= nr * rb
    p = dist.params()
    rc = lib().syn_matrix(ctypes.byref(p), tkey, k_, r0, nr, out.ctypes.data)
    if rc != 0:
        raise ValueError("syn_matrix rejected qtype=%d k=%d" % (dist.qtype, k_))
    return out


def block_fields(dist: QDist, k_: int, r: int, b: int, *, tkey: int) -> dict:
    """Raw drawn fields of block b of row r: q (as stored), sc, m, d and dmin fp16 bits."""
    B = BLOCK_WEIGHTS[dist.qtype]
    q = np.zeros(B, dtype=np.int32)
    sc = np.zeros(16, dtype=np.int32)
    m = np.zeros(16, dtype=np.int32)
    d = np.zeros(1, dtype=np.uint16)
    dmin = np.zeros(1, dtype=np.uint16)
    p = dist.params()
    if lib().syn_block_fields(ctypes.byref(p), tkey, k_, r, b, q.ctypes.data, sc.ctypes.data, m.ctypes.data,
                              d.ctypes.data, dmin.ctypes.data) != 0:
        raise ValueError("bad qtype/k")
    return dict(q=q, sc=sc, m=m, d=int(d[0]), dmin=int(dmin[0]))


def normal_f32(tkey: int, n: int, mean: float = 0.0, sigma: float = 1.0, i0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().syn_normal_f32(tkey, i0, n, mean, sigma, out.ctypes.data)
    return out


def normal_f16(tkey: int, n: int, mean: float = 0.0, sigma: float = 1.0, i0: int = 0) -> np.ndarray:
    """fp16 bit patterns (uint16) of mean + sigma * N(0,1)."""
    out = np.empty(n, dtype=np.uint16)
    lib().syn_normal_f16(tkey, i0, n, mean, sigma, out.ctypes.data)
    return out


def uniform_int(tkey: int, i: int, lo: int, hi: int) -> int:
    return int(lib().syn_uniform_int(tkey, i, lo, hi))


def f16_bits(v: float) -> int:
    return int(lib().syn_f16_bits(float(v)))


# ----------------------------------------------------------------------------------------------
# Model workloads
# ----------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """A synthetic Llama decode workload: shapes, formats and value distributions."""
    name: str
    wid: int                      # workload id, part of every tensor's stream id
    n_layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    n_prior: int                  # KV positions already in the cache (new token goes at this position)
    qtype_attn: int
    qtype_ffn: int
    qtype_embed: int
    qtype_head: int
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5
    near_identity_every: int = 0  # if > 0, layers l % every == every-1 get scaled output projections
    near_identity_mult: float = 1e-3
    n_resident: int = -1          # layers kept in HBM (-1 = all); the rest stream from pinned host RAM
    skip_tau: float = 0.0         # cosine skip threshold (0 = no skipping)
    draft_layers: int = 0         # self-speculative draft depth (0 = off)
    draft_k: int = 0
    n_tokens: int = 32            # greedy tokens generated by the full run
    seed: int = 0
    # per-layer type mix (a stand-in for Q4_K_M, a mix of K-quant types): W_down of layers
    # l % wide_down_every == 0 in wide_qtype (0 = no mix)
    wide_qtype: int = 0
    wide_down_every: int = 0

    @property
    def resident_layers(self) -> int:
        return self.n_layers if self.n_resident < 0 else self.n_resident

    def qtype_of(self, tensor: int, layer: int = -1) -> int:
        if tensor in (WQ, WK, WV, WO):
            return self.qtype_attn
        if tensor == WDOWN and layer >= 0 and self.wide_down_every > 0 and layer % self.wide_down_every == 0:
            return self.wide_qtype
        if tensor in (WGATE, WUP, WDOWN):
            return self.qtype_ffn
        if tensor == EMBED:
            return self.qtype_embed
        if tensor == HEAD:
            return self.qtype_head
        raise ValueError(tensor)

    def shape_of(self, tensor: int):
        """(rows, k) of a weight matrix."""
        H, hd = self.hidden, self.head_dim
        return {
            EMBED: (self.vocab, H), HEAD: (self.vocab, H),
            WQ: (self.n_q * hd, H), WK: (self.n_kv * hd, H), WV: (self.n_kv * hd, H),
            WO: (H, self.n_q * hd), WGATE: (self.ffn, H), WUP: (self.ffn, H), WDOWN: (H, self.ffn),
        }[tensor]

    def is_near_identity(self, layer: int) -> bool:
        e = self.near_identity_every
        return e > 0 and layer % e == e - 1

    def layer_qtypes(self):
        """[n_layers][4] types of (QKV, WO, GATE|UP, DOWN) if layers differ, else None."""
        if self.wide_down_every <= 0:
            return None
        return np.array([[self.qtype_of(WQ, l), self.qtype_of(WO, l), self.qtype_of(WGATE, l), self.qtype_of(WDOWN, l)]
                         for l in range(self.n_layers)], dtype=np.int32)

    def dist_of(self, layer: int, tensor: int) -> QDist:
        d = DEFAULT_DIST[self.qtype_of(tensor, layer)]
        if tensor in (WO, WDOWN) and layer >= 0 and self.is_near_identity(layer):
            d = replace(d, d_mult=self.near_identity_mult)
        return d

    def tkey(self, layer: int, tensor: int) -> int:
        return key(self.seed, stream_id(self.wid, layer, tensor))

    def weight(self, layer: int, tensor: int, r0: int = 0, nr: Optional[int] = None, out=None) -> np.ndarray:
        rows, k_ = self.shape_of(tensor)
        return matrix(self.dist_of(layer, tensor), k_, rows, r0, nr, tkey=self.tkey(layer, tensor), out=out)

    def gain(self, layer: int, which: int) -> np.ndarray:
        """RMSNorm gains 1 + N(0, 0.02), fp32."""
        return normal_f32(self.tkey(layer, which), self.hidden, 1.0, 0.02)

    def kv_prior(self, layer: int, which: int) -> np.ndarray:
        """Prefilled K or V rows N(0,1) as fp16 bits, layout [n_prior][n_kv][head_dim]."""
        n = self.n_prior * self.n_kv * self.head_dim
        return normal_f16(self.tkey(layer, which), n, 0.0, 1.0).reshape(self.n_prior, self.n_kv, self.head_dim)

    def first_token(self) -> int:
        return uniform_int(self.tkey(-1, TOKEN), 0, 0, self.vocab - 1)

    def layer_bytes(self, layer: int = 0) -> int:
        return sum(row_bytes(self.qtype_of(t, layer), self.shape_of(t)[1]) * self.shape_of(t)[0]
                   for t in (WQ, WK, WV, WO, WGATE, WUP, WDOWN))

    def layers_bytes(self) -> int:
        """Canonical bytes of every layer's weights."""
        return sum(self.layer_bytes(l) for l in range(self.n_layers))

    def model_bytes(self) -> int:
        g = sum(row_bytes(self.qtype_of(t), self.shape_of(t)[1]) * self.shape_of(t)[0] for t in (EMBED, HEAD))
        return g + self.layers_bytes()


# Workloads measured by this project.  Ids are part of the random streams.
GEMV_Q8_0_4096 = dict(qtype=Q8_0, rows=4096, k=4096, wid=0)

LLAMA8B_Q8_0 = Workload("llama8b-q8_0-resident", 1, 32, 4096, 32, 8, 128, 14336, 128256, 512,
                        Q8_0, Q8_0, Q8_0, Q8_0)
LLAMA70B_Q4_K = Workload("llama70b-q4_k-resident", 2, 80, 8192, 64, 8, 128, 28672, 128256, 2048,
                         Q4_K, Q4_K, Q4_K, Q4_K)
LLAMA70B_Q6_K_STREAM = Workload("llama70b-q6_k-slep20-skip0.98", 3, 80, 8192, 64, 8, 128, 28672, 128256, 2048,
                                Q6_K, Q6_K, Q6_K, Q6_K, near_identity_every=4, n_resident=20, skip_tau=0.98)
# Q4_K_M stand-in (the pages list Q4_K_M as a mixed 256-weight K-quant type at about 4.5 bits per
# weight): Q4_K matrices with W_down of every other layer and the output head in Q6_K (4.78 bits per
# layer weight).
LLAMA70B_Q4_K_M = Workload("llama70b-q4_k_m-resident", 5, 80, 8192, 64, 8, 128, 28672, 128256, 2048,
                           Q4_K, Q4_K, Q4_K, Q6_K, wide_qtype=Q6_K, wide_down_every=2)
LLAMA70B_Q6_K_Q5_K_SPEC = Workload("llama70b-q6_k-attn-q5_k-ffn-selfspec-k3", 4, 80, 8192, 64, 8, 128, 28672,
                                   128256, 4096, Q6_K, Q5_K, Q6_K, Q6_K, draft_layers=20, draft_k=3)


def tiny(qtype_attn: int, qtype_ffn: Optional[int] = None, wid: int = 100, **kw) -> Workload:
    """A small Llama of the same structure (head_dim 128, GQA) for whole-model parity in seconds."""
    qf = qtype_attn if qtype_ffn is None else qtype_ffn
    base = dict(name="tiny-%s-%s" % (QTYPE_NAMES[qtype_attn], QTYPE_NAMES[qf]), wid=wid, n_layers=4, hidden=512,
                n_q=4, n_kv=2, head_dim=128, ffn=1536, vocab=1000, n_prior=37,
                qtype_attn=qtype_attn, qtype_ffn=qf, qtype_embed=qtype_attn, qtype_head=qtype_attn, n_tokens=4)
    base.update(kw)
    return Workload(**base)
