"""Load a seeded synthetic workload (from the `synth` input generator) into a Model.

The generator writes canonical block bytes; the library packs them on the device.  Nothing here
computes any part of the decode path."""
from __future__ import annotations

import time
from typing import Optional

from . import _lib
from .model import Model


def make_model(wl, *, max_ctx: Optional[int] = None, max_cols: Optional[int] = None,
               n_resident: Optional[int] = None, device: str = "cuda:0") -> Model:
    cols = max_cols if max_cols is not None else (wl.draft_k + 1 if wl.draft_k else 1)
    ctx = max_ctx if max_ctx is not None else wl.n_prior + 64
    res = wl.n_resident if n_resident is None else n_resident
    if res == "auto":  # automatic tier placement from the device's free memory and MemAvailable
        res = plan_residency_of(wl, max_ctx=ctx, max_cols=cols)[0]
    return Model(n_layers=wl.n_layers, hidden=wl.hidden, n_q=wl.n_q, n_kv=wl.n_kv, head_dim=wl.head_dim,
                 ffn=wl.ffn, vocab=wl.vocab, max_ctx=ctx, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps,
                 qtype_attn=wl.qtype_attn, qtype_ffn=wl.qtype_ffn, qtype_embed=wl.qtype_embed,
                 qtype_head=wl.qtype_head, n_resident=res, max_cols=cols, layer_qtypes=wl.layer_qtypes(),
                 device=device)


def plan_residency_of(wl, *, max_ctx: int, max_cols: int = 1, device_budget: int = 0, host_budget: int = 0):
    """(n_resident, arena_bytes, pinned_bytes) of workload `wl` under the given budgets (0 = measured)."""
    from .model import plan_residency
    return plan_residency(n_layers=wl.n_layers, hidden=wl.hidden, n_q=wl.n_q, n_kv=wl.n_kv, head_dim=wl.head_dim,
                          ffn=wl.ffn, vocab=wl.vocab, max_ctx=max_ctx, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps,
                          qtype_attn=wl.qtype_attn, qtype_ffn=wl.qtype_ffn, qtype_embed=wl.qtype_embed,
                          qtype_head=wl.qtype_head, max_cols=max_cols, layer_qtypes=wl.layer_qtypes(),
                          device_budget=device_budget,
                          host_budget=host_budget)


def load(model: Model, wl, *, weights_override=None, log=None) -> float:
    """Load every tensor, gain and prefilled KV row of workload `wl`. Returns seconds spent."""
    import synth
    t0 = time.time()
    ov = weights_override or {}

    def w(layer, t):
        return ov[(layer, t)] if (layer, t) in ov else wl.weight(layer, t)

    for t in (synth.EMBED, synth.HEAD):
        model.set_tensor(-1, t, wl.qtype_of(t), w(-1, t))
    model.set_norm(-1, _lib.NORM_FINAL, wl.gain(-1, synth.G_FINAL))
    for l in range(wl.n_layers):
        for t in (synth.WQ, synth.WK, synth.WV, synth.WO, synth.WGATE, synth.WUP, synth.WDOWN):
            model.set_tensor(l, t, wl.qtype_of(t, l), w(l, t))
        model.set_norm(l, _lib.NORM_ATTN, wl.gain(l, synth.G_ATTN))
        model.set_norm(l, _lib.NORM_FFN, wl.gain(l, synth.G_FFN))
        model.set_kv(l, wl.kv_prior(l, synth.KCACHE), wl.kv_prior(l, synth.VCACHE))
        if log and (l % 10 == 9 or l == wl.n_layers - 1):
            log("loaded layer %d/%d (%.1f s)" % (l + 1, wl.n_layers, time.time() - t0))
    return time.time() - t0
