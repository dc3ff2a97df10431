"""Automatic tier placement (qwg_plan_residency) on the host: with both budgets given it is plain
arithmetic over the arena plan and makes no GPU call.  The tier sizes follow the engine's rule of
sizing the resident tier from device memory and the pinned tier from MemAvailable ([NT] "3-tier
adaptive cache"; [HN] 3-tier cache detail)."""
import ctypes
import os

import numpy as np
import pytest

import synth
from quantized_weight_streaming_gemv_amd import _lib

GIB = 1 << 30


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libqwg.so not built")
    return _lib.lib()


def desc_of(wl, n_res, max_ctx, max_cols=1):
    return _lib.ModelDesc(wl.n_layers, wl.hidden, wl.n_q, wl.n_kv, wl.head_dim, wl.ffn, wl.vocab, max_ctx,
                          wl.rope_theta, wl.rms_eps, n_res, wl.qtype_attn, wl.qtype_ffn, wl.qtype_embed,
                          wl.qtype_head, max_cols)


def arena_of(L, wl, n_res, max_ctx):
    """Arena bytes of an unbound model with n_res resident layers (create/destroy touch no GPU)."""
    h = ctypes.c_void_p()
    _lib.call("qwg_model_create", ctypes.byref(desc_of(wl, n_res, max_ctx)), ctypes.byref(h))
    try:
        return int(L.qwg_model_arena_bytes(h))
    finally:
        L.qwg_model_destroy(h)


def plan(wl, dev, host, max_ctx):
    from quantized_weight_streaming_gemv_amd import synthetic
    return synthetic.plan_residency_of(wl, max_ctx=max_ctx, device_budget=dev, host_budget=host)


def test_everything_fits(L):
    wl = synth.tiny(synth.Q4_K, n_layers=6)
    full = arena_of(L, wl, -1, 64)
    n, arena, pinned = plan(wl, full, GIB, 64)
    assert (n, arena, pinned) == (wl.n_layers, full, 0)


@pytest.mark.parametrize("n_res", [0, 1, 3])
def test_boundary_and_pinned_bytes(L, n_res):
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=6)
    a = arena_of(L, wl, n_res, 64)
    n, arena, pinned = plan(wl, a, 64 * GIB, 64)
    assert (n, arena) == (n_res, a)
    # every streamed layer has one pinned image; the image is what one more resident layer adds
    # to the arena, less the two streaming slots that disappear when nothing streams
    n1, _, pinned1 = plan(wl, arena_of(L, wl, 0, 64), 64 * GIB, 64)
    assert n1 == 0 and pinned1 % wl.n_layers == 0
    assert pinned == (wl.n_layers - n_res) * (pinned1 // wl.n_layers)
    if n_res > 0:
        assert plan(wl, a - 1, 64 * GIB, 64)[0] == n_res - 1


def test_all_resident_is_cheaper_than_one_streamed_layer(L):
    """Streaming needs two HBM slots of a layer image, so one streamed layer costs more device
    memory than none: a budget that holds n_layers - 1 resident layers holds all of them."""
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=6)
    assert arena_of(L, wl, -1, 64) < arena_of(L, wl, 5, 64)
    assert plan(wl, arena_of(L, wl, 5, 64), 64 * GIB, 64)[0] == wl.n_layers


def test_nothing_fits_is_an_error(L):
    wl = synth.tiny(synth.Q4_K, n_layers=6)
    a0 = arena_of(L, wl, 0, 64)
    with pytest.raises(_lib.QwgError) as e:
        plan(wl, a0 - 1, 64 * GIB, 64)
    assert e.value.code == -3
    _, _, pinned = plan(wl, a0, 64 * GIB, 64)
    with pytest.raises(_lib.QwgError) as e:
        plan(wl, a0, pinned - 1, 64)  # the streamed images do not fit pinned host memory
    assert e.value.code == -3


def test_mixed_layer_types(L):
    """A per-layer type table: layers with a wider W_down have larger images; a bad type is refused."""
    wl = synth.replace(synth.tiny(synth.Q4_K, n_layers=4), qtype_head=synth.Q6_K, wide_qtype=synth.Q6_K,
                       wide_down_every=2)
    lt = wl.layer_qtypes()
    assert lt.shape == (4, 4) and list(lt[:, 3]) == [synth.Q6_K, synth.Q4_K, synth.Q6_K, synth.Q4_K]
    assert (lt[:, :3] == synth.Q4_K).all()

    def arena(table, n_res):
        d = desc_of(wl, n_res, 64)
        d.layer_qtypes = None if table is None else table.ctypes.data
        h = ctypes.c_void_p()
        _lib.call("qwg_model_create", ctypes.byref(d), ctypes.byref(h))
        try:
            return int(L.qwg_model_arena_bytes(h))
        finally:
            L.qwg_model_destroy(h)

    plain = np.full((4, 4), synth.Q4_K, dtype=np.int32)
    assert arena(lt, -1) > arena(plain, -1) == arena(None, -1)
    # resident layer 0 (wide) costs more than resident layer 1 (narrow)
    assert arena(lt, 1) - arena(lt, 0) > arena(lt, 2) - arena(lt, 1)
    bad = lt.copy()
    bad[2, 1] = 7
    with pytest.raises(_lib.QwgError) as e:
        arena(bad, -1)
    assert e.value.code == -6


def test_q4_k_m_stand_in_bits_per_weight():
    """The Q4_K_M stand-in averages 4.78 bits per layer weight (Q4_K with half the W_down in Q6_K)."""
    wl = synth.LLAMA70B_Q4_K_M
    n_w = sum(wl.shape_of(t)[0] * wl.shape_of(t)[1] for t in (synth.WQ, synth.WK, synth.WV, synth.WO,
                                                               synth.WGATE, synth.WUP, synth.WDOWN))
    bpw = 8 * wl.layers_bytes() / (wl.n_layers * n_w)
    assert abs(bpw - 4.78) < 0.01
    assert wl.layer_bytes(0) - wl.layer_bytes(1) == (210 - 144) * wl.hidden * wl.ffn // 256


def test_fewer_bits_keep_more_layers_resident(L):
    """The pages' consequence of tier sizing: at the same 24 GB device budget a 4.5-bit 70B model
    keeps about ten more layers in device memory than the 6.6-bit one (36 vs 26 there)."""
    q4 = synth.replace(synth.LLAMA70B_Q4_K, n_resident=-1)
    q6 = synth.replace(synth.LLAMA70B_Q6_K_STREAM, n_resident=-1)
    q4m = synth.LLAMA70B_Q4_K_M
    n4 = plan(q4, 24 * 10**9, 256 * GIB, 2048 + 64)[0]
    n4m = plan(q4m, 24 * 10**9, 256 * GIB, 2048 + 64)[0]
    n6 = plan(q6, 24 * 10**9, 256 * GIB, 2048 + 64)[0]
    assert 0 < n6 < n4m < n4 < 80
    assert n4m - n6 >= 10
