"""Decode state, failure handling and the streaming double buffer's ordering (GPU only).

- resume: the decode state is (KV cache, n_past, skip mask); 16 tokens, a snapshot, a fresh model
  restored from it and 16 more tokens equal 32 uninterrupted tokens bitwise;
- a non-finite fp16 scale written by the host propagates to the logits, and the capture check names
  the layer that produced it, as the oracle's hidden states do;
- a pass that fails with copies in flight leaves a model that continues (or is destroyed) safely;
- the double buffer stays bitwise equal to resident decode with compute forced to lag the copies, and
  with kernels and copies serialized by the runtime (AMD_SERIALIZE_KERNEL / AMD_SERIALIZE_COPY);
- the file-backed third tier matches the oracle."""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import is_tie, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def qwg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_weight_streaming_gemv_amd import synthetic
    synthetic._lib.lib()
    return synthetic


def _greedy(m, t, n):
    toks, lgs = [], []
    for _ in range(n):
        t, lg = m.decode_step(t, want_logits=True)
        toks.append(t)
        lgs.append(lg)
    return toks, lgs


@pytest.mark.parametrize("n_resident", [-1, 2], ids=["resident", "streamed"])
def test_kv_snapshot_restore_equals_uninterrupted(qwg, n_resident):
    wl = synth.tiny(synth.Q4_K, wid=301)
    a = qwg.make_model(wl, n_resident=n_resident)
    qwg.load(a, wl)
    ref_toks, ref_lgs = _greedy(a, wl.first_token(), 32)
    a.close()

    b = qwg.make_model(wl, n_resident=n_resident)
    qwg.load(b, wl)
    toks1, lgs1 = _greedy(b, wl.first_token(), 16)
    n = b.n_past
    snap = [b.get_kv(l, n) for l in range(wl.n_layers)]
    b.close()

    c = qwg.make_model(wl, n_resident=n_resident)
    qwg.load(c, wl)
    for l, (k, v) in enumerate(snap):
        c.set_kv(l, k, v)
    assert c.n_past == n
    toks2, lgs2 = _greedy(c, toks1[-1], 16)
    c.close()
    assert toks1 + toks2 == ref_toks
    for x, y in zip(lgs1 + lgs2, ref_lgs):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def _nan_scale(W, qt, block):
    """A copy of canonical matrix W with the fp16 d of one block set to NaN (0x7E00)."""
    W = np.array(W, copy=True)
    flat = W.reshape(-1, synth.BLOCK_BYTES[qt])
    off = 208 if qt == synth.Q6_K else 0
    flat[block, off:off + 2] = [0x00, 0x7E]
    return W


@pytest.mark.parametrize("qt", [synth.Q4_K, synth.Q6_K, synth.Q8_0])
def test_nan_scale_propagates_and_names_the_layer(qwg, qt):
    """A NaN d in one block of layer 2's W_down: the step's logits are non-finite on both sides, the
    first non-finite hidden state is layer 2's output on both, and every hidden state before it still
    matches the oracle."""
    wl = synth.tiny(qt, wid=310 + qt)
    bad_layer = 2
    W = _nan_scale(wl.weight(bad_layer, synth.WDOWN), qt, 5)
    m = qwg.make_model(wl)
    qwg.load(m, wl, weights_override={(bad_layer, synth.WDOWN): W})
    m.set_capture(True)
    t = wl.first_token()
    nxt, lg = m.decode_step(t, want_logits=True)
    assert not np.isfinite(lg).any()
    assert m.first_nonfinite() == bad_layer
    om = oracle.OracleModel(wl)
    om._keep.append(W)
    om.layers[bad_layer].w[oracle.OracleModel.TENSORS.index(synth.WDOWN)] = W.ctypes.data
    with np.errstate(invalid="ignore", over="ignore"):
        r = om.decode(t, want_hidden=True)
    first = next(l - 1 for l in range(wl.n_layers + 1) if not np.isfinite(r["hidden"][l]).all())
    assert first == bad_layer
    assert not np.isfinite(r["logits"]).any()
    # a NaN logit is the largest: both sides choose the first NaN, index 0 here
    assert nxt == r["next"] == 0
    for l in range(bad_layer + 1):  # hidden[l] is the state after layer l - 1
        assert rel_l2(m.get_hidden(l - 1), r["hidden"][l]) < 2e-3
    m.close()


def test_failure_with_copies_in_flight_then_continue_and_destroy(qwg):
    """A streamed pass forced to fail at layer 3 returns QWG_E_STATE with the copies of layers 3 and 4
    issued and compute still waiting behind a spin; the same model then decodes exactly like a fresh
    one, and a model destroyed right after such a failure frees cleanly (a new one works)."""
    from quantized_weight_streaming_gemv_amd import _lib
    wl = synth.tiny(synth.Q6_K, n_layers=6, wid=320)
    ref = qwg.make_model(wl, n_resident=1)
    qwg.load(ref, wl)
    want, want_lg = _greedy(ref, wl.first_token(), 3)
    ref.close()

    m = qwg.make_model(wl, n_resident=1)
    qwg.load(m, wl)
    m.set_debug(_lib.DEBUG_SPIN_US, 2000)
    m.set_debug(_lib.DEBUG_FAIL_AT_LAYER, 3)
    n0 = m.n_past
    with pytest.raises(_lib.QwgError) as e:
        m.decode_step(wl.first_token())
    assert e.value.code == -5 and "forced failure at layer 3" in str(e.value)
    assert m.n_past == n0
    m.set_debug(_lib.DEBUG_FAIL_AT_LAYER, -1)
    got, got_lg = _greedy(m, wl.first_token(), 3)
    assert got == want
    for x, y in zip(got_lg, want_lg):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    m.close()

    d = qwg.make_model(wl, n_resident=1)
    qwg.load(d, wl)
    d.set_debug(_lib.DEBUG_SPIN_US, 5000)
    d.set_debug(_lib.DEBUG_FAIL_AT_LAYER, 4)
    with pytest.raises(_lib.QwgError):
        d.decode_step(wl.first_token())
    d.close()  # synchronizes both streams, then frees the pinned images
    again = qwg.make_model(wl, n_resident=1)
    qwg.load(again, wl)
    assert _greedy(again, wl.first_token(), 3)[0] == want
    again.close()


def test_double_buffer_with_compute_lagging_copies(qwg):
    """Every streamed layer's compute waits 3 ms before its kernels, so the copy stream runs ahead as far
    as the slot events let it: a copy into a slot still being read would change the results.  Decode
    stays bitwise equal to resident decode."""
    from quantized_weight_streaming_gemv_amd import _lib
    wl = synth.tiny(synth.Q6_K, n_layers=6, wid=330)
    outs = []
    for res, spin in ((-1, 0), (0, 3000), (2, 3000)):
        m = qwg.make_model(wl, n_resident=res)
        qwg.load(m, wl)
        m.set_debug(_lib.DEBUG_SPIN_US, spin)
        outs.append(_greedy(m, wl.first_token(), 3))
        m.close()
    for toks, lgs in outs[1:]:
        assert toks == outs[0][0]
        for x, y in zip(lgs, outs[0][1]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_double_buffer_under_serialized_runtime(qwg):
    """The same streamed decode in a child process with AMD_SERIALIZE_KERNEL=3 and AMD_SERIALIZE_COPY=3
    (the runtime waits after every kernel and copy) equals this process's resident decode bitwise."""
    wl = synth.tiny(synth.Q6_K, n_layers=6, wid=331)
    m = qwg.make_model(wl)
    qwg.load(m, wl)
    toks, lgs = _greedy(m, wl.first_token(), 3)
    m.close()
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", AMD_SERIALIZE_COPY="3")
    child = os.path.join(HERE, "child_stream_decode.py")
    r = subprocess.run([sys.executable, child, "331", "0", "3"], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["h2d_bytes"] > 0 and out["tokens"] == toks
    assert out["logit_sha256"] == [hashlib.sha256(x.tobytes()).hexdigest() for x in lgs]


def test_file_backed_tier_matches_oracle(qwg, tmp_path):
    """Streamed layers spilled to files (host reads into pinned staging, then H2D) against the oracle:
    hidden states and logits within relative L2 2e-3 over four tokens."""
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=5, wid=340)
    m = qwg.make_model(wl, n_resident=1)
    qwg.load(m, wl)
    for l in (1, 3, 4):
        m.spill_layer(l, str(tmp_path / ("layer%d.img" % l)))
    m.set_capture(True)
    om = oracle.OracleModel(wl)
    t = wl.first_token()
    for step in range(4):
        g_next, g_lg = m.decode_step(t, want_logits=True)
        r = om.decode(t, want_hidden=True)
        assert rel_l2(g_lg, r["logits"]) < 2e-3
        for l in range(wl.n_layers + 1):
            assert rel_l2(m.get_hidden(l - 1), r["hidden"][l]) < 2e-3, (step, l)
        if g_next != r["next"]:
            assert is_tie(r["logits"], g_next, r["next"])
        t = r["next"]
    fb, _ = m.file_stats()
    assert fb > 0
    m.close()
