"""Decode-path parity of libqwg.so's model entry points against the CPU oracle (GPU only),
on small Llamas of the same structure (head_dim 128, GQA, SwiGLU) for every format mix.

Per-layer hidden states and logits must be within relative L2 2e-3; greedy tokens must agree
except at near-ties (gap below 1e-4 max|logits|), where the oracle's choice is forced into both."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import is_tie, kv_rows_ok, rel_l2

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MIXES = [(synth.Q8_0, synth.Q8_0), (synth.Q4_K, synth.Q4_K), (synth.Q6_K, synth.Q6_K), (synth.Q6_K, synth.Q5_K),
         (synth.Q4_0, synth.Q4_0)]


@pytest.fixture(scope="module")
def qwg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_weight_streaming_gemv_amd import synthetic
    synthetic._lib.lib()
    return synthetic


def run_pair(qwg, wl, n_tokens, n_resident=None, capture=True):
    m = qwg.make_model(wl, n_resident=n_resident)
    qwg.load(m, wl)
    m.set_capture(capture)
    om = oracle.OracleModel(wl)
    t = wl.first_token()
    records = []
    for step in range(n_tokens):
        g_next, g_logits = m.decode_step(t, want_logits=True)
        r = om.decode(t, want_hidden=True)
        hid = [m.get_hidden(l) for l in range(-1, wl.n_layers)] if capture else None
        records.append((g_next, g_logits, hid, r))
        if g_next != r["next"]:
            assert is_tie(r["logits"], g_next, r["next"]), (step, g_next, r["next"])
        t = r["next"]
    return m, om, records


@pytest.mark.parametrize("mix", MIXES, ids=["%s-%s" % (synth.QTYPE_NAMES[a], synth.QTYPE_NAMES[b]) for a, b in MIXES])
def test_decode_matches_oracle(qwg, mix):
    wl = synth.tiny(mix[0], mix[1], wid=100 + mix[0] * 20 + mix[1])
    m, om, records = run_pair(qwg, wl, 4)
    for g_next, g_logits, hid, r in records:
        assert rel_l2(g_logits, r["logits"]) < 2e-3
        for l in range(wl.n_layers + 1):
            assert rel_l2(hid[l], r["hidden"][l]) < 2e-3, l
    assert m.n_past == om.n_past
    # the KV rows the steps appended, element by element; the prefilled rows are unchanged
    for l in range(wl.n_layers):
        k, v = m.get_kv(l, om.n_past)
        for gpu, ref in ((k, om.kc[l]), (v, om.vc[l])):
            assert np.array_equal(gpu[: wl.n_prior], ref[: wl.n_prior])
            ok, worst = kv_rows_ok(gpu[wl.n_prior: om.n_past], ref[wl.n_prior: om.n_past])
            assert ok.all(), (l, worst)
    m.close()


LONG_FFN = [synth.Q4_K, synth.Q6_K, synth.Q8_0]


@pytest.mark.parametrize("qt", LONG_FFN, ids=[synth.QTYPE_NAMES[q] for q in LONG_FFN])
def test_long_ffn_decode_matches_oracle(qwg, qt):
    """An FFN of 4864 (152 input chunks of the down GEMV): the down GEMV digitizes its fp32 input in
    two segments, the second ragged, while the weights stream (nibble digits for Q4_K, byte digits
    for Q6_K and Q8_0, whose 16-weight chunks take four loop iterations per segment)."""
    wl = synth.tiny(qt, n_layers=2, ffn=4864, wid=240 + qt)
    m, om, records = run_pair(qwg, wl, 2)
    for g_next, g_logits, hid, r in records:
        assert rel_l2(g_logits, r["logits"]) < 2e-3
        for l in range(wl.n_layers + 1):
            assert rel_l2(hid[l], r["hidden"][l]) < 2e-3, l
    m.close()


def tiny_q4_k_m(**kw):
    """A small model with the Q4_K_M stand-in's type mix: Q4_K, with W_down of every other layer and
    the head in Q6_K."""
    base = dict(wid=215, qtype_head=synth.Q6_K, wide_qtype=synth.Q6_K, wide_down_every=2)
    base.update(kw)
    return synth.tiny(synth.Q4_K, **base)


@pytest.mark.parametrize("n_resident", [-1, 1], ids=["resident", "streamed"])
def test_mixed_layer_types_match_oracle(qwg, n_resident):
    """Per-layer types: the down GEMV's input digits take the kind of that layer's W_down, the head's
    input the head's kind; resident and streamed (layer images of two sizes in the slots)."""
    wl = tiny_q4_k_m()
    assert wl.layer_bytes(0) > wl.layer_bytes(1)
    m, om, records = run_pair(qwg, wl, 3, n_resident=n_resident)
    for g_next, g_logits, hid, r in records:
        assert rel_l2(g_logits, r["logits"]) < 2e-3
        for l in range(wl.n_layers + 1):
            assert rel_l2(hid[l], r["hidden"][l]) < 2e-3, l
    m.close()


def test_mixed_layer_types_spec_step(qwg):
    wl = tiny_q4_k_m(wid=216, draft_k=3)
    m = qwg.make_model(wl)
    qwg.load(m, wl)
    om = oracle.OracleModel(wl)
    t = wl.first_token()
    for _ in range(2):
        toks, acc = m.spec_step(t, 2, 3)
        r = om.spec_round(t, 2, 3)
        assert toks == r["tokens"] and acc == r["n_accepted"]
        t = toks[-1]
    m.close()


@pytest.mark.parametrize("case", [(synth.Q4_K, synth.Q4_K, 4, -1, 11), (synth.Q6_K, synth.Q5_K, 4, -1, 11),
                                  (synth.Q4_K, synth.Q4_K, 8, 2, 11), (synth.Q4_K, synth.Q4_K, 64, -1, 40),
                                  (synth.Q6_K, synth.Q5_K, 64, -1, 70), (synth.Q4_K, synth.Q4_K, 16, 2, 37),
                                  (synth.Q8_0, synth.Q8_0, 64, -1, 19), (synth.Q5_K, synth.Q4_K, 64, -1, 97)],
                         ids=["q4k-4col", "q6k-q5k-4col-mfma", "q4k-8col-streamed", "q4k-64col", "q6k-q5k-64col-2pass",
                              "q4k-16col-streamed", "q8_0-64col-falls-back-to-8", "q5k-q4k-64col-then-33"])
def test_prefill_matches_sequential_steps(qwg, case):
    """Prefill of a prompt in passes of max_cols columns (ragged last pass; 9..64-column passes on the
    prefill GEMM, Q8_0 in passes of 8) equals sequential decode steps of the oracle: next token, its
    logits, the KV rows, n_past."""
    qa, qf, cols, res, n_prompt = case
    _prefill_vs_steps(qwg, synth.tiny(qa, qf, wid=230 + cols + res), cols, res, n_prompt)


def test_prefill_three_query_heads_per_kv_head(qwg):
    """12 query heads on 4 KV heads (three per KV head, an attention output of 1536 per column): a
    40-token prompt in one 64-column pass equals sequential decode steps of the oracle."""
    wl = synth.tiny(synth.Q4_K, wid=301, hidden=1536, n_q=12, n_kv=4)
    _prefill_vs_steps(qwg, wl, 64, -1, 40)


def _prefill_vs_steps(qwg, wl, cols, res, n_prompt):
    prompt = [(wl.first_token() + 7919 * i) % wl.vocab for i in range(n_prompt)]
    ctx = wl.n_prior + max(80, n_prompt + 8)
    m = qwg.make_model(wl, max_cols=cols, n_resident=res, max_ctx=ctx)
    qwg.load(m, wl)
    nxt, logits = m.prefill(prompt, want_logits=True)
    om = oracle.OracleModel(wl, max_ctx=ctx)
    for t in prompt:
        r = om.decode(t)
    assert m.n_past == om.n_past == wl.n_prior + len(prompt)
    assert rel_l2(logits, r["logits"]) < 2e-3
    if nxt != r["next"]:
        assert is_tie(r["logits"], nxt, r["next"])
    for l in range(wl.n_layers):
        k, v = m.get_kv(l, om.n_past)
        for gpu, ref in ((k, om.kc[l]), (v, om.vc[l])):
            assert np.array_equal(gpu[: wl.n_prior], ref[: wl.n_prior])
            ok, worst = kv_rows_ok(gpu[wl.n_prior: om.n_past], ref[wl.n_prior: om.n_past])
            assert ok.all(), (l, worst)
    m.close()


def test_streaming_equals_resident_bitwise(qwg):
    wl = synth.tiny(synth.Q6_K, n_layers=5, wid=160)
    outs = []
    for res in (-1, 2, 0):
        m = qwg.make_model(wl, n_resident=res)
        qwg.load(m, wl)
        t, toks, lg = wl.first_token(), [], []
        for _ in range(3):
            t, logits = m.decode_step(t, want_logits=True)
            toks.append(t)
            lg.append(logits)
        b, ms = m.stream_stats()
        assert (b > 0) == (res >= 0)
        outs.append((toks, np.stack(lg)))
        m.close()
    for toks, lg in outs[1:]:
        assert toks == outs[0][0] and np.array_equal(lg, outs[0][1])


def test_file_backed_layers_equal_pinned_bitwise(qwg, tmp_path):
    """The file-backed tier (streamed layers spilled to files, read by the host into pinned staging,
    then copied to HBM) decodes bitwise like the pinned tier, also mixed with pinned layers."""
    from quantized_weight_streaming_gemv_amd import _lib
    wl = synth.tiny(synth.Q6_K, n_layers=5, wid=161)
    runs = []
    for spill in ((), (2, 4), (1, 2, 3, 4)):
        m = qwg.make_model(wl, n_resident=1)
        qwg.load(m, wl)
        for l in spill:
            m.spill_layer(l, str(tmp_path / ("layer%d-%d.img" % (l, len(spill)))))
        t, out = wl.first_token(), []
        for _ in range(3):
            t, lg = m.decode_step(t, want_logits=True)
            out.append((t, lg))
        fb, _ = m.file_stats()
        h2d, _ = m.stream_stats()
        assert h2d > 0 and fb == 3 * len(spill) * (h2d // (3 * 4))
        if spill:
            with pytest.raises(_lib.QwgError) as e:  # a spilled layer's tensors cannot be set again
                m.set_tensor(spill[0], synth.WO, wl.qtype_of(synth.WO, spill[0]), wl.weight(spill[0], synth.WO))
            assert e.value.code == -5
            with pytest.raises(_lib.QwgError):
                m.spill_layer(spill[0], str(tmp_path / "again.img"))
        with pytest.raises(_lib.QwgError):
            m.spill_layer(0, str(tmp_path / "resident.img"))  # layer 0 is resident
        runs.append(out)
        m.close()
    for out in runs[1:]:
        for (t, lg), (rt, rl) in zip(out, runs[0]):
            assert t == rt and np.array_equal(lg, rl)


def test_calibrate_skip_matches_oracle(qwg):
    wl = synth.tiny(synth.Q6_K, n_layers=6, near_identity_every=2, wid=170)
    m = qwg.make_model(wl, n_resident=3)
    qwg.load(m, wl)
    om = oracle.OracleModel(wl)
    t = wl.first_token()
    g_next, g_cos, g_mask = m.calibrate_skip(0.98, t)
    r = om.calibrate_skip(0.98, t)
    assert np.max(np.abs(g_cos - r["cos"])) < 1e-5
    near = np.abs(r["cos"] - 0.98) < 1e-4
    assert np.array_equal(g_mask[~near], r["mask"][~near])
    assert all(g_mask[l] for l in range(wl.n_layers) if l % 2 == 1)  # near-identity layers are skipped
    # later steps bypass the masked layers (both sides), and agree
    om.skip[:] = g_mask
    t = r["next"]
    for _ in range(3):
        g_next, g_logits = m.decode_step(t, want_logits=True)
        rr = om.decode(t)
        assert rel_l2(g_logits, rr["logits"]) < 2e-3
        if g_next != rr["next"]:
            assert is_tie(rr["logits"], g_next, rr["next"])
        t = rr["next"]
    m.close()


@pytest.mark.parametrize("cols", [8, 64], ids=["8col", "64col"])
def test_prefill_after_calibration_skips_like_steps(qwg, cols):
    """A prompt prefilled after skip calibration (Q6_K, near-identity odd layers, 3 of 6 resident)
    bypasses the masked layers as decode steps do: the next token and its logits match the oracle's
    sequential steps with the same mask, new KV rows match element by element in the computed layers,
    and the skipped layers' caches get no new rows on either side.""" 
    wl = synth.tiny(synth.Q6_K, n_layers=6, near_identity_every=2, wid=171)
    max_ctx = wl.n_prior + 40
    m = qwg.make_model(wl, n_resident=3, max_cols=cols, max_ctx=max_ctx)
    qwg.load(m, wl)
    om = oracle.OracleModel(wl, max_ctx=max_ctx)
    t = wl.first_token()
    _, _, g_mask = m.calibrate_skip(0.98, t)
    r = om.calibrate_skip(0.98, t)
    om.skip[:] = g_mask
    assert g_mask.any() and not g_mask.all()
    prompt = [(r["next"] + 7919 * i) % wl.vocab for i in range(19)]
    n0 = m.n_past
    assert om.n_past == n0
    before = [m.get_kv(l, n0 + len(prompt)) for l in range(wl.n_layers)]
    nxt, logits = m.prefill(prompt, want_logits=True)
    for tok in prompt:
        rr = om.decode(tok)
    assert m.n_past == om.n_past == n0 + len(prompt)
    assert rel_l2(logits, rr["logits"]) < 2e-3
    if nxt != rr["next"]:
        assert is_tie(rr["logits"], nxt, rr["next"])
    new = slice(n0, om.n_past)
    for l in range(wl.n_layers):
        k, v = m.get_kv(l, om.n_past)
        for gpu, ref, old in ((k, om.kc[l], before[l][0]), (v, om.vc[l], before[l][1])):
            if g_mask[l]:  # no new rows: the GPU's cache is untouched, the oracle's still zero
                assert np.array_equal(gpu[new], old[new]) and not ref[new].any(), l
            else:
                ok, worst = kv_rows_ok(gpu[new], ref[new])
                assert ok.all(), (l, worst)
    m.close()


@pytest.mark.parametrize("mfma", [True, False], ids=["mfma", "dot"])
def test_verify_columns_equal_sequential_steps(qwg, mfma):
    from quantized_weight_streaming_gemv_amd import ops
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, wid=180, draft_k=3)
    m = qwg.make_model(wl)
    qwg.load(m, wl)
    om = oracle.OracleModel(wl)
    toks = [wl.first_token(), 5, 17, 999]
    ops.set_gemv_mfma(mfma)
    try:
        logits, am = m.verify(toks)
    finally:
        ops.set_gemv_mfma(True)
    assert m.n_past == wl.n_prior
    for j, t in enumerate(toks):
        r = om.decode(t)
        assert rel_l2(logits[j], r["logits"]) < 2e-3, j
        if am[j] != r["next"]:
            assert is_tie(r["logits"], am[j], r["next"])
    m.close()


def _zero_scales(W, qt):
    W = W.copy()
    flat = W.reshape(-1, synth.BLOCK_BYTES[qt])
    if qt == synth.Q6_K:
        flat[:, 208:210] = 0
    elif qt in (synth.Q4_K, synth.Q5_K):
        flat[:, 0:4] = 0
    else:
        flat[:, 0:2] = 0
    return W


@pytest.mark.parametrize("identity_tail", [False, True])
def test_spec_step_matches_oracle(qwg, identity_tail):
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=4, wid=190, draft_k=3)
    draft = 2
    ov = {}
    if identity_tail:
        for l in (2, 3):
            for t in (synth.WO, synth.WDOWN):
                ov[(l, t)] = _zero_scales(wl.weight(l, t), wl.qtype_of(t, l))
    m = qwg.make_model(wl)
    qwg.load(m, wl, weights_override=ov)
    om = oracle.OracleModel(wl)
    for (l, t), W in ov.items():
        om._keep.append(W)
        om.layers[l].w[om.TENSORS.index(t)] = W.ctypes.data
    t = wl.first_token()
    for _ in range(3):
        toks, acc = m.spec_step(t, draft, 3)
        r = om.spec_round(t, draft, 3)
        assert toks == r["tokens"] and acc == r["n_accepted"]
        assert m.n_past == om.n_past
        if identity_tail:
            assert acc == 3
        t = toks[-1]
    m.close()


@pytest.mark.parametrize("identity_tail", [False, True])
def test_spec_step_streamed_verify(qwg, identity_tail):
    """Self-speculative decoding in streaming mode: the draft runs the resident layers only and the
    verify pass streams the others from pinned host memory once per round.  Tokens and acceptance
    match the oracle and the all-resident model bitwise; the H2D bytes of a round are those of one
    full pass (the drafts stream nothing)."""
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=4, wid=195, draft_k=3)
    draft = 2
    ov = {}
    if identity_tail:
        for l in (2, 3):
            for t in (synth.WO, synth.WDOWN):
                ov[(l, t)] = _zero_scales(wl.weight(l, t), wl.qtype_of(t, l))
    om = oracle.OracleModel(wl)
    for (l, t), W in ov.items():
        om._keep.append(W)
        om.layers[l].w[om.TENSORS.index(t)] = W.ctypes.data
    # bytes one full pass streams (layers 2 and 3)
    m = qwg.make_model(wl, n_resident=draft)
    qwg.load(m, wl, weights_override=ov)
    m.decode_step(wl.first_token())
    pass_bytes, _ = m.stream_stats()
    m.close()
    assert pass_bytes > 0
    runs = []
    for res in (draft, -1):
        m = qwg.make_model(wl, n_resident=res)
        qwg.load(m, wl, weights_override=ov)
        t, rounds = wl.first_token(), []
        for _ in range(3):
            toks, acc = m.spec_step(t, draft, 3)
            rounds.append((toks, acc, m.n_past))
            t = toks[-1]
        b, _ = m.stream_stats()
        assert b == (3 * pass_bytes if res == draft else 0)
        runs.append(rounds)
        m.close()
    assert runs[0] == runs[1]
    t = wl.first_token()
    for toks, acc, n_past in runs[0]:
        r = om.spec_round(t, draft, 3)
        assert toks == r["tokens"] and acc == r["n_accepted"] and n_past == om.n_past
        if identity_tail:
            assert acc == 3
        t = toks[-1]


def test_automatic_residency(qwg):
    """n_resident = "auto": the placement from the device's free memory keeps a small model fully
    resident; a placement under a device budget that holds two layers streams the others and decodes
    the same tokens and logits, bitwise, as the resident model."""
    wl = synth.tiny(synth.Q4_K, n_layers=5, wid=165)
    m = qwg.make_model(wl, n_resident="auto")
    assert m.desc.n_resident == wl.n_layers
    qwg.load(m, wl)
    t, ref = wl.first_token(), []
    for _ in range(2):
        t, lg = m.decode_step(t, want_logits=True)
        ref.append((t, lg))
    m.close()
    ctx = wl.n_prior + 64
    full = qwg.plan_residency_of(wl, max_ctx=ctx, device_budget=1 << 40, host_budget=1 << 40)
    two = qwg.make_model(wl, n_resident=0)
    a0 = two.arena_bytes
    two.close()
    image = (full[1] - a0) // (wl.n_layers - 2)  # all resident = 0 resident + n_layers images - 2 slots
    n, arena, pinned = qwg.plan_residency_of(wl, max_ctx=ctx, device_budget=a0 + 2 * image, host_budget=1 << 40)
    assert n == 2 and pinned == (wl.n_layers - 2) * image
    m = qwg.make_model(wl, n_resident=n)
    assert m.arena_bytes == arena
    qwg.load(m, wl)
    t = wl.first_token()
    for rt, rl in ref:
        t, lg = m.decode_step(t, want_logits=True)
        assert t == rt and np.array_equal(lg, rl)
    assert m.stream_stats()[0] > 0
    m.close()


def test_context_overflow_is_an_error(qwg):
    from quantized_weight_streaming_gemv_amd import QwgError
    wl = synth.tiny(synth.Q8_0, wid=200)
    m = qwg.make_model(wl, max_ctx=wl.n_prior + 1)
    qwg.load(m, wl)
    m.decode_step(wl.first_token())
    with pytest.raises(QwgError):
        m.decode_step(1)
    m.truncate(wl.n_prior)
    m.decode_step(wl.first_token())
    m.close()


@pytest.mark.parametrize("geom", [(4, 1, 1, 1), (8, 1, 2, 1), (2, 2, 1, 1), (8, 4, 2, 1), (8, 2, 2, 1),
                                  (8, 2, 1, 2), (4, 4, 1, 2), (2, 4, 1, 2), (8, 4, 1, 1), (8, 2, 1, 4),
                                  (4, 2, 1, 4), (16, 2, 1, 1), (16, 2, 1, 2), (4, 2, 1, 8)],
                         ids=lambda g: "w%d_r%d_d%d_p%d" % g)
def test_decode_under_launch_geometries(qwg, geom):
    """Every launch geometry computes the same step (the pair epilogues need two rows per wave)."""
    from quantized_weight_streaming_gemv_amd import ops
    wl = synth.tiny(synth.Q4_K, synth.Q6_K, wid=210)
    ops.set_gemv_geometry(*geom)
    try:
        m, om, records = run_pair(qwg, wl, 2, capture=False)
        for g_next, g_logits, _, r in records:
            assert rel_l2(g_logits, r["logits"]) < 2e-3
        m.close()
    finally:
        ops.set_gemv_geometry(0, 0, 0, 0)
