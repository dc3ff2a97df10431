"""Full-size parity: the real Llama-8B / 70B shapes of the measured workloads, in the launch
configuration bench.py times (default geometry), on outputs the CPU oracle can compute in seconds.

  * 8B Q8_0: two whole decode steps against the oracle's whole steps (every layer's hidden
    state, logits, greedy token, the K/V rows written).
  * 70B Q4_K: one decode step; all 80 layers recomputed by the oracle from the GPU's own input to
    each layer (teacher-forced), the written K/V rows, and the head on the GPU's final state.
  * 70B Q6_K, 20 layers resident + 60 streamed, cosine skip at 0.98: the calibration step's
    per-layer cosines and skip decisions on sampled layers (streamed and resident, near-identity
    and random), skipped layers passing h through unchanged in the next step, and streaming
    equal to residency bit for bit.
  * 70B Q4_K prefill: one 8-column pass on the matrix cores equal to 8 one-column steps.
  * 70B Q6_K attention / Q5_K FFN, self-speculative k=3: one round; the (k+1)-column verify equal
    to k+1 single steps, acceptance consistent with the verify argmaxes, rollback of n_past, and
    sampled verify layers against the oracle.

Tolerances are the ones of the model-level tests: hidden states and logits within relative L2
2e-3; cosines within 1e-5; greedy decisions equal except at near-ties (gap below 1e-4 max|logits|
for argmax, within 1e-4 of tau for the skip test).

  * 8B Q8_0: the workload's whole 32-token greedy decode against the oracle's, teacher-forced on
    near-ties (about 90 s, most of it the oracle's).

Opt-in with QWG_FULL_LENGTH=1, because the oracle needs about ten minutes of host time for it: two
self-speculative rounds of the 70B Q6_K / Q5_K workload against the oracle's rounds."""
import gc
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import is_tie, rel_l2

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def qwg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_weight_streaming_gemv_amd import ops, synthetic
    synthetic._lib.lib()
    ops.set_gemv_geometry(0, 0, 0, 0)  # the default (benchmarked) launch geometry
    return synthetic


def free(*objs):
    for o in objs:
        if hasattr(o, "close"):
            o.close()
    gc.collect()
    torch.cuda.empty_cache()


def layer_kv(wl, layer, ctx):
    """The layer's prefilled K/V caches as the oracle takes them ([ctx][n_kv][hd] fp16 bits)."""
    kc = np.zeros((ctx, wl.n_kv, wl.head_dim), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kc[: wl.n_prior] = wl.kv_prior(layer, synth.KCACHE)
    vc[: wl.n_prior] = wl.kv_prior(layer, synth.VCACHE)
    return kc, vc


def check_layer(wl, m, layer, h_in, h_out, pos, ctx):
    """Oracle layer `layer` on the GPU's own input h_in and K/V rows before pos (teacher-forced):
    its output and the K/V row written at pos."""
    w = {t: wl.weight(layer, t) for t in oracle.OracleModel.TENSORS}
    kc, vc = layer_kv(wl, layer, ctx)
    if pos > wl.n_prior:
        gk, gv = m.get_kv(layer, pos)
        assert np.array_equal(gk[: wl.n_prior], kc[: wl.n_prior])
        kc[wl.n_prior: pos] = gk[wl.n_prior: pos]
        vc[wl.n_prior: pos] = gv[wl.n_prior: pos]
    ref = oracle.layer_forward(wl, layer, w, h_in, kc, vc, pos)
    err = rel_l2(h_out, ref)
    assert err < 2e-3, (layer, err)
    gk, gv = m.get_kv(layer, pos + 1)
    # fp16 rows: the GPU rounds its fp32 values, the oracle its fp64 values, so last-bit flips are
    # expected; the rows must agree to the hidden-state tolerance
    for g, r in ((gk[pos], kc[pos]), (gv[pos], vc[pos])):
        assert rel_l2(f16(g), f16(r)) < 2e-3, layer
    return ref


def f16(bits):
    return np.asarray(bits).view(np.float16).astype(np.float64)


@pytest.mark.timeout(600)
def test_llama8b_q8_0_two_steps(qwg):
    wl = synth.LLAMA8B_Q8_0
    ctx = wl.n_prior + 8
    m = qwg.make_model(wl, max_ctx=ctx)
    qwg.load(m, wl)
    m.set_capture(True)
    om = oracle.OracleModel(wl, max_ctx=ctx)
    t = wl.first_token()
    for step in range(2):
        g_next, g_logits = m.decode_step(t, want_logits=True)
        hid = [m.get_hidden(l) for l in range(-1, wl.n_layers)]
        r = om.decode(t, want_hidden=True)
        for l in range(wl.n_layers + 1):
            assert rel_l2(hid[l], r["hidden"][l]) < 2e-3, (step, l)
        assert rel_l2(g_logits, r["logits"]) < 2e-3, step
        if g_next != r["next"]:
            assert is_tie(r["logits"], g_next, r["next"]), (step, g_next, r["next"])
        t = r["next"]
    n = om.n_past
    for l in (0, 13, 31):
        k, v = m.get_kv(l, n)
        assert np.array_equal(k[: wl.n_prior], om.kc[l][: wl.n_prior])
        for j in range(wl.n_prior, n):  # the rows the two steps wrote
            assert rel_l2(f16(k[j]), f16(om.kc[l][j])) < 2e-3, (l, j)
            assert rel_l2(f16(v[j]), f16(om.vc[l][j])) < 2e-3, (l, j)
    free(m)
    del om
    gc.collect()


@pytest.mark.timeout(900)
def test_llama70b_q4_k_step_all_layers(qwg):
    wl = synth.LLAMA70B_Q4_K
    ctx = wl.n_prior + 4
    m = qwg.make_model(wl, max_ctx=ctx)
    qwg.load(m, wl)
    m.set_capture(True)
    t = wl.first_token()
    g_next, g_logits = m.decode_step(t, want_logits=True)
    hid = {l: m.get_hidden(l) for l in range(-1, wl.n_layers)}
    # the embedding row is the exact dequantized row
    emb = oracle.dequant(wl.qtype_embed, wl.weight(-1, synth.EMBED, t, 1), 1, wl.hidden)[0]
    assert np.array_equal(hid[-1], emb)
    for l in range(wl.n_layers):  # every layer, from the GPU's own input to it
        check_layer(wl, m, l, hid[l - 1], hid[l], wl.n_prior, ctx)
        if l % 10 == 9:
            print("70B Q4_K: layers 0..%d match the oracle" % l, flush=True)
    ref = oracle.head_logits(wl, wl.weight(-1, synth.HEAD), hid[79])
    assert rel_l2(g_logits, ref) < 2e-3
    r_next = oracle.argmax_f32(ref.astype(np.float32))
    if g_next != r_next:
        assert is_tie(ref, g_next, r_next)
    free(m)


@pytest.mark.timeout(600)
def test_llama70b_q4_k_prefill_on_matrix_cores_equals_steps(qwg):
    """At the 70B Q4_K shape, a prefill of 8 prompt tokens in one 8-column pass (the matrix-core
    GEMVs; K = 8192 split in two, K = 28672 in eight) equals 8 one-column decode steps (the integer-dot
    GEMVs, themselves checked against the oracle above): the next token's logits and the K/V rows
    of the prompt positions on sampled layers."""
    wl = synth.LLAMA70B_Q4_K
    ctx = wl.n_prior + 16
    m = qwg.make_model(wl, max_ctx=ctx, max_cols=8)
    qwg.load(m, wl)
    prompt = [(wl.first_token() + 7919 * i) % wl.vocab for i in range(8)]
    p_next, p_logits = m.prefill(prompt, want_logits=True)
    rows = slice(wl.n_prior, wl.n_prior + 8)
    kv_p = {l: m.get_kv(l, wl.n_prior + 8) for l in (0, 40, 79)}
    m.truncate(wl.n_prior)
    for t in prompt:
        s_next, s_logits = m.decode_step(t, want_logits=True)
    assert m.n_past == wl.n_prior + 8
    assert rel_l2(p_logits, s_logits) < 2e-3
    if p_next != s_next:
        assert is_tie(s_logits, p_next, s_next)
    for l, (pk, pv) in kv_p.items():
        sk, sv = m.get_kv(l, wl.n_prior + 8)
        assert rel_l2(f16(pk[rows]), f16(sk[rows])) < 2e-3, l
        assert rel_l2(f16(pv[rows]), f16(sv[rows])) < 2e-3, l
    free(m)


@pytest.mark.timeout(600)
def test_llama70b_q4_k_prefill_64_tokens_one_pass_equals_steps(qwg):
    """At the 70B Q4_K shape, a 64-token prompt in one pass of the prompt-prefill GEMM (64 columns, every
    weight read once) equals 64 one-column decode steps (themselves checked against the oracle above):
    the next token's logits and the K/V rows of all 64 prompt positions on sampled layers."""
    wl = synth.LLAMA70B_Q4_K
    ctx = wl.n_prior + 72
    m = qwg.make_model(wl, max_ctx=ctx, max_cols=64)
    qwg.load(m, wl)
    prompt = [(wl.first_token() + 7919 * i) % wl.vocab for i in range(64)]
    p_next, p_logits = m.prefill(prompt, want_logits=True)
    rows = slice(wl.n_prior, wl.n_prior + 64)
    kv_p = {l: m.get_kv(l, wl.n_prior + 64) for l in (0, 40, 79)}
    m.truncate(wl.n_prior)
    for t in prompt:
        s_next, s_logits = m.decode_step(t, want_logits=True)
    assert rel_l2(p_logits, s_logits) < 2e-3
    if p_next != s_next:
        assert is_tie(s_logits, p_next, s_next)
    for l, (pk, pv) in kv_p.items():
        sk, sv = m.get_kv(l, wl.n_prior + 64)
        assert rel_l2(f16(pk[rows]), f16(sk[rows])) < 2e-3, l
        assert rel_l2(f16(pv[rows]), f16(sv[rows])) < 2e-3, l
    free(m)


@pytest.mark.timeout(900)
def test_llama70b_q6_k_streamed_skip(qwg):
    wl = synth.LLAMA70B_Q6_K_STREAM
    ctx = wl.n_prior + 4
    tau = wl.skip_tau
    m = qwg.make_model(wl, max_ctx=ctx)  # layers 0..19 resident, 20..79 streamed from pinned host memory
    qwg.load(m, wl)
    m.set_capture(True)
    t = wl.first_token()
    g_next, g_cos, g_mask = m.calibrate_skip(tau, t)
    h2d, _ = m.stream_stats()
    assert h2d >= 60 * wl.layer_bytes()  # the calibration step computes (and streams) every layer
    sample = (3, 17, 20, 58, 79)  # near-identity resident, random resident, first streamed, random, near-identity
    hid = {l: m.get_hidden(l) for l in sorted(set([l - 1 for l in sample] + list(sample)))}
    for l in sample:
        ref = check_layer(wl, m, l, hid[l - 1], hid[l], wl.n_prior, ctx)
        h_in = hid[l - 1].astype(np.float64)
        assert abs(g_cos[l] - oracle.cosine(h_in, hid[l].astype(np.float64))) < 1e-6, l
        c = oracle.cosine(h_in, ref)
        assert abs(g_cos[l] - c) < 1e-4, (l, g_cos[l], c)
        if abs(c - tau) >= 1e-4:
            assert bool(g_mask[l]) == bool(np.float32(c) >= np.float32(tau)), l
    # near-identity layers are skipped; the skip set is reported, not forced
    assert all(g_mask[l] for l in range(3, 80, 4))
    # next step: skipped layers pass h through unchanged, computed ones still match the oracle
    m.decode_step(g_next, want_logits=False)
    hid2 = {l: m.get_hidden(l) for l in range(-1, wl.n_layers)}
    for l in range(wl.n_layers):
        if g_mask[l]:
            assert np.array_equal(hid2[l], hid2[l - 1]), l
    first_run = [l for l in range(20, 80) if not g_mask[l]][:1]
    for l in first_run:
        check_layer(wl, m, l, hid2[l - 1], hid2[l], wl.n_prior + 1, ctx)
    free(m)

    # streaming equals residency bit for bit: the same calibration step with every layer resident
    mr = qwg.make_model(wl, max_ctx=ctx, n_resident=-1)
    qwg.load(mr, wl)
    r_next, r_cos, r_mask = mr.calibrate_skip(tau, t)
    assert r_next == g_next and np.array_equal(r_cos, g_cos) and np.array_equal(r_mask, g_mask)
    free(mr)


@pytest.mark.timeout(900)
def test_llama70b_q6k_q5k_spec_round(qwg):
    wl = synth.LLAMA70B_Q6_K_Q5_K_SPEC
    k = wl.draft_k
    ctx = wl.n_prior + 2 * (k + 1) + 4
    m = qwg.make_model(wl, max_ctx=ctx)
    qwg.load(m, wl)
    p = wl.n_prior
    t = wl.first_token()
    out, n_acc = m.spec_step(t, wl.draft_layers, k)
    assert 1 <= len(out) <= k + 1 and n_acc == len(out) - 1
    assert m.n_past == p + n_acc + 1
    # replay the round's verify: its columns j <= n_acc are [t, d_1, .., d_a] = [t] + out[:a]; the
    # remaining columns are padding (verify equals single steps whatever the tokens)
    m.truncate(p)
    m.set_capture(True)
    cols = ([t] + out + [out[-1]] * (k + 1))[: k + 1]
    v_logits, v_am = m.verify(cols)
    assert m.n_past == p
    # acceptance: accepted drafts and the emitted token are the verify argmaxes of their columns
    for j in range(n_acc + 1):
        assert out[j] == v_am[j], (j, out, list(v_am))
    hid = {l: m.get_hidden(l) for l in (-1, 0, 39, 40, 78, 79)}  # column 0 of the verify pass
    # (k+1)-column verify equals k+1 single steps
    m.truncate(p)
    for j, c in enumerate(cols):
        s_next, s_logits = m.decode_step(c, want_logits=True)
        assert rel_l2(v_logits[j], s_logits) < 2e-3, j
        if s_next != v_am[j]:
            assert is_tie(s_logits, s_next, v_am[j])
    # sampled verify layers (column 0) against the oracle from the GPU's own inputs
    for l in (0, 40, 79):
        check_layer(wl, m, l, hid[l - 1], hid[l], p, ctx)
    ref = oracle.head_logits(wl, wl.weight(-1, synth.HEAD), hid[79])
    assert rel_l2(v_logits[0], ref) < 2e-3
    free(m)


FULL = pytest.mark.skipif(not os.environ.get("QWG_FULL_LENGTH"),
                          reason="needs minutes of oracle time on the host; set QWG_FULL_LENGTH=1")


@pytest.mark.timeout(1200)
def test_llama8b_q8_0_32_tokens_teacher_forced(qwg):
    """The 8B Q8_0 workload's 32-token greedy decode: every step's per-layer hidden states and logits
    against the oracle's; where the greedy tokens differ the logits must be a near-tie, and both sides
    continue with the oracle's token."""
    wl = synth.LLAMA8B_Q8_0
    ctx = wl.n_prior + 40
    m = qwg.make_model(wl, max_ctx=ctx)
    qwg.load(m, wl)
    m.set_capture(True)
    om = oracle.OracleModel(wl, max_ctx=ctx)
    t, ties, toks = wl.first_token(), 0, []
    for step in range(32):
        g_next, g_logits = m.decode_step(t, want_logits=True)
        r = om.decode(t, want_hidden=True)
        for l in range(wl.n_layers + 1):
            assert rel_l2(m.get_hidden(l - 1), r["hidden"][l]) < 2e-3, (step, l)
        assert rel_l2(g_logits, r["logits"]) < 2e-3, step
        if g_next != r["next"]:
            assert is_tie(r["logits"], g_next, r["next"]), (step, g_next, r["next"])
            ties += 1
        t = r["next"]
        toks.append(t)
        print("8B Q8_0 step %d: token %d" % (step, t), flush=True)
    print("8B Q8_0 32 tokens: %d distinct, %d near-ties forced" % (len(set(toks)), ties), flush=True)
    free(m)
    del om
    gc.collect()


@FULL
@pytest.mark.timeout(2400)
def test_llama70b_q6k_q5k_two_spec_rounds_against_oracle(qwg):
    """Two self-speculative rounds (k = 3 drafts from layers 0..19, one 4-column verify over 80 layers)
    against the oracle's rounds (drafts from its 20-layer model, verify as four sequential full steps):
    the same drafts, acceptance and emitted tokens (up to near-ties), and each verify column's logits
    within relative L2 2e-3."""
    wl = synth.LLAMA70B_Q6_K_Q5_K_SPEC
    k = wl.draft_k
    ctx = wl.n_prior + 4 * (k + 1)
    m = qwg.make_model(wl, max_ctx=ctx)
    qwg.load(m, wl)
    om = oracle.OracleModel(wl, max_ctx=ctx)
    t = wl.first_token()
    for rnd in range(2):
        p = m.n_past
        assert p == om.n_past
        r = om.spec_round(t, wl.draft_layers, k, log=lambda msg: print("round %d %s" % (rnd, msg), flush=True))
        # the GPU's verify of the oracle's columns, then its own round from the same state
        v_logits, v_am = m.verify([t] + r["drafts"])
        for j in range(k + 1):
            assert rel_l2(v_logits[j], r["logits"][j]) < 2e-3, (rnd, j)
            if v_am[j] != r["verdict"][j]:
                assert is_tie(r["logits"][j], v_am[j], r["verdict"][j]), (rnd, j)
        out, acc = m.spec_step(t, wl.draft_layers, k)
        if out != r["tokens"]:
            # only a near-tie in one of the round's greedy decisions (a draft or a verify column) may
            # change the round; then both continue from the oracle's round
            def top2(L):
                i = np.argsort(L)[-2:]
                return int(i[1]), int(i[0])
            assert any(is_tie(L, *top2(L)) for L in list(r["draft_logits"]) + list(r["logits"])), \
                (rnd, out, r["tokens"])
            m.truncate(p)
            for c in [t] + r["tokens"][:-1]:  # the oracle's columns p .. p + a into the GPU's cache
                m.decode_step(c)
        assert m.n_past == om.n_past
        print("round %d: drafts %s, accepted %d, emitted %s" % (rnd, r["drafts"], r["n_accepted"], r["tokens"]),
              flush=True)
        t = r["tokens"][-1]
    free(m)
    del om
    gc.collect()
