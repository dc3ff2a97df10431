"""Pins of the CPU oracle against facts other than itself: the pages' printed sizes,
hand-built blocks with closed-form values, exact rational arithmetic, textbook special
cases and invariants of the Llama decoder (each test names what it pins)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _block(size, ranges, default=0):
    b = np.full(size, default, dtype=np.uint8)
    for s, e, v in ranges:
        b[s:e] = v
    return b


def _expected(entry, n):
    if "runs" in entry:
        out = []
        for cnt, v in entry["runs"]:
            out += [float.fromhex(v) if isinstance(v, str) else float(v)] * cnt
        return np.array(out, dtype=np.float64)
    sp = entry["sparse"]
    out = np.full(n, float.fromhex(sp["default"]))
    for i, v in sp["at"].items():
        out[int(i)] = float.fromhex(v)
    return out


# ---------------------------------------------------------------- pages' numbers

def test_block_sizes_match_quant_table():
    """Show HN page quantization-format table: bits/weight and block sizes."""
    pages = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["quant_table"]["rows"]
    for row in pages:
        qt = row["qtype"]
        assert oracle.lib().orc_block_weights(qt) == row["block"]
        bpw = oracle.lib().orc_block_bytes(qt) * 8 / row["block"]
        step = row.get("printed_rounded_to", 0.0)
        assert abs(bpw - row["bits_per_weight"]) <= step / 2 + 1e-12, (row, bpw)
        assert synth.BLOCK_BYTES[qt] == oracle.lib().orc_block_bytes(qt)


def test_70b_q6k_layer_size_matches_pages():
    """NTransformer page: one 70B Q6_K layer is about 670 MB (NVMe direct streaming section)."""
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["layer_70b_q6_k_mb"]
    b = synth.LLAMA70B_Q6_K_STREAM.layer_bytes()
    assert b == 701890560
    assert abs(b / 2**20 - g["value_mb"]) <= g["tolerance_mb"]


def test_8b_q8_0_fits_pages_vram():
    """Show HN page: 8B Q8_0 fully resident in about 10 GB of VRAM."""
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["vram_8b_q8_0_gb"]
    assert synth.LLAMA8B_Q8_0.model_bytes() / 1e9 < g["upper_bound_gb"]


# ---------------------------------------------------------------- dequant closed forms

BLOCKS = json.load(open(os.path.join(GOLDEN, "blocks.json")))


@pytest.mark.parametrize("entry", BLOCKS["blocks"], ids=[b["name"] for b in BLOCKS["blocks"]])
def test_dequant_hand_built_block(entry):
    qt, size = entry["qtype"], entry["size"]
    B = oracle.lib().orc_block_weights(qt)
    blk = _block(size, entry["set"])
    w = oracle.dequant(qt, blk, 1, B)[0]
    exp = _expected(entry, B)
    assert np.array_equal(w.astype(np.float64), exp), (entry["name"], w[:40], exp[:40])
    if entry.get("positive_zero"):
        assert not np.any(np.signbit(w[w == 0]))


@pytest.mark.parametrize("group", BLOCKS["onehot"], ids=lambda g: str(g["qtype"]))
def test_dequant_onehot_positions(group):
    qt, size = group["qtype"], group["size"]
    B = oracle.lib().orc_block_weights(qt)
    for ranges, idx, val in group["cases"]:
        blk = _block(size, group["base"] + ranges)
        w = oracle.dequant(qt, blk, 1, B)[0]
        exp = np.full(B, float(group["default"]))
        exp[idx] = val
        assert np.array_equal(w.astype(np.float64), exp), (ranges, np.nonzero(w != group["default"]))


@pytest.mark.parametrize("qt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q5_K, synth.Q6_K])
def test_dequant_recovers_drawn_fields(qt):
    """decode(bytes) equals the exact value of the fields the generator drew, rounded once to fp32."""
    dist = synth.DEFAULT_DIST[qt]
    B = synth.BLOCK_WEIGHTS[qt]
    k, rows = 2 * B, 3
    tk = synth.key(7, 1000 + qt)
    W = synth.matrix(dist, k, rows, tkey=tk)
    w = oracle.dequant(qt, W, rows, k)
    for r in range(rows):
        for b in range(k // B):
            f = synth.block_fields(dist, k, r, b, tkey=tk)
            d = Fraction(oracle.half_value(f["d"]))
            dm = Fraction(oracle.half_value(f["dmin"]))
            for i in range(B):
                q = int(f["q"][i])
                if qt == synth.Q8_0:
                    v = d * q
                elif qt == synth.Q4_0:
                    v = d * (q - 8)
                elif qt in (synth.Q4_K, synth.Q5_K):
                    s = i // 32
                    v = d * int(f["sc"][s]) * q - dm * int(f["m"][s])
                else:
                    v = d * int(f["sc"][i // 16]) * (q - 32)
                assert float(np.float32(float(v))) == float(w[r, b * B + i]), (qt, r, b, i)


# ---------------------------------------------------------------- GEMV

def test_gemv_identity_q8_0():
    """W = I built from Q8_0 blocks with d = 1 gives y = x exactly."""
    n = 64
    W = np.zeros((n, 2 * 34), dtype=np.uint8)
    for r in range(n):
        for b in range(2):
            W[r, b * 34 + 1] = 0x3C  # d = 1.0
        W[r, (r // 32) * 34 + 2 + (r % 32)] = 1
    x = synth.normal_f32(synth.key(0, 5), n)
    y, a = oracle.gemv(synth.Q8_0, W, n, n, x)
    assert np.array_equal(y, x.astype(np.float64))
    assert np.array_equal(a, np.abs(x.astype(np.float64)))


@pytest.mark.parametrize("qt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q5_K, synth.Q6_K])
@pytest.mark.parametrize("k", [256, 512])
def test_gemv_exact_rational(qt, k):
    """Brute force with exact rationals on rows <= 4: the fp64 sum is within K * 2^-53 * A."""
    rows = 3
    tk = synth.key(11, 2000 + qt * 10 + k)
    W = synth.matrix(synth.DEFAULT_DIST[qt], k, rows, tkey=tk)
    x = synth.normal_f32(synth.key(11, 3000 + k), 2 * k).reshape(2, k)
    y, a = oracle.gemv(qt, W, rows, k, x)
    w = oracle.dequant(qt, W, rows, k)
    for j in range(2):
        for r in range(rows):
            exact = sum(Fraction(float(w[r, c])) * Fraction(float(x[j, c])) for c in range(k))
            absum = sum(abs(Fraction(float(w[r, c])) * Fraction(float(x[j, c]))) for c in range(k))
            assert abs(Fraction(y[j, r]) - exact) <= Fraction(k) * Fraction(2) ** -53 * absum
            assert abs(Fraction(a[j, r]) - absum) <= Fraction(k) * Fraction(2) ** -53 * absum
    # columns are independent: one column at a time gives the same numbers
    y0, _ = oracle.gemv(qt, W, rows, k, x[1])
    assert np.array_equal(y0, y[1])


def test_gemv_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.gemv(synth.Q4_K, np.zeros(144, np.uint8), 1, 200, np.zeros(200))


# ---------------------------------------------------------------- norm, rope, attention, act

def test_rmsnorm_unit_rms_times_gain():
    x = synth.normal_f32(synth.key(1, 1), 4096, 0.3, 5.0).astype(np.float64)
    g = synth.normal_f32(synth.key(1, 2), 4096, 1.0, 0.02)
    y = oracle.rmsnorm(x, g, 0.0)
    assert abs(math.sqrt(np.mean((y / g) ** 2)) - 1.0) < 1e-12
    assert np.allclose(oracle.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-13, atol=0)


def test_rmsnorm_eps_closed_form():
    # x = 1 everywhere, eps = 3: 1 / sqrt(1 + 3) = 1/2
    g = np.array([1.0, 2.0, -4.0, 0.5], dtype=np.float32)
    assert np.array_equal(oracle.rmsnorm(np.ones(4), g, 3.0), 0.5 * g.astype(np.float64))


def test_rope_identity_at_zero_and_norms():
    hd, nh = 128, 3
    v = synth.normal_f32(synth.key(2, 1), nh * hd).astype(np.float64)
    assert np.array_equal(oracle.rope(v, nh, hd, 0, 5e5), v)
    r = oracle.rope(v, nh, hd, 1234, 5e5)
    pn = lambda a: np.hypot(a[0::2], a[1::2])
    assert np.allclose(pn(r), pn(v), rtol=1e-13)


def test_rope_composition_and_relative_position():
    hd = 128
    v = synth.normal_f32(synth.key(2, 2), hd).astype(np.float64)
    w = synth.normal_f32(synth.key(2, 3), hd).astype(np.float64)
    a = oracle.rope(oracle.rope(v, 1, hd, 300, 5e5), 1, hd, 4000, 5e5)
    assert np.allclose(a, oracle.rope(v, 1, hd, 4300, 5e5), rtol=0, atol=1e-9)
    d1 = oracle.rope(v, 1, hd, 1000, 5e5) @ oracle.rope(w, 1, hd, 990, 5e5)
    d2 = oracle.rope(v, 1, hd, 17, 5e5) @ oracle.rope(w, 1, hd, 7, 5e5)
    assert abs(d1 - d2) < 1e-9 * (np.abs(v) @ np.abs(w))


def test_rope_pairs_and_frequencies():
    """Adjacent pairs (2i, 2i+1) rotate; pair 0 turns by pos radians; pair hd/4 has frequency
    base^-1/2, so at pos = pi * sqrt(base) it has turned by pi."""
    hd, base = 128, 5e5
    e0 = np.zeros(hd)
    e0[0] = 1.0
    r = oracle.rope(e0, 1, hd, 3, base)
    assert np.count_nonzero(r) == 2 and r[0] == math.cos(3.0) and r[1] == math.sin(3.0)
    e = np.zeros(hd)
    e[64] = 1.0  # pair 32 = hd/4
    p = math.pi * math.sqrt(base)
    r = oracle.rope(e, 1, hd, int(round(p)), base)
    ang = round(p) / math.sqrt(base)
    assert abs(r[64] - math.cos(ang)) < 1e-9 and abs(r[65] - math.sin(ang)) < 1e-9
    assert r[64] < -0.9999


def _f16(a):
    return np.array([oracle.half_from_double(v) for v in np.ravel(a)], dtype=np.uint16).reshape(np.shape(a))


def test_attention_one_position_is_v0():
    nq, nkv, hd = 4, 2, 128
    k = synth.normal_f16(synth.key(3, 1), nkv * hd).reshape(1, nkv, hd)
    v = synth.normal_f16(synth.key(3, 2), nkv * hd).reshape(1, nkv, hd)
    q = synth.normal_f32(synth.key(3, 3), nq * hd) * 10
    o = oracle.attention(q, k, v, 1, nq, nkv, hd).reshape(nq, hd)
    vv = np.array([oracle.half_value(b) for b in v.ravel()]).reshape(nkv, hd)
    for h in range(nq):  # contiguous groups: heads 0,1 -> kv 0; heads 2,3 -> kv 1
        assert np.array_equal(o[h], vv[h // 2])


def test_attention_identical_keys_is_mean_and_weights_sum_to_one():
    nq, nkv, hd, n = 2, 1, 128, 9
    k1 = synth.normal_f16(synth.key(3, 4), hd)
    kc = np.tile(k1, (n, 1)).reshape(n, 1, hd)
    vc = synth.normal_f16(synth.key(3, 5), n * hd).reshape(n, 1, hd)
    q = synth.normal_f32(synth.key(3, 6), nq * hd)
    o = oracle.attention(q, kc, vc, n, nq, nkv, hd).reshape(nq, hd)
    vv = np.array([oracle.half_value(b) for b in vc.ravel()]).reshape(n, hd)
    assert np.allclose(o[0], vv.mean(axis=0), rtol=1e-12, atol=1e-14)
    ones = np.full((n, 1, hd), 0x3C00, dtype=np.uint16)
    kc2 = synth.normal_f16(synth.key(3, 7), n * hd).reshape(n, 1, hd)
    o1 = oracle.attention(q * 3, kc2, ones, n, nq, nkv, hd)
    assert np.allclose(o1, 1.0, rtol=1e-14)


def test_attention_two_positions_closed_form():
    """q = c e0, k0 = e0, k1 = 0: weight on position 0 is 1 / (1 + exp(-c / sqrt(128)))."""
    hd, c = 128, 8.0
    kc = np.zeros((2, 1, hd), dtype=np.uint16)
    kc[0, 0, 0] = 0x3C00
    vc = np.zeros((2, 1, hd), dtype=np.uint16)
    vc[0, 0, 0] = 0x3C00  # v0 = e0, v1 = e1
    vc[1, 0, 1] = 0x3C00
    q = np.zeros(hd)
    q[0] = c
    o = oracle.attention(q, kc, vc, 2, 1, 1, hd)
    p0 = 1.0 / (1.0 + math.exp(-c / math.sqrt(128.0)))
    assert abs(o[0] - p0) < 1e-15 and abs(o[1] - (1 - p0)) < 1e-15


def test_attention_ignores_cache_rows_at_and_past_n_pos():
    """Only positions 0 .. n_pos - 1 count: rows from n_pos on hold keys that would dominate the
    softmax and values far from the rest, yet the output equals that of a cache cut at n_pos, and
    admitting one more position changes it."""
    nq, nkv, hd, n_pos, ctx = 4, 2, 128, 3, 6
    kc = synth.normal_f16(synth.key(3, 8), ctx * nkv * hd).reshape(ctx, nkv, hd)
    vc = synth.normal_f16(synth.key(3, 9), ctx * nkv * hd).reshape(ctx, nkv, hd)
    q = synth.normal_f32(synth.key(3, 10), nq * hd)
    big = oracle.half_from_double(60000.0)
    for t in range(n_pos, ctx):  # k_t = 60000 sign(q) per head group: scores far above the others
        for g in range(nkv):
            qh = q[(g * (nq // nkv)) * hd:(g * (nq // nkv) + 1) * hd]
            kc[t, g] = np.where(qh >= 0, big, big | 0x8000).astype(np.uint16)
        vc[t] = big
    o = oracle.attention(q, kc, vc, n_pos, nq, nkv, hd)
    o_cut = oracle.attention(q, kc[:n_pos].copy(), vc[:n_pos].copy(), n_pos, nq, nkv, hd)
    assert np.array_equal(o, o_cut)
    o_more = oracle.attention(q, kc, vc, n_pos + 1, nq, nkv, hd)
    assert np.abs(o_more - o).max() > 1000.0


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(60.0) == 60.0
    s = oracle.silu(-100.0)
    assert s == 0.0 or abs(s) < 1e-40
    z = oracle.silu(-1e6)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    g = np.array([0.0, 2.0, -1e6]); u = np.array([5.0, 3.0, 7.0])
    sw = oracle.swiglu(g, u)
    assert sw[0] == 0.0 and not np.isnan(sw).any()


def test_cosine_special_values():
    v = synth.normal_f32(synth.key(4, 1), 1000).astype(np.float64)
    assert abs(oracle.cosine(v, v) - 1.0) < 1e-15
    assert abs(oracle.cosine(v, -v) + 1.0) < 1e-15
    assert oracle.cosine(np.array([1.0, 0.0]), np.array([0.0, 3.0])) == 0.0
    assert oracle.cosine(np.zeros(4), np.ones(4)) == 0.0


def test_argmax_lowest_index_on_fp32_ties():
    assert oracle.argmax_f32(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    # 1 and 1 + 1e-12 are the same fp32 number: the decision is taken in fp32, lowest index wins
    assert oracle.argmax_f32(np.array([0.5, 1.0, 1.0 + 1e-12])) == 1


def test_half_rounding_through_fp32():
    h = oracle.half_from_double
    assert h(1.0) == 0x3C00 and h(65504.0) == 0x7BFF and h(65520.0) == 0x7C00 and h(-70000.0) == 0xFC00
    assert h(2.0 ** -24) == 0x0001 and h(2.0 ** -25) == 0x0000 and h(3 * 2.0 ** -26) == 0x0001
    assert h(1 + 2.0 ** -11) == 0x3C00 and h(1 + 3 * 2.0 ** -11) == 0x3C02  # ties to even
    # 1 + 2^-11 + 2^-40 is 1 + 2^-11 in fp32 (a tie in fp16 -> even), though in fp64 it is above the tie
    assert h(1 + 2.0 ** -11 + 2.0 ** -40) == 0x3C00
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xC000):
        assert h(oracle.half_value(b)) == b


# ---------------------------------------------------------------- model-level invariants

def _zero_d(W, qt):
    """Set every block scale of a canonical matrix to zero (the matrix becomes exactly 0)."""
    W = W.copy()
    bb = synth.BLOCK_BYTES[qt]
    flat = W.reshape(-1, bb)
    if qt == synth.Q6_K:
        flat[:, 208:210] = 0
    elif qt in (synth.Q4_K, synth.Q5_K):
        flat[:, 0:4] = 0
    else:
        flat[:, 0:2] = 0
    return W


def _model_with_identity_layers(wl, layers):
    om = oracle.OracleModel(wl)
    for l in layers:
        for i, t in enumerate(om.TENSORS):
            if t in (synth.WO, synth.WDOWN):
                z = _zero_d(wl.weight(l, t), wl.qtype_of(t, l))
                om._keep.append(z)
                om.layers[l].w[i] = z.ctypes.data
    return om


def test_identity_layer_skip_equals_compute():
    wl = synth.tiny(synth.Q8_0)
    a = _model_with_identity_layers(wl, [1, 2])
    r = a.step(wl.first_token(), want_hidden=True)
    assert np.array_equal(r["hidden"][2], r["hidden"][1]) and np.array_equal(r["hidden"][3], r["hidden"][2])
    assert abs(r["cos"][1] - 1.0) < 1e-15 and abs(r["cos"][2] - 1.0) < 1e-15 and r["cos"][0] < 0.999
    b = _model_with_identity_layers(wl, [1, 2])
    b.skip[:] = [0, 1, 1, 0]
    r2 = b.step(wl.first_token())
    assert np.array_equal(r["logits"], r2["logits"])


def test_calibration_marks_identity_layers():
    wl = synth.tiny(synth.Q6_K)
    m = _model_with_identity_layers(wl, [3])
    r = m.calibrate_skip(0.98, wl.first_token())
    assert r["mask"][3] == 1 and m.n_past == wl.n_prior + 1


def test_step_writes_kv_only_at_position():
    wl = synth.tiny(synth.Q4_K)
    m = oracle.OracleModel(wl)
    before = [k.copy() for k in m.kc]
    m.decode(wl.first_token())
    for l in range(wl.n_layers):
        changed = np.nonzero(np.any(m.kc[l] != before[l], axis=(1, 2)))[0]
        assert list(changed) == [wl.n_prior]


def test_spec_round_is_lossless_and_accepts_all_when_tail_is_identity():
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=4)
    draft = 2
    # tail layers are exact identities: the draft model equals the full model, all k accepted
    full = _model_with_identity_layers(wl, [2, 3])
    res = full.spec_round(wl.first_token(), draft, 3)
    assert res["n_accepted"] == 3 and res["tokens"] == res["drafts"] + [res["verdict"][3]]
    # greedy decode gives the same tokens (self-speculation never changes the output)
    ref = _model_with_identity_layers(wl, [2, 3])
    t, toks = wl.first_token(), []
    for _ in range(4):
        t = ref.decode(t)["next"]
        toks.append(t)
    assert toks == res["tokens"] and full.n_past == ref.n_past


def test_spec_round_rejection_rolls_back():
    wl = synth.tiny(synth.Q6_K, synth.Q5_K, n_layers=4)
    m = oracle.OracleModel(wl)
    ref = oracle.OracleModel(wl)
    t0 = wl.first_token()
    res = m.spec_round(t0, 2, 3)
    a = res["n_accepted"]
    assert m.n_past == wl.n_prior + a + 1 and len(res["tokens"]) == a + 1
    t, toks = t0, []
    for _ in range(a + 1):
        t = ref.decode(t)["next"]
        toks.append(t)
    assert toks == res["tokens"]


# ---------------------------------------------------------------- layer and head composition
#
# Hand-built Q8_0 layers (d = 1, integer quants: the matrices are exact integers) with closed-form
# outputs.  H = 256, two query heads sharing one KV head of 128, FFN 64, eps = 0, and a residual
# input u of +-1 entries (mean square exactly 1), so every RMSNorm output is gain * u exactly.
# Each case fixes one wiring choice of the pre-norm Llama layer that the Llama architecture list
# of the NTransformer page ("Key features": RoPE, GQA, SwiGLU, RMSNorm, KV cache) implies:
# which gain feeds which norm, gate vs up, RoPE on q and k (not v) before the cache write, the new
# token's K/V appended before it attends, and the final norm's gain in the head.

H_, NQ_, NKV_, HD_, F_ = 256, 2, 1, 128, 64
G_ATTN_, G_FFN_, G_FINAL_ = 0.5, 2.0, 3.0


def _q8(M):
    """Canonical Q8_0 bytes of an integer matrix with entries in [-127, 127] (d = 1.0)."""
    M = np.asarray(M, dtype=np.int64)
    rows, k = M.shape
    out = np.zeros((rows, k // 32, 34), np.uint8)
    out[:, :, 0:2] = [0x00, 0x3C]  # fp16 1.0
    out[:, :, 2:] = M.reshape(rows, k // 32, 32).astype(np.int8).view(np.uint8)
    return out.reshape(rows, -1)


def _u():
    i = np.arange(H_)
    return np.where((i * 7 + i // 3) % 5 < 2, -1.0, 1.0)


class _Layer:
    """One hand-built layer driven through orc_layer_forward, with its own fp16 caches."""

    def __init__(self, mats, max_ctx=16):
        import ctypes
        O = oracle.oracle
        zero = {2: (NQ_ * HD_, H_), 3: (NKV_ * HD_, H_), 4: (NKV_ * HD_, H_), 5: (H_, NQ_ * HD_),
                6: (F_, H_), 7: (F_, H_), 8: (H_, F_)}
        self.keep = []
        self.dims = O.Dims(1, H_, NQ_, NKV_, HD_, F_, 1000, max_ctx, 500000.0, 0.0)
        self.lay = O.Layer()
        for i, t in enumerate((2, 3, 4, 5, 6, 7, 8)):
            W = _q8(mats.get(t, np.zeros(zero[t], np.int64)))
            self.keep.append(W)
            self.lay.w[i] = W.ctypes.data
            self.lay.qt[i] = synth.Q8_0
        self.ga = np.full(H_, G_ATTN_, np.float32)
        self.gf = np.full(H_, G_FFN_, np.float32)
        self.lay.g_attn, self.lay.g_ffn = self.ga.ctypes.data, self.gf.ctypes.data
        self.kc = np.zeros((max_ctx, NKV_, HD_), np.uint16)
        self.vc = np.zeros_like(self.kc)
        self.lay.kc, self.lay.vc = self.kc.ctypes.data, self.vc.ctypes.data
        self.ctypes = ctypes

    def run(self, h, pos):
        out = np.ascontiguousarray(h, dtype=np.float64).copy()
        rc = oracle.oracle.lib().orc_layer_forward(self.ctypes.byref(self.dims), self.ctypes.byref(self.lay),
                                                   out.ctypes.data, pos)
        assert rc == 0
        return out


def _eye(rows, k, col0=0):
    M = np.zeros((rows, k), np.int64)
    M[np.arange(rows), col0 + np.arange(rows)] = 1
    return M


def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def test_layer_uniform_attention_is_mean_of_v_through_wo():
    """Wq = Wk = 0: every score is 0 and attention is the plain mean of V over positions 0..pos,
    including the new token's V = Wv n1 = g_attn * u[128:] (appended before attending); both query
    heads read the one KV head; Wo = I adds that mean into both halves of the residual; the zero FFN
    adds nothing."""
    L = _Layer({4: _eye(HD_, H_, 128), 5: _eye(H_, H_)})
    pos = 6
    prior = synth.normal_f16(synth.key(31, 1), pos * HD_).reshape(pos, 1, HD_)
    L.vc[:pos] = prior
    L.kc[:pos] = synth.normal_f16(synth.key(31, 2), pos * HD_).reshape(pos, 1, HD_)
    u = _u()
    out = L.run(u, pos)
    v_new = G_ATTN_ * u[128:]
    assert np.array_equal(L.vc[pos, 0], _f16(v_new))          # V row: no RoPE
    assert np.all(L.kc[pos, 0].view(np.float16) == 0)              # rope(0) = +-0
    mean = (prior.view(np.float16).astype(np.float64)[:, 0, :].sum(axis=0) + v_new) / (pos + 1)
    assert np.max(np.abs(out - (u + np.concatenate([mean, mean])))) < 1e-12


def test_layer_caches_rotated_k_and_unrotated_v():
    """Wk = [I 0], Wv = [0 I]: at position 0 the cached K row is g_attn * u[:128] exactly (RoPE is
    the identity there); at position 7 it is that row rotated (every pair keeps its norm, the row
    differs from the unrotated one) while the cached V row stays unrotated."""
    u = _u()
    for pos in (0, 7):
        L = _Layer({3: _eye(HD_, H_), 4: _eye(HD_, H_, 128)})
        L.run(u, pos)
        k = L.kc[pos, 0].view(np.float16).astype(np.float64)
        a = G_ATTN_ * u[:128]
        assert np.array_equal(L.vc[pos, 0], _f16(G_ATTN_ * u[128:]))
        if pos == 0:
            assert np.array_equal(L.kc[0, 0], _f16(a))
        else:
            pn = k[0::2] ** 2 + k[1::2] ** 2
            assert np.all(np.abs(pn - 0.5) < 2e-3)            # (0.5^2 + 0.5^2), fp16-rounded
            assert not np.array_equal(L.kc[pos, 0], _f16(a))
            assert np.array_equal(L.kc[pos, 0], _f16(oracle.rope(a, 1, HD_, pos, 500000.0)))


def test_layer_rotates_q_like_k():
    """Position 1, Wq = Wk = [I 0]: q and the new key are the same vector a rotated by the same angle,
    so their score is |a|^2 / sqrt(128) = 2.83 whatever the angle (up to the fp16 rounding of the
    cached key, below 1.5e-3); the prior key is 0 (score 0).  The output is (V0 + e^s V1) / (1 + e^s),
    in both halves of the residual through Wo = I.  A q left unrotated would score a . rope(a) =
    2.65 instead, moving the output by about 0.04."""
    L = _Layer({2: np.vstack([_eye(HD_, H_), _eye(HD_, H_)]), 3: _eye(HD_, H_), 4: _eye(HD_, H_, 128),
                5: _eye(H_, H_)})
    A = synth.normal_f16(synth.key(31, 3), HD_).reshape(1, 1, HD_)
    L.vc[0] = A[0]
    u = _u()
    out = L.run(u, 1)
    a = G_ATTN_ * u[:128]
    s = float(a @ a) / np.sqrt(HD_)
    v0 = A.view(np.float16).astype(np.float64)[0, 0]
    v1 = G_ATTN_ * u[128:]
    o = (v0 + np.exp(s) * v1) / (1.0 + np.exp(s))
    assert np.max(np.abs(out - (u + np.concatenate([o, o])))) < 2e-3


def test_layer_ffn_gate_up_down_and_ffn_gain():
    """Attention adds 0 (Wo = 0).  n2 = g_ffn * u; gate row 0 picks n2[a] = +2, up row 0 picks
    n2[b] = -2, down column 0 puts silu(gate) * up at output c:
    h[c] += silu(2) * (-2) = -4 / (1 + e^-2).  Swapping gate and up would give silu(-2) * 2, using
    g_attn would give silu(0.5) * (-0.5)."""
    u = _u()
    a = int(np.nonzero(u > 0)[0][0])
    b = int(np.nonzero(u < 0)[0][1])
    c = 77
    Wg = np.zeros((F_, H_), np.int64)
    Wu = np.zeros((F_, H_), np.int64)
    Wd = np.zeros((H_, F_), np.int64)
    Wg[0, a] = 1
    Wu[0, b] = 1
    Wd[c, 0] = 1
    L = _Layer({6: Wg, 7: Wu, 8: Wd})
    out = L.run(u, 3)
    want = u.copy()
    want[c] += -4.0 / (1.0 + np.exp(-2.0))
    assert np.max(np.abs(out - want)) < 1e-15


def test_head_uses_final_gain_and_step_wiring():
    """orc_head: logits = W_head (g_final * h / rms(h)); with rms(h) = 1 and eps = 0 and a one-hot
    head row v -> column v, logits[v] = g_final * u[v] = +-3 exactly.  orc_step on a model whose
    embedding row is u and whose layers are exact identities (Wo = W_down = 0) returns those logits
    and the first index of the largest (the first +1 of u)."""
    import ctypes
    O = oracle.oracle
    V = H_
    u = _u()
    head = _q8(_eye(V, H_))
    emb = np.zeros((V, H_), np.int64)
    tok = 5
    emb[tok] = u.astype(np.int64)
    embb = _q8(emb)
    gfin = np.full(H_, G_FINAL_, np.float32)
    L = _Layer({})  # all-zero matrices: an exact identity layer
    dims = O.Dims(1, H_, NQ_, NKV_, HD_, F_, V, 16, 500000.0, 0.0)
    m = O.Model()
    m.dims = dims
    m.layers = ctypes.cast(ctypes.pointer(L.lay), ctypes.POINTER(O.Layer))
    m.embed, m.qt_embed = embb.ctypes.data, synth.Q8_0
    m.head, m.qt_head = head.ctypes.data, synth.Q8_0
    m.g_final = gfin.ctypes.data
    logits = np.empty(V)
    assert O.lib().orc_head(ctypes.byref(m), u.ctypes.data, logits.ctypes.data) == 0
    assert np.array_equal(logits, G_FINAL_ * u)
    lg = np.empty(V)
    nxt = ctypes.c_int32(-1)
    assert O.lib().orc_step(ctypes.byref(m), tok, 2, 1, None, None, None, lg.ctypes.data, ctypes.byref(nxt)) == 0
    assert np.array_equal(lg, G_FINAL_ * u) and nxt.value == int(np.argmax(u))
