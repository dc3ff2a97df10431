"""The seeded input generator: deterministic, random-access, in range, fp16 correctly rounded."""
import os
import subprocess
import sys

import numpy as np
import pytest

import synth


def test_rows_are_random_access():
    d = synth.DEFAULT_DIST[synth.Q4_K]
    tk = synth.key(0, 42)
    full = synth.matrix(d, 1024, 40, tkey=tk)
    part = synth.matrix(d, 1024, 40, 13, 9, tkey=tk)
    assert np.array_equal(full[13:22], part)


def test_independent_of_thread_count():
    code = ("import synth,hashlib;w=synth.LLAMA8B_Q8_0.weight(3,synth.WO,0,64);"
            "print(hashlib.sha256(w.tobytes()).hexdigest())")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for t in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=t, PYTHONPATH=root)
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env, cwd=root).strip())
    assert outs[0] == outs[1]


@pytest.mark.parametrize("qt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q5_K, synth.Q6_K])
def test_field_ranges(qt):
    d = synth.DEFAULT_DIST[qt]
    B = synth.BLOCK_WEIGHTS[qt]
    tk = synth.key(0, 77)
    qs, scs = [], []
    for b in range(64):
        f = synth.block_fields(d, 64 * B, 0, b, tkey=tk)
        qs.append(f["q"])
        scs.append(f["sc"][: (16 if qt == synth.Q6_K else 8)])
    q = np.concatenate(qs)
    assert q.min() == d.q[0] and q.max() == d.q[1]
    if qt in (synth.Q4_K, synth.Q5_K, synth.Q6_K):
        sc = np.concatenate(scs)
        assert sc.min() == d.sc[0] and sc.max() == d.sc[1]


def test_f16_matches_numpy_rounding():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.normal(size=2000) * 10.0 ** rng.integers(-9, 6, size=2000),
                           [65504.0, 65519.9, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, -0.0, 0.0]])
    ours = np.array([synth.f16_bits(v) for v in vals], dtype=np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normals_look_standard():
    x = synth.normal_f32(synth.key(0, 9), 200000).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
