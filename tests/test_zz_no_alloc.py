"""The allocation-free GEMV entry point (qwg_gemv_noalloc) against qwg_gemv with a caller work buffer
(GPU only): two calls in a row, the second smaller, each bitwise equal to the existing entry point
(same kernels) and within the oracle's row bound; a shape whose scratch exceeds the static array is
refused before anything runs."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import gemv_ok

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_gemv_noalloc_equals_gemv_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_weight_streaming_gemv_amd import QwgError, ops
    # the first call needs K-split partial sums (8 columns over K = 8192) as well as digits; the
    # second is smaller, so the static array still holds the first call's larger contents
    cases = [(synth.Q4_K, 4096, 8192, 8), (synth.Q6_K, 300, 2048, 1)]
    for i, (qt, rows, k, nc) in enumerate(cases):
        assert ops.gemv_work_bytes(qt, rows, k, nc) <= ops.NOALLOC_SCRATCH_BYTES
        W = synth.matrix(synth.DEFAULT_DIST[qt], k, rows, tkey=synth.key(41, i))
        x = synth.normal_f32(synth.key(41, 10 + i), nc * k).reshape(nc, k)
        P = ops.repack(qt, torch.from_numpy(W).to(DEV), rows, k)
        dx = torch.from_numpy(x).to(DEV)
        want = ops.gemv(qt, P, rows, k, dx)
        out = torch.full((nc, rows), float("nan"), dtype=torch.float32, device=DEV)
        ops.gemv_noalloc(qt, P, rows, k, dx, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.cpu().numpy().reshape(nc, rows).view(np.uint32)), i
        yr, ar = oracle.gemv(qt, W, rows, k, x)
        assert gemv_ok(got, yr, ar).all(), i
    # 8 columns over K = 65536 and 50000 rows: 16 K splits of partial sums, beyond 16 MiB
    qt, rows, k, nc = synth.Q4_K, 50000, 65536, 8
    assert ops.gemv_work_bytes(qt, rows, k, nc) > ops.NOALLOC_SCRATCH_BYTES
    small = torch.zeros(4096, dtype=torch.float32, device=DEV)
    xs = torch.zeros((nc, k), dtype=torch.float32, device=DEV)
    with pytest.raises(QwgError) as e:
        ops.gemv_noalloc(qt, small, rows, k, xs, small)
    assert e.value.code == -3 and "static scratch" in str(e.value)
