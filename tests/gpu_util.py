"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def gemv_ok(y, y_ref, a_ref):
    """The row bound |y - y_ref| <= 1e-4 * sum|w x| + 1e-6."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= 1e-4 * a_ref + 1e-6


def is_tie(logits_ref, i, j, rel=1e-4):
    """Two argmax candidates count as a tie when their gap is below rel * max|logits|."""
    L = np.asarray(logits_ref, dtype=np.float64)
    return abs(L[i] - L[j]) <= rel * np.max(np.abs(L))


def kv_rows_ok(gpu_bits, ref_bits, rel=2e-3):
    """Newly written fp16 K/V rows, element by element: |g - r| <= one fp16 step at r + rel * RMS of
    r's row (the stored value is the fp16 rounding of a value that carries the GEMV's error, which is
    bounded relative to the row's magnitude, not to each element).  Returns (ok mask, worst ratio)."""
    g = np.asarray(gpu_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    r = np.asarray(ref_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    step = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    bound = step + rel * rms
    err = np.abs(g - r)
    return err <= bound, float(np.max(err / bound))
