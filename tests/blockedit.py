"""Edits of canonical block bytes for building special test inputs (no arithmetic of the method).

`zero_columns` rewrites matrix columns so that every weight in them dequantizes to exactly zero,
following the canonical GGUF block layouts (the K-quants also get dmin = 0 in the touched blocks,
since their zero needs d*sc*q = dmin*m).  Tests confirm the result with the oracle's own decoder
before using it, so a mistake here shows up as a failed precondition, not as a false parity."""
import numpy as np

import synth


def _set_nibble(byte_arr, idx, hi, val):
    b = int(byte_arr[idx])
    byte_arr[idx] = ((b & 0x0F) | (val << 4)) if hi else ((b & 0xF0) | val)


def zero_columns(qtype: int, W: np.ndarray, rows: int, k: int, cols) -> np.ndarray:
    """A copy of canonical matrix W (rows x row_bytes) with weight columns `cols` set to zero."""
    B, S = synth.BLOCK_WEIGHTS[qtype], synth.BLOCK_BYTES[qtype]
    out = np.array(W, dtype=np.uint8, copy=True).reshape(rows, (k // B) * S)
    for r in range(rows):
        row = out[r]
        for c in cols:
            blk = row[(c // B) * S:(c // B + 1) * S]
            i = c % B
            if qtype == synth.Q8_0:
                blk[2 + i] = 0
            elif qtype == synth.Q4_0:
                _set_nibble(blk, 2 + (i % 16), i >= 16, 8)
            elif qtype in (synth.Q4_K, synth.Q5_K):
                blk[2] = blk[3] = 0  # dmin = +0
                qs = 16 if qtype == synth.Q4_K else 48
                g, t = i // 64, i % 64
                _set_nibble(blk, qs + 32 * g + (t % 32), t >= 32, 0)
                if qtype == synth.Q5_K:
                    bit = 2 * g + (1 if t >= 32 else 0)
                    blk[16 + (t % 32)] &= ~(1 << bit) & 0xFF
            elif qtype == synth.Q6_K:
                n, rr = i // 128, i % 128
                u, l = rr // 32, rr % 32
                _set_nibble(blk, 64 * n + l + 32 * (u & 1), u >= 2, 0)
                q = int(blk[128 + 32 * n + l])
                blk[128 + 32 * n + l] = (q & ~(3 << (2 * u)) | (2 << (2 * u))) & 0xFF  # q = 32: weight 0
            else:
                raise ValueError(qtype)
    return out
