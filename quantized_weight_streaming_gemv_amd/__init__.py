"""MI355X (gfx950) decode hot path of a layer-streaming Llama engine with block-quantized weights.

The compute lives in libqwg.so (hand-written HIP kernels behind the C ABI in include/qwg.h);
this package is its thin ctypes binding.  Import is cheap: the library is loaded on first use
and every entry point raises if it is missing (there is no CPU fallback)."""
from ._lib import (LIB_PATH, NORM_ATTN, NORM_FFN, NORM_FINAL, Q4_0, Q4_K, Q5_K, Q6_K, Q8_0, T_EMBED, T_HEAD, T_WDOWN,
                   T_WGATE, T_WK, T_WO, T_WQ, T_WUP, T_WV, QwgError, lib)

__all__ = ["LIB_PATH", "lib", "QwgError", "Q4_0", "Q8_0", "Q4_K", "Q5_K", "Q6_K"]
