"""fp64 CPU oracle for tiled online-softmax attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
library and is never a fallback for it.
"""
from .attention import (MOD_ALIBI, MOD_CHECKERBOARD, MOD_CUSTOM, MOD_NONE, as_f64, backward, decode,
                        default_alibi_slopes, forward, magnitudes, score_bias)

__all__ = ["MOD_NONE", "MOD_ALIBI", "MOD_CHECKERBOARD", "MOD_CUSTOM", "as_f64", "forward", "backward",
           "decode", "default_alibi_slopes", "magnitudes", "score_bias"]
