"""fp64 CPU oracle for the fused attention forward pass and the tensorized
online softmax (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU path.
Every function here is a thin ctypes marshaller around ``oracle.c``; the
arithmetic lives there, in plain loops that follow the FlashAttention-T page
(sections A2 and A3, Fig 2(a), Algorithm 1).
"""
from .oracle import (Oracle, attn_exact, attn_surrogate, round_bf16, round_e4m3,  # noqa: F401
                     round_f16, max_threads, FALLBACK_OFF, FALLBACK_AUTO, FALLBACK_FORCE,
                     P_EXACT, P_BF16, P_E4M3, P_F16)
