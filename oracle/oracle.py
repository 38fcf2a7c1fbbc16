"""ctypes binding of the fp64 oracle (test infrastructure only; see oracle.c).

Arrays are numpy float64, shaped [BH, N, d] (or [B, H, N, d], which is folded to
[B*H, N, d]).  The functions only marshal arguments; all arithmetic is in C.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FALLBACK_OFF, FALLBACK_AUTO, FALLBACK_FORCE = 0, 1, 2
P_EXACT, P_BF16, P_E4M3, P_F16 = 0, 1, 2, 3

_default = None


def _bind(path):
    """Load one build of oracle.c and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64 = ctypes.c_int64
    lib.oracle_attn_exact.argtypes = [dp, dp, dp, i64, i64, i64, ctypes.c_int,
                                      ctypes.c_double, i64p, i64, dp, dp, ctypes.c_int]
    lib.oracle_attn_exact.restype = ctypes.c_int
    lib.oracle_attn_surrogate.argtypes = [dp, dp, dp, i64, i64, i64, ctypes.c_int,
                                          ctypes.c_double, i64, i64, i64p,
                                          ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                          ctypes.c_int, dp, dp, dp, dp, u8p, i64p,
                                          ctypes.c_int]
    lib.oracle_attn_surrogate.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_round_e4m3.argtypes = [ctypes.c_double]
    lib.oracle_round_e4m3.restype = ctypes.c_double
    lib.oracle_round_f16.argtypes = [ctypes.c_double]
    lib.oracle_round_f16.restype = ctypes.c_double
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_abi_version.restype = ctypes.c_int
    return lib


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = _bind(_build.LIB)
    return _default


class Oracle:
    """The same functions, bound to a given build of oracle.c (default: liboracle.so)."""

    def __init__(self, path=None):
        self._lib = _bind(path) if path else _load()

    def attn_exact(self, *a, **kw):
        return attn_exact(*a, _lib=self._lib, **kw)

    def attn_surrogate(self, *a, **kw):
        return attn_surrogate(*a, _lib=self._lib, **kw)

    def round_bf16(self, x):
        return round_bf16(x, _lib=self._lib)

    def round_e4m3(self, x):
        return round_e4m3(x, _lib=self._lib)

    def round_f16(self, x):
        return round_f16(x, _lib=self._lib)


def _ptr(a, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


def _fold(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    if x.ndim == 4:
        x = x.reshape(x.shape[0] * x.shape[1], x.shape[2], x.shape[3])
    if x.ndim != 3:
        raise ValueError("expected [BH, N, d] or [B, H, N, d]")
    return x


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def attn_exact(q, k, v, causal, scale, rows=None, threads=0, _lib=None):
    """Exact attention (the plain definition) in fp64.

    Returns (o, lse): o [BH, N, d] and lse [BH, N] when rows is None, else
    o [len(rows), d] and lse [len(rows)] for the flat rows bh*N + i.
    """
    lib = _lib or _load()
    q, k, v = _fold(q), _fold(k), _fold(v)
    BH, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if rows is None:
        o = np.empty((BH, N, d))
        lse = np.empty((BH, N))
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, d))
        lse = np.empty(rows.size)
        rp, nr = _ptr(rows, ctypes.c_int64), rows.size
    rc = lib.oracle_attn_exact(_ptr(q), _ptr(k), _ptr(v), BH, N, d, int(bool(causal)),
                               float(scale), rp, nr, _ptr(o), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_exact failed ({rc})")
    return o, lse


def attn_surrogate(q, k, v, causal, scale, X, Bc, order=None, fallback=FALLBACK_OFF,
                   tau=100.0, p_round=P_EXACT, p_shift=0, threads=0, _lib=None):
    """Algorithm 1 (surrogate-max online softmax) in fp64, block by block.

    Returns a dict with o [BH,N,d], lse [BH,N], ref [BH,N] (final reference max per
    row, raw dot-product units), gap [BH,N] (largest c*(m^ - m_i) seen),
    switched [BH, ceil(N/X)] and the invariant counters.
    """
    lib = _lib or _load()
    q, k, v = _fold(q), _fold(k), _fold(v)
    BH, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    ntile = (N + X - 1) // X if X > 0 else 0
    o = np.empty((BH, N, d))
    lse = np.empty((BH, N))
    ref = np.empty((BH, N))
    gap = np.empty((BH, N))
    sw = np.zeros((BH, max(ntile, 0)), dtype=np.uint8)
    cnt = np.zeros(4, dtype=np.int64)
    op = None
    if order is not None:
        order = np.ascontiguousarray(order, dtype=np.int64)
        op = _ptr(order, ctypes.c_int64)
    rc = lib.oracle_attn_surrogate(_ptr(q), _ptr(k), _ptr(v), BH, N, d, int(bool(causal)),
                                   float(scale), int(X), int(Bc), op, int(fallback),
                                   float(tau), int(p_round), int(p_shift), _ptr(o), _ptr(lse),
                                   _ptr(ref), _ptr(gap), _ptr(sw, ctypes.c_uint8),
                                   _ptr(cnt, ctypes.c_int64), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_surrogate failed ({rc})")
    return {"o": o, "lse": lse, "ref": ref, "gap": gap, "switched": sw,
            "n_mhat_below_m": int(cnt[0]), "n_z_positive": int(cnt[1]),
            "n_nonfinite_rows": int(cnt[2]), "n_tiles_per_row": int(cnt[3])}


def round_bf16(x, _lib=None):
    f = (_lib or _load()).oracle_round_bf16
    return np.vectorize(lambda t: f(float(t)), otypes=[np.float64])(x)


def round_e4m3(x, _lib=None):
    f = (_lib or _load()).oracle_round_e4m3
    return np.vectorize(lambda t: f(float(t)), otypes=[np.float64])(x)


def round_f16(x, _lib=None):
    f = (_lib or _load()).oracle_round_f16
    return np.vectorize(lambda t: f(float(t)), otypes=[np.float64])(x)
