"""The C ABI without a GPU: the library loads, exports every function declared
in include/tos.h, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from tensorized_online_softmax_amd import binding as tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tos.h")

# distinct, 16-byte aligned fake device addresses: every call below returns
# before anything is launched or dereferenced
Q, K, V, O, L = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(tos_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(tb.EXPORTED), names
    lib = tb.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    # nm agrees (dynamic symbol table)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", tb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_helpers():
    assert tb.tos_version() == 1
    assert tb.tos_attn_fwd_flops(2, 32, 4096, 128, 1) == 4.0 * 2 * 32 * 4096 ** 2 * 128 / 2
    assert tb.tos_attn_fwd_flops(4, 16, 1024, 64, 0) == 4.0 * 4 * 16 * 1024 ** 2 * 64
    assert tb.tos_attn_fwd_flops(0, 16, 1024, 64, 0) == 0.0
    assert tb.tos_status_string(tb.TOS_OK) == "TOS_OK"
    assert tb.tos_status_string(tb.TOS_ERR_UNSUPPORTED) == "TOS_ERR_UNSUPPORTED"
    assert tb.tos_status_string(99) == "TOS_UNKNOWN_STATUS"
    op = tb.tos_fwd_opts_default()
    assert op.size == ctypes.sizeof(tb.tos_fwd_opts)
    assert (op.x_tile, op.softmax_split, op.fallback) == (32, 0, 0)
    assert (op.q_descale, op.k_descale, op.v_descale) == (1.0, 1.0, 1.0)
    assert tb.lib().tos_fwd_opts_default(None) == tb.TOS_ERR_INVALID_ARG


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=64, d=64, causal=0, scale=0.125,
         dtype=tb.TOS_BF16, opts=None):
    return tb.lib().tos_attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype,
                                 ctypes.byref(opts) if opts is not None else None, None)


def opts(**kw):
    op = tb.tos_fwd_opts_default()
    for key, val in kw.items():
        setattr(op, key, val)
    return op


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), tb.TOS_ERR_INVALID_ARG),
    (dict(k=None), tb.TOS_ERR_INVALID_ARG),
    (dict(v=None), tb.TOS_ERR_INVALID_ARG),
    (dict(o=None), tb.TOS_ERR_INVALID_ARG),
    (dict(B=-1), tb.TOS_ERR_INVALID_ARG),
    (dict(N=-5), tb.TOS_ERR_INVALID_ARG),
    (dict(scale=0.0), tb.TOS_ERR_INVALID_ARG),
    (dict(scale=-1.0), tb.TOS_ERR_INVALID_ARG),
    (dict(scale=float("nan")), tb.TOS_ERR_INVALID_ARG),
    (dict(scale=float("inf")), tb.TOS_ERR_INVALID_ARG),
    (dict(causal=2), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=7), tb.TOS_ERR_INVALID_ARG),
    (dict(o=Q), tb.TOS_ERR_INVALID_ARG),                    # output aliases q
    (dict(o=K + 64), tb.TOS_ERR_INVALID_ARG),               # output overlaps k
    (dict(lse=O + 128), tb.TOS_ERR_INVALID_ARG),            # lse inside o
    (dict(q=Q + 8), tb.TOS_ERR_INVALID_ARG),                # misaligned
    (dict(lse=L + 2), tb.TOS_ERR_INVALID_ARG),
    (dict(d=96), tb.TOS_ERR_UNSUPPORTED),
    (dict(d=256), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(size=4)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(x_tile=8)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(x_tile=128)), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=tb.TOS_F32, opts=opts(x_tile=64)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(x_tile=64)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(x_tile=64, softmax_split=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(x_tile=64, schedule=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=5)), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=tb.TOS_F32, opts=opts(softmax_split=2)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(softmax_split=2)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=2, x_tile=16)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=2, fallback=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=2, schedule=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(fallback=3)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(fallback_tau=-1.0)), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(q_descale=0.0)), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(v_descale=float("nan"))), tb.TOS_ERR_INVALID_ARG),
    (dict(dtype=tb.TOS_F32, opts=opts(softmax_split=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, d=96), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_F16, d=96), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(schedule=2)), tb.TOS_ERR_INVALID_ARG),
    # the sequential schedule: 16-bit inputs, VALU row sum, no AUTO, X = 1 or 32
    (dict(dtype=tb.TOS_F32, opts=opts(schedule=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(schedule=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(schedule=1, softmax_split=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(schedule=1, x_tile=16)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(schedule=1, fallback=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=4), tb.TOS_ERR_INVALID_ARG),
    (dict(B=70000, H=70000), tb.TOS_ERR_UNSUPPORTED),       # grid beyond 2^31
    # empty problems: nothing to do, and no pointer is needed
    (dict(B=0, q=None, k=None, v=None, o=None), tb.TOS_OK),
    (dict(H=0), tb.TOS_OK),
    (dict(N=0), tb.TOS_OK),
])
def test_validation(kw, status):
    assert call(**kw) == status
