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
    assert tb.tos_version() == 2
    assert tb.tos_attn_fwd_flops(2, 32, 4096, 128, 1) == 4.0 * 2 * 32 * 4096 ** 2 * 128 / 2
    assert tb.tos_attn_fwd_flops(4, 16, 1024, 64, 0) == 4.0 * 4 * 16 * 1024 ** 2 * 64
    assert tb.tos_attn_fwd_flops(0, 16, 1024, 64, 0) == 0.0
    assert tb.tos_status_string(tb.TOS_OK) == "TOS_OK"
    assert tb.tos_status_string(tb.TOS_ERR_UNSUPPORTED) == "TOS_ERR_UNSUPPORTED"
    assert tb.tos_status_string(tb.TOS_ERR_SCRATCH) == "TOS_ERR_SCRATCH"
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
    # tau above 126: the switch's rescale by up to 2^tau would overflow fp32
    (dict(opts=opts(fallback=1, fallback_tau=127.0)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(fallback=1, fallback_tau=float("inf"))), tb.TOS_ERR_INVALID_ARG),
    # split values and shares
    (dict(opts=opts(softmax_split=6)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=-1)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=1, split_num=3, split_den=2)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=1, split_num=1, split_den=0)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=1, split_num=-1, split_den=4)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=0, split_num=1, split_den=2)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(softmax_split=1, split_num=1, split_den=3)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=3)), tb.TOS_ERR_UNSUPPORTED),          # HSPLIT needs a share
    (dict(opts=opts(softmax_split=3, split_num=1, split_den=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=4, split_num=1, split_den=4)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=1, split_num=1, split_den=2, x_tile=16)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=1, split_num=1, split_den=2, fallback=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=3, split_num=1, split_den=2, fallback=2)), tb.TOS_ERR_UNSUPPORTED),
    (dict(opts=opts(softmax_split=5, schedule=1)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_F32, opts=opts(softmax_split=5)), tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(softmax_split=3, split_num=1, split_den=2)),
     tb.TOS_ERR_UNSUPPORTED),
    (dict(dtype=tb.TOS_FP8_E4M3, opts=opts(softmax_split=1, split_num=1, split_den=2)),
     tb.TOS_ERR_UNSUPPORTED),
    (dict(B=70000, H=70000), tb.TOS_ERR_UNSUPPORTED),       # grid beyond 2^31
    # empty problems: nothing to do, and no pointer is needed
    # a workspace size with no workspace, a misaligned or overlapping workspace
    (dict(opts=opts(workspace_bytes=64)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(workspace=0x600008, workspace_bytes=64)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(workspace=Q + 64, workspace_bytes=64)), tb.TOS_ERR_INVALID_ARG),
    (dict(opts=opts(workspace=O, workspace_bytes=64)), tb.TOS_ERR_INVALID_ARG),
    (dict(B=0, q=None, k=None, v=None, o=None), tb.TOS_OK),
    (dict(H=0), tb.TOS_OK),
    (dict(N=0), tb.TOS_OK),
])
def test_validation(kw, status):
    assert call(**kw) == status


# ---- the Python binding's tensor checks (CPU tensors: every check below fires
# before the library is called)

def _t(shape=(1, 2, 8, 64), dtype=None, **kw):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16, **kw)


def test_binding_rejects_bad_tensors():
    import torch
    q = _t()
    good = dict(q=q, k=_t(), v=_t())
    with pytest.raises(ValueError, match="4-D"):
        tb.check_tensors(_t((2, 8, 64)), _t(), _t())
    with pytest.raises(ValueError, match="shapes differ"):
        tb.check_tensors(q, _t((1, 2, 9, 64)), _t())
    with pytest.raises(ValueError, match="needs"):
        tb.check_tensors(q, _t(), _t(), dtype="f32")            # bf16 data, f32 named
    with pytest.raises(ValueError, match="needs"):
        tb.check_tensors(q, _t(dtype=torch.float16), _t())      # mixed input dtypes
    with pytest.raises(ValueError, match="contiguous"):
        tb.check_tensors(_t((1, 8, 2, 64)).transpose(1, 2), _t(), _t())
    with pytest.raises(ValueError, match="out must be"):
        tb.check_tensors(**good, out=_t((1, 2, 8, 32)))          # undersized out
    with pytest.raises(ValueError, match="out must be"):
        tb.check_tensors(**good, out=_t(dtype=torch.float32))   # wrong O dtype
    with pytest.raises(ValueError, match="lse must be"):
        tb.check_tensors(**good, lse=torch.zeros(1, 2, 7))
    with pytest.raises(ValueError, match="lse must be"):
        tb.check_tensors(**good, lse=torch.zeros(1, 2, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="fallback_tiles"):
        tb.check_tensors(**good, fallback_tiles=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="unsupported input dtype"):
        tb.check_tensors(_t(dtype=torch.float64), _t(dtype=torch.float64), _t(dtype=torch.float64))
    # everything well formed but on the CPU: rejected as not being on the GPU
    with pytest.raises(ValueError, match="CUDA"):
        tb.check_tensors(**good, out=_t(), lse=torch.zeros(1, 2, 8))
    # attn_fwd runs the same checks before it allocates or launches
    with pytest.raises(ValueError, match="needs"):
        tb.attn_fwd(q, _t(), _t(), dtype="f16")
    with pytest.raises(ValueError, match="CUDA"):
        tb.attn_fwd(q, _t(), _t())


def test_workspace_size():
    """Pieces only where query blocks are fewer than compute units (256 when no
    device is visible), 16-bit inputs and the fallback off; at most 256 units of
    256 rows x (2d + 8) bytes (fp16 O, then lse and the row scale's exponent)."""
    ws = tb.tos_attn_fwd_workspace_size
    cap = 256 * 256 * (2 * 128 + 8)
    assert ws(2, 4, 4096, 128, 1, tb.TOS_BF16) == cap      # one GPU's share of 8: 128 blocks
    assert ws(2, 32, 4096, 128, 1, tb.TOS_BF16) == 0       # 1024 query blocks
    assert ws(4, 16, 1024, 64, 0, tb.TOS_BF16) == 0        # 256 query blocks
    assert 0 < ws(1, 4, 1000, 64, 1, tb.TOS_F16) <= 256 * 256 * (2 * 64 + 8)
    assert ws(1, 1, 128, 64, 0, tb.TOS_BF16) == 0          # 2 key blocks: nothing to cut
    assert ws(1, 2, 4096, 128, 0, tb.TOS_F32) == 0
    assert ws(1, 2, 4096, 128, 0, tb.TOS_FP8_E4M3, opts(q_descale=1.0)) == 0
    assert ws(1, 2, 4096, 128, 0, tb.TOS_BF16, opts(fallback=1)) == 0
    assert ws(0, 2, 4096, 128, 0, tb.TOS_BF16) == 0
    with pytest.raises(tb.TosError):
        ws(1, 2, 4096, 96, 0, tb.TOS_BF16)
    with pytest.raises(tb.TosError):
        ws(1, 2, 4096, 128, 0, tb.TOS_BF16, opts(x_tile=8))
    assert tb.lib().tos_attn_fwd_workspace_size(1, 1, 64, 64, 0, 1, None, None) == tb.TOS_ERR_INVALID_ARG
