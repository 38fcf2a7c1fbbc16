"""libtos.so through its C ABI alone: tests/c_abi/attn_fwd_c.c (gcc, the HIP
runtime's C API, no Python binding and no torch in that process) draws seeded
inputs, calls tos_attn_fwd and writes inputs and outputs to a file; the fp64
oracle checks the outputs against the stored inputs."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import TOL_LSE_REL, TOL_O  # noqa: E402
import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "attn_fwd_c")
_DT = {0: ("f32", np.float32, 4), 1: ("bf16", torch.bfloat16, 2), 3: ("f16", np.float16, 2)}


def test_c_program_builds():
    """The C consumer compiles against include/tos.h and links libtos.so (CPU)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("tos_c_abi_build",
                                                  os.path.join(HERE, "c_abi", "build.py"))
    c_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(c_build)
    assert os.path.exists(c_build.build())


def _decode(buf, dt, n):
    name, typ, esz = _DT[dt]
    raw = np.frombuffer(buf, dtype=np.uint8, count=n * esz)
    if name == "bf16":
        return torch.from_numpy(raw.copy()).view(torch.bfloat16).to(torch.float64).numpy()
    return raw.view(typ).astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,N,d,causal,dtype", [
    (1, 3, 300, 128, 1, 1),
    (2, 2, 130, 64, 0, 3),
    (1, 2, 100, 64, 0, 0),
    (2, 150, 260, 128, 1, 1),   # more query blocks than compute units
])
def test_c_abi_call(tmp_path, B, H, N, d, causal, dtype):
    assert os.path.exists(EXE), "build tests/c_abi/attn_fwd_c first (__graft_entry__.build())"
    out = tmp_path / "out.bin"
    r = subprocess.run([EXE, str(B), str(H), str(N), str(d), str(causal), str(dtype), "77",
                        str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    blob = out.read_bytes()
    hdr = np.frombuffer(blob[:48], dtype=np.int64)
    assert list(hdr) == [B, H, N, d, causal, dtype]
    esz = _DT[dtype][2]
    n = B * H * N * d
    off = 48
    arrs = []
    for _ in range(4):
        arrs.append(_decode(blob[off:off + n * esz], dtype, n).reshape(B * H, N, d))
        off += n * esz
    q, k, v, o = arrs
    lse = np.frombuffer(blob[off:off + 4 * B * H * N], dtype=np.float32).astype(np.float64)
    assert off + 4 * B * H * N == len(blob)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))   # the program's float32 scale
    o_ref, lse_ref = oracle.attn_exact(q, k, v, bool(causal), scale)
    tmax, tmean = TOL_O[_DT[dtype][0]]
    err = np.abs(o - o_ref.reshape(o.shape))
    assert err.max() <= tmax and err.mean() <= tmean, (err.max(), err.mean())
    lerr = np.abs(lse - lse_ref.reshape(-1)) / np.maximum(1.0, np.abs(lse_ref.reshape(-1)))
    assert lerr.max() <= TOL_LSE_REL, lerr.max()
