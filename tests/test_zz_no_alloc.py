"""tos_attn_fwd_noalloc through the C ABI: two calls in a row, the second on a
smaller problem, each checked against tos_attn_fwd with a caller workspace
(same kernels and pieces: identical output) and against the fp64 oracle."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import assert_close, oracle_exact, to_device  # noqa: E402
from tensorized_online_softmax_amd import binding as tb  # noqa: E402
from tensorized_online_softmax_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(entry, dev, B, H, N, d, causal, scale, workspace):
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    op = tb.make_opts()
    if workspace is not None:
        op.workspace, op.workspace_bytes = workspace.data_ptr(), workspace.numel()
    rc = entry(dev["q"], dev["k"], dev["v"], o, lse, B, H, N, d, causal, scale, tb.TOS_BF16, op)
    assert rc == tb.TOS_OK, tb.tos_status_string(rc)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("shapes", [[(2, 4, 4096, 128, 1), (1, 2, 1000, 64, 1)],
                                    [(1, 3, 3000, 64, 0), (1, 1, 700, 128, 0)]])
def test_noalloc_matches_workspace_entry(shapes):
    for (B, H, N, d, causal) in shapes:          # the second call is the smaller one
        need = tb.tos_attn_fwd_workspace_size(B, H, N, d, causal, tb.TOS_BF16)
        assert need > 0                           # the pieces path, which uses the scratch
        print(f"[noalloc] B={B} H={H} N={N} d={d} causal={causal} workspace {need} B", flush=True)
        inp = inputs.make(B, H, N, d, "bf16", seed=800 + N + d)
        dev = to_device(inp)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ref_gpu, lse_ref_gpu = _run(tb.tos_attn_fwd, dev, B, H, N, d, causal, inp["scale"], ws)
        o, lse = _run(tb.tos_attn_fwd_noalloc, dev, B, H, N, d, causal, inp["scale"], None)
        assert torch.equal(o, o_ref_gpu) and torch.equal(lse, lse_ref_gpu)
        o_ref, lse_ref = oracle_exact(inp, bool(causal))
        assert_close(o.to(torch.float64).cpu().numpy().reshape(o_ref.shape), o_ref,
                     lse.to(torch.float64).cpu().numpy().reshape(lse_ref.shape), lse_ref, "bf16",
                     f"noalloc B={B} H={H} N={N} d={d} causal={causal}")


def test_noalloc_rejects_a_caller_workspace():
    B, H, N, d = 1, 1, 64, 64
    inp = inputs.make(B, H, N, d, "bf16", seed=5)
    dev = to_device(inp)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    op = tb.make_opts()
    op.workspace, op.workspace_bytes = ws.data_ptr(), ws.numel()
    rc = tb.tos_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], o, None, B, H, N, d, 0,
                                 inp["scale"], tb.TOS_BF16, op)
    assert rc == tb.TOS_ERR_INVALID_ARG
