"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the fp64 oracle on the same stored inputs, compare element by element."""
import math

import numpy as np
import torch

import oracle
from tensorized_online_softmax_amd import binding as tb
from tensorized_online_softmax_amd import inputs

# tolerances on O vs the exact fp64 oracle, per input dtype (max abs, mean abs).
# bf16's 1e-2 is about 5 units of its rounding (2^-9); fp16 takes the same 5
# units of its own (5 * 2^-11), and the mean a tenth of the max throughout.
TOL_O = {"f32": (1e-4, 1e-5), "bf16": (1e-2, 1e-3), "f16": (5 * 2.0 ** -11, 0.5 * 2.0 ** -11),
         "fp8": (6e-2, 6e-3)}
TOL_LSE_REL = 1e-3          # |dlse| <= 1e-3 * max(1, |lse|)


def to_device(inp):
    return {n: inp[n].cuda() for n in ("q", "k", "v")}


def run_gpu(inp, causal, x_tile=32, split="valu", fallback="off", tau=0.0, counter=False,
            dev=None):
    """Run the HIP kernels; returns (o float64 numpy, lse float64 numpy, tiles)."""
    dev = dev or to_device(inp)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda") if counter else None
    o, lse = tb.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=inp["scale"],
                         dtype=inp["dtype"], x_tile=x_tile, split=split, fallback=fallback,
                         tau=tau, descale=inp["descale"] if inp["dtype"] == "fp8" else None,
                         fallback_tiles=cnt)
    torch.cuda.synchronize()
    tiles = int(cnt.item()) if counter else None
    return (o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy(), tiles)


def real_inputs(inp):
    d = inp["descale"]
    return (inputs.real_values(inp["q"], d["q"]), inputs.real_values(inp["k"], d["k"]),
            inputs.real_values(inp["v"], d["v"]))


def oracle_exact(inp, causal, rows=None):
    q, k, v = real_inputs(inp)
    return oracle.attn_exact(q, k, v, causal, inp["scale"], rows=rows)


def errors(o, o_ref, lse, lse_ref):
    e = np.abs(o - o_ref)
    el = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    return float(e.max()), float(e.mean()), float(el.max())


def storage_ulp(x, dtype):
    """Spacing of the output type's numbers at |x|: bf16 (8 significant bits)
    or fp16 (11 significant bits, subnormal spacing 2^-24)."""
    ax = np.abs(x)
    if dtype == "f16":
        return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -14))) - 10)
    return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -126))) - 7)


def round_to_output(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float16 if dtype == "f16" else torch.bfloat16).double().numpy()


def assert_close(o, o_ref, lse, lse_ref, dtype, what="", storage_ulp_rule=True, **_):
    """Max and mean abs error of O within TOL_O[dtype], lse within 1e-3 relative.

    16-bit outputs (bf16 for bf16 and fp8 inputs, fp16 for fp16): an element whose
    error exceeds the max bound still passes when it is within one unit of the
    output type of the oracle value rounded to that type -- storing |O| >= 2 in
    bf16 alone can be off by 2^-8 (half its spacing there), beyond 1e-2 once the
    computation's own error is added, so the bound cannot be met element by
    element in early causal rows, which average only a few values of V.
    """
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    mx, mean, lrel = errors(o, o_ref, lse, lse_ref)
    tmax, tmean = TOL_O[dtype]
    if storage_ulp_rule and dtype != "f32" and mx > tmax:
        out = "f16" if dtype == "f16" else "bf16"
        ref16 = round_to_output(o_ref, out)
        bad = (np.abs(o - o_ref) > tmax) & (np.abs(o - ref16) > storage_ulp(ref16, out))
        assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {tmax} and 1 {out} unit "
                               f"(max {mx:.3e})")
    else:
        assert mx <= tmax, f"{what}: O max {mx:.3e} (tol {tmax})"
    assert mean <= tmean, f"{what}: O mean {mean:.3e} (tol {tmean})"
    assert lrel <= TOL_LSE_REL, f"{what}: lse rel err {lrel:.3e}"
    return mx, mean, lrel
