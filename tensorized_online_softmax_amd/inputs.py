"""Seeded synthetic inputs for the attention forward pass.

This module only draws and stores inputs; it holds none of the method's
arithmetic, and both the GPU path's tests and the CPU oracle take their inputs
from it.

Recipe (shared by every workload):
  * numpy ``default_rng(seed)`` (PCG64) draws float32 N(0, 1) values on the host,
    in [B, H, N, d] order, one generator per tensor (seed + 1 for Q, + 2 for K,
    + 3 for V, + 4 for the spike placement);
  * bf16 and fp16 storage: a round-to-nearest-even cast of those float32 values;
  * fp8 storage (OCP e4m3fn): per-tensor descale s = amax / 448, values x / s
    clamped to [-448, 448] and cast with round-to-nearest-even; the real value of
    a stored code c is s * c.

The workloads reproduce the shapes the FlashAttention-T page evaluates
(section A4: sequence lengths 512 to 8k, head dims 64 and 128, FP16/FP8
inputs with FP32 accumulation; Fig 11's outlier-variance stress data) at the
sizes used for this implementation's own measurements.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

DTYPES = ("f32", "bf16", "f16", "fp8")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" | "bf16" | "f16" | "fp8"
    causal: bool
    x_tile: int           # surrogate tile rows X
    seed: int             # base seed: Q = seed+1, K = seed+2, V = seed+3, spikes = seed+4
    std: float = 1.0      # standard deviation of the Q and K draws
    spike_frac: float = 0.0     # fraction of query rows that get one spiked key
    spike_logit: float = 0.0    # logit offset (in scaled units) of the spiked key
    fallback: str = "off"       # all-underflow fallback the workload runs with
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def exps(self) -> float:
        """Exponentials of the algorithm: one per (query, key) element, halved
        when causal (the diagonal elements aside)."""
        e = float(self.B * self.H * self.N * self.N)
        return e / 2 if self.causal else e


WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 128, 64, "f32", False, 16, 1000,
                                note="single head, fp32, non-causal, X=16"),
    "mha_bf16": Workload("mha_bf16", 4, 16, 1024, 64, "bf16", False, 32, 2000,
                         note="multi-head, bf16, d=64, non-causal"),
    "causal_bf16": Workload("causal_bf16", 2, 32, 4096, 128, "bf16", True, 32, 3000,
                            note="causal, bf16, d=128, N=4096"),
    "long_causal_bf16": Workload("long_causal_bf16", 1, 16, 16384, 128, "bf16", True, 32, 4000,
                                 note="long-sequence causal, bf16, d=128, N=16384"),
    # one GPU's share of the causal workload on an 8-GPU node sharded by heads
    # (no exchange between GPUs): 4 of the 32 heads
    "causal_bf16_shard8": Workload("causal_bf16_shard8", 2, 4, 4096, 128, "bf16", True, 32, 3000,
                                   note="causal bf16 N=4096 d=128, one GPU's share of 8 (H=4)"),
    "causal_f16": Workload("causal_f16", 2, 32, 4096, 128, "f16", True, 32, 3000,
                           note="causal, fp16, d=128, N=4096"),
    "fp8_spiky": Workload("fp8_spiky", 1, 16, 8192, 128, "fp8", False, 32, 5000,
                          std=math.sqrt(8.0), spike_frac=0.2, spike_logit=40.0, fallback="auto",
                          note="fp8 e4m3 stress: logit std 8, 20% of rows with one +40 key"),
}


def _normal(seed, shape, std=1.0):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _spike(q, k, scale, frac, logit, seed):
    """Raise one scaled logit per chosen row by exactly `logit`.

    For each head, floor(frac*N) distinct rows i are drawn, each with one key j*;
    q_i += (logit/scale) * k_j* / |k_j*|^2 in float64, so that
    scale*<q_i, k_j*> grows by `logit` (before quantisation).
    """
    if frac <= 0.0:
        return q
    B, H, N, d = q.shape
    rng = np.random.default_rng(seed)
    q = q.astype(np.float64)
    kk = k.astype(np.float64)
    nrow = int(math.floor(frac * N))
    for b in range(B):
        for h in range(H):
            rows = rng.choice(N, size=nrow, replace=False)
            keys = rng.integers(0, N, size=nrow)
            kv = kk[b, h, keys]                                   # [nrow, d]
            q[b, h, rows] += (logit / scale) * kv / np.sum(kv * kv, axis=1, keepdims=True)
    return q.astype(np.float32)


def to_fp8(x: np.ndarray):
    """Per-tensor e4m3 storage: returns (codes as torch.float8_e4m3fn, descale)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = amax / 448.0 if amax > 0 else 1.0
    y = np.clip(x.astype(np.float64) / s, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn), float(np.float32(s))


# The FlashAttention-T page's benchmark grid (section A4, "experimental
# setup"): 16k tokens in total and a hidden size of 2048 at every sequence
# length, so B = 16384 / N and H = 2048 / d.
GRID_TOKENS = 16384
GRID_HIDDEN = 2048
GRID_N = (512, 1024, 2048, 4096, 8192)
GRID_D = (64, 128)


def grid_workload(N, d, dtype, causal, x_tile=32, seed=6000):
    """One point of the page's grid as a Workload (named grid_<dtype>_<c|nc>_N<N>_d<d>)."""
    if GRID_TOKENS % N or GRID_HIDDEN % d:
        raise ValueError("N must divide 16384 and d must divide 2048")
    name = f"grid_{dtype}_{'c' if causal else 'nc'}_N{N}_d{d}"
    return Workload(name, GRID_TOKENS // N, GRID_HIDDEN // d, N, d, dtype, bool(causal), x_tile,
                    seed + N + d, note="16k tokens, hidden 2048")


def grid(dtypes=("bf16", "f16", "fp8"), causal=(False, True)):
    """Every point of the page's grid, for the given dtypes."""
    out = []
    for dt in dtypes:
        for c in causal:
            for d in GRID_D:
                for n in GRID_N:
                    out.append(grid_workload(n, d, dt, c))
    return out


def make(B, H, N, d, dtype, seed, std=1.0, spike_frac=0.0, spike_logit=0.0, scale=None):
    """Draw Q, K, V for one problem.

    Returns a dict: q, k, v (CPU torch tensors in the storage dtype, [B,H,N,d]),
    descale (dict of per-tensor fp32 descales; 1.0 unless fp8), dtype, scale.
    """
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = (B, H, N, d)
    q = _normal(seed + 1, shape, std)
    k = _normal(seed + 2, shape, std)
    v = _normal(seed + 3, shape)
    q = _spike(q, k, scale, spike_frac, spike_logit, seed + 4)
    descale = {"q": 1.0, "k": 1.0, "v": 1.0}
    if dtype == "f32":
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    elif dtype in ("bf16", "f16"):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)).to(tdt) for a in (q, k, v))
    else:
        (tq, sq), (tk, sk), (tv, sv) = to_fp8(q), to_fp8(k), to_fp8(v)
        descale = {"q": sq, "k": sk, "v": sv}
    return {"q": tq, "k": tk, "v": tv, "descale": descale, "dtype": dtype, "scale": scale}


def make_workload(w: Workload):
    return make(w.B, w.H, w.N, w.d, w.dtype, w.seed, std=w.std,
                spike_frac=w.spike_frac, spike_logit=w.spike_logit, scale=w.scale)


def real_values(t: torch.Tensor, descale: float = 1.0) -> np.ndarray:
    """The exact real values a stored tensor represents, as float64 numpy."""
    x = t.detach().to("cpu").to(torch.float64).numpy()
    return x * descale if descale != 1.0 else x
