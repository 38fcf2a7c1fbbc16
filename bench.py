"""Throughput of the fused attention forward pass (tensorized online softmax) on
one MI355X, as one JSON line.

A step is one call of tos_attn_fwd over the whole workload (all key blocks, the
softmax, both products, the epilogue) with inputs already resident in HBM.
Default workload: causal bf16 attention, B=2, H=32, N=4096, d=128 (X = 32).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--split PLAN] [--share NUM/DEN] [--schedule cosched|sequential]
                    [--x-tile X] [--fallback off|auto|force] [--no-cpu-baseline]
                    [--no-fp8] [--cpu-rows R] [--copy-calib-mib M]

--copy-calib-mib M also runs one plain device-to-device copy of M MiB after the
timed region; rocprofv3 counter runs of this command use it to calibrate the
FETCH_SIZE / WRITE_SIZE counters against a kernel of known traffic.

Other modes, each printing its own JSON lines instead of the bench line:
--ablation (the knob settings, launch by launch), --grid DTYPES (the page's
workload grid), --vector-interval (phase-stamped instances), --mfma-ceiling (the
vendor bf16 GEMM), --item-cost (per-step and per-item cost from plain launches).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "f32": 157.3}   # MI355X dense MFMA
# whole-chip v_exp_f32 rate at the published clock: 256 CUs x 4 SIMDs x 8 lanes
# per clock (a wave64 v_exp_f32 takes 8 clocks of issue, measured) x 2.4 GHz
EXP_PER_S = 256 * 4 * 8 * 2.4e9
HBM_GBPS = 8000.0
# sources of each dtype's kernel: a committed traffic summary is used only
# while these are unchanged
_CSRC = "tensorized_online_softmax_amd/csrc/"
KERNEL_SOURCES = {
    "bf16": [_CSRC + f for f in ("attn_fwd_kernels.hpp", "softmax_tile.hpp", "pieces.hpp")],
    "f16": [_CSRC + f for f in ("attn_fwd_kernels.hpp", "softmax_tile.hpp", "pieces.hpp")],
    "f32": [_CSRC + f for f in ("attn_fwd_kernels.hpp", "attn_fwd_f32_slab.hpp", "softmax_tile.hpp",
                                "pieces.hpp")],
    "fp8": [_CSRC + f for f in ("attn_fwd_kernels.hpp", "attn_fwd_fp8.hpp", "softmax_tile.hpp",
                                "pieces.hpp")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{workload}.txt")


def kernel_hash(dtype):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[dtype]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload, dtype):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_hash(dtype):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def block_shape(w, x_tile, fallback):
    """Query rows and keys per step of the kernel the library picks for the
    workload: fp32 at X = 1 or 16 without the fallback runs in 16-row slabs of
    16-key chunks (with 1, 2 or 4 workgroups sharing the head dim) while 128-row
    workgroups would number fewer than the compute units; other fp32 calls take
    128-row workgroups, the 16-bit and fp8 kernels 256-row ones, of 64-key blocks."""
    import torch
    if w.dtype != "f32":
        return {"Br": 256, "Bc": 64}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    BH = w.B * w.H
    if x_tile in (1, 16) and fallback == "off" and BH * -(-w.N // 128) < cus:
        slabs = BH * -(-w.N // 16)
        return {"Br": 16, "Bc": 16, "head_dim_shares": 4 if 4 * slabs <= cus else 2 if 2 * slabs <= cus else 1}
    return {"Br": 128, "Bc": 64}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, target_rows):
    """The fp64 oracle (exact attention) on a seeded sample of the workload's
    rows, on every host core this process may use."""
    import numpy as np
    import oracle
    from tensorized_online_softmax_amd import inputs
    threads = min(len(os.sched_getaffinity(0)),
                  int(os.environ.get("OMP_NUM_THREADS", "0")) or 1 << 30)
    q, k, v = (inputs.real_values(inp[n], inp["descale"][n]) for n in ("q", "k", "v"))
    BH = w.B * w.H
    if target_rows <= 0 or target_rows >= BH * w.N:
        target_rows = BH * w.N
        rows = np.arange(BH * w.N, dtype=np.int64)
    else:
        rows = np.sort(np.random.default_rng(w.seed + 99).choice(BH * w.N, size=target_rows,
                                                                  replace=False))
    i = rows % w.N
    keys = (i + 1) if w.causal else np.full(rows.shape, w.N)
    flops = float(np.sum(4.0 * w.d * keys))
    t0 = time.perf_counter()
    oracle.attn_exact(q, k, v, w.causal, w.scale, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    what = ("every query row" if target_rows == BH * w.N
            else f"{target_rows} of {BH * w.N} query rows (seeded uniform)")
    # the method's own recurrence (oracle_attn_surrogate: Algorithm 1 block by
    # block in fp64) beside the plain definition, on a bounded sample of heads
    nh = max(1, min(BH, BH // 8))
    q3, k3, v3 = (x.reshape(BH, w.N, w.d)[:nh] for x in (q, k, v))
    fb = {"off": oracle.FALLBACK_OFF, "auto": oracle.FALLBACK_AUTO,
          "force": oracle.FALLBACK_FORCE}[w.fallback]
    t0 = time.perf_counter()
    oracle.attn_surrogate(q3, k3, v3, w.causal, w.scale, X=w.x_tile, Bc=64, fallback=fb,
                          tau=12.0 if w.dtype == "fp8" else 100.0, threads=threads)
    dt2 = time.perf_counter() - t0
    flops2 = flops * nh / BH if target_rows == BH * w.N else w.flops() * nh / BH
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "seconds": round(dt, 3),
            "gflops_fp64": round(flops / dt / 1e9, 3),
            "sample": f"{what} of the workload, each over its full key range; fp64 exact "
                      f"attention (oracle_attn_exact), {dt:.1f} s",
            "surrogate": {"value": round(flops2 / dt2 / 1e12, 6), "unit": "TFLOP/s",
                          "seconds": round(dt2, 3), "gflops_fp64": round(flops2 / dt2 / 1e9, 3),
                          "sample": f"{nh} of {BH} heads, every row; fp64 surrogate-maximum "
                                    f"recurrence (oracle_attn_surrogate, X={w.x_tile}, Bc=64)"}}


def mfma_ceiling():
    """Dense bf16 GEMM throughput of the vendor library (torch.matmul) on this
    GPU: the practical MFMA ceiling that the published peak overstates when the
    data are random (power-limited clock)."""
    import torch
    torch.cuda.set_device(0)
    out = {"metric": "bf16 GEMM TFLOP/s (torch.matmul), context for the MFMA roofline",
           "unit": "TFLOP/s", "peak_published": PEAK_TFLOPS["bf16"], "runs": []}
    for n, data in ((8192, "randn"), (16384, "randn"), (8192, "zeros")):
        make = torch.randn if data == "randn" else torch.zeros
        a = make(n, n, device="cuda", dtype=torch.bfloat16)
        b = make(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(5):
            a @ b
        torch.cuda.synchronize()
        it = 20 if n <= 8192 else 6
        t0 = time.perf_counter()
        for _ in range(it):
            a @ b
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / it
        tf = 2.0 * n ** 3 / dt / 1e12
        out["runs"].append({"m=n=k": n, "data": data, "tflops": round(tf, 1),
                            "frac_of_published_peak": round(tf / PEAK_TFLOPS["bf16"], 4)})
        print(f"[bench] bf16 GEMM {n}^3 {data}: {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def grid_sweep(dtypes, steps, warmup):
    """The page's workload grid: per point, the kernel at X = 32 (the surrogate
    tile) and at X = 1 (the per-row online softmax, the FlashAttention-2 analog),
    both with the vector-unit row sum.  The two settings alternate launch by
    launch, so that clock and power drift falls on both alike; each reports
    the median of its launches."""
    import torch
    from tensorized_online_softmax_amd import binding, inputs
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    for w in inputs.grid(tuple(dtypes)):
        inp = inputs.make_workload(w)
        q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
        odt = {"f32": torch.float32, "f16": torch.float16}.get(w.dtype, torch.bfloat16)
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=odt, device="cuda")
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        descale = inp["descale"] if w.dtype == "fp8" else None

        def step(x):
            binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, dtype=w.dtype,
                             x_tile=x, descale=descale, out=o, lse=lse)
        xs = (32, 1)
        for _ in range(warmup):
            for x in xs:
                step(x)
        ev = {x: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)] for x in xs}
        torch.cuda.synchronize()
        for i in range(steps):
            for x in xs:
                ev[x][i][0].record(stream)
                step(x)
                ev[x][i][1].record(stream)
        torch.cuda.synchronize()
        line = {"workload": w.name, "dtype": w.dtype, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                "causal": w.causal, "flops": w.flops(), "launches": steps}
        for x in xs:
            t = sorted(a.elapsed_time(b) / 1e3 for a, b in ev[x])
            med = t[len(t) // 2]
            tf = w.flops() / med / 1e12
            line[f"x{x}_us"] = round(med * 1e6, 2)
            line[f"x{x}_tflops"] = round(tf, 1)
            line[f"x{x}_frac"] = round(tf / PEAK_TFLOPS[w.dtype], 4)
        line["speedup_x32_over_x1"] = round(line["x1_us"] / line["x32_us"], 4)
        print(json.dumps(line), flush=True)
        del q, k, v, o, lse, inp


# The ablation's knob settings, after FlashAttention-T's evaluation (section
# A4, Fig 9 and Fig 10: FA2, FA2 + Max16, AllTensor, FA-T) and its
# tensor-vector split (section A2, Fig 6): name, X, softmax split, schedule,
# matrix-unit share.  The pages' AllTensor puts scaling, FMA and the row sum on
# the tensor unit; gfx950 has no TF32 matrix instruction, so here the scaling
# and the FMA are fp32 products.
ABLATION = [
    ("per_row_sequential", 1, "valu", "sequential", None),     # FA2 analog
    ("per_row_cosched", 1, "valu", "cosched", None),
    ("tile16_cosched", 16, "valu", "cosched", None),           # Max16 analog
    ("tile32_sequential", 32, "valu", "sequential", None),
    ("tile32_cosched", 32, "valu", "cosched", None),           # FA-T analog (the default)
    ("tile64_cosched", 64, "valu", "cosched", None),           # tiles of two waves
    ("tile32_rowsum_mfma", 32, "rowsum_mfma", "cosched", None),
    ("tile32_rowsum_1_4", 32, "rowsum_mfma", "cosched", (1, 4)),
    ("tile32_rowsum_1_2", 32, "rowsum_mfma", "cosched", (1, 2)),
    ("tile32_rowsum_3_4", 32, "rowsum_mfma", "cosched", (3, 4)),
    ("tile32_scale_mfma", 32, "scale_mfma", "cosched", None),  # O rescale on the matrix unit
    ("tile32_hsplit_1_4", 32, "hsplit", "cosched", (1, 4)),
    ("tile32_hsplit_1_2", 32, "hsplit", "cosched", (1, 2)),
    ("tile32_vsplit_1_2", 32, "vsplit", "cosched", (1, 2)),
    ("tile32_all_mfma", 32, "all_mfma", "cosched", None),      # AllTensor analog
]


def ablation(workload, steps, warmup, reps=3):
    """Median launch time of each knob setting on one workload.  Each setting
    runs in blocks (a few warmup launches, then timed ones) so that it is
    measured at its own power and clock state, and the round of blocks repeats
    `reps` times so that drift falls on every setting alike.  (Alternating the
    settings launch by launch instead lets a low-power neighbour raise the
    clock of the next launch.)"""
    import torch
    from tensorized_online_softmax_amd import binding, inputs
    w = inputs.WORKLOADS[workload]
    if w.dtype not in ("bf16", "f16"):
        raise SystemExit("the ablation runs the 16-bit kernels")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    inp = inputs.make_workload(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    odt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=odt, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    per_block = max(3, min(steps, 60) // reps)
    warm = max(2, min(warmup, 5))
    times = [[] for _ in ABLATION]
    for _ in range(reps):
        for si, (name, x, split, sched, share) in enumerate(ABLATION):
            def f():
                binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, dtype=w.dtype,
                                 x_tile=x, split=split, schedule=sched, share=share,
                                 out=o, lse=lse)
            for _ in range(warm):
                f()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(per_block)]
            for a, b in ev:
                a.record(stream)
                f()
                b.record(stream)
            torch.cuda.synchronize()
            times[si] += [a.elapsed_time(b) / 1e3 for a, b in ev]
    med = [sorted(t)[len(t) // 2] for t in times]
    for (name, x, split, sched, share), m, t in zip(ABLATION, med, times):
        tf = w.flops() / m / 1e12
        print(json.dumps({"workload": w.name, "setting": name, "x_tile": x, "softmax_split": split,
                          "share": f"{share[0]}/{share[1]}" if share else None,
                          "schedule": sched, "launches": len(t), "median_us": round(m * 1e6, 2),
                          "tflops": round(tf, 1), "frac": round(tf / PEAK_TFLOPS[w.dtype], 4),
                          "speedup_over_first": round(med[0] / m, 4)}), flush=True)


def time_workload(w, inp, x_tile, split, fallback, schedule, share, steps, warmup):
    """Warmup, then `steps` timed launches of one workload (inputs resident in
    HBM), each bracketed by HIP events on the launch stream; returns the
    wall-clock throughput, the config and the roofline of the launch."""
    import torch
    from tensorized_online_softmax_amd import binding
    print(f"[bench] workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} "
          f"causal={w.causal} X={x_tile} split={split} fallback={fallback}",
          file=sys.stderr, flush=True)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=binding.out_dtype(w.dtype), device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    descale = inp["descale"] if w.dtype == "fp8" else None

    def step():
        binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, dtype=w.dtype,
                         x_tile=x_tile, split=split, fallback=fallback,
                         descale=descale, out=o, lse=lse, schedule=schedule, share=share)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()   # the stream the kernels are launched on
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    med_launch_s = sorted(launch_ms)[len(launch_ms) // 2] / 1e3
    ms_per_step = wall * 1e3 / steps
    flops = w.flops()
    print(f"[bench] {steps} steps in {wall:.3f} s; launch avg {avg_launch_s * 1e6:.1f} us "
          f"min {min(launch_ms) * 1e3:.1f} us max {max(launch_ms) * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    peak = PEAK_TFLOPS[w.dtype]
    achieved = flops / avg_launch_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": read_traffic(w.name, w.dtype),
                # the secondary (vector) ceiling: one v_exp_f32 per attention element
                "exp_per_launch": w.exps(), "exp_floor_us": round(w.exps() / EXP_PER_S * 1e6, 2),
                "launch_us": {"mean": round(avg_launch_s * 1e6, 2),
                              "median": round(med_launch_s * 1e6, 2),
                              "min": round(min(launch_ms) * 1e3, 2)},
                "achieved_at_median": round(flops / med_launch_s / 1e12, 2)}
    config = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
              "causal": w.causal, "x_tile": x_tile,
              # e4m3 P~ pairs have no vector dot form: fp8 sums them on the matrix unit
              "softmax_split": "rowsum_mfma" if w.dtype == "fp8" else split,
              "share": f"{share[0]}/{share[1]}" if share else None,
              "schedule": schedule,
              "fallback": fallback, **block_shape(w, x_tile, fallback),
              "flops_per_step": flops, "pct_of_peak": round(100 * achieved / peak, 2)}
    del q, k, v, o, lse
    return {"value": round(flops / (ms_per_step / 1e3) / 1e12, 2),
            "ms_per_step": round(ms_per_step, 4), "config": config, "roofline": roofline}


# Settings of the vector-interval table (FlashAttention-T, section A4, Fig 9:
# the share of the iteration in which the matrix unit waits for vector work),
# each with the matrix-unit cycles of one steady step of a SIMD (two waves of 32
# query rows x 64 keys): 32 bf16 32x32x16 MFMAs of 32 clocks per wave, 4 more
# for the matrix-unit row sum, and for everything on the matrix unit also 34
# fp32 32x32x2 MFMAs of 64 clocks (Z: two tiles of one offset and 16 slices).
VECTOR_INTERVAL = [
    ("per_row_sequential", 1, "valu", "sequential", 2 * 32 * 32),   # FA2 analog
    ("tile32_sequential", 32, "valu", "sequential", 2 * 32 * 32),
    ("per_row_cosched", 1, "valu", "cosched", 2 * 32 * 32),
    ("tile16_cosched", 16, "valu", "cosched", 2 * 32 * 32),         # Max16 analog
    ("tile32_cosched", 32, "valu", "cosched", 2 * 32 * 32),         # FA-T analog
    ("tile32_rowsum_mfma", 32, "rowsum_mfma", "cosched", 2 * 36 * 32),
    ("tile32_all_mfma", 32, "all_mfma", "cosched", 2 * (36 * 32 + 34 * 64)),   # AllTensor analog
]


def vector_interval(workload, steps, warmup):
    """Phase-stamped runs of each setting (s_memtime cycles per wave, as the last
    launch wrote them): the step cycles of a SIMD against its matrix-unit cycles give
    the share of the step in which the matrix unit is idle; the sequential
    schedule's softmax section is its vector-only time.  The stamps wait for
    themselves, so a traced launch is slower than a plain one (both reported)."""
    import torch
    from tensorized_online_softmax_amd import binding, inputs
    w = inputs.WORKLOADS[workload]
    if w.dtype != "bf16" or w.d != 128:
        raise SystemExit("the phase-stamped kernels are the bf16 d=128 ones")
    torch.cuda.set_device(0)
    inp = inputs.make_workload(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    trace = torch.zeros(1024 * 1024 // 8, dtype=torch.int64, device="cuda")
    n = max(3, min(steps, 20))
    for name, x, split, sched, mfma_clk in VECTOR_INTERVAL:
        def f(tr=None):
            binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, x_tile=x, split=split,
                             schedule=sched, out=o, lse=lse, trace=tr)
        times = {}
        for kind in ("plain", "traced"):
            for _ in range(max(2, min(warmup, 5))):
                f(trace if kind == "traced" else None)
            trace.zero_()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            for i in range(n):
                ev[i].record()
                f(trace if kind == "traced" else None)
            ev[n].record()
            torch.cuda.synchronize()
            t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
            times[kind] = t[len(t) // 2]
        raw = trace.view(-1, 16).cpu().numpy()
        raw = raw[raw[:, 0] > 0]
        tr = raw.astype("float64")
        tot = tr.sum(axis=0)
        line = {"workload": w.name, "setting": name, "x_tile": x, "softmax_split": split,
                "schedule": sched, "launches": n,
                "plain_median_us": round(times["plain"], 2),
                "traced_median_us": round(times["traced"], 2),
                "waves": int(tr.shape[0])}
        if tot[1] > 0:
            step = tot[2] / tot[1]
            line.update({"steady_steps": int(tot[1]), "steady_step_clk": round(step, 1),
                         "phase_a_clk": round(tot[3] / tot[1], 1),
                         "phase_b_clk": round(tot[4] / tot[1], 1),
                         "barrier_clk": round(tot[5] / tot[1], 1)})
        if tot[6] > 0:
            line.update({"edge_steps": int(tot[6]), "edge_step_clk": round(tot[7] / tot[6], 1),
                         "edge_softmax_clk": round(tot[8] / tot[6], 1),
                         "edge_barrier_clk": round(tot[9] / tot[6], 1)})
        # the shader clock from the wave spans against the fixed 100 MHz counter;
        # the last launch's span (its waves' first to last stamps on that counter)
        # against each wave's own: the share of the launch a wave is running
        line["shader_clock_ghz"] = round(tot[0] / tot[10] * 0.1, 3)
        line["wave_clk"] = round(tot[0] / tr.shape[0], 1)
        line["steps_share_of_wave"] = round((tot[2] + tot[7]) / tot[0], 4)
        span = int(raw[:, 12].max()) - int(raw[:, 11].min())
        if span > 0:
            line["launch_span_us"] = round(span / 100.0, 2)
            line["wave_span_share_mean"] = round(float(tot[10] / tr.shape[0]) / span, 4)
        # the matrix unit's idle share of a step of a SIMD (two waves), from the
        # steady steps when the schedule has them, else from all steps
        step = line.get("steady_step_clk") or line.get("edge_step_clk")
        line["mfma_clk_per_simd_step"] = mfma_clk
        line["vector_interval_ratio"] = round(max(0.0, 1.0 - mfma_clk / step), 4)
        if sched == "sequential":
            line["softmax_share_of_step"] = round(tot[8] / tot[7], 4)
        print(json.dumps(line), flush=True)


def item_cost(steps, warmup):
    """Plain launches of the persistent bf16 kernel (d = 128, not causal, X = 32)
    with k = 1, 2, 4 and 8 items per workgroup (256-row query blocks; k times
    the compute-unit count of them) of s = N/64 key-block steps, N = 1024 and
    4096, each timed over interleaved rounds; then the least-squares fit
    time = a + k * (c_item + s * c_step): what a key-block step and an item's
    boundary (its prologue, first and last steps, epilogue) cost on this GPU."""
    import numpy as np
    import torch
    from tensorized_online_softmax_amd import binding
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    cases = []
    for N in (1024, 4096):
        for k in (1, 2, 4, 8):
            BH = k * cus * 256 // N
            g = torch.Generator(device="cuda").manual_seed(BH * 7 + N)
            q, kk, v = (torch.randn(1, BH, N, 128, device="cuda", generator=g).to(torch.bfloat16)
                        for _ in range(3))
            o = torch.empty_like(q)
            lse = torch.empty(1, BH, N, device="cuda")
            cases.append({"N": N, "items_per_workgroup": k, "steps_per_item": N // 64, "heads": BH,
                          "t": [], "f": (lambda q=q, kk=kk, v=v, o=o, lse=lse: binding.attn_fwd(
                              q, kk, v, causal=False, out=o, lse=lse))})
    n = max(5, min(steps, 20))
    for c in cases:
        for _ in range(max(2, min(warmup, 5))):
            c["f"]()
    torch.cuda.synchronize()
    for _ in range(3):   # rounds: the cases alternate, so that clock drift falls on all alike
        for c in cases:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            for i in range(n):
                ev[i].record(stream)
                c["f"]()
            ev[n].record(stream)
            torch.cuda.synchronize()
            c["t"] += [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]
    for c in cases:
        c["median_us"] = round(float(np.median(c["t"])), 2)
    A = np.array([[1.0, c["items_per_workgroup"], c["items_per_workgroup"] * c["steps_per_item"]]
                  for c in cases])
    y = np.array([c["median_us"] for c in cases])
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    out = {"metric": "per-item and per-step cost of the persistent bf16 kernel (d=128, not causal, X=32)",
           "unit": "us", "compute_units": cus, "launches_per_case": 3 * n,
           "cases": [{k: c[k] for k in ("N", "heads", "items_per_workgroup", "steps_per_item", "median_us")}
                     for c in cases],
           "fit": {"fixed_us": round(float(coef[0]), 2), "per_item_us": round(float(coef[1]), 2),
                   "per_step_us": round(float(coef[2]), 3),
                   "residuals_us": [round(float(r), 1) for r in y - A @ coef]}}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="causal_bf16")
    ap.add_argument("--split", default="valu",
                    choices=["valu", "rowsum_mfma", "scale_mfma", "hsplit", "vsplit", "all_mfma"])
    ap.add_argument("--share", default=None, metavar="NUM/DEN",
                    help="the matrix unit's share of the --split value (e.g. 1/2)")
    ap.add_argument("--schedule", default="cosched", choices=["cosched", "sequential"],
                    help="sequential: the no-co-scheduling ablation (16-bit inputs)")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the attention bench: time the knob settings of the "
                         "ablation (X, row-sum split, schedule) on the workload, alternating "
                         "them launch by launch; one JSON line per setting")
    ap.add_argument("--x-tile", type=int, default=None)
    ap.add_argument("--fallback", default=None, choices=["off", "auto", "force"],
                    help="default: the workload's own (AUTO for the fp8 stress workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8 stress workload's block after the bf16 headline")
    ap.add_argument("--cpu-rows", type=int, default=0, help="0 = every row")
    ap.add_argument("--copy-calib-mib", type=int, default=0)
    ap.add_argument("--grid", default=None, metavar="DTYPES",
                    help="instead of the attention bench: time every point of the page's "
                         "workload grid (16k tokens, hidden 2048) for the comma-separated "
                         "dtypes (bf16,f16,fp8), at X = 32 and X = 1; one JSON line per point")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the attention bench: time torch's bf16 GEMM (the vendor "
                         "library) on random and on all-zero data, for the MFMA throughput this "
                         "GPU sustains under its power limit")
    ap.add_argument("--item-cost", action="store_true",
                    help="instead of the attention bench: plain launches of the bf16 d=128 kernel "
                         "at 1, 2, 4 and 8 items per workgroup and two sequence lengths, fitted "
                         "to a per-step and a per-item cost; one JSON line")
    ap.add_argument("--vector-interval", action="store_true",
                    help="instead of the attention bench: phase-stamped runs of the ablation's "
                         "settings (bf16, d=128 workloads) and the matrix unit's idle share of "
                         "a step; one JSON line per setting")
    args = ap.parse_args()
    if args.vector_interval:
        vector_interval(args.workload, args.steps, args.warmup)
        return
    if args.item_cost:
        item_cost(args.steps, args.warmup)
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.grid:
        grid_sweep(args.grid.split(","), args.steps, args.warmup)
        return
    if args.ablation:
        ablation(args.workload, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(heads shard across GPUs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from tensorized_online_softmax_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    x_tile = args.x_tile or w.x_tile
    fallback = args.fallback or w.fallback
    share = tuple(int(x) for x in args.share.split("/")) if args.share else None
    torch.cuda.set_device(0)
    inp = inputs.make_workload(w)
    t = time_workload(w, inp, x_tile, args.split, fallback, args.schedule, share, args.steps,
                      args.warmup)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {args.copy_calib_mib} MiB read + written",
              file=sys.stderr, flush=True)

    result = {
        "metric": "fused attention fwd TFLOP/s at 1 GPU and % of MFMA peak (bf16, fp8)",
        "value": t["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, numpy PCG64)",
        "config": t["config"],
        "roofline": t["roofline"],
    }
    # the metric names two precisions: the fp8 stress workload rides along as a
    # second block with its own roofline (the headline stays the bf16 line)
    if args.workload == "causal_bf16" and not args.no_fp8:
        w8 = inputs.WORKLOADS["fp8_spiky"]
        inp8 = inputs.make_workload(w8)
        t8 = time_workload(w8, inp8, w8.x_tile, "valu", w8.fallback, "cosched", None,
                           args.steps, args.warmup)
        result["fp8"] = {"value": t8["value"], "unit": "TFLOP/s", "dtype": "fp8",
                         "ms_per_step": t8["ms_per_step"], "config": t8["config"],
                         "roofline": t8["roofline"]}
        del inp8
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
