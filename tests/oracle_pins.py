"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with:
  * closed forms derived by hand from the definition of attention
    (tests/golden/closed_forms.json; FlashAttention-T page, section A3, Fig 2(a));
  * a library routine: torch's CPU scaled-dot-product attention in float64,
    which returns O and the log-sum-exp;
  * special cases: Q = 0, N = 1, constant V, equal keys, one-hot V, joint
    permutation of K and V rows;
  * the surrogate-maximum guarantees of section A2 (m^ >= m, Z <= 0, no
    non-finite values) and the value of m^ itself (the tile's largest logit);
  * the textbook per-row online softmax (the X = 1 special case);
  * the all-underflow failure mode and the fallback (section A2, numerical
    stability guarantees);
  * torch's round-to-nearest-even casts to bfloat16 and float8_e4m3fn.

The same functions run against deliberately broken builds of oracle.c
(test_oracle_mutants.py), which shows that the pins catch plausible mistakes.
"""
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def _rel_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b) / np.maximum(1.0, np.abs(b))
    assert err.max(initial=0.0) <= tol, f"{what}: max rel err {err.max():.3e} > {tol:.1e}"


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _torch_ref(q, k, v, causal, scale):
    """O and lse from torch's CPU flash-attention routine in float64 ([BH,N,d] in)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None] for x in (q, k, v))
    o, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, bool(causal), attn_mask=None, scale=float(scale))
    return o[0].numpy(), lse[0].numpy()


def _all_variants(orc, q, k, v, causal, scale):
    """The exact oracle and a spread of surrogate settings, as (label, o, lse)."""
    o, lse = orc.attn_exact(q, k, v, causal, scale)
    out = [("exact", o, lse)]
    N = q.shape[1]
    for X, Bc in ((1, 1), (2, 3), (4, 5), (16, 16), (32, 64), (max(N, 1), 7)):
        r = orc.attn_surrogate(q, k, v, causal, scale, X=X, Bc=Bc)
        out.append((f"surrogate X={X} Bc={Bc}", r["o"], r["lse"]))
    return out


# --------------------------------------------------------------------------
def pin_golden_closed_forms(orc):
    spec = json.load(open(GOLDEN))
    for case in spec["cases"]:
        N, d = case["N"], case["d"]
        env = {"math": math}
        if "Q" in case:
            q = np.array(case["Q"], dtype=np.float64)[None]
            k = np.array(case["K"], dtype=np.float64)[None]
            v = np.array(case["V"], dtype=np.float64)[None]
            o_ref = np.array(case["O"], dtype=np.float64)
            lse_ref = np.array(case["LSE"], dtype=np.float64)
        else:
            q = np.array([[eval(case["q"], env, {"i": i})] for i in range(N)])[None]
            k = np.array([[eval(case["k"], env, {"j": j})] for j in range(N)])[None]
            v = np.array([[eval(case["v"], env, {"j": j})] for j in range(N)])[None]
            o_ref = np.array([[eval(case["o"], env, {"i": i})] for i in range(N)])
            lse_ref = np.array([eval(case["lse"], env, {"i": i}) for i in range(N)])
        for label, o, lse in _all_variants(orc, q, k, v, case["causal"], case["scale"]):
            _rel_close(o[0], o_ref, 1e-12, f"{case['name']} {label} O")
            _rel_close(lse[0], lse_ref, 1e-12, f"{case['name']} {label} lse")


def pin_library_sdpa(orc):
    rng = np.random.default_rng(11)
    for (BH, N, d) in ((1, 1, 1), (2, 7, 8), (3, 33, 16), (2, 64, 32), (1, 100, 64)):
        for causal in (False, True):
            for std in (1.0, 3.0):
                q, k, v = (_rand(rng, BH, N, d, std=std) for _ in range(3))
                scale = 1.0 / math.sqrt(d)
                o_ref, lse_ref = _torch_ref(q, k, v, causal, scale)
                for label, o, lse in _all_variants(orc, q, k, v, causal, scale):
                    tag = f"BH={BH} N={N} d={d} causal={causal} std={std} {label}"
                    _rel_close(o, o_ref, 1e-11, tag + " O")
                    _rel_close(lse, lse_ref, 1e-11, tag + " lse")
    # selected rows give the same numbers as the full pass
    q, k, v = (_rand(rng, 2, 50, 8) for _ in range(3))
    o, lse = orc.attn_exact(q, k, v, True, 0.4)
    rows = np.array([0, 7, 49, 50, 77, 99])
    os_, ls_ = orc.attn_exact(q, k, v, True, 0.4, rows=rows)
    _rel_close(os_, o.reshape(-1, 8)[rows], 0.0, "row-sampled O")
    _rel_close(ls_, lse.reshape(-1)[rows], 0.0, "row-sampled lse")


def pin_special_cases(orc):
    rng = np.random.default_rng(12)
    BH, N, d = 2, 23, 24
    k, v = _rand(rng, BH, N, d), _rand(rng, BH, N, d)
    scale = 0.35
    for causal in (False, True):
        # Q = 0: uniform weights over the valid keys
        q = np.zeros((BH, N, d))
        cnt = np.array([(i + 1) if causal else N for i in range(N)], dtype=np.float64)
        mean = np.stack([np.stack([v[b, :(i + 1 if causal else N)].mean(0) for i in range(N)])
                         for b in range(BH)])
        for label, o, lse in _all_variants(orc, q, k, v, causal, scale):
            _rel_close(o, mean, 1e-12, f"Q=0 causal={causal} {label} O")
            _rel_close(lse, np.broadcast_to(np.log(cnt), (BH, N)), 1e-12, f"Q=0 {label} lse")
        # all keys equal: same weights, lse shifted by the common logit
        q = _rand(rng, BH, N, d)
        keq = np.broadcast_to(k[:, :1], k.shape).copy()
        common = scale * np.einsum("bnd,bd->bn", q, keq[:, 0])
        for label, o, lse in _all_variants(orc, q, keq, v, causal, scale):
            _rel_close(o, mean, 1e-12, f"equal keys causal={causal} {label} O")
            _rel_close(lse, common + np.log(cnt), 1e-12, f"equal keys {label} lse")
        # V constant: O = that constant
        vc = np.full((BH, N, d), -2.5)
        for label, o, _ in _all_variants(orc, q, k, vc, causal, scale):
            _rel_close(o, vc, 1e-12, f"const V causal={causal} {label} O")
        # one-hot V (v_j = e_j): O is the probability matrix, rows sum to 1,
        # masked entries are exactly 0
        qn = _rand(rng, 1, N, N, std=2.0)
        kn = _rand(rng, 1, N, N, std=2.0)
        eye = np.eye(N)[None]
        for label, o, _ in _all_variants(orc, qn, kn, eye, causal, 1.0 / math.sqrt(N)):
            _rel_close(o.sum(-1), np.ones((1, N)), 1e-12, f"one-hot V {label} row sums")
            assert np.all(o >= 0.0), f"{label}: negative probability"
            if causal:
                assert np.all(np.triu(o[0], 1) == 0.0), f"{label}: weight on a masked key"
    # N = 1: O = v_0, lse = scale * <q_0, k_0>
    q1, k1, v1 = (_rand(rng, 3, 1, 5) for _ in range(3))
    for causal in (False, True):
        for label, o, lse in _all_variants(orc, q1, k1, v1, causal, 0.7):
            _rel_close(o, v1, 1e-14, f"N=1 {label} O")
            _rel_close(lse[:, 0], 0.7 * np.sum(q1 * k1, -1)[:, 0], 1e-14, f"N=1 {label} lse")
    # joint permutation of K and V rows leaves non-causal attention unchanged
    q, k, v = (_rand(rng, 2, 31, 8) for _ in range(3))
    perm = rng.permutation(31)
    for label, o, lse in _all_variants(orc, q, k, v, False, 0.5):
        for label2, o2, lse2 in _all_variants(orc, q, k[:, perm], v[:, perm], False, 0.5)[:2]:
            _rel_close(o2, o, 1e-12, f"permuted K/V {label}/{label2} O")
            _rel_close(lse2, lse, 1e-12, f"permuted K/V {label}/{label2} lse")


def pin_surrogate_equals_exact(orc):
    """Algorithm 1 reaches the plain definition for every tile size, block size,
    mask and block order (brute force over small shapes)."""
    rng = np.random.default_rng(13)
    for N in (1, 2, 3, 5, 16, 17, 33):
        for d in (1, 2, 4, 8):
            q, k, v = (_rand(rng, 2, N, d, std=2.0) for _ in range(3))
            for causal in (False, True):
                o_ref, lse_ref = orc.attn_exact(q, k, v, causal, 0.6)
                for X in sorted({1, 2, 3, 16, 32, N}):
                    for Bc in (1, 2, 5, 16, 64):
                        nblk = (N + Bc - 1) // Bc
                        for order in (None, rng.permutation(nblk)):
                            r = orc.attn_surrogate(q, k, v, causal, 0.6, X=X, Bc=Bc, order=order)
                            tag = f"N={N} d={d} causal={causal} X={X} Bc={Bc} order={order}"
                            _rel_close(r["o"], o_ref, 1e-12, tag + " O")
                            _rel_close(r["lse"], lse_ref, 1e-12, tag + " lse")
                            assert r["n_mhat_below_m"] == 0 and r["n_z_positive"] == 0, tag
                            assert r["n_nonfinite_rows"] == 0 and r["n_tiles_per_row"] == 0, tag


def pin_surrogate_invariants(orc):
    """m^ is the tile's largest logit, m^ >= every row max, Z <= 0, all finite."""
    rng = np.random.default_rng(14)
    BH, N, d = 3, 200, 16
    for std in (1.0, 4.0):
        q, k, v = (_rand(rng, BH, N, d, std=std) for _ in range(3))
        for causal in (False, True):
            logits = np.einsum("bid,bjd->bij", q, k)
            if causal:
                logits = np.where(np.tril(np.ones((N, N), dtype=bool)), logits, -np.inf)
            rowmax = logits.max(-1)
            for X in (1, 7, 16, 32):
                r = orc.attn_surrogate(q, k, v, causal, 0.25, X=X, Bc=16)
                tag = f"std={std} causal={causal} X={X}"
                assert r["n_mhat_below_m"] == 0 and r["n_z_positive"] == 0, tag
                assert r["n_nonfinite_rows"] == 0, tag
                ntile = (N + X - 1) // X
                pad = ntile * X - N
                tm = np.pad(rowmax, ((0, 0), (0, pad)), constant_values=-np.inf)
                tm = tm.reshape(BH, ntile, X).max(-1)
                expect = np.repeat(tm, X, axis=1)[:, :N]
                # logits here come from numpy's einsum, so allow its rounding
                _rel_close(r["ref"], expect, 1e-14, tag + " final m^ = tile max of logits")
                assert np.all(r["ref"] >= rowmax - 1e-13 * np.abs(rowmax)), tag
                # largest gap c*(m^ - m_i) over the blocks, from running maxima
                Bc = 16
                nblk = (N + Bc - 1) // Bc
                lp = np.pad(logits, ((0, 0), (0, 0), (0, nblk * Bc - N)), constant_values=-np.inf)
                run = np.maximum.accumulate(lp.reshape(BH, N, nblk, Bc).max(-1), axis=2)
                rp = np.pad(run, ((0, 0), (0, pad), (0, 0)), constant_values=-np.inf)
                tmax = np.repeat(rp.reshape(BH, ntile, X, nblk).max(2), X, axis=1)[:, :N]
                with np.errstate(invalid="ignore"):
                    g = 0.25 * math.log2(math.e) * (tmax - run)
                g = np.where(np.isfinite(run), g, 0.0).max(-1)
                assert np.abs(r["gap"] - g).max() <= 1e-12, tag + " largest gap"


def pin_per_row_textbook(orc):
    """X = 1 is the textbook online softmax (Milakov & Gimelshein 2018): per row,
    m_new = max(m, max_j s_j); l = l*exp(m - m_new) + sum_j exp(s_j - m_new);
    o = o*exp(m - m_new) + sum_j exp(s_j - m_new) v_j.  Written here with
    natural exponentials in plain Python loops, on tiny inputs."""
    rng = np.random.default_rng(15)
    BH, N, d, Bc, scale = 2, 13, 3, 4, 0.8
    q, k, v = (_rand(rng, BH, N, d, std=1.5) for _ in range(3))
    for causal in (False, True):
        o_ref = np.zeros((BH, N, d))
        lse_ref = np.zeros((BH, N))
        for b in range(BH):
            for i in range(N):
                m, l, acc = -math.inf, 0.0, [0.0] * d
                for j0 in range(0, N, Bc):
                    js = [j for j in range(j0, min(j0 + Bc, N)) if (not causal or j <= i)]
                    if not js:
                        continue
                    s = {j: scale * sum(q[b, i, t] * k[b, j, t] for t in range(d)) for j in js}
                    m_new = max(m, max(s.values()))
                    a = math.exp(m - m_new) if m > -math.inf else 0.0
                    l = l * a + sum(math.exp(s[j] - m_new) for j in js)
                    acc = [acc[t] * a + sum(math.exp(s[j] - m_new) * v[b, j, t] for j in js)
                           for t in range(d)]
                    m = m_new
                o_ref[b, i] = [x / l for x in acc]
                lse_ref[b, i] = m + math.log(l)
        for X, fb in ((1, 0), (5, 2)):
            r = orc.attn_surrogate(q, k, v, causal, scale, X=X, Bc=Bc, fallback=fb)
            _rel_close(r["o"], o_ref, 1e-12, f"per-row causal={causal} X={X} fallback={fb} O")
            _rel_close(r["lse"], lse_ref, 1e-12, f"per-row causal={causal} X={X} lse")
        r1 = orc.attn_surrogate(q, k, v, causal, scale, X=1, Bc=Bc)
        rf = orc.attn_surrogate(q, k, v, causal, scale, X=5, Bc=Bc, fallback=2)
        assert np.array_equal(r1["o"], rf["o"]), "FORCE must be the per-row recurrence"
        assert rf["switched"].all() and rf["n_tiles_per_row"] == rf["switched"].size


def _spiky(rng, BH, N, d, std, frac, logit, scale):
    """Logits of std `std`; in a fraction of rows one key raised by `logit`."""
    s = math.sqrt(std / (math.sqrt(d) * scale))
    q = rng.standard_normal((BH, N, d)) * s
    k = rng.standard_normal((BH, N, d)) * s
    v = rng.standard_normal((BH, N, d))
    for b in range(BH):
        rows = rng.choice(N, size=int(frac * N), replace=False)
        keys = rng.integers(0, N, size=rows.size)
        kk = k[b, keys]
        q[b, rows] += (logit / scale) * kk / np.sum(kk * kk, 1, keepdims=True)
    return q, k, v


def pin_fallback(orc):
    """With P~ stored as e4m3 (x 2^8), spiky rows next to flat rows make the
    surrogate flush whole rows (section A2, all-underflow); the per-row fallback
    (AUTO with tau = 12, or FORCE) removes the failure."""
    rng = np.random.default_rng(16)
    BH, N, d = 2, 256, 64
    scale = 1.0 / math.sqrt(d)
    q, k, v = _spiky(rng, BH, N, d, 8.0, 0.2, 40.0, scale)
    o_ref, lse_ref = orc.attn_exact(q, k, v, False, scale)
    off = orc.attn_surrogate(q, k, v, False, scale, X=32, Bc=64, p_round=2, p_shift=8)
    err_off = np.abs(off["o"] - o_ref).max(-1)
    assert (np.isneginf(off["lse"]).any() or err_off.max() > 0.1), "no failure without fallback"
    flushed = np.isneginf(off["lse"])
    assert np.all(off["o"][flushed] == 0.0), "flushed rows must give O = 0"
    for fb in (1, 2):
        r = orc.attn_surrogate(q, k, v, False, scale, X=32, Bc=64, fallback=fb, tau=12.0,
                               p_round=2, p_shift=8)
        assert r["switched"].sum() > 0, f"fallback={fb}: no tile switched"
        err = np.abs(r["o"] - o_ref)
        assert err.max() <= 6e-2, f"fallback={fb}: max err {err.max():.3e}"
        # e4m3 keeps 4 significant bits: each P~ is within 2^-4 relative, so
        # ln(l) is within ln(1 + 2^-4) < 0.065 of the exact value
        assert np.abs(r["lse"] - lse_ref).max() <= 0.065, f"fallback={fb} lse"
    # the same setting without spikes never switches and matches to P rounding
    # (non-causal: every row averages 256 keys, so e4m3 weight rounding averages out)
    q, k, v = (_rand(rng, BH, N, d) for _ in range(3))
    for causal in (False, True):
        r = orc.attn_surrogate(q, k, v, causal, scale, X=32, Bc=64, fallback=1, tau=12.0,
                               p_round=2, p_shift=8)
        o_ref, lse_ref = orc.attn_exact(q, k, v, causal, scale)
        assert r["switched"].sum() == 0, "switched on N(0,1) inputs"
        if not causal:
            assert np.abs(r["o"] - o_ref).max() <= 6e-2
        assert np.abs(r["lse"] - lse_ref).max() <= 0.065, "no-spike lse"
        # bf16 P rounding: same answer to bf16 precision
        rb = orc.attn_surrogate(q, k, v, causal, scale, X=32, Bc=64, p_round=1)
        assert np.abs(rb["o"] - o_ref).max() <= 1e-2


def pin_fallback_f16(orc):
    """fp16 P~ (x 2^15, normals down to 2^-14) flushes the flat rows of a tile that
    holds a spiked row (a gap of about 58 log2 units) without the fallback; AUTO
    at the fp16 default tau = 24 switches those tiles and recovers exact
    attention to fp16 precision, and N(0,1) inputs never switch."""
    rng = np.random.default_rng(16)
    BH, N, d = 2, 256, 64
    scale = 1.0 / math.sqrt(d)
    q, k, v = _spiky(rng, BH, N, d, 8.0, 0.2, 40.0, scale)
    o_ref, lse_ref = orc.attn_exact(q, k, v, False, scale)
    off = orc.attn_surrogate(q, k, v, False, scale, X=32, Bc=64, p_round=3, p_shift=15)
    flushed = np.isneginf(off["lse"])
    assert flushed.any(), "no row flushed without the fallback"
    assert np.all(off["o"][flushed] == 0.0), "flushed rows must give O = 0"
    r = orc.attn_surrogate(q, k, v, False, scale, X=32, Bc=64, fallback=1, tau=24.0,
                           p_round=3, p_shift=15)
    assert r["switched"].sum() > 0 and not np.isneginf(r["lse"]).any()
    # 11 significant bits: each P~ within 2^-11 relative, O a convex combination
    # of V rows with |v| < 8 moves by at most about 8 * 2^-11
    assert np.abs(r["o"] - o_ref).max() <= 8 * 2.0 ** -11
    assert np.abs(r["lse"] - lse_ref).max() <= math.log1p(2.0 ** -11)
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    for causal in (False, True):
        r = orc.attn_surrogate(q, k, v, causal, scale, X=32, Bc=64, fallback=1, tau=24.0,
                               p_round=3, p_shift=15)
        o_ref, lse_ref = orc.attn_exact(q, k, v, causal, scale)
        assert r["switched"].sum() == 0, "switched on N(0,1) inputs"
        assert np.abs(r["o"] - o_ref).max() <= 8 * 2.0 ** -11


def pin_rounding(orc):
    """Round-to-nearest-even models agree with torch's casts on float32 inputs."""
    rng = np.random.default_rng(17)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-3).astype(np.float32),
        (rng.standard_normal(2000) * 1e-37).astype(np.float32),      # bf16 subnormals
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want), "bf16 rounding differs from torch"
    y = np.concatenate([
        rng.uniform(-448, 448, 4000).astype(np.float32),
        (rng.standard_normal(3000) * 0.01).astype(np.float32),         # e4m3 subnormals
        np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 0.0], dtype=np.float32),  # ties
    ])
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.round_e4m3(y.astype(np.float64))
    assert np.array_equal(got, want), "e4m3 rounding differs from torch"
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = codes[np.isfinite(codes)]
    assert np.array_equal(orc.round_e4m3(codes), codes), "e4m3 codes are not fixed points"
    z = np.concatenate([
        (rng.standard_normal(4000) * 100).astype(np.float32),
        (rng.standard_normal(2000) * 1e-6).astype(np.float32),         # fp16 subnormals
        np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25,
                  65504.0, 65519.0, 65520.0, -65520.0, 2.0 ** -14], dtype=np.float32),  # ties, overflow
    ])
    want = torch.from_numpy(z).to(torch.float16).to(torch.float64).numpy()
    got = orc.round_f16(z.astype(np.float64))
    assert np.array_equal(got, want), "fp16 rounding differs from torch"


ALL_PINS = [pin_golden_closed_forms, pin_library_sdpa, pin_special_cases,
            pin_surrogate_equals_exact, pin_surrogate_invariants, pin_per_row_textbook,
            pin_fallback, pin_fallback_f16, pin_rounding]
