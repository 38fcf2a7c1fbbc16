/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the fused attention forward pass
 * and for the tensorized online softmax (surrogate-maximum recurrence).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code, header,
 * table or helper with the GPU path, and the GPU path never calls it.
 *
 * Sources (the pages are cited by title and section):
 *   [FA-T]  "FlashAttention-T: Towards Fully Tensorized Attention by Exploiting
 *           Tensor-Vector Parallelism" (papercache deepnotes summary).
 *     - section A3 "fused attention algorithm flow", Fig 2(a): the per-block
 *       iteration (1) logits S, (2) row max m, (3)(5)(6) exponentiate with m and
 *       m_old, (4) rescale O, (7) update row sum l, (8) accumulate P~ V into O.
 *     - section A2 "surrogate maximum": m^[i] is the largest running row maximum
 *       over the X-row tile that holds row i (tile size X, e.g. 16 or 64).
 *     - section A2 "numerical stability guarantees": m^ >= m makes every
 *       exponential <= 1 (no overflow); all-underflow of a row is possible for
 *       extreme inputs, and an implementation may fall back to per-row (vector)
 *       computation.
 *     - section A2 "algorithm flow" (Algorithm 1): step 1 tile max, steps 2-3
 *       O <- exp(m^_old - m^) O, steps 4-5 Z <- log2(e) S - log2(e) m^,
 *       step 6 P~ <- exp2(Z), step 7 row-sum update of l.
 *     - section A4 "numerical stability and accuracy", Fig 11: the method is
 *       judged against an FP64 reference attention.
 *
 * Readings where the pages are silent or garbled (each is also listed in the
 * design notes of the repository):
 *   R-1  the tile of row i is the half-open range [floor(i/X)X, min(floor(i/X)X+X, N)),
 *        so the last tile may be partial;
 *   R-2  m^ is the maximum over the tile's rows of their running row maxima, hence
 *        non-decreasing from block to block;
 *   R-3  the term subtracted in steps 4-5 is the surrogate m^ (the step assigns it);
 *   R-4  the softmax scale multiplies the raw dot products: c = scale*log2(e),
 *        Z = c*r - c*m^ on raw dot products r, scale > 0;
 *   R-6  l <- alpha*l + rowsum(P~) with the same alpha as O (Fig 2(a) step 7);
 *   R-7  O = O/l and lse = scale*m^ + ln(l) = ln sum_j exp(scale*<q_i,k_j>);
 *   R-8  causal = key j <= query i (square, top-left aligned); masked logits are
 *        -inf before any max; blocks with no valid entry for the tile are skipped;
 *   R-10 the optional fallback: before exponentiating a block, a tile whose gap
 *        c*(m^_new - min_i m_i) exceeds tau switches (for good) to the per-row
 *        recurrence; FORCE uses the per-row recurrence from the first block;
 *        with the fallback OFF a row whose exponentials all flushed to zero gets
 *        O = 0 and lse = -inf.
 *
 * Memory layout: every tensor is contiguous row-major fp64; q, k, v, o are
 * [BH][N][d] (B and H folded into BH = B*H; head bh = b*H + h), lse is [BH][N].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI_VERSION 1

int oracle_abi_version(void) { return ORACLE_ABI_VERSION; }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* ------------------------------------------------------------------------- */
/* Rounding models for the P~ operand fed to the P~V product.                 */
/* Written from the number formats' definitions (round to nearest, ties to    */
/* even); used only when a caller asks the surrogate recurrence to model the  */
/* precision of the matrix-unit operand.                                      */
/* ------------------------------------------------------------------------- */

/* bfloat16: 8 significant bits, exponent range of binary32 (min normal 2^-126,
 * subnormal spacing 2^-133, largest finite (2 - 2^-7) * 2^127). */
double oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    double ax = fabs(x), r;
    if (ax < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(ax, 133)), -133);
    } else {
        int e;
        double f = frexp(ax, &e);           /* ax = f * 2^e, f in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(f, 8)), e - 8);
        if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) r = INFINITY;
    }
    return x < 0 ? -r : r;
}

/* OCP float8 e4m3 ("fn": no infinities): 4 significant bits, exponent bias 7,
 * min normal 2^-6, subnormal spacing 2^-9, largest finite 448.  Values beyond
 * 448 saturate to 448 (the model is used only on values the generators keep in
 * range). */
double oracle_round_e4m3(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    double ax = fabs(x), r;
    if (ax < ldexp(1.0, -6)) {
        r = ldexp(nearbyint(ldexp(ax, 9)), -9);
    } else {
        int e;
        double f = frexp(ax, &e);
        r = ldexp(nearbyint(ldexp(f, 4)), e - 4);
    }
    if (r > 448.0) r = 448.0;
    return x < 0 ? -r : r;
}

/* IEEE binary16: 11 significant bits, min normal 2^-14, subnormal spacing
 * 2^-24, largest finite 65504; values that round past it become infinite. */
double oracle_round_f16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    double ax = fabs(x), r;
    if (ax < ldexp(1.0, -14)) {
        r = ldexp(nearbyint(ldexp(ax, 24)), -24);
    } else {
        int e;
        double f = frexp(ax, &e);
        r = ldexp(nearbyint(ldexp(f, 11)), e - 11);
        if (r > 65504.0) r = INFINITY;
    }
    return x < 0 ? -r : r;
}

/* p_round: 0 = exact (fp64), 1 = bf16, 2 = e4m3, 3 = fp16, after multiplying
 * by 2^p_shift */
static double round_p(double p, int p_round, int p_shift)
{
    switch (p_round) {
    case 1: return oracle_round_bf16(ldexp(p, p_shift));
    case 2: return oracle_round_e4m3(ldexp(p, p_shift));
    case 3: return oracle_round_f16(ldexp(p, p_shift));
    default: return ldexp(p, p_shift);
    }
}

static int key_valid(int64_t i, int64_t j, int causal) { return !causal || j <= i; }

static double dot(const double* a, const double* b, int64_t d)
{
    double s = 0.0;
    for (int64_t t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/* ------------------------------------------------------------------------- */
/* O-1: exact attention, the plain definition (Fig 2(a) problem statement;    */
/* Fig 11's FP64 reference).  For each selected row i of head bh:             */
/*   s_j  = scale * <q_i, k_j>      for valid keys j (all j, or j <= i causal) */
/*   m    = max_j s_j                                                         */
/*   e_j  = exp(s_j - m),  l = sum_j e_j                                      */
/*   o_i  = sum_j e_j v_j / l,  lse_i = m + ln l                              */
/* rows == NULL selects every row and writes o as [BH][N][d], lse as [BH][N]; */
/* otherwise rows[r] = bh*N + i and o is [nrows][d], lse is [nrows].          */
/* Returns 0, or -1 on a bad argument.                                        */
/* ------------------------------------------------------------------------- */
int oracle_attn_exact(const double* q, const double* k, const double* v,
                      int64_t BH, int64_t N, int64_t d, int causal, double scale,
                      const int64_t* rows, int64_t nrows,
                      double* o, double* lse, int nthreads)
{
    if (BH < 0 || N < 0 || d < 1 || !(scale > 0.0) || !isfinite(scale)) return -1;
    int64_t total = rows ? nrows : BH * N;
    if (total < 0) return -1;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= BH * N) return -1;
    }
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double* e = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!e) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < total; ++r) {
            if (!e) continue;
            int64_t flat = rows ? rows[r] : r;
            int64_t bh = flat / N, i = flat % N;
            const double* qi = q + (bh * N + i) * d;
            const double* kh = k + bh * N * d;
            const double* vh = v + bh * N * d;
            double m = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                if (!key_valid(i, j, causal)) { e[j] = -INFINITY; continue; }
                e[j] = scale * dot(qi, kh + j * d, d);
                if (e[j] > m) m = e[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                e[j] = key_valid(i, j, causal) ? exp(e[j] - m) : 0.0;
                l += e[j];
            }
            double* oi = o + r * d;
            for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                if (e[j] == 0.0) continue;
                const double* vj = vh + j * d;
                for (int64_t t = 0; t < d; ++t) oi[t] += e[j] * vj[t];
            }
            for (int64_t t = 0; t < d; ++t) oi[t] /= l;
            lse[r] = m + log(l);
        }
        free(e);
    }
    return err ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* O-2: Algorithm 1, the tensorized online softmax, run block by block in the */
/* pages' order, one X-row tile at a time (section A2).                       */
/*                                                                            */
/* Work is in raw dot products r_ij = <q_i, k_j> (masked: -inf) and the base-2 */
/* constant c = scale*log2(e).  Per tile T and per key block J (in `order`,   */
/* default ascending, skipping blocks with no valid entry for T):             */
/*   m_i   <- max(m_i, max_{j in J} r_ij)                   running row max   */
/*   SURROGATE mode:                                                          */
/*     m^_new <- max_{i in T} m_i                           step 1 (tilemax)  */
/*     [fallback AUTO: if c*(m^_new - min_i m_i) > tau, switch T to PER_ROW   */
/*      with ref_i <- m^ (state is relative to the old m^)]                   */
/*     alpha <- exp2(c*(m^ - m^_new)) (0 on the first block)  steps 2-3       */
/*     O_i <- alpha O_i, l_i <- alpha l_i, m^ <- m^_new                       */
/*     Z_ij <- c*r_ij - c*m^                                  steps 4-5       */
/*     P_ij <- round(exp2(Z_ij))                              step 6          */
/*   PER_ROW mode (the textbook recurrence, per row):                         */
/*     alpha_i <- exp2(c*(ref_i - m_i)); O_i, l_i scaled; ref_i <- m_i        */
/*     P_ij <- round(exp2(c*r_ij - c*ref_i))                                  */
/*   l_i <- l_i + sum_j P_ij                                  step 7          */
/*   O_i <- O_i + sum_j P_ij v_j                              Fig 2(a) (8)    */
/* End: o_i = O_i / l_i, lse_i = scale*ref_i + ln(l_i) - p_shift*ln 2, with   */
/* ref_i = m^ in SURROGATE mode; a row with l_i = 0 gets o_i = 0, lse = -inf. */
/*                                                                            */
/* Arguments                                                                  */
/*   X        tile rows (>= 1; X = 1 is the per-row recurrence)               */
/*   Bc       keys per block (>= 1)                                           */
/*   order    NULL or a permutation of 0..ceil(N/Bc)-1: block visiting order  */
/*   fallback 0 OFF, 1 AUTO (threshold tau, in log2 units), 2 FORCE          */
/*   p_round  0 exact, 1 bf16, 2 e4m3, 3 fp16 -- rounding of P~ (x 2^p_shift)  */
/* Outputs (any may be NULL except o and lse)                                  */
/*   o [BH][N][d], lse [BH][N]                                                */
/*   ref_out [BH][N]  final reference max of each row (raw dot-product units) */
/*   gap_out [BH][N]  largest c*(m^ - m_i) seen by the row over the blocks    */
/*   switched [BH][ceil(N/X)]  1 where the tile ended in PER_ROW mode         */
/*   counters[4]: {m^ < m_i events, Z > 0 events, rows with l > 0 whose o or   */
/*                 lse is not finite, tiles that ended in PER_ROW mode}        */
/* Returns 0, -1 on a bad argument, -2 on allocation failure.                 */
/* ------------------------------------------------------------------------- */
enum { MODE_SURROGATE = 0, MODE_PER_ROW = 1 };

int oracle_attn_surrogate(const double* q, const double* k, const double* v,
                          int64_t BH, int64_t N, int64_t d, int causal, double scale,
                          int64_t X, int64_t Bc, const int64_t* order,
                          int fallback, double tau, int p_round, int p_shift,
                          double* o, double* lse,
                          double* ref_out, double* gap_out, uint8_t* switched,
                          int64_t* counters, int nthreads)
{
    if (BH < 0 || N < 0 || d < 1 || X < 1 || Bc < 1) return -1;
    if (!(scale > 0.0) || !isfinite(scale)) return -1;
    if (fallback < 0 || fallback > 2 || p_round < 0 || p_round > 3) return -1;
    const int64_t nblk = (N + Bc - 1) / Bc;
    const int64_t ntile = (N + X - 1) / X;
    if (order) {
        /* must be a permutation */
        uint8_t* seen = (uint8_t*)calloc((size_t)(nblk > 0 ? nblk : 1), 1);
        if (!seen) return -2;
        int bad = 0;
        for (int64_t b = 0; b < nblk; ++b) {
            if (order[b] < 0 || order[b] >= nblk || seen[order[b]]) { bad = 1; break; }
            seen[order[b]] = 1;
        }
        free(seen);
        if (bad) return -1;
    }
    const double c = scale * 1.4426950408889634073599246810018921; /* scale*log2(e) */
    int64_t cnt_mhat = 0, cnt_z = 0, cnt_nonfinite = 0, cnt_switch = 0;
    set_threads(nthreads);
    int err = 0;

#pragma omp parallel reduction(+:cnt_mhat, cnt_z, cnt_nonfinite, cnt_switch)
    {
        double* r   = (double*)malloc(sizeof(double) * (size_t)(X * Bc));
        double* m   = (double*)malloc(sizeof(double) * (size_t)X);
        double* ref = (double*)malloc(sizeof(double) * (size_t)X);
        double* l   = (double*)malloc(sizeof(double) * (size_t)X);
        double* gap = (double*)malloc(sizeof(double) * (size_t)X);
        double* O   = (double*)malloc(sizeof(double) * (size_t)(X * d));
        const int ok = r && m && ref && l && gap && O;
        if (!ok) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t tt = 0; tt < BH * ntile; ++tt) {
            if (!ok) continue;
            const int64_t bh = tt / ntile, t = tt % ntile;
            const int64_t i0 = t * X, i1 = (i0 + X < N) ? i0 + X : N, nt = i1 - i0;
            const double* kh = k + bh * N * d;
            const double* vh = v + bh * N * d;
            double mhat = -INFINITY;
            int mode = (fallback == 2) ? MODE_PER_ROW : MODE_SURROGATE;
            for (int64_t a = 0; a < nt; ++a) {
                m[a] = -INFINITY; ref[a] = -INFINITY; l[a] = 0.0; gap[a] = 0.0;
                for (int64_t u = 0; u < d; ++u) O[a * d + u] = 0.0;
            }
            for (int64_t bi = 0; bi < nblk; ++bi) {
                const int64_t jb = order ? order[bi] : bi;
                const int64_t j0 = jb * Bc, j1 = (j0 + Bc < N) ? j0 + Bc : N, nb = j1 - j0;
                /* R-8: skip a block with no valid (i, j) for any row of the tile */
                int any = 0;
                for (int64_t a = 0; a < nt && !any; ++a)
                    for (int64_t jj = 0; jj < nb && !any; ++jj)
                        any = key_valid(i0 + a, j0 + jj, causal);
                if (!any) continue;

                /* logits of the block and running row maxima (Fig 2(a) (1), (2)) */
                for (int64_t a = 0; a < nt; ++a) {
                    const double* qi = q + (bh * N + i0 + a) * d;
                    for (int64_t jj = 0; jj < nb; ++jj) {
                        double x = key_valid(i0 + a, j0 + jj, causal)
                                       ? dot(qi, kh + (j0 + jj) * d, d) : -INFINITY;
                        r[a * Bc + jj] = x;
                        if (x > m[a]) m[a] = x;
                    }
                }

                if (mode == MODE_SURROGATE) {
                    /* step 1: surrogate max = max of the tile's running row maxima */
                    double mhat_new = -INFINITY, mmin = INFINITY;
                    for (int64_t a = 0; a < nt; ++a) {
                        if (m[a] > mhat_new) mhat_new = m[a];
                        if (m[a] > -INFINITY && m[a] < mmin) mmin = m[a];
                    }
                    for (int64_t a = 0; a < nt; ++a) {
                        if (mhat_new < m[a]) cnt_mhat++;          /* m^ >= m must hold */
                        if (m[a] > -INFINITY) {
                            double g = c * (mhat_new - m[a]);
                            if (g > gap[a]) gap[a] = g;
                        }
                    }
                    if (fallback == 1 && mmin < INFINITY && c * (mhat_new - mmin) > tau) {
                        /* all-underflow risk: leave the surrogate for this tile */
                        mode = MODE_PER_ROW;
                        for (int64_t a = 0; a < nt; ++a) ref[a] = mhat;
                    } else {
                        /* steps 2-3: one uniform rescale factor for the whole tile */
                        double alpha = (mhat == -INFINITY) ? 0.0 : exp2(c * (mhat - mhat_new));
                        for (int64_t a = 0; a < nt; ++a) {
                            l[a] *= alpha;
                            for (int64_t u = 0; u < d; ++u) O[a * d + u] *= alpha;
                        }
                        mhat = mhat_new;
                        /* steps 4-6: Z = c*r - c*m^, P~ = exp2(Z) */
                        for (int64_t a = 0; a < nt; ++a)
                            for (int64_t jj = 0; jj < nb; ++jj) {
                                double x = r[a * Bc + jj];
                                if (x == -INFINITY) { r[a * Bc + jj] = 0.0; continue; }
                                double z = c * x - c * mhat;
                                if (z > 0.0) cnt_z++;               /* no overflow: Z <= 0 */
                                r[a * Bc + jj] = round_p(exp2(z), p_round, p_shift);
                            }
                    }
                }
                if (mode == MODE_PER_ROW) {
                    /* the per-row recurrence (what the fallback and X = 1 compute) */
                    for (int64_t a = 0; a < nt; ++a) {
                        double alpha = (ref[a] == -INFINITY) ? 0.0 : exp2(c * (ref[a] - m[a]));
                        if (m[a] == -INFINITY) alpha = 1.0;        /* row has no key yet */
                        l[a] *= alpha;
                        for (int64_t u = 0; u < d; ++u) O[a * d + u] *= alpha;
                        ref[a] = m[a];
                        for (int64_t jj = 0; jj < nb; ++jj) {
                            double x = r[a * Bc + jj];
                            if (x == -INFINITY) { r[a * Bc + jj] = 0.0; continue; }
                            double z = c * x - c * ref[a];
                            if (z > 0.0) cnt_z++;
                            r[a * Bc + jj] = round_p(exp2(z), p_round, p_shift);
                        }
                    }
                }
                /* step 7 and Fig 2(a) (8): l += rowsum(P~), O += P~ V */
                for (int64_t a = 0; a < nt; ++a)
                    for (int64_t jj = 0; jj < nb; ++jj) {
                        double p = r[a * Bc + jj];
                        if (p == 0.0) continue;
                        l[a] += p;
                        const double* vj = vh + (j0 + jj) * d;
                        for (int64_t u = 0; u < d; ++u) O[a * d + u] += p * vj[u];
                    }
            }
            /* final normalisation and log-sum-exp (reading R-7) */
            for (int64_t a = 0; a < nt; ++a) {
                const int64_t row = bh * N + i0 + a;
                const double rf = (mode == MODE_SURROGATE) ? mhat : ref[a];
                double* oi = o + row * d;
                if (l[a] > 0.0) {
                    for (int64_t u = 0; u < d; ++u) oi[u] = O[a * d + u] / l[a];
                    lse[row] = scale * rf + log(l[a]) - p_shift * 0.69314718055994530941723212145818;
                    int bad = !isfinite(lse[row]);
                    for (int64_t u = 0; u < d; ++u) bad |= !isfinite(oi[u]);
                    cnt_nonfinite += bad;
                } else {
                    for (int64_t u = 0; u < d; ++u) oi[u] = 0.0;
                    lse[row] = -INFINITY;
                }
                if (ref_out) ref_out[row] = rf;
                if (gap_out) gap_out[row] = gap[a];
            }
            if (switched) switched[bh * ntile + t] = (uint8_t)(mode == MODE_PER_ROW);
            cnt_switch += (mode == MODE_PER_ROW);
        }
        free(r); free(m); free(ref); free(l); free(gap); free(O);
    }
    if (err) return -2;
    if (counters) {
        counters[0] = cnt_mhat; counters[1] = cnt_z;
        counters[2] = cnt_nonfinite; counters[3] = cnt_switch;
    }
    return 0;
}
