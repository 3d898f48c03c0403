/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of the two causal-attention forwards
 * that the HIP library computes.  It exists so that tests, the smoke check and
 * the benchmark's CPU-baseline leg have something independent to compare the
 * GPU against.  It shares no code, header, table or constant with the HIP
 * library, and no product code path may call it.
 *
 * Inputs are the exact values handed to the GPU: either fp32 arrays or bf16
 * bit patterns (uint16), widened exactly to double here.  Every sum, product,
 * log, sqrt, pow and exp below is carried out in double precision in the
 * order the definition states it (no tiling, no fusion, no reordering).
 *
 * Threshold Rectified Attention
 *   source: snap-research/TDA, page "triton_threshold_attention.py",
 *   module docstring (the formula out = ReLU(Q K^T - tau)^p V with
 *   tau(i) = beta*sqrt(2*log(i+1)/d)) and `_threshold_rela_fwd_kernel`
 *   (query position is 0-based, so the log takes position+1; natural log;
 *   d is the head dimension; key j contributes only when j <= i).
 *
 * NSA selection branch
 *   source: msb-msb/openbox-llm, page "nsa_selection_kernel.py", module
 *   docstring (GQA layout, kv head = h // G, slots of -1 are padding, causal
 *   j <= i, softmax, a query with no valid block outputs 0) and
 *   `selection_forward_reference` (the selected blocks form a SET: a block
 *   listed twice is attended once; scale = D^-0.5); `_selection_fwd_kernel`
 *   (lse = max + log(sum) over the scaled scores, natural log, with the
 *   finite sentinel -1e9 for an empty row).
 *
 * Threshold Rectified Attention backward
 *   source: the same page, `_threshold_rela_bwd_kernel_dq`,
 *   `_threshold_rela_bwd_kernel_dkv` and `ThresholdRelaFunction.backward`
 *   (gradients of q, k and v only; with x = q_i.k_j - tau_i the weight's
 *   derivative is p * max(x, 0)^(p-1) for x > 0 and 0 otherwise).
 *
 * NSA selection-branch backward
 *   source: the same page's forward (its attended set, scale and softmax) and
 *   its statement that the lse output feeds a backward pass that the page does
 *   not show; the gradients here are those of that forward's definition with
 *   respect to q, k and v (block_idx is an integer index, not differentiated).
 *
 * Threshold Differential Attention
 *   source: snap-research/TDA, page "triton_threshold_attention.py",
 *   `differential_threshold_rela_triton` (optionally L2-normalise q1, k1, q2,
 *   k2 along the head dimension; two Threshold Rectified Attention outputs
 *   over the same v, beta and p; combined as out1 - clamp(lambda, 0, 1)*out2)
 *   and torch.nn.functional.normalize's definition x / max(||x||_2, 1e-12).
 *
 * Threading: rows are independent; OpenMP spreads them over threads.  Each
 * row is computed by exactly one thread in a fixed order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes for the input arrays */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Widen element `idx` of an fp32 or bf16 array to double (exact). */
static double widen(const void *p, int dtype, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float *)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Threshold Rectified Attention forward for a list of output rows.
 *
 *   q, k, v : [B, H, T, D] dense row-major, fp32 or bf16 bits (dtype)
 *   rows    : flat row ids r = (b*H + h)*T + i, or NULL for all B*H*T rows
 *   out     : [nrows, D] doubles, row n holds out[rows[n], :]
 *
 *   out[b,h,i,:] = sum_{j=0..i} max(q_i . k_j - tau_i, 0)^p * v_j
 *   tau_i        = beta * sqrt(2 * ln(i + 1) / D)
 *
 * No 1/sqrt(D) scale, no softmax, no normalisation.  x^p is libm pow(); a
 * non-positive x contributes nothing (ReLU).  Returns 0, or -1 on bad args.
 */
int oracle_tra_rows(const void *q, const void *k, const void *v, int dtype,
                    int64_t B, int64_t H, int64_t T, int64_t D,
                    double beta, double p,
                    const int64_t *rows, int64_t nrows,
                    double *out, int nthreads) {
    if (!q || !k || !v || !out || B < 0 || H < 0 || T < 0 || D <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const int64_t total = B * H * T;
    if (!rows) nrows = total;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t n = 0; n < nrows; ++n) {
        const int64_t r = rows ? rows[n] : n;
        double *o = out + n * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (r < 0 || r >= total) { bad = 1; continue; }
        const int64_t bh = r / T, i = r % T;
        const int64_t head = bh * T * D;           /* start of this (b,h) slab */
        const double tau = beta * sqrt(2.0 * log((double)(i + 1)) / (double)D);
        for (int64_t j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int64_t d = 0; d < D; ++d)
                s += widen(q, dtype, head + i * D + d) * widen(k, dtype, head + j * D + d);
            const double x = s - tau;
            if (!(x > 0.0)) continue;
            const double w = pow(x, p);
            for (int64_t d = 0; d < D; ++d)
                o[d] += w * widen(v, dtype, head + j * D + d);
        }
    }
    return bad ? -1 : 0;
}

/*
 * NSA selection-branch forward for a list of output rows.
 *
 *   q         : [B, Hq, T, D]   fp32 or bf16 bits (dtype)
 *   k, v      : [B, Hkv, T, D]
 *   block_idx : [B, Hkv, T, S]  int32; any negative value is padding
 *   rows      : flat row ids r = (b*Hq + h)*T + i, or NULL for all rows
 *   out       : [nrows, D] doubles;  lse : [nrows] doubles (may be NULL)
 *
 * For query i of head h (group G = Hq/Hkv, kv head = h / G) the attended set
 * A is the union over slots of the tokens of block blk = block_idx[b,kv,i,s]
 * (tokens blk*bs .. blk*bs+bs-1) that satisfy j <= i.  A slot that is
 * negative or names a block at or past T/bs adds nothing; a block listed in
 * several slots is counted once.  Then, with scale = 1/sqrt(D),
 *
 *   s_j  = scale * (q_i . k_j)             for j in A
 *   out  = sum_j exp(s_j - M) v_j / sum_j exp(s_j - M),  M = max_j s_j
 *   lse  = M + ln(sum_j exp(s_j - M))      (= ln sum_j exp(s_j))
 *
 * and an empty A gives out = 0, lse = -1e9.  Keys are visited in increasing
 * position order.  Returns 0, or -1 on bad arguments.
 */
int oracle_nsa_rows(const void *q, const void *k, const void *v, int dtype,
                    const int32_t *block_idx,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                    int64_t bs, int64_t S,
                    const int64_t *rows, int64_t nrows,
                    double *out, double *lse, int nthreads) {
    if (!q || !k || !v || !block_idx || !out) return -1;
    if (B < 0 || Hq < 0 || Hkv <= 0 || T < 0 || D <= 0 || bs <= 0 || S < 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const int64_t G = Hq / Hkv;
    const int64_t nblk = T / bs;
    const int64_t total = B * Hq * T;
    const double scale = 1.0 / sqrt((double)D);
    if (!rows) nrows = total;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        unsigned char *chosen = (unsigned char *)calloc((size_t)(nblk > 0 ? nblk : 1), 1);
        double *sc = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        if (!chosen || !sc) bad = 1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < nrows; ++n) {
            if (!chosen || !sc) continue;
            const int64_t r = rows ? rows[n] : n;
            double *o = out + n * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            if (lse) lse[n] = -1e9;
            if (r < 0 || r >= total) { bad = 1; continue; }
            const int64_t bh = r / T, i = r % T;
            const int64_t b = bh / Hq, h = bh % Hq;
            const int64_t kvh = h / G;
            const int64_t qrow = (bh * T + i) * D;
            const int64_t kvslab = (b * Hkv + kvh) * T * D;
            const int32_t *slots = block_idx + ((b * Hkv + kvh) * T + i) * S;

            /* the set of selected blocks */
            memset(chosen, 0, (size_t)(nblk > 0 ? nblk : 1));
            for (int64_t s = 0; s < S; ++s) {
                const int64_t blk = slots[s];
                if (blk >= 0 && blk < nblk) chosen[blk] = 1;
            }
            /* scores over the attended tokens, increasing position */
            int64_t na = 0;
            double M = -INFINITY;
            for (int64_t blk = 0; blk < nblk; ++blk) {
                if (!chosen[blk]) continue;
                for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += widen(q, dtype, qrow + d) * widen(k, dtype, kvslab + j * D + d);
                    const double s = scale * dot;
                    sc[j] = s;
                    if (s > M) M = s;
                    ++na;
                }
            }
            if (na == 0) continue;                 /* empty row: 0 and -1e9 */
            double l = 0.0;
            for (int64_t blk = 0; blk < nblk; ++blk) {
                if (!chosen[blk]) continue;
                for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) {
                    const double e = exp(sc[j] - M);
                    l += e;
                    for (int64_t d = 0; d < D; ++d) o[d] += e * widen(v, dtype, kvslab + j * D + d);
                }
            }
            for (int64_t d = 0; d < D; ++d) o[d] /= l;
            if (lse) lse[n] = M + log(l);
        }
        free(chosen);
        free(sc);
    }
    return bad ? -1 : 0;
}

/* x rounded to the nearest value of the input dtype (ties to even): fp32, or
 * bfloat16 (8 significant bits, fp32's exponent range). */
static double round_to_dtype(double x, int dtype) {
    if (dtype == ORACLE_F32) return (double)(float)x;
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    const double m = frexp(x, &e);              /* x = m * 2^e, 0.5 <= |m| < 1 */
    if (e < -125) e = -125;                     /* below the normal range: fixed quantum */
    const double q = ldexp(x, 8 - e);           /* 8 significant bits before the point */
    const double r = nearbyint(q);              /* default rounding: to nearest, ties even */
    (void)m;
    return ldexp(r, e - 8);
}

/* Row `row` (D values) of a [.., D] array, widened; with `normalize` it is
 * normalised as torch.nn.functional.normalize(p=2, dim=-1) does on a tensor of
 * the input dtype: the norm is itself a value of that dtype (the exact 2-norm,
 * rounded once to nearest-even), clamped below at 1e-12 (as a value of that
 * dtype), and each quotient x / norm is rounded to the dtype.  The page
 * normalises tensors of the input dtype and hands the normalised tensors, in
 * that dtype, to the attention. */
static void load_row(const void *x, int dtype, int64_t row, int64_t D, int normalize,
                     double *dst) {
    double ss = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        dst[d] = widen(x, dtype, row * D + d);
        ss += dst[d] * dst[d];
    }
    if (!normalize) return;
    double nrm = round_to_dtype(sqrt(ss), dtype);
    const double eps = round_to_dtype(1e-12, dtype);
    if (nrm < eps) nrm = eps;
    for (int64_t d = 0; d < D; ++d) dst[d] = round_to_dtype(dst[d] / nrm, dtype);
}

/*
 * The normalised rows that the Threshold Differential Attention forward below
 * works on (normalize != 0): rows [nrows, D] of fp32 or bf16 bits in, doubles
 * out (each a value of the input dtype).  Exposed so that tests can compare the
 * normalisation on its own with torch's.  Returns 0, or -1 on bad arguments.
 */
int oracle_l2norm_rows(const void *x, int dtype, int64_t nrows, int64_t D, double *out) {
    if (!x || !out || nrows < 0 || D <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    for (int64_t r = 0; r < nrows; ++r) load_row(x, dtype, r, D, 1, out + r * D);
    return 0;
}

/*
 * Threshold Differential Attention forward for a list of output rows.
 *
 *   q1, q2, k1, k2, v : [B, H, T, D] dense row-major, fp32 or bf16 bits (dtype)
 *   rows              : flat row ids r = (b*H + h)*T + i, or NULL for all rows
 *   out               : [nrows, D] doubles
 *
 * With normalize != 0 every row of q1, q2, k1, k2 is first normalised as
 * load_row states: divided by its 2-norm rounded to the input dtype (at least
 * 1e-12), each quotient rounded to the dtype (bf16 or fp32, nearest-even), as
 * the page's normalised tensors are.  Then, the two paths
 * taken one after the other as the page does,
 *
 *   out1 = sum_{j<=i} max(q1_i . k1_j - tau_i, 0)^p v_j
 *   out2 = sum_{j<=i} max(q2_i . k2_j - tau_i, 0)^p v_j
 *   out  = out1 - min(max(lambda, 0), 1) * out2,   tau_i = beta*sqrt(2 ln(i+1)/D)
 *
 * Returns 0, or -1 on bad arguments.
 */
int oracle_tda_rows(const void *q1, const void *q2, const void *k1, const void *k2,
                    const void *v, int dtype,
                    int64_t B, int64_t H, int64_t T, int64_t D,
                    double beta, double lambda, double p, int normalize,
                    const int64_t *rows, int64_t nrows,
                    double *out, int nthreads) {
    if (!q1 || !q2 || !k1 || !k2 || !v || !out || B < 0 || H < 0 || T < 0 || D <= 0)
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const int64_t total = B * H * T;
    const double lam = lambda < 0.0 ? 0.0 : (lambda > 1.0 ? 1.0 : lambda);
    if (!rows) nrows = total;
    set_threads(nthreads);
    /* every key row as load_row gives it, computed once (the same values that
     * loading it again for each query would give) */
    double *nk1 = (double *)malloc(sizeof(double) * (size_t)(total * D));
    double *nk2 = (double *)malloc(sizeof(double) * (size_t)(total * D));
    if (total > 0 && (!nk1 || !nk2)) {
        free(nk1);
        free(nk2);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < total; ++r) {
        load_row(k1, dtype, r, D, normalize, nk1 + r * D);
        load_row(k2, dtype, r, D, normalize, nk2 + r * D);
    }
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
        double *buf = (double *)malloc(sizeof(double) * (size_t)(4 * D));
        if (!buf) bad = 1;
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < nrows; ++n) {
            if (!buf) continue;
            const int64_t r = rows ? rows[n] : n;
            double *o = out + n * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            if (r < 0 || r >= total) { bad = 1; continue; }
            const int64_t bh = r / T, i = r % T;
            double *qa = buf, *qb = buf + D;
            double *o1 = buf + 2 * D, *o2 = buf + 3 * D;
            load_row(q1, dtype, bh * T + i, D, normalize, qa);
            load_row(q2, dtype, bh * T + i, D, normalize, qb);
            const double tau = beta * sqrt(2.0 * log((double)(i + 1)) / (double)D);
            for (int64_t d = 0; d < D; ++d) o1[d] = o2[d] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                const double *ka = nk1 + (bh * T + j) * D;
                const double *kb = nk2 + (bh * T + j) * D;
                double s1 = 0.0, s2 = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    s1 += qa[d] * ka[d];
                    s2 += qb[d] * kb[d];
                }
                const double x1 = s1 - tau, x2 = s2 - tau;
                const double w1 = x1 > 0.0 ? pow(x1, p) : 0.0;
                const double w2 = x2 > 0.0 ? pow(x2, p) : 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    const double vd = widen(v, dtype, bh * T * D + j * D + d);
                    o1[d] += w1 * vd;
                    o2[d] += w2 * vd;
                }
            }
            for (int64_t d = 0; d < D; ++d) o[d] = o1[d] - lam * o2[d];
        }
        free(buf);
    }
    free(nk1);
    free(nk2);
    return bad ? -1 : 0;
}

/*
 * Threshold Rectified Attention backward, for a list of query rows (dq) and a
 * list of key rows (dk, dv).
 *
 *   q, k, v, dout : [B, H, T, D] dense row-major, fp32 or bf16 bits (dtype)
 *   qrows, nq     : flat query-row ids (b*H + h)*T + i, or NULL for all rows
 *   dq            : [nq, D] doubles (may be NULL to skip)
 *   krows, nk     : flat key-row ids (b*H + h)*T + j, or NULL for all rows
 *   dk, dv        : [nk, D] doubles (each may be NULL to skip)
 *
 * With x_ij = q_i . k_j - tau_i (tau_i = beta*sqrt(2 ln(i+1)/D)) and, for the
 * causal pairs j <= i with x_ij > 0,
 *   w_ij = x_ij^p,   g_ij = p * x_ij^(p-1),   a_ij = (dout_i . v_j) * g_ij
 * (pairs with x_ij <= 0 or j > i have w = a = 0):
 *   dq_i = sum_{j<=i} a_ij k_j,   dk_j = sum_{i>=j} a_ij q_i,   dv_j = sum_{i>=j} w_ij dout_i
 * Returns 0, or -1 on bad arguments.
 */
int oracle_tra_bwd_rows(const void *q, const void *k, const void *v, const void *dout,
                        int dtype, int64_t B, int64_t H, int64_t T, int64_t D,
                        double beta, double p,
                        const int64_t *qrows, int64_t nq, double *dq,
                        const int64_t *krows, int64_t nk, double *dk, double *dv,
                        int nthreads) {
    if (!q || !k || !v || !dout || B < 0 || H < 0 || T < 0 || D <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const int64_t total = B * H * T;
    if (!qrows) nq = total;
    if (!krows) nk = total;
    set_threads(nthreads);
    int bad = 0;
    if (dq) {
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
        for (int64_t n = 0; n < nq; ++n) {
            const int64_t r = qrows ? qrows[n] : n;
            double *o = dq + n * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            if (r < 0 || r >= total) { bad = 1; continue; }
            const int64_t bh = r / T, i = r % T, head = bh * T * D;
            const double tau = beta * sqrt(2.0 * log((double)(i + 1)) / (double)D);
            for (int64_t j = 0; j <= i; ++j) {
                double s = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    s += widen(q, dtype, head + i * D + d) * widen(k, dtype, head + j * D + d);
                    dp += widen(dout, dtype, head + i * D + d) * widen(v, dtype, head + j * D + d);
                }
                const double x = s - tau;
                if (!(x > 0.0)) continue;
                const double a = dp * p * pow(x, p - 1.0);
                for (int64_t d = 0; d < D; ++d) o[d] += a * widen(k, dtype, head + j * D + d);
            }
        }
    }
    if (dk || dv) {
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
        for (int64_t n = 0; n < nk; ++n) {
            const int64_t r = krows ? krows[n] : n;
            if (dk) for (int64_t d = 0; d < D; ++d) dk[n * D + d] = 0.0;
            if (dv) for (int64_t d = 0; d < D; ++d) dv[n * D + d] = 0.0;
            if (r < 0 || r >= total) { bad = 1; continue; }
            const int64_t bh = r / T, j = r % T, head = bh * T * D;
            for (int64_t i = j; i < T; ++i) {
                const double tau = beta * sqrt(2.0 * log((double)(i + 1)) / (double)D);
                double s = 0.0, dp = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    s += widen(q, dtype, head + i * D + d) * widen(k, dtype, head + j * D + d);
                    dp += widen(dout, dtype, head + i * D + d) * widen(v, dtype, head + j * D + d);
                }
                const double x = s - tau;
                if (!(x > 0.0)) continue;
                const double w = pow(x, p);
                const double a = dp * p * pow(x, p - 1.0);
                for (int64_t d = 0; d < D; ++d) {
                    if (dk) dk[n * D + d] += a * widen(q, dtype, head + i * D + d);
                    if (dv) dv[n * D + d] += w * widen(dout, dtype, head + i * D + d);
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* The attended set of row (b, kv, i): chosen[blk] for each selected block id in
 * range (duplicates once); returns the number of attended tokens (j <= i). */
static int64_t nsa_attended(const int32_t *slots, int64_t S, int64_t nblk, int64_t bs,
                            int64_t i, unsigned char *chosen) {
    memset(chosen, 0, (size_t)(nblk > 0 ? nblk : 1));
    for (int64_t s = 0; s < S; ++s) {
        const int64_t blk = slots[s];
        if (blk >= 0 && blk < nblk) chosen[blk] = 1;
    }
    int64_t na = 0;
    for (int64_t blk = 0; blk < nblk; ++blk)
        if (chosen[blk])
            for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) ++na;
    return na;
}

/* Whether block blk (0 <= blk < nblk) is in the attended set of a query row whose
 * S slots are given: the membership test of nsa_attended for one block, without
 * building the whole set (j <= i holds wherever the key-row loop asks). */
static int nsa_slot_holds(const int32_t *slots, int64_t S, int64_t blk) {
    for (int64_t s = 0; s < S; ++s)
        if (slots[s] == blk) return 1;
    return 0;
}

/* Softmax statistics of query row (b, h, i) over its attended set:
 * M = max_j s_j and l = sum_j exp(s_j - M), s_j = scale * q_i . k_j; and
 * delta = sum_j P_j (dout_i . v_j) with P_j = exp(s_j - M) / l.  Returns 0 if
 * the set is empty (then nothing flows through the row). */
static int nsa_row_stats(const void *q, const void *k, const void *v, const void *dout,
                         int dtype, const unsigned char *chosen, int64_t nblk, int64_t bs,
                         int64_t i, int64_t qrow, int64_t kvslab, int64_t D, double scale,
                         double *M, double *l, double *delta) {
    double m = -INFINITY;
    int64_t na = 0;
    for (int64_t blk = 0; blk < nblk; ++blk) {
        if (!chosen[blk]) continue;
        for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += widen(q, dtype, qrow + d) * widen(k, dtype, kvslab + j * D + d);
            if (scale * dot > m) m = scale * dot;
            ++na;
        }
    }
    if (na == 0) return 0;
    double sum = 0.0, dl = 0.0;
    for (int64_t blk = 0; blk < nblk; ++blk) {
        if (!chosen[blk]) continue;
        for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) {
            double dot = 0.0, dp = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                dot += widen(q, dtype, qrow + d) * widen(k, dtype, kvslab + j * D + d);
                dp += widen(dout, dtype, qrow + d) * widen(v, dtype, kvslab + j * D + d);
            }
            const double e = exp(scale * dot - m);
            sum += e;
            dl += e * dp;
        }
    }
    *M = m;
    *l = sum;
    *delta = dl / sum;
    return 1;
}

/*
 * NSA selection-branch backward for a list of query rows (dq) and key rows (dk, dv).
 *
 *   q, dout    : [B, Hq, T, D];  k, v : [B, Hkv, T, D]  (dtype)
 *   block_idx  : [B, Hkv, T, S] int32, as for the forward
 *   qrows, nq  : flat rows (b*Hq + h)*T + i (NULL: all), dq [nq, D] (may be NULL)
 *   krows, nk  : flat rows (b*Hkv + kv)*T + j (NULL: all), dk, dv [nk, D] (may be NULL)
 *
 * With A_i the attended set of row i (as in the forward), s_ij = scale q_i.k_j,
 * P_ij = softmax over A_i, dP_ij = dout_i . v_j, delta_i = sum_{j in A_i} P_ij dP_ij
 * and dS_ij = P_ij (dP_ij - delta_i), per query head h of kv group kv = h / G:
 *   dq_i   = scale * sum_{j in A_i} dS_ij k_j
 *   dk_j   = scale * sum_{h in group} sum_{i : j in A_i} dS_ij q_i
 *   dv_j   =         sum_{h in group} sum_{i : j in A_i} P_ij dout_i
 * A row with an empty set contributes nothing.  Returns 0, or -1 on bad args.
 */
int oracle_nsa_bwd_rows(const void *q, const void *k, const void *v, const void *dout,
                        int dtype, const int32_t *block_idx,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D,
                        int64_t bs, int64_t S,
                        const int64_t *qrows, int64_t nq, double *dq,
                        const int64_t *krows, int64_t nk, double *dk, double *dv,
                        int nthreads) {
    if (!q || !k || !v || !dout || !block_idx) return -1;
    if (B < 0 || Hq < 0 || Hkv <= 0 || T < 0 || D <= 0 || bs <= 0 || S < 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    const int64_t G = Hq / Hkv, nblk = T / bs;
    const double scale = 1.0 / sqrt((double)D);
    if (!qrows) nq = B * Hq * T;
    if (!krows) nk = B * Hkv * T;
    set_threads(nthreads);
    /* every query row's (M, l, delta), computed once per call by nsa_row_stats (the
     * same values that computing them again for each query or key row would give);
     * l = 0 marks a row with an empty set */
    double *stats = NULL;
    if (dq || dk || dv) {
        stats = (double *)malloc(sizeof(double) * (size_t)(3 * B * Hq * T + 1));
        if (!stats) return -1;
    }
    int bad = 0;
    if (stats) {
#pragma omp parallel reduction(| : bad)
        {
            unsigned char *chosen = (unsigned char *)calloc((size_t)(nblk > 0 ? nblk : 1), 1);
            if (!chosen) bad = 1;
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < B * Hq * T; ++r) {
                if (!chosen) continue;
                const int64_t bh = r / T, i = r % T, b = bh / Hq, h = bh % Hq, kv = h / G;
                const int64_t qrow = (bh * T + i) * D, kvslab = (b * Hkv + kv) * T * D;
                nsa_attended(block_idx + ((b * Hkv + kv) * T + i) * S, S, nblk, bs, i, chosen);
                double M = 0.0, l = 0.0, delta = 0.0;
                if (!nsa_row_stats(q, k, v, dout, dtype, chosen, nblk, bs, i, qrow, kvslab, D,
                                   scale, &M, &l, &delta))
                    l = 0.0;
                stats[3 * r] = M;
                stats[3 * r + 1] = l;
                stats[3 * r + 2] = delta;
            }
            free(chosen);
        }
        if (bad) {
            free(stats);
            return -1;
        }
    }
#pragma omp parallel reduction(| : bad)
    {
        unsigned char *chosen = (unsigned char *)calloc((size_t)(nblk > 0 ? nblk : 1), 1);
        if (!chosen) bad = 1;
        if (dq) {
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < nq; ++n) {
                if (!chosen) continue;
                const int64_t r = qrows ? qrows[n] : n;
                double *o = dq + n * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                if (r < 0 || r >= B * Hq * T) { bad = 1; continue; }
                const int64_t bh = r / T, i = r % T, b = bh / Hq, h = bh % Hq, kv = h / G;
                const int64_t qrow = (bh * T + i) * D, kvslab = (b * Hkv + kv) * T * D;
                nsa_attended(block_idx + ((b * Hkv + kv) * T + i) * S, S, nblk, bs, i, chosen);
                const double M = stats[3 * r], l = stats[3 * r + 1], delta = stats[3 * r + 2];
                if (l == 0.0) continue;
                for (int64_t blk = 0; blk < nblk; ++blk) {
                    if (!chosen[blk]) continue;
                    for (int64_t j = blk * bs; j < (blk + 1) * bs && j <= i; ++j) {
                        double dot = 0.0, dp = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            dot += widen(q, dtype, qrow + d) * widen(k, dtype, kvslab + j * D + d);
                            dp += widen(dout, dtype, qrow + d) * widen(v, dtype, kvslab + j * D + d);
                        }
                        const double P = exp(scale * dot - M) / l;
                        const double ds = P * (dp - delta);
                        for (int64_t d = 0; d < D; ++d)
                            o[d] += scale * ds * widen(k, dtype, kvslab + j * D + d);
                    }
                }
            }
        }
        if (dk || dv) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t n = 0; n < nk; ++n) {
                if (!chosen) continue;
                const int64_t r = krows ? krows[n] : n;
                if (dk) for (int64_t d = 0; d < D; ++d) dk[n * D + d] = 0.0;
                if (dv) for (int64_t d = 0; d < D; ++d) dv[n * D + d] = 0.0;
                if (r < 0 || r >= B * Hkv * T) { bad = 1; continue; }
                const int64_t bkv = r / T, j = r % T, b = bkv / Hkv, kv = bkv % Hkv;
                const int64_t kvslab = bkv * T * D, blk = j / bs;
                if (blk >= nblk) continue;
                for (int64_t i = j; i < T; ++i) {
                    if (!nsa_slot_holds(block_idx + (bkv * T + i) * S, S, blk)) continue;
                    for (int64_t g = 0; g < G; ++g) {
                        const int64_t h = kv * G + g;
                        const int64_t qr = (b * Hq + h) * T + i, qrow = qr * D;
                        const double M = stats[3 * qr], l = stats[3 * qr + 1];
                        const double delta = stats[3 * qr + 2];
                        if (l == 0.0) continue;
                        double dot = 0.0, dp = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            dot += widen(q, dtype, qrow + d) * widen(k, dtype, kvslab + j * D + d);
                            dp += widen(dout, dtype, qrow + d) * widen(v, dtype, kvslab + j * D + d);
                        }
                        const double P = exp(scale * dot - M) / l;
                        const double ds = P * (dp - delta);
                        for (int64_t d = 0; d < D; ++d) {
                            if (dk) dk[n * D + d] += scale * ds * widen(q, dtype, qrow + d);
                            if (dv) dv[n * D + d] += P * widen(dout, dtype, qrow + d);
                        }
                    }
                }
            }
        }
        free(chosen);
    }
    free(stats);
    return bad ? -1 : 0;
}
