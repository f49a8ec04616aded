/*
 * lssar_ref.c -- fp64 CPU oracle for LSSAR causal attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline of the bench; never by the HIP library, and it shares no code
 * with it.
 *
 * Source: paper note "Softplus Attention with Re-weighting Boosts Length
 * Extrapolation in Large Language Models" (papernotes.org, ICML 2026),
 * section Method details.  The steps below follow that section's order:
 *
 *   Overall framework + Key design 1 (LSSA, the normalisation stage):
 *     Q_i <- Q_i/|Q_i|_2,  K_j <- K_j/|K_j|_2
 *     A   = Softplus((log d . log N) (.) Q K^T) (.) M'
 *           N: L x L, every element of row i equals i; M': lower triangle 1
 *     A_i <- A_i / |A_i|_1
 *   Key design 2 (re-weighting, the sharpening stage):
 *     A   <- ReLU^p(A (.) N - O),  O = ones except its first 3 rows = 0
 *     A_i <- A_i / |A_i|_1
 *   Key design 3 (integration): the result replaces Softmax(.), so the
 *     attention output is A V; the mask multiplies (0/1) instead of adding
 *     -inf because Softplus is non-negative.
 *
 * Readings where the note is silent or loose (each one is a choice):
 *   R1  "log" is the natural logarithm; d is the head dimension.
 *   R2  Row index i of N is 1-based (row i attends to i tokens), so row 1
 *       has scale log 1 = 0.
 *   R3  No 1/sqrt(d) temperature: log d . log i replaces it.
 *   R4  Softplus(x) = log(1 + e^x), beta = 1, no linear cut-over.
 *   R5  M' multiplies AFTER Softplus: a masked entry is exactly 0 and adds
 *       nothing to the row's L1 norm.
 *   R6  A zero row of Q or K is normalised with its norm clamped to 1e-12.
 *   R7  o_i = 0 for rows i = 1, 2, 3 and 1 for i >= 4, at every length.
 *   R8  Stage 2 acts on the stage-1 L1-normalised A.
 *   R9  p is an integer >= 1; ReLU(0)^p = 0.
 *   R10 Degenerate rows: when m_i = max_j (i A_ij - o_i) <= eps, every
 *       ReLU^p entry is (numerically) zero and the stage-2 L1 normalisation
 *       has no meaningful value; the output row is then 0.  This is the
 *       scale-invariant form of clamping the stage-2 denominator (the page
 *       "Softmax alternatives and the attention-sink problem", Practical
 *       advice, asks that the denominator never be zero).
 *   R11 Square causal self-attention, one K/V head per Q head; q, k are the
 *       post-RoPE vectors.
 *
 * Two variants from the note's ablation table (section Key experimental
 * data, ablation), selected by arguments of the _ex entry points:
 *   R14 phi = Sigmoid ("Sigmoid + L1 + re-weighting"): the non-negative map
 *       of Key design 1 becomes the logistic sigmoid 1/(1 + e^-x); the
 *       scores, mask, both L1 normalisations, N, O and ReLU^p stay as above.
 *   R15 LSSA only ("LSSA only, no re-weighting"; also the main-results row
 *       "LSSA, normalisation stage only"): stage 1, then out = A V; p and
 *       eps play no part and no row is degenerate (every A_ij with j <= i
 *       is positive).
 *
 * Backward (lssar_ref_bwd_f64): the chain rule through the same steps in
 * reverse, for the loss sum_i dout_i . out_i:
 *   R16 A degenerate row (R10) has the constant output 0 and passes no
 *       gradient to q, k or v.  ReLU'(0) = 0, so p = 1 entries exactly at
 *       the threshold pass none either.
 *   R17 The norm clamp of R6 is differentiated as written: for |x| > 1e-12
 *       d(x/|x|) = (I - x^ x^T) / |x|; below it, I / 1e-12.
 *
 * Row statistics (lssar_ref_rowstats_f64), what a training forward keeps for
 * its backward:
 *   R19 Per row, the stage-1 L1 norm before normalisation,
 *       S_i = sum_{j<=i} Softplus(s_ij), and the largest unmasked scaled
 *       score m_i = max_{j<=i} s_ij with s_ij = log d log i q^_i . k^_j.
 *       Given the row's own scores, stage 2's row constants (the threshold
 *       o_i S_i / i and the row maximum i Softplus(m_i) / S_i - o_i)
 *       depend on nothing else.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC lssar_ref.c -lm (no -ffast-math).
 */
#include "lssar_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Softplus(x) = log(1 + e^x)  (R4), evaluated without overflow:
 * for x > 0, log(1 + e^x) = x + log(1 + e^-x). */
static double softplus(double x)
{
    if (x > 0.0)
        return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* Logistic sigmoid 1/(1 + e^-x) (R14), evaluated without overflow. */
static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    const double e = exp(x);
    return e / (1.0 + e);
}

/* The non-negative map of stage 1: Softplus (R4) or Sigmoid (R14). */
static double phi_fn(int phi, double x)
{
    return phi == LSSAR_REF_PHI_SIGMOID ? sigmoid(x) : softplus(x);
}

/* x^p by repeated multiplication (R9: integer p >= 1). */
static double ipow(double x, int p)
{
    double r = 1.0;
    for (int e = 0; e < p; ++e)
        r *= x;
    return r;
}

/* Row L2 normalisation (Key design 1): y = x / max(|x|_2, 1e-12)  (R6). */
static void l2_normalise(const double* x, double* y, int d)
{
    double ss = 0.0;
    for (int e = 0; e < d; ++e)
        ss += x[e] * x[e];
    double nrm = sqrt(ss);
    if (nrm < 1e-12)
        nrm = 1e-12;
    for (int e = 0; e < d; ++e)
        y[e] = x[e] / nrm;
}

/* One output row.  qh: the normalised query row i (0-based row = i-1);
 * kh: all L normalised key rows of the head; v: the head's V; a: scratch of
 * 2 L doubles.  Every j in 1..L is computed and then multiplied by the mask
 * M'_ij, as the matrix form on the page does.  phi picks the stage-1 map
 * (R4/R14); reweight = 0 skips stage 2 (R15).
 *
 * Self-check of stage 2: with m the row's largest entry of A (.) N - O,
 * ReLU(x)^p and (ReLU(x)/m)^p differ by the constant factor m^-p, which the
 * second L1 normalisation removes, so both give the same weights in exact
 * arithmetic.  The second form stays in [0, 1] at every p; the literal one
 * can leave fp64's range (x can reach i - 1).  Returns 0, or 1 when the two
 * normalised weight rows differ anywhere by more than 1e-12. */
static int lssar_row(const double* qh, const double* kh, const double* v,
                     int L, int d, int p, double eps, int phi, int reweight,
                     int row, double* a, double* out)
{
    const int i = row + 1;                       /* R2: 1-based row index */
    const double scale = log((double)d) * log((double)i);   /* log d . log N_ij, R1 */

    /* Stage 1 (Key design 1): A_ij = phi(scale * q^_i . k^_j) * M'_ij */
    double l1 = 0.0;
    for (int j = 1; j <= L; ++j) {
        const double* kj = kh + (size_t)(j - 1) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qh[e] * kj[e];
        double mask = (j <= i) ? 1.0 : 0.0;     /* M': lower triangle = 1 (R5) */
        a[j - 1] = phi_fn(phi, scale * dot) * mask;
        l1 += a[j - 1];
    }
    for (int j = 0; j < L; ++j)                  /* A_i <- A_i / |A_i|_1 */
        a[j] /= l1;

    if (reweight) {
        /* Stage 2 (Key design 2): A <- ReLU^p(A * N - O), then L1 again */
        const double o = (i <= 3) ? 0.0 : 1.0;       /* O: first 3 rows zero (R7) */
        double m = -INFINITY;
        for (int j = 0; j < L; ++j) {
            a[j] = a[j] * (double)i - o;             /* A (.) N - O */
            if (a[j] > m)
                m = a[j];
        }
        if (!(m > eps)) {                            /* degenerate row (R10) */
            memset(out, 0, sizeof(double) * (size_t)d);
            return 0;
        }
        double* b = a + L;                           /* the rescaled form */
        double l1b = 0.0, l1c = 0.0;
        for (int j = 0; j < L; ++j) {
            b[j] = ipow(fmax(a[j], 0.0) / m, p);
            l1c += b[j];
            double r = a[j] > 0.0 ? a[j] : 0.0;      /* ReLU */
            a[j] = ipow(r, p);                       /* ^p */
            l1b += a[j];
        }
        for (int j = 0; j < L; ++j)
            if (!(fabs(a[j] / l1b - b[j] / l1c) <= 1e-12))
                return 1;
        for (int j = 0; j < L; ++j)                  /* A_i <- A_i / |A_i|_1 */
            a[j] /= l1b;
    }

    /* Attention output (Key design 3): out_i = sum_j A_ij v_j */
    for (int e = 0; e < d; ++e)
        out[e] = 0.0;
    for (int j = 0; j < L; ++j) {
        const double* vj = v + (size_t)j * d;
        for (int e = 0; e < d; ++e)
            out[e] += a[j] * vj[e];
    }
    return 0;
}

static int bad_args(const void* q, const void* k, const void* v, const void* out,
                    int L, int d, int p, double eps, int phi, int reweight)
{
    return !q || !k || !v || !out || L < 1 || d < 1 || p < 1 || !(eps >= 0.0) ||
           (phi != LSSAR_REF_PHI_SOFTPLUS && phi != LSSAR_REF_PHI_SIGMOID) ||
           (reweight != 0 && reweight != 1);
}

int lssar_ref_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Normalise the rows of one head's Q and K (Key design 1). */
static void normalise_head(const double* q, const double* k, double* qh,
                           double* kh, int L, int d)
{
    for (int r = 0; r < L; ++r) {
        l2_normalise(q + (size_t)r * d, qh + (size_t)r * d, d);
        l2_normalise(k + (size_t)r * d, kh + (size_t)r * d, d);
    }
}

int lssar_ref_head_rows_ex_f64(const double* q, const double* k, const double* v,
                               int L, int d, int p, double eps, int phi,
                               int reweight, const int* rows, int nrows,
                               double* out, int nthreads)
{
    if (bad_args(q, k, v, out, L, d, p, eps, phi, reweight) || nrows < 0 ||
        (nrows && !rows))
        return -1;
    for (int r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= L)
            return -1;
    double* qh = malloc(sizeof(double) * (size_t)L * d);
    double* kh = malloc(sizeof(double) * (size_t)L * d);
    if (!qh || !kh) {
        free(qh);
        free(kh);
        return -2;
    }
    normalise_head(q, k, qh, kh, L, d);
    int fail = 0, range = 0;
#pragma omp parallel num_threads(lssar_ref_threads(nthreads))
    {
        double* a = malloc(sizeof(double) * 2 * (size_t)L);
        if (!a) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < nrows; ++r)
                if (lssar_row(qh + (size_t)rows[r] * d, kh, v, L, d, p, eps, phi,
                              reweight, rows[r], a, out + (size_t)r * d)) {
#pragma omp atomic write
                    range = 1;
                }
        }
        free(a);
    }
    free(qh);
    free(kh);
    return fail ? -2 : range ? -3 : 0;
}

int lssar_ref_fwd_ex_f64(const double* q, const double* k, const double* v,
                         double* out, int B, int H, int L, int d, int p,
                         double eps, int phi, int reweight, int nthreads)
{
    if (bad_args(q, k, v, out, L, d, p, eps, phi, reweight) || B < 1 || H < 1)
        return -1;
    const size_t head = (size_t)L * d;
    const long nheads = (long)B * H;
    double* qh = malloc(sizeof(double) * head * (size_t)nheads);
    double* kh = malloc(sizeof(double) * head * (size_t)nheads);
    if (!qh || !kh) {
        free(qh);
        free(kh);
        return -2;
    }
    const int nt = lssar_ref_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (long bh = 0; bh < nheads; ++bh)
        normalise_head(q + bh * head, k + bh * head, qh + bh * head,
                       kh + bh * head, L, d);
    int fail = 0, range = 0;
#pragma omp parallel num_threads(nt)
    {
        double* a = malloc(sizeof(double) * 2 * (size_t)L);
        if (!a) {
#pragma omp atomic write
            fail = 1;
        } else {
            /* rows are independent; row i costs O(L d), schedule dynamically */
#pragma omp for schedule(dynamic, 4)
            for (long t = 0; t < nheads * L; ++t) {
                long bh = t / L;
                int row = (int)(t % L);
                if (lssar_row(qh + bh * head + (size_t)row * d, kh + bh * head,
                              v + bh * head, L, d, p, eps, phi, reweight, row, a,
                              out + bh * head + (size_t)row * d)) {
#pragma omp atomic write
                    range = 1;
                }
            }
        }
        free(a);
    }
    free(qh);
    free(kh);
    return fail ? -2 : range ? -3 : 0;
}

int lssar_ref_head_rows_f64(const double* q, const double* k, const double* v,
                            int L, int d, int p, double eps,
                            const int* rows, int nrows, double* out,
                            int nthreads)
{
    return lssar_ref_head_rows_ex_f64(q, k, v, L, d, p, eps, LSSAR_REF_PHI_SOFTPLUS,
                                      1, rows, nrows, out, nthreads);
}

int lssar_ref_fwd_f64(const double* q, const double* k, const double* v,
                      double* out, int B, int H, int L, int d, int p,
                      double eps, int nthreads)
{
    return lssar_ref_fwd_ex_f64(q, k, v, out, B, H, L, d, p, eps,
                                LSSAR_REF_PHI_SOFTPLUS, 1, nthreads);
}

/* R19 for one row: the stage-1 loop of lssar_row (same scale, same mask
 * M' applied after Softplus) keeping the L1 norm and the largest unmasked
 * scaled score instead of normalising. */
static void lssar_row_stats(const double* qh, const double* kh, int L, int d,
                            int row, double* st)
{
    const int i = row + 1;                       /* R2 */
    const double scale = log((double)d) * log((double)i);   /* R1 */
    double l1 = 0.0, smax = -INFINITY;
    for (int j = 1; j <= L; ++j) {
        const double* kj = kh + (size_t)(j - 1) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += qh[e] * kj[e];
        const double s = scale * dot;
        const double mask = (j <= i) ? 1.0 : 0.0;   /* M' (R5) */
        l1 += softplus(s) * mask;
        if (mask == 1.0 && s > smax)
            smax = s;
    }
    st[0] = l1;
    st[1] = smax;
}

int lssar_ref_rowstats_f64(const double* q, const double* k, double* stats,
                           int B, int H, int L, int d, int nthreads)
{
    if (!q || !k || !stats || B < 1 || H < 1 || L < 1 || d < 1)
        return -1;
    const size_t head = (size_t)L * d;
    const long nheads = (long)B * H;
    double* qh = malloc(sizeof(double) * head);
    double* kh = malloc(sizeof(double) * head);
    if (!qh || !kh) {
        free(qh);
        free(kh);
        return -2;
    }
    for (long bh = 0; bh < nheads; ++bh) {
        normalise_head(q + bh * head, k + bh * head, qh, kh, L, d);
#pragma omp parallel for num_threads(lssar_ref_threads(nthreads)) schedule(dynamic, 16)
        for (int row = 0; row < L; ++row)
            lssar_row_stats(qh + (size_t)row * d, kh, L, d, row,
                            stats + ((size_t)bh * L + row) * 2);
    }
    free(qh);
    free(kh);
    return 0;
}

/* ------------------------------------------------------------------------
 * Backward
 * ------------------------------------------------------------------------ */

/* d(x / max(|x|, 1e-12)) applied to the gradient g of the normalised row
 * (R17). */
static void l2_normalise_bwd(const double* x, const double* g, double* out, int d)
{
    double ss = 0.0;
    for (int e = 0; e < d; ++e)
        ss += x[e] * x[e];
    const double nrm = sqrt(ss);
    if (!(nrm > 1e-12)) {
        for (int e = 0; e < d; ++e)
            out[e] = g[e] / 1e-12;
        return;
    }
    double gx = 0.0;
    for (int e = 0; e < d; ++e)
        gx += g[e] * x[e] / nrm;
    for (int e = 0; e < d; ++e)
        out[e] = (g[e] - gx * x[e] / nrm) / nrm;
}

/* One head: accumulate the gradients of every row into dqh (per row, the
 * gradient of the normalised query), dkh (normalised keys) and dv.
 * Scratch: 6 * L doubles. */
static void lssar_head_bwd(const double* qh, const double* kh, const double* v,
                           const double* dout, int L, int d, int p, double eps,
                           double* dqh, double* dkh, double* dv, double* scr)
{
    double* s = scr;            /* scores s_j           */
    double* a = scr + L;        /* Softplus values a_j  */
    double* x = scr + 2 * L;    /* i A_j - o            */
    double* w = scr + 3 * L;    /* final weights W_j    */
    double* g = scr + 4 * L;    /* gradients, reused    */
    double* A = scr + 5 * L;    /* stage-1 weights A_j  */
    for (int row = 0; row < L; ++row) {
        const int i = 1 + row;                   /* R2 */
        const double lam = log((double)d) * log((double)i);
        const double* qi = qh + (size_t)row * d;
        const double* gi = dout + (size_t)row * d;
        /* forward of the row (Key designs 1-2), keys 1..i */
        double S = 0.0;
        for (int j = 0; j < i; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += qi[e] * kh[(size_t)j * d + e];
            s[j] = lam * dot;
            a[j] = softplus(s[j]);
            S += a[j];
        }
        const double o = (i <= 3) ? 0.0 : 1.0;
        double m = -INFINITY;
        for (int j = 0; j < i; ++j) {
            A[j] = a[j] / S;
            x[j] = A[j] * (double)i - o;
            if (x[j] > m)
                m = x[j];
        }
        if (!(m > eps))
            continue;                            /* R16: no gradient */
        double R = 0.0;
        for (int j = 0; j < i; ++j) {
            w[j] = x[j] > 0.0 ? ipow(x[j], p) : 0.0;
            R += w[j];
        }
        for (int j = 0; j < i; ++j)
            w[j] /= R;
        /* dW_j = dout_i . v_j; through W = r / R */
        double delta = 0.0;
        for (int j = 0; j < i; ++j) {
            double dw = 0.0;
            for (int e = 0; e < d; ++e)
                dw += gi[e] * v[(size_t)j * d + e];
            g[j] = dw;
            delta += w[j] * dw;
        }
        /* dr_j = (dW_j - delta) / R; dx_j = dr_j p x^(p-1) for x > 0;
           dA_j = i dx_j */
        double eps1 = 0.0;
        for (int j = 0; j < i; ++j) {
            const double dr = (g[j] - delta) / R;
            const double dx = x[j] > 0.0 ? dr * (double)p * ipow(x[j], p - 1) : 0.0;
            g[j] = (double)i * dx;
            eps1 += A[j] * g[j];
        }
        /* through A = a / S, a = Softplus(s) (derivative: the logistic
           sigmoid), s = lam (q^ . k^) */
        for (int j = 0; j < i; ++j) {
            const double da = (g[j] - eps1) / S;
            const double ds = da * sigmoid(s[j]);
            const double dc = lam * ds;
            for (int e = 0; e < d; ++e) {
                dqh[(size_t)row * d + e] += dc * kh[(size_t)j * d + e];
                dkh[(size_t)j * d + e] += dc * qi[e];
                dv[(size_t)j * d + e] += w[j] * gi[e];
            }
        }
    }
}

int lssar_ref_bwd_f64(const double* q, const double* k, const double* v,
                      const double* dout, double* dq, double* dk, double* dv,
                      int B, int H, int L, int d, int p, double eps, int nthreads)
{
    if (bad_args(q, k, v, dout, L, d, p, eps, LSSAR_REF_PHI_SOFTPLUS, 1) ||
        !dq || !dk || !dv || B < 1 || H < 1)
        return -1;
    const size_t head = (size_t)L * d;
    const long nheads = (long)B * H;
    int fail = 0;
#pragma omp parallel num_threads(lssar_ref_threads(nthreads))
    {
        double* qh = malloc(sizeof(double) * head);
        double* kh = malloc(sizeof(double) * head);
        double* dqh = malloc(sizeof(double) * head);
        double* dkh = malloc(sizeof(double) * head);
        double* scr = malloc(sizeof(double) * 6 * (size_t)L);
        if (!qh || !kh || !dqh || !dkh || !scr) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < nheads; ++bh) {
                const size_t off = (size_t)bh * head;
                normalise_head(q + off, k + off, qh, kh, L, d);
                memset(dqh, 0, sizeof(double) * head);
                memset(dkh, 0, sizeof(double) * head);
                memset(dv + off, 0, sizeof(double) * head);
                lssar_head_bwd(qh, kh, v + off, dout + off, L, d, p, eps, dqh, dkh,
                               dv + off, scr);
                for (int r = 0; r < L; ++r) {
                    l2_normalise_bwd(q + off + (size_t)r * d, dqh + (size_t)r * d,
                                     dq + off + (size_t)r * d, d);
                    l2_normalise_bwd(k + off + (size_t)r * d, dkh + (size_t)r * d,
                                     dk + off + (size_t)r * d, d);
                }
            }
        }
        free(qh);
        free(kh);
        free(dqh);
        free(dkh);
        free(scr);
    }
    return fail ? -2 : 0;
}
