/*
 * lssar_ref.h -- fp64 CPU oracle for LSSAR causal attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the bench may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes is the definition in the paper note "Softplus Attention
 * with Re-weighting Boosts Length Extrapolation in Large Language Models"
 * (papernotes.org), section Method details: Overall framework, Key design 1
 * (LSSA) and Key design 2 (re-weighting), written out as a plain loop in
 * fp64.  Readings where the note is silent are listed in lssar_ref.c.
 *
 * Layout: every tensor is a contiguous row-major [B, H, L, d] array of
 * doubles (the exact values of the dtype-rounded inputs).  Rows are queries
 * (1-based position i = row index + 1); the output has the same layout.
 */
#ifndef LSSAR_REF_H
#define LSSAR_REF_H

#ifdef __cplusplus
extern "C" {
#endif

/* Full forward over all B*H heads and L rows.  nthreads <= 0 uses the
 * OpenMP default.  Returns 0, or -1 on invalid arguments (null pointer,
 * B/H/L/d < 1, p < 1, eps < 0 or NaN), -2 if scratch allocation fails, or
 * -3 if a row's literal ReLU^p weights (Key design 2) left fp64's range:
 * every re-weighted row is also computed with its entries divided by the
 * row maximum before the power, which the L1 normalisation makes
 * equivalent, and the two must agree to 1e-12 (the output is then not
 * trustworthy; x^p can reach (i - 1)^p). */
int lssar_ref_fwd_f64(const double* q, const double* k, const double* v,
                      double* out, int B, int H, int L, int d, int p,
                      double eps, int nthreads);

/* A chosen set of rows of ONE head: q, k, v are that head's [L, d] arrays,
 * rows[r] is a 0-based query row, out is [nrows, d].  Same return codes. */
int lssar_ref_head_rows_f64(const double* q, const double* k, const double* v,
                            int L, int d, int p, double eps,
                            const int* rows, int nrows, double* out,
                            int nthreads);

/* Stage-1 map for the _ex entry points: Softplus (the method) or the
 * logistic Sigmoid of the note's ablation ("Sigmoid + L1 + re-weighting"). */
enum { LSSAR_REF_PHI_SOFTPLUS = 0, LSSAR_REF_PHI_SIGMOID = 1 };

/* As lssar_ref_fwd_f64 with the stage-1 map phi and reweight = 1 (both
 * stages) or 0 (stage 1 only, then A V: the ablation's "LSSA only"; p and
 * eps are then checked but unused).  -1 also for an unknown phi/reweight. */
int lssar_ref_fwd_ex_f64(const double* q, const double* k, const double* v,
                         double* out, int B, int H, int L, int d, int p,
                         double eps, int phi, int reweight, int nthreads);

/* As lssar_ref_head_rows_f64 with phi and reweight as above. */
int lssar_ref_head_rows_ex_f64(const double* q, const double* k, const double* v,
                               int L, int d, int p, double eps, int phi,
                               int reweight, const int* rows, int nrows,
                               double* out, int nthreads);

/* Backward of lssar_ref_fwd_f64 for the loss sum over rows of
 * dout_i . out_i: writes dq, dk, dv ([B, H, L, d], same layout).  The
 * chain rule through the same steps in reverse; a degenerate row passes no
 * gradient.  Same return codes (dout and the outputs must be non-null). */
int lssar_ref_bwd_f64(const double* q, const double* k, const double* v,
                      const double* dout, double* dq, double* dk, double* dv,
                      int B, int H, int L, int d, int p, double eps, int nthreads);

/* Row statistics of stage 1 (the lssar_ref.c reading R19): for every row,
 * stats[2 r] = S_i = sum_{j<=i} Softplus(s_ij), the L1 norm of Key design
 * 1's row before it is normalised, and stats[2 r + 1] = m_i = max_{j<=i}
 * s_ij, the largest unmasked scaled score (s_ij = log d log i q^_i . k^_j).
 * stats is [B, H, L, 2].  Returns 0, -1 on invalid arguments, -2 if scratch
 * allocation fails. */
int lssar_ref_rowstats_f64(const double* q, const double* k, double* stats,
                           int B, int H, int L, int d, int nthreads);

/* Number of OpenMP threads a call with this nthreads argument would use. */
int lssar_ref_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
