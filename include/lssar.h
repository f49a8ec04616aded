/*
 * lssar.h -- C ABI of the MI355X (gfx950) LSSAR causal attention: forward,
 * its ablation variants, the decode step over a key/value cache, and the
 * backward.
 *
 * LSSAR = Length Scaled Softplus Attention with Re-weighting, defined in the
 * paper note "Softplus Attention with Re-weighting Boosts Length
 * Extrapolation in Large Language Models" (papernotes.org, ICML 2026),
 * section Method details:
 *   Key design 1 (LSSA): L2-normalise every row of Q and K; for j <= i take
 *     A_ij = Softplus(ln d * ln i * q^_i . k^_j); entries above the diagonal
 *     are multiplied by 0 (the mask multiplies because Softplus >= 0, Key
 *     design 3); divide each row by its L1 norm.
 *   Key design 2 (re-weighting): A_ij <- ReLU(i * A_ij - o_i)^p with o_i = 0
 *     for rows 1-3 and 1 otherwise; divide each row by its L1 norm again.
 *   Key design 3: the weights replace Softmax, so out = A V.
 * Rows are 1-based positions i; d is the head dimension; log is natural.
 *
 * Degenerate rows.  When m_i = max_j (i A_ij - o_i) <= eps every re-weighted
 * entry is (numerically) zero and the second L1 normalisation has no value;
 * such a row's output is all zeros.  The page "Softmax alternatives and the
 * attention-sink problem" (Practical advice, implementation notes) asks that
 * this denominator never be zero; this is its scale-invariant form.
 *
 * Conventions for every entry point:
 *  - q, k, v, out: DEVICE pointers to contiguous row-major [B, H, L, d]
 *    tensors of one dtype (fp32 or bf16), each 16-byte aligned.  out must
 *    not overlap q, k or v.  The caller owns all buffers and the stream; the
 *    library keeps no pointer after a call returns and holds no mutable
 *    global state (calls on different streams may run concurrently).
 *  - stream: a hipStream_t (NULL = the legacy default stream).  Calls are
 *    asynchronous with respect to the host and ordered on the stream.
 *  - Square causal self-attention: query i sees keys 1..i; one K/V head per
 *    Q head; q and k are the vectors after any positional rotation.
 *  - Arithmetic, bf16 inputs: the Softplus forward's scores contract
 *    lambda_i q^_i against k^_j, each rounded to f16, on f16 MFMA; a query
 *    block with an ill-conditioned or deep row is computed again, and every
 *    other entry point's scores computed, from the raw inputs on bf16 MFMA;
 *    fp32 accumulation throughout.  Norms, Softplus, row sums and the
 *    re-weighting run in fp32; bf16 weights feed the P.V contraction (fp32
 *    accumulation).
 *    fp32 inputs: scores on fp64 MFMA, norms and the score -> Softplus ->
 *    re-weighting chain in fp64, fp32 weights and P.V on fp32 MFMA.  The
 *    output is rounded to the input dtype (nearest-even).
 *  - Every argument is validated on the host before any HIP call; invalid
 *    input returns an error code and launches nothing.
 */
#ifndef LSSAR_H
#define LSSAR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum { LSSAR_F32 = 0, LSSAR_BF16 = 1 } lssar_dtype;

/* Stage-1 maps for lssar_attn_fwd_phi_ws: Softplus (the method) or the
 * logistic Sigmoid 1/(1 + e^-x) that the note's ablation table (section Key
 * experimental data, ablation, row "Sigmoid + L1 + re-weighting") puts in
 * its place. */
typedef enum { LSSAR_PHI_SOFTPLUS = 0, LSSAR_PHI_SIGMOID = 1 } lssar_phi;

/* Status codes. */
enum {
    LSSAR_OK = 0,
    LSSAR_EINVAL = -1,       /* null/misaligned/overlapping pointer, B,H,L < 1,
                                p < 1, eps < 0 or not finite, sizes overflow */
    LSSAR_EUNSUPPORTED = -2, /* d not in {64, 128}, unknown dtype or phi,
                                p > 1024, L > 2^22 */
    LSSAR_EWORKSPACE = -3,   /* workspace null, misaligned, too small or
                                overlapping a tensor */
    LSSAR_EHIP = -4,         /* a HIP call or kernel launch failed; see
                                lssar_last_hip_error() */
    LSSAR_ESCRATCH = -5      /* lssar_attn_fwd_noalloc: the input needs more
                                than its static scratch */
};

/* Workspace for every forward entry point that takes one, in bytes, each
 * part rounded up to 256: one key factor per key row (fp32 for bf16 inputs:
 * 4*B*H*L; fp64 for fp32 inputs: 8*B*H*L); for bf16 inputs also the
 * normalised rows of K in f16 (B*H*L*d f16) and the attention kernel's
 * dispatch table (8 bytes per workgroup, lssar_fwd_schedule).  Returns 0
 * for invalid sizes. */
size_t lssar_workspace_bytes(int B, int H, int L, int d, int dtype);

/* LSSAR causal attention forward (Key designs 1-3 above) with a
 * caller-provided device workspace of at least lssar_workspace_bytes()
 * bytes, 256-byte aligned, overlapping no tensor.  Allocates nothing.
 * Equivalent to lssar_prep followed by lssar_attn_fwd_prepped on `stream`.
 * p: integer exponent >= 1 (the note reports 3 and 15).
 * eps: degenerate-row threshold >= 0 (1e-4 is the reference choice). */
int lssar_attn_fwd_ws(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int L, int d, int p, float eps, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* As lssar_attn_fwd_ws, but takes its workspace stream-ordered from the
 * device's default memory pool (hipMallocAsync / hipFreeAsync on `stream`). */
int lssar_attn_fwd(const void* q, const void* k, const void* v, void* out,
                   int B, int H, int L, int d, int p, float eps, int dtype,
                   void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * lssar_attn_fwd with no allocation and no workspace argument.  Its
 * workspace is a static device array of the library, one per GPU, of
 * lssar_noalloc_scratch_bytes() = 64 MiB, held from the library's first use
 * on that GPU until the process ends (bf16 at d = 64 fits up to about 500 K
 * query rows B*H*L, e.g. B1 H12 L32768).
 *  - Arguments, layout and output as for lssar_attn_fwd_ws on the CURRENT
 *    device; `stream` must belong to it.
 *  - LSSAR_ESCRATCH (checked on the host, before any HIP call) if
 *    lssar_workspace_bytes(B, H, L, d, dtype) exceeds the scratch; other
 *    errors as for lssar_attn_fwd_ws.
 *  - Calls no allocator.  Every call on a GPU shares that GPU's scratch:
 *    calls that overlap in time on one GPU (other streams, other threads)
 *    race; issue them on one stream.  Each call rewrites all of the scratch
 *    it reads (nothing needs to start at zero). */
int lssar_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                           void* out, int B, int H, int L, int d, int p,
                           float eps, int dtype, void* stream);

/* Size of lssar_attn_fwd_noalloc's per-GPU scratch, in bytes. */
size_t lssar_noalloc_scratch_bytes(void);

/* The prep step alone (the prep kernel; it reads K only).  Writes into the
 * workspace the key factors (Key design 1's K_j <- K_j / |K_j|_2, kept as a
 * factor of the score): for fp32 inputs fk[bh*L + j] = 1 / max(|k_j|_2,
 * 1e-12) in fp64; for bf16 inputs fk[bh*L + j] = 1 / max(|k_j|_2, 1e-12)
 * (fp64, rounded to fp32), the normalised row k_j / max(|k_j|_2, 1e-12)
 * rounded to f16, and the attention kernel's dispatch table.  Workspace
 * rules as for
 * lssar_attn_fwd_ws (it must not overlap k); a bad workspace is
 * LSSAR_EWORKSPACE. */
int lssar_prep(const void* k, void* workspace, size_t workspace_bytes, int B,
               int H, int L, int d, int dtype, void* stream);

/* The attention kernel alone (fused, two passes), reading the workspace
 * that lssar_prep filled for this k (stream-ordered after it). */
int lssar_attn_fwd_prepped(const void* q, const void* k, const void* v,
                           void* workspace, size_t workspace_bytes, void* out,
                           int B, int H, int L, int d, int p, float eps,
                           int dtype, void* stream);

/* Ablation variant (Key experimental data, ablation, "Sigmoid + L1 +
 * re-weighting"): as lssar_attn_fwd_ws with the stage-1 map chosen by phi.
 * With LSSAR_PHI_SOFTPLUS it computes exactly what lssar_attn_fwd_ws does;
 * with LSSAR_PHI_SIGMOID, A_ij = Sigmoid(ln d * ln i * q^_i . k^_j) for
 * j <= i, and every later step (mask, both L1 normalisations, N, O, ReLU^p,
 * the degenerate-row rule) is unchanged.  Same arguments, workspace and
 * errors; an unknown phi is LSSAR_EUNSUPPORTED. */
int lssar_attn_fwd_phi_ws(const void* q, const void* k, const void* v, void* out,
                          int B, int H, int L, int d, int p, float eps, int phi,
                          int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Stage 1 alone, then A V: the note's "LSSA only" (Key experimental data,
 * main results row "LSSA, normalisation stage only", and the ablation row
 * "LSSA only, no re-weighting").  out_i = sum_(j<=i) A_ij v_j with A the
 * L1-normalised Softplus row of Key design 1; no row is degenerate.  One
 * pass over the keys.  Arguments, workspace (lssar_workspace_bytes) and
 * errors as for lssar_attn_fwd_ws, without p and eps. */
int lssar_lssa_fwd_ws(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int L, int d, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace of lssar_decode_ws, in bytes (0 for invalid sizes): per cache
 * row one score, per chunk of 16384/d rows of every head 2 + (d + 1) partial
 * sums;
 * fp32 values for bf16 inputs, fp64 for fp32 inputs; each part rounded up
 * to 256 bytes. */
size_t lssar_decode_workspace_bytes(int B, int H, int Lmax, int d, int dtype);

/* Decode step over a key/value cache: for every (b, h) one new query at
 * 1-based position i = lens[b] attends to cache rows 1..i, and out[b, h] is
 * row i of the causal forward (Key designs 1-3, same readings, same
 * degenerate-row rule).  The note's Limitations and main results concern
 * this use: extrapolation to 8-16x the training length at inference.
 *  - q, out: DEVICE [B, H, d]; k_cache, v_cache: DEVICE [B, H, Lmax, d] with
 *    the new token's key and value already written at row i - 1 (0-based);
 *    rows at or past lens[b] are never read.  One dtype, 16-byte aligned;
 *    out overlaps nothing.
 *  - lens: DEVICE int32 [B] (4-byte aligned) or NULL (every sequence uses
 *    all Lmax rows).  Read by the kernels, so it can change between calls
 *    (and between replays of a captured graph) without host involvement.
 *    Values are clamped to [0, Lmax]; a sequence of length 0 gets zeros.
 *  - p, eps, dtype, errors: as for lssar_attn_fwd_ws.  d in {64, 128}.
 *  - workspace: lssar_decode_workspace_bytes(), 256-byte aligned, overlapping
 *    no argument.  Allocates nothing; three kernel launches on `stream`
 *    (bf16 with B*H >= 176: one launch, one workgroup per head, which uses
 *    only the per-row part of the workspace).  Either way the output is
 *    deterministic; the two schedules sum in different orders and agree to
 *    rounding. */
int lssar_decode_ws(const void* q, const void* k_cache, const void* v_cache,
                    const int* lens, void* out, int B, int H, int Lmax, int d,
                    int p, float eps, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace of lssar_attn_bwd_ws and lssar_attn_bwd_stats_ws, in bytes (0
 * for invalid sizes): per row of Q and K one inverse norm, and 8
 * coefficients per query row (fp32 for bf16 inputs, fp64 for fp32 inputs);
 * each part rounded up to 256 bytes. */
size_t lssar_bwd_workspace_bytes(int B, int H, int L, int d, int dtype);

/* Backward of lssar_attn_fwd_ws for the loss sum over rows of dout_i .
 * out_i: the gradients dq, dk, dv of the causal forward (Key designs 1-3,
 * the same readings and degenerate-row rule; a degenerate row passes no
 * gradient), by the chain rule through its steps in reverse: the stage-2 L1
 * normalisation, ReLU^p, N and O, the stage-1 L1 normalisation, Softplus
 * (derivative: the logistic sigmoid), the scores and the L2 norms (clamped
 * at 1e-12 as in the forward).  The forward's row statistics are
 * recomputed; nothing from the forward call is needed.
 *  - q, k, v, dout: DEVICE [B, H, L, d] inputs; dq, dk, dv: DEVICE
 *    [B, H, L, d] outputs, same dtype, 16-byte aligned; no output overlaps
 *    an input or another output.
 *  - Arithmetic: fp32 for bf16 inputs (outputs rounded to bf16), fp64 for
 *    fp32 inputs.
 *  - p, eps, dtype, d, errors: as for lssar_attn_fwd_ws.  workspace:
 *    lssar_bwd_workspace_bytes(), 256-byte aligned, overlapping no tensor.
 *    Allocates nothing; four kernel launches on `stream`. */
int lssar_attn_bwd_ws(const void* q, const void* k, const void* v,
                      const void* dout, void* dq, void* dk, void* dv, int B,
                      int H, int L, int d, int p, float eps, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Training forward: lssar_attn_fwd_ws (the Softplus method), which also
 * stores each row's stage-1 statistics for lssar_attn_bwd_stats_ws
 * (Key design 1: the L1 norm that normalises the Softplus row, and the
 * largest scaled score of the row; Key design 2's threshold and row maximum
 * follow from them):
 *  - row_stats: DEVICE fp64 [B, H, L, 2], 16-byte aligned, overlapping no
 *    other buffer.  row_stats[r][0] = S_i = sum_{j<=i} Softplus(s_ij) and
 *    row_stats[r][1] = m_i = max_{j<=i} s_ij, with s_ij = log d log i
 *    q^_i . k^_j (natural logarithms).  Rows r are (b, h, i - 1) row-major.
 *  - Values come from the kernels' arithmetic (fp32 for bf16 inputs, fp64
 *    for fp32 inputs), rounded to fp64.
 *  - For bf16 inputs the scores come from the raw query and key rows (bf16
 *    products, exact in fp32) with the fp32 factors applied to the
 *    accumulator; lssar_attn_fwd_ws folds the row factor into the query
 *    operand and rounds it to f16, so the two outputs agree to the bf16
 *    parity bar, not bitwise.  fp32 inputs: bitwise the same output.
 *  - Everything else, including errors, as for lssar_attn_fwd_ws (EINVAL
 *    also for a null, misaligned or overlapping row_stats).  Allocates
 *    nothing. */
int lssar_attn_fwd_stats_ws(const void* q, const void* k, const void* v,
                            void* out, double* row_stats, int B, int H, int L,
                            int d, int p, float eps, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/* lssar_attn_bwd_ws with what lssar_attn_fwd_stats_ws produced for the same
 * q, k, v, p and eps: its output out and its row statistics.  The backward
 * reads S_i and m_i instead of recomputing them (one pass over the keys per
 * query row fewer).  For bf16 inputs at d = 64 the row coefficients and dq
 * come from a single pass: dout_i . out_i serves as a first value of the
 * stage-2 L1 normalisation's row term delta_i = sum_j W_ij dout_i . v_j,
 * which the pass then corrects to its own weights' value.  The other paths
 * compute delta_i from the weights alone and do not read out.
 *  - out: DEVICE [B, H, L, d], the forward's output (same dtype);
 *    row_stats: DEVICE fp64 [B, H, L, 2]; both 16-byte aligned inputs that
 *    overlap no output and not the workspace.
 *  - Everything else as for lssar_attn_bwd_ws. */
int lssar_attn_bwd_stats_ws(const void* q, const void* k, const void* v,
                            const void* out, const void* dout,
                            const double* row_stats, void* dq, void* dk, void* dv,
                            int B, int H, int L, int d, int p, float eps, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* lssar_status_str(int status);

/* The hipError_t of the last LSSAR_EHIP returned on this host thread
 * (0 if none). */
int lssar_last_hip_error(void);

/* ABI version: 10000 * major + 100 * minor + patch. */
int lssar_version(void);

/* Dispatch order of the bf16 forward kernel (lssar_attn_fwd_ws and its
 * variants, d = 64 or 128) for the shape B, H, L: no part of the method,
 * a query of how the work is spread over the GPU.  The kernel has one
 * workgroup per 64-row query block; each of the 8 XCDs takes a contiguous
 * slice of the heads' block pairs {pi, nqb - 1 - pi} (equal work per XCD)
 * and runs its blocks largest first; workgroup w runs on XCD w % 8.
 *  - Returns the number of workgroups launched (>= B * H * ceil(L / 64)),
 *    or LSSAR_EINVAL for a shape the forward rejects.
 *  - items: HOST int array, or NULL to query the count only; else it needs
 *    room for the returned count (capacity, in elements; LSSAR_EINVAL if
 *    smaller) and receives for workgroup w the block (b H + h) nqb + qb it
 *    computes, or -1 for a workgroup that exits at once.
 *  - No HIP call; thread-safe. */
long long lssar_fwd_schedule(int B, int H, int L, int* items, long long capacity);

#ifdef __cplusplus
}
#endif
#endif /* LSSAR_H */
