/*
 * selective_scan_ref.c -- plain fp64 CPU oracle for the right-to-left (R2L) and
 * left-to-right selective scans of the Bifocal dLLM / R2LM method.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg may
 * load it. It shares no code, header, table or helper with the HIP library and
 * includes nothing from it.
 *
 * What it computes, and where that comes from:
 *
 *  - "Bifocal Diffusion Language Models" (gist.science, nl and fr technical
 *    summaries, section 2 "Methodology"): the R2L stream takes the backbone's
 *    hidden states, reverses the sequence, applies a Mamba selective scan and
 *    reverses the result back; the output is a residual correction Delta^R2L
 *    added to the hidden states through a learnable scalar s that starts at 0,
 *    so that at initialisation the model is (bit for bit, per the fr summary)
 *    the causal baseline. During denoising the R2L scan runs over the
 *    generation tokens only.
 *  - "Training Hybrid Block Diffusion Language Models with Partial
 *    Bidirectionality" (gist.science nl summary, "Methodology" items 1-3):
 *    the reverse scan is restricted to the active block; completed prefix
 *    blocks are stored as forward-only Mamba boundary states, which depend on
 *    the clean prefix alone.
 *
 * The pages never write the recurrence out. This oracle takes the plainest
 * reading of "Mamba selective scan": per channel d and state index n,
 *     abar = exp(Delta_t * A[d,n])            (zero-order hold for A)
 *     h    = abar * h_prev + Delta_t * B[t,n] * x[t,d]   (Euler step for B)
 *     y_t  = sum_n C[t,n] * h_n + Dskip[d] * x[t,d]
 * with Delta_t = softplus(dt[t,d]) when softplus is on. "h_prev" is the state
 * of the token to the right (reverse scan) or to the left (forward scan).
 *
 * Everything is fp64 with libm's exp/log1p; no blocking, fusion or reordering.
 * Independent (sequence, channel) pairs run in parallel under OpenMP; each pair
 * is a plain sequential loop, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Numerically stable log(1 + exp(v)). The pages do not name the map from the
 * raw step input to Delta; softplus is the usual Mamba choice and the one this
 * path takes (a reading). */
static double ref_softplus(double v)
{
    double pos = v > 0.0 ? v : 0.0;
    return pos + log1p(exp(-fabs(v)));
}

/*
 * One selective scan over every sequence of a packed batch.
 *
 *   reverse        1: visit each sequence right to left (the R2L stream);
 *                  0: left to right (the forward prefix scan).
 *   batch          number of sequences.
 *   seq_off        [batch+1] token offsets, non-decreasing, seq_off[0] == 0.
 *                  Sequence b owns tokens seq_off[b] .. seq_off[b+1]-1.
 *   D, N           channels and state size.
 *   x, dt          [tokens, D] row-major; dt is the raw step input.
 *   Bm             [tokens, N] row-major, shared by all channels.
 *   Cm             [tokens, N] row-major, or NULL for a state-only scan.
 *   A              [D, N] row-major.
 *   Dskip          [D] or NULL (treated as zero).
 *   delta_softplus 1: Delta = softplus(dt); 0: Delta = dt.
 *   h_in           [batch, D, N] initial state (the state beyond the first
 *                  visited token), or NULL for zero.
 *   h_out          [batch, D, N] state after the last visited token, or NULL.
 *   y              [tokens, D] scan readout, or NULL. Needs Cm.
 *   res            [tokens, D] residual base, or NULL.
 *   s              residual gate.
 *   out            [tokens, D], or NULL. Needs Cm. out = y when res is NULL;
 *                  otherwise out = res when s == 0 (a copy, so that the result
 *                  is exactly the residual), else res + s * y.
 *   nthreads       OpenMP threads (<= 0: the runtime default).
 *
 * Returns 0 on success, -1 on an invalid argument (nothing is written then).
 */
int ref_selective_scan(int reverse, int64_t batch, const int64_t *seq_off,
                       int64_t D, int64_t N,
                       const double *x, const double *dt,
                       const double *Bm, const double *Cm,
                       const double *A, const double *Dskip,
                       int delta_softplus,
                       const double *h_in, double *h_out,
                       double *y, const double *res, double s, double *out,
                       int nthreads)
{
    if (batch < 0 || D <= 0 || N <= 0 || N > 4096 || !seq_off)
        return -1;
    if (!x || !dt || !Bm || !A)
        return -1;
    if ((y || out) && !Cm)
        return -1;
    if (seq_off[0] != 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b)
        if (seq_off[b + 1] < seq_off[b])
            return -1;

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif

    const int64_t pairs = batch * D;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t b = p / D;
        const int64_t d = p % D;
        const int64_t start = seq_off[b];
        const int64_t len = seq_off[b + 1] - start;
        double *h = (double *)malloc((size_t)N * sizeof(double));
        if (!h)
            abort();

        for (int64_t n = 0; n < N; ++n)
            h[n] = h_in ? h_in[(b * D + d) * N + n] : 0.0;

        for (int64_t i = 0; i < len; ++i) {
            /* The reversal is the visiting order; outputs go back to the
             * token's own position, which is the "reverse back" step. */
            const int64_t t = reverse ? start + len - 1 - i : start + i;
            const double xv = x[t * D + d];
            const double raw = dt[t * D + d];
            const double delta = delta_softplus ? ref_softplus(raw) : raw;

            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(delta * A[d * N + n]);
                h[n] = abar * h[n] + (delta * Bm[t * N + n]) * xv;
            }

            if (Cm) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += Cm[t * N + n] * h[n];
                const double yv = acc + (Dskip ? Dskip[d] : 0.0) * xv;
                if (y)
                    y[t * D + d] = yv;
                if (out) {
                    if (!res)
                        out[t * D + d] = yv;
                    else if (s == 0.0)
                        out[t * D + d] = res[t * D + d];
                    else
                        out[t * D + d] = res[t * D + d] + s * yv;
                }
            }
        }

        if (h_out)
            for (int64_t n = 0; n < N; ++n)
                h_out[(b * D + d) * N + n] = h[n];
        free(h);
    }
    return 0;
}

/* Thread count the runtime would use, for reporting. */
int ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
