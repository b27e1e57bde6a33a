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

/* d softplus(v) / dv = 1 / (1 + exp(-v)), in a form that does not overflow. */
static double ref_sigmoid(double v)
{
    if (v >= 0.0)
        return 1.0 / (1.0 + exp(-v));
    const double e = exp(v);
    return e / (1.0 + e);
}

/*
 * Gradients of one selective scan (the same forward as ref_selective_scan,
 * with readout), for training the R2L stream: "Bifocal Diffusion Language
 * Models" trains the sidecar (and, plug-in, only the sidecar and s); this
 * is the reverse-mode derivative of the loop above, written out.
 *
 * Given dout = dL/dout [tokens, D] and dh_out = dL/dh_out [batch, D, N] (or
 * NULL), with dy = s * dout when there is a residual and dout otherwise, and
 * g the gradient with respect to the state, visiting the tokens of each
 * sequence in the opposite order of the forward scan:
 *     g  += dy_t * Cm[t,:]                 (the readout of token t)
 *     dCm[t,:] += dy_t * h_t               (summed over channels)
 *     dx_t = dy_t * Dskip + Delta_t * sum_n g_n * Bm[t,n]  (+ dout_t if res is x)
 *     dBm[t,:] += g * Delta_t * x_t        (summed over channels)
 *     dDelta_t = sum_n g_n * (Bm[t,n] * x_t + A[d,n] * abar_n * h_prev_n)
 *     dA[d,:] += g * Delta_t * abar * h_prev   (summed over tokens and sequences)
 *     g *= abar                            (now the gradient of h_prev)
 *     ddt_t = dDelta_t * sigmoid(dt_t) (softplus on) or dDelta_t
 * then dh_in = g; dDskip[d] = sum_t dy_t * x_t; ds = sum dout * y.
 *
 *   res_kind   0: no residual (out = y); 1: the residual is x; 2: a separate
 *              residual (its gradient is dout itself and is not written).
 *   outputs    dx, ddt [tokens, D]; dBm, dCm [tokens, N]; dA [D, N];
 *              dDskip [D]; dh_in [batch, D, N]; ds [1]: each may be NULL.
 *
 * Work runs in parallel over (sequence, group of 64 channels); the sums over
 * channel groups and over sequences are then taken in a fixed order, so the
 * result does not depend on the thread count.
 * Returns 0, or -1 on an invalid argument (nothing is written then).
 */
int ref_selective_scan_backward(int reverse, int64_t batch, const int64_t *seq_off,
                                int64_t D, int64_t N,
                                const double *x, const double *dt,
                                const double *Bm, const double *Cm,
                                const double *A, const double *Dskip,
                                int delta_softplus, const double *h_in,
                                int res_kind, double s,
                                const double *dout, const double *dh_out,
                                double *dx, double *ddt, double *dBm, double *dCm,
                                double *dA, double *dDskip, double *dh_in, double *ds,
                                int nthreads)
{
    if (batch < 0 || D <= 0 || N <= 0 || N > 4096 || !seq_off)
        return -1;
    if (!x || !dt || !Bm || !Cm || !A || !dout || res_kind < 0 || res_kind > 2)
        return -1;
    if (seq_off[0] != 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b)
        if (seq_off[b + 1] < seq_off[b])
            return -1;
    const int64_t tokens = seq_off[batch];
    const int64_t G = 64;                       /* channels per task */
    const int64_t groups = (D + G - 1) / G;

#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#else
    (void)nthreads;
#endif

    /* per-task partial sums, reduced in a fixed order afterwards */
    double *pB = calloc((size_t)(tokens * groups * N) + 1, sizeof(double));
    double *pC = calloc((size_t)(tokens * groups * N) + 1, sizeof(double));
    double *pA = calloc((size_t)(batch * D * N) + 1, sizeof(double));
    double *pD = calloc((size_t)(batch * D) + 1, sizeof(double));
    double *pS = calloc((size_t)(batch * groups) + 1, sizeof(double));
    if (!pB || !pC || !pA || !pD || !pS)
        abort();

    const int64_t tasks = batch * groups;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t task = 0; task < tasks; ++task) {
        const int64_t b = task / groups;
        const int64_t grp = task % groups;
        const int64_t start = seq_off[b];
        const int64_t len = seq_off[b + 1] - start;
        /* H[i*N + n]: state before visiting position i (H[0] = h_in), and
         * after the last one at i = len */
        double *H = malloc((size_t)((len + 1) * N) * sizeof(double));
        double *abar = malloc((size_t)(len * N + 1) * sizeof(double));
        double *delta = malloc((size_t)(len + 1) * sizeof(double));
        double *g = malloc((size_t)N * sizeof(double));
        if (!H || !abar || !delta || !g)
            abort();

        for (int64_t d = grp * G; d < D && d < (grp + 1) * G; ++d) {
            /* forward, keeping every state */
            for (int64_t n = 0; n < N; ++n)
                H[n] = h_in ? h_in[(b * D + d) * N + n] : 0.0;
            for (int64_t i = 0; i < len; ++i) {
                const int64_t t = reverse ? start + len - 1 - i : start + i;
                const double xv = x[t * D + d];
                const double raw = dt[t * D + d];
                delta[i] = delta_softplus ? ref_softplus(raw) : raw;
                for (int64_t n = 0; n < N; ++n) {
                    abar[i * N + n] = exp(delta[i] * A[d * N + n]);
                    H[(i + 1) * N + n] = abar[i * N + n] * H[i * N + n] +
                                         (delta[i] * Bm[t * N + n]) * xv;
                }
            }

            /* backward, in the opposite visiting order */
            for (int64_t n = 0; n < N; ++n)
                g[n] = dh_out ? dh_out[(b * D + d) * N + n] : 0.0;
            const double dsk = Dskip ? Dskip[d] : 0.0;
            for (int64_t i = len - 1; i >= 0; --i) {
                const int64_t t = reverse ? start + len - 1 - i : start + i;
                const double xv = x[t * D + d];
                const double dv = dout[t * D + d];
                const double dy = res_kind ? s * dv : dv;
                const double *h_now = H + (i + 1) * N;
                const double *h_prev = H + i * N;

                double yv = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    yv += Cm[t * N + n] * h_now[n];
                yv += dsk * xv;
                if (res_kind)
                    pS[task] += dv * yv;

                for (int64_t n = 0; n < N; ++n) {
                    g[n] += dy * Cm[t * N + n];
                    pC[(t * groups + grp) * N + n] += dy * h_now[n];
                }
                pD[b * D + d] += dy * xv;

                double dxv = dy * dsk + (res_kind == 1 ? dv : 0.0);
                double ddelta = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = abar[i * N + n];
                    dxv += g[n] * delta[i] * Bm[t * N + n];
                    pB[(t * groups + grp) * N + n] += g[n] * delta[i] * xv;
                    ddelta += g[n] * (Bm[t * N + n] * xv + A[d * N + n] * a * h_prev[n]);
                    pA[(b * D + d) * N + n] += g[n] * delta[i] * a * h_prev[n];
                    g[n] *= a;
                }
                if (dx)
                    dx[t * D + d] = dxv;
                if (ddt)
                    ddt[t * D + d] = delta_softplus ? ddelta * ref_sigmoid(dt[t * D + d]) : ddelta;
            }
            if (dh_in)
                for (int64_t n = 0; n < N; ++n)
                    dh_in[(b * D + d) * N + n] = g[n];
        }
        free(H);
        free(abar);
        free(delta);
        free(g);
    }

    /* the fixed-order sums */
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double sb = 0.0, sc = 0.0;
            for (int64_t grp = 0; grp < groups; ++grp) {
                sb += pB[(t * groups + grp) * N + n];
                sc += pC[(t * groups + grp) * N + n];
            }
            if (dBm)
                dBm[t * N + n] = sb;
            if (dCm)
                dCm[t * N + n] = sc;
        }
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t n = 0; n < N; ++n) {
            double sa = 0.0;
            for (int64_t b = 0; b < batch; ++b)
                sa += pA[(b * D + d) * N + n];
            if (dA)
                dA[d * N + n] = sa;
        }
        double sd = 0.0;
        for (int64_t b = 0; b < batch; ++b)
            sd += pD[b * D + d];
        if (dDskip)
            dDskip[d] = sd;
    }
    if (ds) {
        double ss = 0.0;
        for (int64_t task = 0; task < tasks; ++task)
            ss += pS[task];
        ds[0] = ss;
    }
    free(pB);
    free(pC);
    free(pA);
    free(pD);
    free(pS);
    return 0;
}

/*
 * The bidirectional full-window scan that the block-diffusion page contrasts
 * with its partial reverse scan ("Training Hybrid Block Diffusion Language
 * Models with Partial Bidirectionality", nl summary, "Probleemstelling", the
 * problem statement: the earlier hybrids, DiffuMamba among them, scan the
 * whole denoising window in both directions), and the left-to-right and
 * right-to-left streams that "Bifocal Diffusion Language Models" compares in
 * its ablations (section 4, experimental results).
 * The pages do not say how the two directions combine. The plain reading
 * taken here: each direction is the scan above with its own parameter set
 * (dt, Bm, Cm, A, Dskip; _f forward, _r reverse, which may be the same
 * arrays), both read the same x, and their readouts add:
 *     y_t = y_t(forward from h_in) + y_t(reverse from zero)
 *     out = res == NULL ? y : (s == 0 ? res : res + s * y)
 * h_out receives the forward direction's final state (the reverse one
 * depends on the whole window and is not a cacheable boundary state).
 * Arguments otherwise as in ref_selective_scan; y and out may be NULL.
 */
int ref_bidir_scan(int64_t batch, const int64_t *seq_off, int64_t D, int64_t N,
                   const double *x,
                   const double *dt_f, const double *Bm_f, const double *Cm_f,
                   const double *A_f, const double *Dskip_f,
                   const double *dt_r, const double *Bm_r, const double *Cm_r,
                   const double *A_r, const double *Dskip_r,
                   int delta_softplus, const double *h_in, double *h_out,
                   double *y, const double *res, double s, double *out, int nthreads)
{
    if (batch < 0 || D <= 0 || !seq_off || !Cm_f || !Cm_r)
        return -1;
    const int64_t tokens = seq_off[batch];
    if (tokens < 0)
        return -1;
    const size_t cells = (size_t)tokens * (size_t)D;
    double *yf = (double *)malloc((cells ? cells : 1) * sizeof(double));
    double *yr = (double *)malloc((cells ? cells : 1) * sizeof(double));
    if (!yf || !yr)
        abort();
    int rc = ref_selective_scan(0, batch, seq_off, D, N, x, dt_f, Bm_f, Cm_f, A_f, Dskip_f,
                                delta_softplus, h_in, h_out, yf, NULL, 0.0, NULL, nthreads);
    if (rc == 0)
        rc = ref_selective_scan(1, batch, seq_off, D, N, x, dt_r, Bm_r, Cm_r, A_r, Dskip_r,
                                delta_softplus, NULL, NULL, yr, NULL, 0.0, NULL, nthreads);
    if (rc == 0) {
        for (size_t i = 0; i < cells; ++i) {
            const double yv = yf[i] + yr[i];
            if (y)
                y[i] = yv;
            if (out) {
                if (!res)
                    out[i] = yv;
                else if (s == 0.0)
                    out[i] = res[i];
                else
                    out[i] = res[i] + s * yv;
            }
        }
    }
    free(yf);
    free(yr);
    return rc;
}
