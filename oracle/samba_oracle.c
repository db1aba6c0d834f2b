/*
 * samba_oracle.c -- plain, sequential, fp64 CPU oracle for the Mamba selective-scan
 * layer core of the Samba hybrid model.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists so that tests, the smoke check and the
 * CPU-baseline leg of the benchmark can compare the HIP path against an obviously
 * correct definition.  The product library never links, loads or calls it, and it
 * shares no source, header, table or helper with the HIP path.
 *
 * Sources (page titles, with the section each step follows):
 *   [P1] "Samba: Simple Hybrid State Space Models for Efficient Unlimited Context
 *        Language Modeling" (paper-graph-ui summary), section 3.4 "Detailed,
 *        Sentence-Based Technical Breakdown", subsections
 *          - "Input Projection and Short Convolution"      (U = SiLU(DepthwiseConv(H, W_conv)), k = 4)
 *          - "Input-Dependent Selective Gating"            (Delta = Softplus(. + b))
 *          - "The State Space Model Update (S6)"           (Z_t = exp(Delta A) Z_{t-1} + Delta (B_t x U_t);
 *                                                           Y_t = Z_t C_t + D * U_t; Z_0 = 0)
 *          - "Gated Output"                                (O = Y * SiLU(gate))
 *   [P4] "Samba Guide: Hybrid Mamba & Sliding Window Architecture" (aifetchly blog),
 *        section "Hands-On Implementation", "Step 1: The Selective State Space (Mamba)
 *        Layer": fixes what [P1] leaves open -- the conv is causal with zero left
 *        padding of k-1 and the first L outputs kept (so tap k-1 multiplies the current
 *        token); A enters as A = -exp(A_log); the skip and the input term use the
 *        post-conv, post-SiLU activation; the gate is SiLU(z).
 *
 * Readings where the pages are silent (each one listed with its reason in the design notes):
 *   - A is passed as the matrix that multiplies Delta (normally negative): Abar = exp(Delta*A).
 *   - Bbar*u = Delta * B_t[n] * u_t (the Euler form both printed formulas use).
 *   - Conv history before a sequence start is zero unless an initial history is given.
 *   - A null gate pointer means "no gating" (the layer output is Y itself).
 *
 * Everything is evaluated in double precision, sequentially in time, in the order the
 * pages state the steps.  The only parallelism is OpenMP over independent channels.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_K 4 /* short-convolution kernel size k = 4 ([P1] "Input Projection and Short Convolution") */

/* Softplus(a) = log(1 + e^a), written in the overflow-safe form
 * max(a, 0) + log1p(exp(-|a|)).  [P1] "Input-Dependent Selective Gating". */
double oracle_softplus(double a)
{
    return (a > 0.0 ? a : 0.0) + log1p(exp(-fabs(a)));
}

/* SiLU(v) = v * sigmoid(v) = v / (1 + e^-v).  [P1] "Input Projection and Short Convolution". */
double oracle_silu(double v)
{
    return v / (1.0 + exp(-v));
}

/*
 * One sequence of length L over channels [0, nch), all arrays row-major:
 *   x, dt, z  [L][ldx]   (token-major; channel d of token t at t*ldx + d)
 *   B, C      [L][N]     (shared by every channel: [P1] "Input-Dependent SSM Parameters")
 *   A         [nch][N]   Dskip, dt_bias, conv_b [nch]   conv_w [nch][4]
 *   h         [nch][N]   in: initial state Z_0 (zeros for a fresh sequence); out: final state
 *   hist      [3][ldh]   in: the 3 pre-conv inputs before token 0, oldest first (zeros for a
 *                        fresh sequence); out: the last 3 pre-conv inputs, oldest first
 *   y         [L][ldx]   out: gated layer output
 * z may be NULL (no gate); Dskip, dt_bias, conv_b may be NULL (zero).
 */
void oracle_scan_sequence(int L, int nch, int N, int ldx, int ldh,
                          const double *x, const double *dt, const double *B, const double *C,
                          const double *z, const double *A, const double *Dskip,
                          const double *dt_bias, const double *conv_w, const double *conv_b,
                          double *h, double *hist, double *y)
{
    int d;
#pragma omp parallel for schedule(static)
    for (d = 0; d < nch; ++d) {
        double win[ORACLE_K]; /* win[0..2] = x[t-3..t-1], win[3] = x[t] */
        double hs[64];
        const double *w = conv_w + (size_t)d * ORACLE_K;
        const double cb = conv_b ? conv_b[d] : 0.0;
        const double dsk = Dskip ? Dskip[d] : 0.0;
        const double bias = dt_bias ? dt_bias[d] : 0.0;
        int n, t, k;
        for (k = 0; k < ORACLE_K - 1; ++k) win[k] = hist[(size_t)k * ldh + d];
        for (n = 0; n < N; ++n) hs[n] = h[(size_t)d * N + n];
        for (t = 0; t < L; ++t) {
            const size_t ix = (size_t)t * ldx + d;
            /* Short convolution, depthwise and causal: tap k multiplies x[t-3+k]
             * ([P1] "Input Projection and Short Convolution"; tap order and zero left
             * padding from [P4] Step 1). */
            double pre = cb, u, delta, du, acc;
            win[ORACLE_K - 1] = x[ix];
            for (k = 0; k < ORACLE_K; ++k) pre += w[k] * win[k];
            u = oracle_silu(pre);
            for (k = 0; k < ORACLE_K - 1; ++k) win[k] = win[k + 1];
            /* Delta = Softplus(dt + b)  ([P1] "Input-Dependent Selective Gating"). */
            delta = oracle_softplus(dt[ix] + bias);
            /* Z_t = exp(Delta A) . Z_{t-1} + Delta (B_t x U_t);  Y_t = Z_t C_t + D U_t
             * ([P1] "The State Space Model Update (S6)"). */
            du = delta * u;
            acc = 0.0;
            for (n = 0; n < N; ++n) {
                const double abar = exp(delta * A[(size_t)d * N + n]);
                hs[n] = abar * hs[n] + du * B[(size_t)t * N + n];
                acc += C[(size_t)t * N + n] * hs[n];
            }
            acc += dsk * u;
            /* O = Y . SiLU(gate)  ([P1] "Gated Output"; gate = z per [P4] Step 1). */
            y[ix] = z ? acc * oracle_silu(z[ix]) : acc;
        }
        for (n = 0; n < N; ++n) h[(size_t)d * N + n] = hs[n];
        for (k = 0; k < ORACLE_K - 1; ++k) hist[(size_t)k * ldh + d] = win[k];
    }
}

/* Fixed-length batch: sequence s uses rows [s*L, (s+1)*L) of x/dt/z/y and of B/C,
 * h[s] = [nch][N] and hist[s] = [3][nch].  Each sequence is independent. */
void oracle_prefill(int batch, int L, int nch, int N,
                    const double *x, const double *dt, const double *B, const double *C,
                    const double *z, const double *A, const double *Dskip,
                    const double *dt_bias, const double *conv_w, const double *conv_b,
                    double *h, double *hist, double *y)
{
    int s;
    for (s = 0; s < batch; ++s) {
        const size_t o = (size_t)s * L * nch, ob = (size_t)s * L * N;
        oracle_scan_sequence(L, nch, N, nch, nch, x + o, dt + o, B + ob, C + ob,
                             z ? z + o : NULL, A, Dskip, dt_bias, conv_w, conv_b,
                             h + (size_t)s * nch * N, hist + (size_t)s * 3 * nch, y + o);
    }
}

/* Packed variable-length batch: sequence s covers tokens [cu[s], cu[s+1]) of the packed
 * arrays; its state and conv history start from h[s] / hist[s] (the caller zeroes them
 * for fresh sequences) and end there. */
void oracle_varlen(int nseq, const int32_t *cu, int nch, int N,
                   const double *x, const double *dt, const double *B, const double *C,
                   const double *z, const double *A, const double *Dskip,
                   const double *dt_bias, const double *conv_w, const double *conv_b,
                   double *h, double *hist, double *y)
{
    int s;
    for (s = 0; s < nseq; ++s) {
        const size_t t0 = (size_t)cu[s];
        const int L = cu[s + 1] - cu[s];
        oracle_scan_sequence(L, nch, N, nch, nch, x + t0 * nch, dt + t0 * nch, B + t0 * N,
                             C + t0 * N, z ? z + t0 * nch : NULL, A, Dskip, dt_bias, conv_w,
                             conv_b, h + (size_t)s * nch * N, hist + (size_t)s * 3 * nch,
                             y + t0 * nch);
    }
}

/* One decode step for nseq sequences: token arrays are [nseq][nch] (B, C: [nseq][N]);
 * h [nseq][nch][N] and hist [nseq][3][nch] are the resident state, updated in place.
 * This is the same recurrence with L = 1 ([P1] section 5, constant per-token
 * generation cost from the fixed-size state). */
void oracle_decode_step(int nseq, int nch, int N,
                        const double *x, const double *dt, const double *B, const double *C,
                        const double *z, const double *A, const double *Dskip,
                        const double *dt_bias, const double *conv_w, const double *conv_b,
                        double *h, double *hist, double *y)
{
    oracle_prefill(nseq, 1, nch, N, x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h, hist, y);
}

/*
 * The short convolution and its SiLU alone, U = SiLU(DepthwiseConv(H, W_conv)) ([P1]
 * "Input Projection and Short Convolution"; causal, tap k multiplying x[t-3+k], per [P4]
 * Step 1): the activation a full layer feeds to its x_proj as well as to the scan.  One
 * sequence of L tokens, conventions as in oracle_scan_sequence: x, u [L][ldx];
 * hist [3][ldh] in: the 3 inputs before token 0 (oldest first), out: the last 3 inputs.
 */
void oracle_conv_silu_sequence(int L, int nch, int ldx, int ldh, const double *x,
                               const double *conv_w, const double *conv_b, double *hist, double *u)
{
    int d;
#pragma omp parallel for schedule(static)
    for (d = 0; d < nch; ++d) {
        double win[ORACLE_K]; /* win[0..2] = x[t-3..t-1], win[3] = x[t] */
        const double *w = conv_w + (size_t)d * ORACLE_K;
        const double cb = conv_b ? conv_b[d] : 0.0;
        int t, k;
        for (k = 0; k < ORACLE_K - 1; ++k) win[k] = hist[(size_t)k * ldh + d];
        for (t = 0; t < L; ++t) {
            const size_t ix = (size_t)t * ldx + d;
            double pre = cb;
            win[ORACLE_K - 1] = x[ix];
            for (k = 0; k < ORACLE_K; ++k) pre += w[k] * win[k];
            u[ix] = oracle_silu(pre);
            for (k = 0; k < ORACLE_K - 1; ++k) win[k] = win[k + 1];
        }
        for (k = 0; k < ORACLE_K - 1; ++k) hist[(size_t)k * ldh + d] = win[k];
    }
}

/* Packed sequences for the conv alone: sequence s covers tokens [cu[s], cu[s+1]) of x / u
 * ([T][nch]); its history starts from hist[s] ([3][nch]; the caller zeroes it for fresh
 * sequences) and ends there. */
void oracle_conv_silu_varlen(int nseq, const int32_t *cu, int nch, const double *x,
                             const double *conv_w, const double *conv_b, double *hist, double *u)
{
    int s;
    for (s = 0; s < nseq; ++s) {
        const size_t t0 = (size_t)cu[s];
        oracle_conv_silu_sequence(cu[s + 1] - cu[s], nch, nch, nch, x + t0 * nch, conv_w, conv_b,
                                  hist + (size_t)s * 3 * nch, u + t0 * nch);
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the channel-parallel loops (timing of the CPU baseline only). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
