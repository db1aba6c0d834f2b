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
#include <stdlib.h>

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

/*
 * The scan from a precomputed activation U (the post-conv, post-SiLU input; [P1] "Input-
 * Dependent SSM Parameters": in a full layer Delta, B and C are projections of U, so U is
 * computed before the scan).  Packed sequences as in oracle_varlen (fixed length: cu[s] =
 * s*L); per channel and token, in the order of [P1] section 3.4:
 *   Delta = Softplus(dt + b);  Z_t = exp(Delta A) . Z_{t-1} + Delta (B_t x U_t);
 *   Y_t = Z_t C_t + D U_t;     O = Y . SiLU(z)
 * u, dt, z, y [T][nch]; B, C [T][N]; h [nseq][nch][N] in: initial state, out: final state.
 */
void oracle_scan_u_varlen(int nseq, const int32_t *cu, int nch, int N,
                          const double *u, const double *dt, const double *B, const double *C,
                          const double *z, const double *A, const double *Dskip,
                          const double *dt_bias, double *h, double *y)
{
    int s;
    for (s = 0; s < nseq; ++s) {
        const int t0 = cu[s], t1 = cu[s + 1];
        double *hseq = h + (size_t)s * nch * N;
        int d;
#pragma omp parallel for schedule(static)
        for (d = 0; d < nch; ++d) {
            double hs[64];
            const double dsk = Dskip ? Dskip[d] : 0.0;
            const double bias = dt_bias ? dt_bias[d] : 0.0;
            int n, t;
            for (n = 0; n < N; ++n) hs[n] = hseq[(size_t)d * N + n];
            for (t = t0; t < t1; ++t) {
                const size_t ix = (size_t)t * nch + d;
                const double uu = u[ix];
                const double delta = oracle_softplus(dt[ix] + bias);
                const double du = delta * uu;
                double acc = 0.0;
                for (n = 0; n < N; ++n) {
                    const double abar = exp(delta * A[(size_t)d * N + n]);
                    hs[n] = abar * hs[n] + du * B[(size_t)t * N + n];
                    acc += C[(size_t)t * N + n] * hs[n];
                }
                acc += dsk * uu;
                y[ix] = z ? acc * oracle_silu(z[ix]) : acc;
            }
            for (n = 0; n < N; ++n) hseq[(size_t)d * N + n] = hs[n];
        }
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

/*
 * Gradients of one sequence (reverse-mode differentiation of oracle_scan_sequence, written
 * step by step from the same formulas).  The loss is taken to be
 *     sum_t dout[t] . y[t]  +  dh_final . h_final  +  dconv_final . hist_final,
 * i.e. dout, dh_final and dconv_final are the incoming gradients of the layer output,
 * the final state and the outgoing conv history (either of the last two may be NULL).
 * Conventions as in oracle_scan_sequence; in addition
 *   dout, dx, ddt, dz [L][ldx]   dz may be NULL when z is NULL
 *   dB, dC [L][N]                accumulated (+=) over the channels
 *   dA [nch][N], dD, ddt_bias, dconv_b [nch], dconv_w [nch][4]   accumulated (+=)
 *   dh0 [nch][N], dconv0 [3][ldh]   overwritten: gradients of the initial state / history
 * work must hold L * (N + 5) doubles (the recomputed forward values).
 *
 * For each token, in reverse: with G[n] = dLoss/dh_t[n] (from y_t and from h_{t+1}),
 *   y_t = sum_n C h_t + D u_t, out = y SiLU(z):  dz = dout y SiLU'(z),  gy = dout SiLU(z)
 *   G[n] = gy C_t[n] + (adjoint from h_{t+1}[n]);  dC_t[n] += gy h_t[n]
 *   h_t = Abar h_{t-1} + Delta u B,  Abar = exp(Delta A):
 *     dB_t[n] += G Delta u,  dA[n] += G Abar h_{t-1} Delta,  adjoint to h_{t-1}[n] = G Abar
 *     dDelta = sum_n G (A Abar h_{t-1} + u B),  du = gy D + Delta sum_n G B
 *   Delta = softplus(a), a = dt + b:  da = dDelta sigmoid(a) = ddt = (share of) ddt_bias
 *   u = SiLU(pre):  dpre = du SiLU'(pre);  pre = b + sum_k w_k x_{t-3+k}:
 *     dconv_b += dpre,  dconv_w[k] += dpre x_{t-3+k},  dx_{t-3+k} += w_k dpre
 * with SiLU'(v) = s (1 + v (1 - s)), s = sigmoid(v).
 */
static double sigm(double v) { return 1.0 / (1.0 + exp(-v)); }

void oracle_backward_sequence(int L, int nch, int N, int ldx, int ldh,
                              const double *x, const double *dt, const double *B, const double *C,
                              const double *z, const double *A, const double *Dskip,
                              const double *dt_bias, const double *conv_w, const double *conv_b,
                              const double *h0, const double *hist0, const double *dout,
                              const double *dh_final, const double *dconv_final,
                              double *dx, double *ddt, double *dz, double *dB, double *dC,
                              double *dA, double *dD, double *ddt_bias, double *dconv_w, double *dconv_b,
                              double *dh0, double *dconv0, double *work)
{
    int d, t, n, k;
    for (d = 0; d < nch; ++d) {
        /* forward recompute: hs[t][n] = h_t[n]; pre, u, a, delta, y per token */
        double *hs = work, *pre = work + (size_t)L * N, *u = pre + L, *av = u + L, *delta = av + L, *y = delta + L;
        const double *w = conv_w + (size_t)d * ORACLE_K;
        const double cb = conv_b ? conv_b[d] : 0.0;
        const double dsk = Dskip ? Dskip[d] : 0.0;
        const double bias = dt_bias ? dt_bias[d] : 0.0;
        double hcur[64], R[64], P1, P2, P3;
        for (n = 0; n < N; ++n) hcur[n] = h0[(size_t)d * N + n];
        {
            double win[ORACLE_K];
            for (k = 0; k < ORACLE_K - 1; ++k) win[k] = hist0[(size_t)k * ldh + d];
            for (t = 0; t < L; ++t) {
                const size_t ix = (size_t)t * ldx + d;
                double p = cb, acc = 0.0;
                win[ORACLE_K - 1] = x[ix];
                for (k = 0; k < ORACLE_K; ++k) p += w[k] * win[k];
                for (k = 0; k < ORACLE_K - 1; ++k) win[k] = win[k + 1];
                pre[t] = p;
                u[t] = oracle_silu(p);
                av[t] = dt[ix] + bias;
                delta[t] = oracle_softplus(av[t]);
                for (n = 0; n < N; ++n) {
                    hcur[n] = exp(delta[t] * A[(size_t)d * N + n]) * hcur[n] + delta[t] * u[t] * B[(size_t)t * N + n];
                    hs[(size_t)t * N + n] = hcur[n];
                    acc += C[(size_t)t * N + n] * hcur[n];
                }
                y[t] = acc + dsk * u[t];
            }
        }
        /* reverse */
        for (n = 0; n < N; ++n) R[n] = dh_final ? dh_final[(size_t)d * N + n] : 0.0;
        /* P1, P2, P3: pending gradient of x_{t}, x_{t-1}, x_{t-2} before step t */
        P1 = dconv_final ? dconv_final[(size_t)2 * ldh + d] : 0.0;
        P2 = dconv_final ? dconv_final[(size_t)1 * ldh + d] : 0.0;
        P3 = dconv_final ? dconv_final[(size_t)0 * ldh + d] : 0.0;
        for (t = L - 1; t >= 0; --t) {
            const size_t ix = (size_t)t * ldx + d;
            double gy, du, S1 = 0.0, S2 = 0.0, ddel, da, sp, dpre, xin[ORACLE_K];
            if (z) {
                const double sz = sigm(z[ix]);
                dz[ix] = dout[ix] * y[t] * sz * (1.0 + z[ix] * (1.0 - sz));
                gy = dout[ix] * z[ix] * sz;
            } else {
                gy = dout[ix];
            }
            dD[d] += gy * u[t];
            du = gy * dsk;
            for (n = 0; n < N; ++n) {
                const double an = A[(size_t)d * N + n];
                const double abar = exp(delta[t] * an);
                const double hp = t > 0 ? hs[(size_t)(t - 1) * N + n] : h0[(size_t)d * N + n];
                const double G = gy * C[(size_t)t * N + n] + R[n];
                dC[(size_t)t * N + n] += gy * hs[(size_t)t * N + n];
                dB[(size_t)t * N + n] += G * delta[t] * u[t];
                dA[(size_t)d * N + n] += G * abar * hp * delta[t];
                S1 += G * an * abar * hp;
                S2 += G * B[(size_t)t * N + n];
                R[n] = G * abar;
            }
            ddel = S1 + u[t] * S2;
            du += delta[t] * S2;
            da = ddel * sigm(av[t]);
            ddt[ix] = da;
            ddt_bias[d] += da;
            sp = sigm(pre[t]);
            dpre = du * sp * (1.0 + pre[t] * (1.0 - sp));
            dconv_b[d] += dpre;
            for (k = 0; k < ORACLE_K; ++k) {
                const int tk = t - 3 + k;
                xin[k] = tk >= 0 ? x[(size_t)tk * ldx + d] : hist0[(size_t)(tk + 3) * ldh + d];
                dconv_w[(size_t)d * ORACLE_K + k] += dpre * xin[k];
            }
            dx[ix] = P1 + w[3] * dpre;
            P1 = P2 + w[2] * dpre;
            P2 = P3 + w[1] * dpre;
            P3 = w[0] * dpre;
        }
        for (n = 0; n < N; ++n) dh0[(size_t)d * N + n] = R[n];
        dconv0[(size_t)0 * ldh + d] = P3;
        dconv0[(size_t)1 * ldh + d] = P2;
        dconv0[(size_t)2 * ldh + d] = P1;
    }
}

/* Packed sequences (cu as in oracle_varlen; fixed length is cu[s] = s * L): arrays as in
 * oracle_backward_sequence with the token arrays packed [T][nch] / [T][N], and h0, hist0,
 * dh_final, dconv_final, dh0, dconv0 per sequence ([nseq][nch][N], [nseq][3][nch]).
 * Parameter gradients are summed over the sequences.  Channels are split over threads;
 * each thread accumulates its own dB / dC, and the per-thread sums are added in thread
 * order afterwards. */
void oracle_backward(int nseq, const int32_t *cu, int nch, int N,
                     const double *x, const double *dt, const double *B, const double *C,
                     const double *z, const double *A, const double *Dskip,
                     const double *dt_bias, const double *conv_w, const double *conv_b,
                     const double *h0, const double *hist0, const double *dout,
                     const double *dh_final, const double *dconv_final,
                     double *dx, double *ddt, double *dz, double *dB, double *dC,
                     double *dA, double *dD, double *ddt_bias, double *dconv_w, double *dconv_b,
                     double *dh0, double *dconv0)
{
    const int T = cu[nseq];
    int maxL = 0, s, nt = 1, i, th;
    double **lB, **lC;
    for (s = 0; s < nseq; ++s)
        if (cu[s + 1] - cu[s] > maxL) maxL = cu[s + 1] - cu[s];
#ifdef _OPENMP
    {
        extern int omp_get_max_threads(void);
        nt = omp_get_max_threads();
    }
#endif
    if (nt > nch) nt = nch > 0 ? nch : 1;
    lB = (double **)calloc((size_t)nt, sizeof(double *));
    lC = (double **)calloc((size_t)nt, sizeof(double *));
#pragma omp parallel for schedule(static, 1) num_threads(nt)
    for (th = 0; th < nt; ++th) {
        const int d0 = (int)((long long)nch * th / nt), d1 = (int)((long long)nch * (th + 1) / nt);
        double *work = (double *)calloc((size_t)maxL * (N + 5) + 1, sizeof(double));
        int ss;
        lB[th] = (double *)calloc((size_t)T * N + 1, sizeof(double));
        lC[th] = (double *)calloc((size_t)T * N + 1, sizeof(double));
        for (ss = 0; ss < nseq && d1 > d0; ++ss) {
            const size_t t0 = (size_t)cu[ss];
            const int L = cu[ss + 1] - cu[ss];
            const size_t o = t0 * nch + d0, oh = (size_t)ss * nch * N + (size_t)d0 * N, oc = (size_t)ss * 3 * nch + d0;
            oracle_backward_sequence(L, d1 - d0, N, nch, nch, x + o, dt + o, B + t0 * N, C + t0 * N,
                                     z ? z + o : NULL, A + (size_t)d0 * N, Dskip ? Dskip + d0 : NULL,
                                     dt_bias ? dt_bias + d0 : NULL, conv_w + (size_t)d0 * ORACLE_K,
                                     conv_b ? conv_b + d0 : NULL, h0 + oh, hist0 + oc, dout + o,
                                     dh_final ? dh_final + oh : NULL, dconv_final ? dconv_final + oc : NULL,
                                     dx + o, ddt + o, dz ? dz + o : NULL, lB[th] + t0 * N, lC[th] + t0 * N,
                                     dA + (size_t)d0 * N, dD + d0, ddt_bias + d0, dconv_w + (size_t)d0 * ORACLE_K,
                                     dconv_b + d0, dh0 + oh, dconv0 + oc, work);
        }
        free(work);
    }
    for (th = 0; th < nt; ++th) {
        for (i = 0; i < T * N; ++i) {
            dB[i] += lB[th][i];
            dC[i] += lC[th][i];
        }
        free(lB[th]);
        free(lC[th]);
    }
    free(lB);
    free(lC);
}

/*
 * Sliding window attention ([P1] "The Sliding Window Attention (SWA) Layer": "Window
 * Specification", "Positional Encoding").
 *
 * RoPE as in Su et al. (the formulation [P1] names): the pairs (2i, 2i+1) of a head vector at
 * position p are rotated by the angle p * base^(-2i/dh).  The angle is formed in double
 * precision.
 */
void oracle_rope(double *v, int dh, double pos, double base)
{
    int i;
    for (i = 0; i < dh / 2; ++i) {
        const double th = pos * pow(base, -2.0 * i / dh);
        const double c = cos(th), sn = sin(th), a = v[2 * i], b = v[2 * i + 1];
        v[2 * i] = a * c - b * sn;
        v[2 * i + 1] = a * sn + b * c;
    }
}

/*
 * Causal attention restricted to a window: the query at position t of a sequence attends to
 * the keys at positions t - window .. t of the same sequence ("for position t, the attention
 * computation includes positions t-w through t"), after RoPE on queries and keys; scores
 * are scaled by 1/sqrt(dh) and normalised by softmax.  Grouped-query attention: query head
 * h reads key/value head h / (Hq / Hkv).
 *   q [T][Hq][dh], k, v [T][Hkv][dh], out [T][Hq][dh]; sequence s covers tokens
 *   [cu[s], cu[s+1]) and its positions start at 0.
 *   rows (nrows entries, or NULL for all T): the query tokens to compute (out rows of the
 *   others are left untouched).
 */
void oracle_swa(int nseq, const int32_t *cu, int Hq, int Hkv, int dh, int window, double base,
                const double *q, const double *k, const double *v, double *out, const int32_t *rows,
                int nrows)
{
    const int T = cu[nseq];
    const int nr = rows ? nrows : T;
    const int group = Hq / Hkv;
    int it;
#pragma omp parallel for schedule(dynamic, 4)
    for (it = 0; it < nr; ++it) {
        const int t = rows ? rows[it] : it;
        int s = 0, h, j, e;
        double *qv = (double *)malloc(sizeof(double) * dh), *kv = (double *)malloc(sizeof(double) * dh);
        double *sc = (double *)malloc(sizeof(double) * (window + 1));
        while (!(cu[s] <= t && t < cu[s + 1])) ++s;
        for (h = 0; h < Hq; ++h) {
            const int hk = h / group;
            const int t0 = cu[s];
            const int lo = t - window > t0 ? t - window : t0;
            double mx = -INFINITY, sum = 0.0;
            for (e = 0; e < dh; ++e) qv[e] = q[((size_t)t * Hq + h) * dh + e];
            oracle_rope(qv, dh, (double)(t - t0), base);
            for (j = lo; j <= t; ++j) {
                double dot = 0.0;
                for (e = 0; e < dh; ++e) kv[e] = k[((size_t)j * Hkv + hk) * dh + e];
                oracle_rope(kv, dh, (double)(j - t0), base);
                for (e = 0; e < dh; ++e) dot += qv[e] * kv[e];
                sc[j - lo] = dot / sqrt((double)dh);
                if (sc[j - lo] > mx) mx = sc[j - lo];
            }
            for (j = lo; j <= t; ++j) {
                sc[j - lo] = exp(sc[j - lo] - mx);
                sum += sc[j - lo];
            }
            for (e = 0; e < dh; ++e) {
                double acc = 0.0;
                for (j = lo; j <= t; ++j) acc += sc[j - lo] * v[((size_t)j * Hkv + hk) * dh + e];
                out[((size_t)t * Hq + h) * dh + e] = acc / sum;
            }
        }
        free(qv);
        free(kv);
        free(sc);
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
