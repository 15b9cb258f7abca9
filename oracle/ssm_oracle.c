/*
 * ssm_oracle.c -- plain fp64 CPU reference of the Mamba-1 selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it; the library itself never does, and the two
 * share no code, header, table or helper.
 *
 * It is written from the equations on these pages, as direct nested loops over
 * batch, channel, time and state, in double precision, with libm's exp/expm1/
 * log1p and no reordering beyond what the definitions state:
 *
 *   [P1] "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 *        (paper summary page): sec. 4a (block: Conv1d -> SiLU -> SSM -> x SiLU
 *        gate), sec. 4b eq. (1a)/(1b) (continuous SSM), eq. (4) (ZOH rule),
 *        eq. (2a)/(2b) (recurrence), Algorithm 2 (S6 shapes: A (D,N), B and C
 *        (B,L,N), Delta (B,L,D)), the softplus tau_Delta parameterisation.
 *   [P2] "2. Mamba 상세" (EulerStack mixer tutorial): the YAML example
 *        (d_conv: 4, ssm_state kept for inference).
 *   [P4] "14.1 SSM(State Space Models)과 Mamba 아키텍처의 부상": sec. 3.1
 *        (y = C h + D x, the D skip term), sec. 3.2 (ZOH), sec. 4.1 (selection),
 *        sec. 5.1 (SSD: a scalar-times-identity state matrix per head).
 *
 * Readings taken where the pages leave a step open (each one is listed in the
 * design notes):
 *   - B-bar is the exact ZOH form of eq. (4) for a diagonal A, element-wise
 *     (Delta a)^-1 (exp(Delta a) - 1) Delta b; at Delta a == 0 the removable
 *     singularity takes its limit, B-bar = Delta b.
 *   - the D skip multiplies the SSM input u (after the conv prologue if any).
 *   - the gate multiplies the whole output: y = (C h + D u) * silu(z).
 *   - the initial state is zero unless h0 is given.
 *   - the conv prologue is a causal cross-correlation with zero left padding:
 *     u_t = silu(sum_k w[k] x_{t-(K-1)+k} + b), so w[K-1] weighs the current
 *     token.
 *   - the conv state carried between calls ([P2] keeps a state for inference)
 *     is the last K-1 inputs x, oldest first, laid out (B, K-1, D); a scan
 *     may start from one (the inputs before t = 0) and return the one after
 *     its last step, and a decode step shifts it by one input.
 *
 * All arrays are row-major with the last index fastest, host memory, double.
 * Threads (OpenMP) split only independent (batch, channel) pairs.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* SiLU (swish), the activation named in [P1] sec. 4a / 4d: v * sigmoid(v). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* softplus, the tau_Delta of [P1] Algorithm 2, in the overflow-free form
 * max(v,0) + log(1 + exp(-|v|)). */
static double softplus(double v) { return (v > 0 ? v : 0.0) + log1p(exp(-fabs(v))); }

/* ZOH discretisation of one diagonal entry, [P1] eq. (4) / [P4] sec. 3.2:
 *   Abar = exp(Delta a),  Bbar = (Delta a)^-1 (exp(Delta a) - 1) Delta b.
 * expm1 keeps the bracket accurate for small Delta a; at Delta a == 0 the
 * quotient takes its limit 1. */
static void zoh(double dt, double a, double b, double *abar, double *bbar)
{
    double za = dt * a;
    *abar = exp(za);
    double phi = (za == 0.0) ? 1.0 : expm1(za) / za;
    *bbar = phi * dt * b;
}

/* One channel's input at time s.  x points at element (b, 0, d), times are
 * `stride` apart.  Times before 0 come from hist, the K-1 inputs before the
 * sequence (oldest first, also `stride` apart), or are 0 without it. */
static double x_at(const double *x, const double *hist, int64_t stride, int64_t s, int64_t K)
{
    if (s >= 0) return x[s * stride];
    if (hist && s >= -(K - 1)) return hist[(K - 1 + s) * stride];
    return 0.0;
}

/* Causal depthwise conv1d(K) + SiLU on one channel's input at time t. */
static double conv_silu_at(const double *x, const double *hist, int64_t stride, int64_t t,
                           int64_t K, const double *wd, double bias)
{
    double acc = bias;
    for (int64_t k = 0; k < K; ++k) acc += wd[k] * x_at(x, hist, stride, t - (K - 1) + k, K);
    return silu(acc);
}

int oracle_abi_version(void) { return 3; }

/*
 * Selective scan forward ([P1] Algorithm 2 with the block's gate and the
 * [P4] sec. 3.1 skip term):
 *   u_t   = x_t, or conv1d+SiLU of x when conv_w is given          ([P1] 4a)
 *   dt    = delta_t, or softplus(delta_t + bias) when requested     ([P1] Alg. 2)
 *   h_t,n = Abar h_{t-1},n + Bbar u_t         with eq. (4) per n    ([P1] eq. 2a)
 *   y_t   = (sum_n C_t,n h_t,n + Dskip u_t) * silu(z_t)             ([P1] eq. 2b, 4a)
 *
 * Shapes: x, delta, z, y (B,L,D); A (D,N); Bm, Cm (B,L,N); Dskip, delta_bias,
 * conv_b (D); conv_w (D,K); h0, h_final (B,D,N); conv_state_in and
 * conv_state_out (B,K-1,D): the inputs before t = 0 and the last K-1 inputs
 * (earlier than t = 0 where L < K-1).  Optional arguments may be NULL.
 * Returns 0, or -1 on a bad size.
 */
int oracle_selective_scan_f64(int64_t Bsz, int64_t L, int64_t D, int64_t N,
                              const double *x, const double *delta, const double *A,
                              const double *Bm, const double *Cm, const double *Dskip,
                              const double *z, const double *delta_bias, int delta_softplus,
                              const double *conv_w, const double *conv_b, int64_t conv_k,
                              const double *conv_state_in, double *conv_state_out,
                              const double *h0, double *y, double *h_final, int nthreads)
{
    if (Bsz < 0 || L < 0 || D < 0 || N < 1 || (conv_w && conv_k < 1)) return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t nch = Bsz * D;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / D, d = ch % D;
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        const double *xbd = x + b * L * D + d;
        const double *hist = conv_state_in ? conv_state_in + b * (conv_k - 1) * D + d : NULL;
        for (int64_t t = 0; t < L; ++t) {
            int64_t i = (b * L + t) * D + d;
            double u = conv_w ? conv_silu_at(xbd, hist, D, t, conv_k, conv_w + d * conv_k,
                                             conv_b ? conv_b[d] : 0.0)
                              : x[i];
            double dt = delta[i];
            if (delta_softplus) dt = softplus(dt + (delta_bias ? delta_bias[d] : 0.0));
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double abar, bbar;
                zoh(dt, A[d * N + n], Bm[(b * L + t) * N + n], &abar, &bbar);
                h[n] = abar * h[n] + bbar * u;
                acc += Cm[(b * L + t) * N + n] * h[n];
            }
            double yv = acc + (Dskip ? Dskip[d] * u : 0.0);
            if (z) yv *= silu(z[i]);
            y[i] = yv;
        }
        if (h_final)
            for (int64_t n = 0; n < N; ++n) h_final[(b * D + d) * N + n] = h[n];
        if (conv_state_out)
            for (int64_t k = 0; k < conv_k - 1; ++k)
                conv_state_out[(b * (conv_k - 1) + k) * D + d] =
                    x_at(xbd, hist, D, L - (conv_k - 1) + k, conv_k);
        free(h);
    }
    return 0;
}

/*
 * Depthwise causal conv1d(K) followed by SiLU ([P1] sec. 4a, [P2] d_conv: 4):
 *   u[b,t,d] = silu(sum_k w[d,k] x[b,t-(K-1)+k,d] + bias[d]), x at t<0 is 0.
 * x, u (B,L,D); w (D,K); bias (D) or NULL.
 */
int oracle_causal_conv1d_silu_f64(int64_t Bsz, int64_t L, int64_t D, int64_t K,
                                  const double *x, const double *w, const double *bias,
                                  double *u, int nthreads)
{
    if (Bsz < 0 || L < 0 || D < 0 || K < 1) return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t nch = Bsz * D;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / D, d = ch % D;
        const double *xbd = x + b * L * D + d;
        for (int64_t t = 0; t < L; ++t)
            u[(b * L + t) * D + d] = conv_silu_at(xbd, NULL, D, t, K, w + d * K, bias ? bias[d] : 0.0);
    }
    return 0;
}

/*
 * One recurrent (decode) step ([P1] eq. (2a)/(2b) used as a recurrence, one
 * token at a time, with the state carried between calls as in [P2]'s
 * ssm_state option):
 *   u             = x[b,d], or with conv_w the prologue of [P1] sec. 4a on the
 *                   window (conv_state[b,0..K-2,d], x[b,d]), after which the
 *                   window drops its oldest input and appends x[b,d]
 *   state[b,d,n] <- Abar state[b,d,n] + Bbar u           (eq. 4 per n)
 *   y[b,d]        = (sum_n C[b,n] state[b,d,n] + Dskip[d] u) * silu(z[b,d])
 * state (B,D,N) and conv_state (B,K-1,D) are updated in place; x, delta, z,
 * y (B,D); Bm, Cm (B,N); conv_w (D,K); conv_b (D).
 */
int oracle_state_update_f64(int64_t Bsz, int64_t D, int64_t N, double *state,
                            const double *x, const double *delta, const double *A,
                            const double *Bm, const double *Cm, const double *Dskip,
                            const double *z, const double *delta_bias, int delta_softplus,
                            const double *conv_w, const double *conv_b, int64_t conv_k,
                            double *conv_state, double *y, int nthreads)
{
    if (Bsz < 0 || D < 0 || N < 1 || (conv_w && conv_k < 1) || (conv_w && conv_k > 1 && !conv_state))
        return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t nch = Bsz * D;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t ch = 0; ch < nch; ++ch) {
        int64_t b = ch / D, d = ch % D;
        double u = x[ch];
        if (conv_w) {
            const double *wd = conv_w + d * conv_k;
            double *win = conv_w && conv_k > 1 ? conv_state + b * (conv_k - 1) * D + d : NULL;
            double acc = conv_b ? conv_b[d] : 0.0;
            for (int64_t k = 0; k < conv_k - 1; ++k) acc += wd[k] * win[k * D];
            acc += wd[conv_k - 1] * x[ch];
            u = silu(acc);
            for (int64_t k = 0; k + 1 < conv_k - 1; ++k) win[k * D] = win[(k + 1) * D];
            if (conv_k > 1) win[(conv_k - 2) * D] = x[ch];
        }
        double dt = delta[ch];
        if (delta_softplus) dt = softplus(dt + (delta_bias ? delta_bias[d] : 0.0));
        double *h = state + ch * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double abar, bbar;
            zoh(dt, A[d * N + n], Bm[b * N + n], &abar, &bbar);
            h[n] = abar * h[n] + bbar * u;
            acc += Cm[b * N + n] * h[n];
        }
        double yv = acc + (Dskip ? Dskip[d] * u : 0.0);
        if (z) yv *= silu(z[ch]);
        y[ch] = yv;
    }
    return 0;
}

/* d/dz of phi(z) = (e^z - 1)/z, i.e. psi(z) = (e^z (z - 1) + 1) / z^2, with
 * psi(0) = 1/2; a Taylor series near 0 avoids the cancellation. */
static double psi(double zv)
{
    if (fabs(zv) < 0.1) {
        /* sum_k (k+1) z^k / (k+2)! for k = 0..9 */
        double s = 0.0, fact = 2.0, p = 1.0;
        for (int k = 0; k < 10; ++k) {
            s += (double)(k + 1) * p / fact;
            p *= zv;
            fact *= (double)(k + 3);
        }
        return s;
    }
    return (exp(zv) * (zv - 1.0) + 1.0) / (zv * zv);
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* d silu(v) / dv = sigma(v) (1 + v (1 - sigma(v))). */
static double dsilu(double v)
{
    double s = sigmoid(v);
    return s * (1.0 + v * (1.0 - s));
}

/*
 * Gradients of the selective scan above for a scalar loss L whose gradient
 * with respect to y is dy (B,L,D) and with respect to h_final is dh_final
 * (B,D,N, or NULL for 0): reverse-mode differentiation of the same loops
 * (the adjoint of eq. (2a)/(2b) with the ZOH of eq. (4), [P1] sec. 4b; the
 * pages recompute the states instead of storing them, sec. 4c, which this
 * plain reference does not need to do).  Per batch row, channel and entry,
 * with lambda_t = dL/dh_t:
 *   lambda_t   = C_t gy_t + Abar_{t+1} lambda_{t+1},   gy_t = dy_t silu(z_t)
 *   dAbar_t    = lambda_t h_{t-1},   dBbar_t = lambda_t u_t,
 *   du_t      += sum_n lambda_t Bbar_t + Dskip gy_t
 *   ddt_t     += sum_n (dAbar_t a e_t + dBbar_t B_t e_t)   (Bbar = B (e - 1)/a)
 *   dA        += sum_t (dAbar_t dt_t e_t + dBbar_t B_t dt_t^2 psi(dt_t a))
 *   dB_t      += sum_d dBbar_t dt_t phi(dt_t a),   dC_t += sum_d gy_t h_t
 *   dz_t       = dy_t (C_t h_t + Dskip u_t) silu'(z_t),  dDskip += sum gy_t u_t
 *   dh0        = Abar_0 lambda_0
 * then through softplus (ddelta = ddt sigma(delta + bias)) and the conv
 * prologue (dc_t = du_t silu'(c_t), c_t the pre-activation; dx, dconv_w,
 * dconv_b by the chain rule of the causal cross-correlation).  With
 * conv_state_in (B,K-1,D), the inputs before t = 0 that the forward's conv
 * reads in place of zeros, dconv_state_in (B,K-1,D) receives their gradient
 * by the same chain rule.  Outputs (all written, optional ones when
 * non-NULL): dx, ddelta, dz (B,L,D); dA (D,N); dBm, dCm (B,L,N); dDskip,
 * ddelta_bias, dconv_b (D); dconv_w (D,K); dh0 (B,D,N); dconv_state_in
 * (B,K-1,D).  Threads split batch rows.  Returns 0 or -1.
 */
int oracle_selective_scan_bwd_f64(int64_t Bsz, int64_t L, int64_t D, int64_t N,
                                  const double *x, const double *delta, const double *A,
                                  const double *Bm, const double *Cm, const double *Dskip,
                                  const double *z, const double *delta_bias, int delta_softplus,
                                  const double *conv_w, const double *conv_b, int64_t conv_k,
                                  const double *conv_state_in, const double *h0,
                                  const double *dy, const double *dh_final,
                                  double *dx, double *ddelta, double *dz, double *dA, double *dBm,
                                  double *dCm, double *dDskip, double *ddelta_bias,
                                  double *dconv_w, double *dconv_b, double *dh0,
                                  double *dconv_state_in, int nthreads)
{
    if (Bsz < 0 || L < 0 || D < 0 || N < 1 || (conv_w && conv_k < 1)) return -1;
    if ((conv_state_in || dconv_state_in) && !conv_w) return -1;
    if (nthreads < 1) nthreads = 1;
    int64_t K = conv_w ? conv_k : 0;
    /* per batch row partial sums of the per-channel parameters */
    double *pA = (double *)calloc((size_t)(Bsz * D * N + 1), sizeof(double));
    double *pD = (double *)calloc((size_t)(Bsz * D + 1), sizeof(double));
    double *pbias = (double *)calloc((size_t)(Bsz * D + 1), sizeof(double));
    double *pw = (double *)calloc((size_t)(Bsz * D * (K > 0 ? K : 1) + 1), sizeof(double));
    double *pb = (double *)calloc((size_t)(Bsz * D + 1), sizeof(double));
    for (int64_t i = 0; i < Bsz * L * N; ++i) { dBm[i] = 0.0; dCm[i] = 0.0; }
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t b = 0; b < Bsz; ++b) {
        double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));  /* h_{t-1} at row t */
        double *us = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double *cs = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double *dts = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double *duv = (double *)malloc(sizeof(double) * (size_t)(L + 1));
        double *lam = (double *)malloc(sizeof(double) * (size_t)N);
        for (int64_t d = 0; d < D; ++d) {
            const double *xbd = x + b * L * D + d;
            const double *hist = conv_state_in ? conv_state_in + b * (conv_k - 1) * D + d : NULL;
            double *dhist = dconv_state_in ? dconv_state_in + b * (conv_k - 1) * D + d : NULL;
            /* forward, keeping h_{t-1}, u_t, the conv pre-activation and dt */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                int64_t i = (b * L + t) * D + d;
                double u = x[i];
                if (K > 0) {
                    double c = conv_b ? conv_b[d] : 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        c += conv_w[d * K + k] * x_at(xbd, hist, D, t - (K - 1) + k, K);
                    cs[t] = c;
                    u = silu(c);
                }
                us[t] = u;
                double dt = delta[i];
                if (delta_softplus) dt = softplus(dt + (delta_bias ? delta_bias[d] : 0.0));
                dts[t] = dt;
                for (int64_t n = 0; n < N; ++n) {
                    double abar, bbar;
                    zoh(dt, A[d * N + n], Bm[(b * L + t) * N + n], &abar, &bbar);
                    hs[(t + 1) * N + n] = abar * hs[t * N + n] + bbar * u;
                }
            }
            /* backward */
            for (int64_t n = 0; n < N; ++n) lam[n] = dh_final ? dh_final[(b * D + d) * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                int64_t i = (b * L + t) * D + d;
                double u = us[t], dt = dts[t];
                double gy = dy[i];
                if (z) {
                    double yhat = (Dskip ? Dskip[d] * u : 0.0);
                    for (int64_t n = 0; n < N; ++n) yhat += Cm[(b * L + t) * N + n] * hs[(t + 1) * N + n];
                    if (dz) dz[i] = dy[i] * yhat * dsilu(z[i]);
                    gy = dy[i] * silu(z[i]);
                }
                double du = Dskip ? Dskip[d] * gy : 0.0;
                if (Dskip) pD[b * D + d] += gy * u;
                double ddt = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    double a = A[d * N + n], bb = Bm[(b * L + t) * N + n];
                    double cc = Cm[(b * L + t) * N + n];
                    double hprev = hs[t * N + n], hcur = hs[(t + 1) * N + n];
                    dCm[(b * L + t) * N + n] += gy * hcur;
                    double l = lam[n] + cc * gy;           /* dL/dh_t */
                    double zz = dt * a, e = exp(zz);
                    double phi = (zz == 0.0) ? 1.0 : expm1(zz) / zz;
                    double bbar = phi * dt * bb;
                    double dabar = l * hprev, dbbar = l * u;
                    du += l * bbar;
                    ddt += dabar * a * e + dbbar * bb * e;
                    pA[(b * D + d) * N + n] += dabar * dt * e + dbbar * bb * dt * dt * psi(zz);
                    dBm[(b * L + t) * N + n] += dbbar * dt * phi;
                    lam[n] = e * l;                         /* dL/dh_{t-1} */
                }
                double draw = ddt;
                if (delta_softplus) {
                    double sg = sigmoid(delta[i] + (delta_bias ? delta_bias[d] : 0.0));
                    draw = ddt * sg;
                    pbias[b * D + d] += draw;
                }
                ddelta[i] = draw;
                duv[t] = du;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = lam[n];
            /* through the conv prologue */
            for (int64_t t = 0; t < L; ++t) dx[(b * L + t) * D + d] = K > 0 ? 0.0 : duv[t];
            if (dhist)
                for (int64_t k = 0; k < K - 1; ++k) dhist[k * D] = 0.0;
            if (K > 0) {
                for (int64_t t = 0; t < L; ++t) {
                    double dc = duv[t] * dsilu(cs[t]);
                    pb[b * D + d] += dc;
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t s = t - (K - 1) + k;
                        pw[(b * D + d) * K + k] += dc * x_at(xbd, hist, D, s, K);
                        if (s >= 0)
                            dx[(b * L + s) * D + d] += dc * conv_w[d * K + k];
                        else if (dhist)
                            dhist[(K - 1 + s) * D] += dc * conv_w[d * K + k];
                    }
                }
            }
        }
        free(hs); free(us); free(cs); free(dts); free(duv); free(lam);
    }
    /* sum the per-row partials in a fixed order */
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t b = 0; b < Bsz; ++b) s += pA[(b * D + d) * N + n];
            dA[d * N + n] = s;
        }
        double sd = 0.0, sb = 0.0, sc = 0.0;
        for (int64_t b = 0; b < Bsz; ++b) { sd += pD[b * D + d]; sb += pbias[b * D + d]; sc += pb[b * D + d]; }
        if (dDskip) dDskip[d] = sd;
        if (ddelta_bias) ddelta_bias[d] = sb;
        if (dconv_b) dconv_b[d] = sc;
        if (dconv_w)
            for (int64_t k = 0; k < K; ++k) {
                double s = 0.0;
                for (int64_t b = 0; b < Bsz; ++b) s += pw[(b * D + d) * K + k];
                dconv_w[d * K + k] = s;
            }
    }
    free(pA); free(pD); free(pbias); free(pw); free(pb);
    return 0;
}

/*
 * Structured state-space duality (SSD, the Mamba-2 layer) in its recurrent
 * ("linear") mode, from [P4] sec. 5.1: the state matrix is a scalar times the
 * identity, A_t = a_t I, with one scalar per head, so every channel of a head
 * decays by the same factor.  Discretised like the rest of this oracle by the
 * ZOH rule of [P1] eq. (4) / [P4] sec. 3.2, which for A = a I reduces to
 *   alpha_t = exp(dt_t a_h),   w_t = (dt_t a_h)^-1 (exp(dt_t a_h) - 1) dt_t
 * (= dt_t when dt_t a_h == 0).  Per batch b, head h, head channel p and state
 * entry n, with g the group of the head (heads split evenly over G groups,
 * which share B and C):
 *   S_t[p,n] = alpha_t S_{t-1}[p,n] + w_t B_t[g,n] x_t[h,p]
 *   y_t[h,p] = (sum_n C_t[g,n] S_t[p,n] + Dskip[h] x_t[h,p]) * silu(z_t[h,p])
 *
 * Shapes: x, z, y (B,L,H,P); delta (B,L,H); A, Dskip, delta_bias (H);
 * Bm, Cm (B,L,G,N); h0, h_final (B,H,P,N).  dt is delta, or softplus(delta +
 * bias) when requested.  Optional arguments may be NULL.  Threads split the
 * independent (batch, head) pairs.  Returns 0, or -1 on a bad size.
 */
int oracle_ssd_f64(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                   const double *x, const double *delta, const double *A, const double *Bm,
                   const double *Cm, const double *Dskip, const double *z,
                   const double *delta_bias, int delta_softplus, const double *h0, double *y,
                   double *h_final, int nthreads)
{
    if (Bsz < 0 || L < 0 || H < 1 || P < 1 || G < 1 || N < 1 || H % G != 0) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t heads_per_group = H / G;
    const int64_t npairs = Bsz * H;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t bh = 0; bh < npairs; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / heads_per_group;
        double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
        for (int64_t i = 0; i < P * N; ++i) S[i] = h0 ? h0[bh * P * N + i] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dt = delta[(b * L + t) * H + h];
            if (delta_softplus) dt = softplus(dt + (delta_bias ? delta_bias[h] : 0.0));
            const double *Bt = Bm + ((b * L + t) * G + g) * N;
            const double *Ct = Cm + ((b * L + t) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const int64_t i = ((b * L + t) * H + h) * P + p;
                const double u = x[i];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    double abar, bbar;
                    zoh(dt, A[h], Bt[n], &abar, &bbar);
                    double *s = S + p * N + n;
                    *s = abar * *s + bbar * u;
                    acc += Ct[n] * *s;
                }
                double yv = acc + (Dskip ? Dskip[h] * u : 0.0);
                if (z) yv *= silu(z[i]);
                y[i] = yv;
            }
        }
        if (h_final)
            for (int64_t i = 0; i < P * N; ++i) h_final[bh * P * N + i] = S[i];
        free(S);
    }
    return 0;
}
