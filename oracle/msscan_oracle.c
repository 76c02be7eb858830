/*
 * msscan_oracle.c -- plain, slow, fp64 CPU oracle for the selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this file's library.  It shares
 * no code, header, table or helper with the HIP library; the HIP library never
 * includes, links or calls it.
 *
 * Every function below follows the pages' statement of the method:
 *
 *   * The recurrence and its readout are the per-timestep loop of the naive
 *     PyTorch selective scan on the lmnt.cn page (news/271401; its text
 *     carries no title line and opens with section 1, "从RNN到Mamba"),
 *     section 3.2: A_bar = exp(dt*A),
 *     B_bar = dt*B_t (broadcast over channels), h = A_bar*h + B_bar*x_t,
 *     y_t = sum_n h*C_t, then y += x*D, then y * silu(z).
 *   * The step size is softplus of a linear map plus bias: page "Mamba架构原理与
 *     工业级长文本处理实战指南" (jsqmd.com/news/861956), section 2.2, first
 *     equation; softplus is log(1+e^x) there.
 *   * The zero-order-hold alternative B_bar = (exp(dt*A) - 1)/A * B is the
 *     discretisation of page "Mamba模型解析：从状态空间到序列建模实践"
 *     (intelliparadigm.com), section 3.2, and the integral form of the jsqmd
 *     page, section 2.3; for a diagonal A the matrix inverse is a division.
 *   * Inference runs the same recurrence one token at a time with one kept
 *     state (lmnt page, sections 2.2 and 5.3): oracle_step.
 *
 * Readings where the pages are silent:
 *   the state starts at zero unless h0 is given; "Euler" keeps A_bar=exp(dt*A)
 *   and only replaces B_bar by dt*B; the bias goes inside softplus; D*u is added
 *   before the gate; silu(z) = z/(1+exp(-z)); B_t and C_t are shared by all
 *   channels; at A == 0 the ZOH factor takes its limit dt.
 *
 * Arithmetic: every input is first converted to double by the caller (bf16 and
 * fp32 convert exactly); all arithmetic here is double precision libm.
 * Layouts (row-major, contiguous):
 *   u, delta_raw, z, y : [batch][L][Dn]
 *   B, C               : [batch][L][N]
 *   A                  : [Dn][N]
 *   D, delta_bias      : [Dn]
 *   h0, h_last, h      : [batch][Dn][N]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), written so that neither e^x overflows nor the
 * 1 + small sum loses digits: max(x,0) + log1p(e^-|x|).  Same value as the
 * pages' definition, in exact arithmetic. */
static double sp_softplus(double x) {
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* silu(v) = v * sigmoid(v). */
static double sp_silu(double v) {
    return v / (1.0 + exp(-v));
}

/* Step size of one element: dt = softplus(delta_raw + bias) when softplus is
 * on, else delta_raw + bias. */
static double step_size(double draw, const double* delta_bias, int64_t d, int softplus) {
    double v = draw + (delta_bias ? delta_bias[d] : 0.0);
    return softplus ? sp_softplus(v) : v;
}

/* One timestep of one channel: updates h[0..N) in place, returns the gated
 * output.  The body is the loop body of the lmnt page section 3.2.  The
 * discretisation `disc` picks A_bar and the factor of B*u:
 *   0 Euler     A_bar = exp(dt*A),  dt
 *   1 ZOH       A_bar = exp(dt*A),  (exp(dt*A) - 1)/A  (dt at A == 0)
 *               (intelliparadigm page, section 3.2)
 *   2 bilinear  A_bar = (1 + dt*A/2)/(1 - dt*A/2),  dt/(1 - dt*A/2)
 *               (the bilinear transform the intelliparadigm page's section 3.2
 *               code names; its printed code is garbled, so this is the
 *               textbook form for a diagonal A). */
static double one_step(double* h, double ut, double dt, const double* Arow,
                       const double* Bt, const double* Ct, int64_t N,
                       double Dd, int has_D, double zt, int has_z, int disc) {
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double a = Arow[n];
        double abar, bfac;
        if (disc == 2) {
            const double half = 0.5 * dt * a;
            abar = (1.0 + half) / (1.0 - half);
            bfac = dt / (1.0 - half);
        } else {
            abar = exp(dt * a);
            if (disc == 1)
                bfac = (a == 0.0) ? dt : expm1(dt * a) / a;
            else
                bfac = dt;
        }
        h[n] = abar * h[n] + bfac * Bt[n] * ut;
        acc += Ct[n] * h[n];
    }
    if (has_D) acc += Dd * ut;
    if (has_z) acc *= sp_silu(zt);
    return acc;
}

/* Full-sequence scan.  Channels (b, d) are independent; OpenMP runs them in
 * parallel, each channel strictly in time order.  Returns 0 on success,
 * -1 on bad arguments, -2 on allocation failure. */
int oracle_scan(const double* u, const double* delta_raw, const double* A,
                const double* B, const double* C, const double* D,
                const double* z, const double* delta_bias, const double* h0,
                int softplus, int disc, int64_t batch, int64_t L, int64_t Dn,
                int64_t N, double* y, double* h_last, int nthreads) {
    if (!u || !delta_raw || !A || !B || !C || !y) return -1;
    if (batch < 0 || L < 0 || Dn < 0 || N < 1) return -1;
    int64_t nch = batch * Dn;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        if (!h) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t ch = 0; ch < nch; ++ch) {
            if (!h) continue;
            int64_t b = ch / Dn, d = ch % Dn;
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                int64_t e = (b * L + t) * Dn + d;
                const double* Bt = B + (b * L + t) * N;
                const double* Ct = C + (b * L + t) * N;
                double dt = step_size(delta_raw[e], delta_bias, d, softplus);
                y[e] = one_step(h, u[e], dt, A + d * N, Bt, Ct, N,
                                D ? D[d] : 0.0, D != NULL, z ? z[e] : 0.0,
                                z != NULL, disc);
            }
            if (h_last)
                for (int64_t n = 0; n < N; ++n) h_last[(b * Dn + d) * N + n] = h[n];
        }
        free(h);
    }
    return failed ? -2 : 0;
}

/* One decode step with the state kept by the caller (lmnt page, section 5.3:
 * generation token by token with one fixed-size state).  h is [batch][Dn][N]
 * and is updated in place; x, delta_raw, z, y are [batch][Dn]; B, C are
 * [batch][N].  Same body as one timestep of oracle_scan. */
int oracle_step(double* h, const double* x, const double* delta_raw,
                const double* A, const double* B, const double* C,
                const double* D, const double* z, const double* delta_bias,
                int softplus, int disc, int64_t batch, int64_t Dn, int64_t N,
                double* y) {
    if (!h || !x || !delta_raw || !A || !B || !C || !y) return -1;
    if (batch < 0 || Dn < 0 || N < 1) return -1;
    int64_t nch = batch * Dn;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t e = 0; e < nch; ++e) {
        int64_t b = e / Dn, d = e % Dn;
        double dt = step_size(delta_raw[e], delta_bias, d, softplus);
        y[e] = one_step(h + e * N, x[e], dt, A + d * N, B + b * N, C + b * N,
                        N, D ? D[d] : 0.0, D != NULL, z ? z[e] : 0.0,
                        z != NULL, disc);
    }
    return 0;
}

/* Derivatives of A_bar and of the B*u factor with respect to dt and to a,
 * for the three discretisations of one_step:
 *   Euler:    A_bar = e^{dt a}, f = dt
 *   ZOH:      A_bar = e^{dt a}, f = (e^{dt a} - 1)/a  (dt at a = 0)
 *   bilinear: A_bar = (1 + dt a/2)/(1 - dt a/2), f = dt/(1 - dt a/2)      */
static void disc_parts(double dt, double a, int disc, double* abar, double* f, double* dabar_ddt,
                       double* dabar_da, double* df_ddt, double* df_da) {
    if (disc == 2) {
        const double q = 1.0 - 0.5 * dt * a;
        *abar = (1.0 + 0.5 * dt * a) / q;
        *f = dt / q;
        *dabar_ddt = a / (q * q);
        *dabar_da = dt / (q * q);
        *df_ddt = 1.0 / (q * q);
        *df_da = 0.5 * dt * dt / (q * q);
        return;
    }
    const double e = exp(dt * a);
    *abar = e;
    *dabar_ddt = a * e;
    *dabar_da = dt * e;
    if (disc == 1) {
        if (a == 0.0) {
            *f = dt;
            *df_ddt = 1.0;
            *df_da = 0.5 * dt * dt;
        } else {
            *f = expm1(dt * a) / a;
            *df_ddt = e;
            *df_da = (dt * e - *f) / a;
        }
    } else {
        *f = dt;
        *df_ddt = 1.0;
        *df_da = 0.0;
    }
}

/* Gradients of the scan (the reverse-mode derivative of oracle_scan), for
 * training.  Given dy = dL/dy (and dh_last = dL/dh_last, or none), returns
 * dL/d of every input: du, ddelta (w.r.t. delta_raw), dz, dA, dB, dC, dD,
 * dbias, dh0.  The pages train the model end to end by gradient descent
 * (jsqmd page, section 4.2; the lmnt page's training loop in section 4.2) but
 * print no derivative, so this is the chain rule applied to one_step, run
 * backwards in time: with lambda_t = dL/dh_t,
 *   lambda_t = C_t g_t + A_bar_{t+1} lambda_{t+1}   (g_t = dL/dy_pre_t),
 * and every input's gradient collects its terms from each step.  The forward
 * states are recomputed per channel first.
 * Layouts as oracle_scan; dA, dB, dC, dD, dbias accumulate sums over the
 * channels / batch rows / timesteps that share the parameter.  Outputs dz,
 * dD, dbias, dh0 may be NULL (dz and dD must be given when z and D are).
 * Runs channels of one batch row in parallel with per-thread partial sums of
 * dB and dC, reduced in thread order (deterministic for a fixed thread count). */
int oracle_scan_bwd(const double* u, const double* delta_raw, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* delta_bias,
                    const double* h0, int softplus, int disc, int64_t batch, int64_t L,
                    int64_t Dn, int64_t N, const double* dy, const double* dh_last, double* du,
                    double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dz,
                    double* dbias, double* dh0, int nthreads) {
    if (!u || !delta_raw || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
        return -1;
    if ((z && !dz) || (D && !dD)) return -1;
    if (batch < 0 || L < 0 || Dn < 0 || N < 1) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    const int nt = omp_get_max_threads();
#else
    const int nt = 1;
#endif
    for (int64_t i = 0; i < Dn * N; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < batch * L * N; ++i) dB[i] = dC[i] = 0.0;
    if (dD)
        for (int64_t i = 0; i < Dn; ++i) dD[i] = 0.0;
    if (dbias)
        for (int64_t i = 0; i < Dn; ++i) dbias[i] = 0.0;
    /* per-thread partial sums: dB, dC of the current batch row; dA, dD, dbias */
    double* part = (double*)calloc((size_t)nt * (size_t)(2 * L * N + Dn * N + 2 * Dn),
                                   sizeof(double));
    if (!part) return -2;
    int failed = 0;
    for (int64_t b = 0; b < batch; ++b) {
#ifdef _OPENMP
#pragma omp parallel
#endif
        {
#ifdef _OPENMP
            const int tid = omp_get_thread_num();
#else
            const int tid = 0;
#endif
            double* pB = part + (size_t)tid * (size_t)(2 * L * N + Dn * N + 2 * Dn);
            double* pC = pB + L * N;
            double* pA = pC + L * N;
            double* pD = pA + Dn * N;
            double* pbias = pD + Dn;
            for (int64_t i = 0; i < 2 * L * N; ++i) pB[i] = 0.0;
            double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
            double* lam = (double*)malloc(sizeof(double) * (size_t)N);
            if (!hs || !lam) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
                failed = 1;
            }
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
            for (int64_t d = 0; d < Dn; ++d) {
                if (!hs || !lam) continue;
                const double* Arow = A + d * N;
                /* forward: hs[(t+1)*N + n] = h_t, hs[n] = h_{-1} */
                for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t e = (b * L + t) * Dn + d;
                    const double dt = step_size(delta_raw[e], delta_bias, d, softplus);
                    for (int64_t n = 0; n < N; ++n) {
                        double abar, f, x1, x2, x3, x4;
                        disc_parts(dt, Arow[n], disc, &abar, &f, &x1, &x2, &x3, &x4);
                        hs[(t + 1) * N + n] =
                            abar * hs[t * N + n] + f * B[(b * L + t) * N + n] * u[e];
                    }
                }
                /* backward */
                for (int64_t n = 0; n < N; ++n) lam[n] = dh_last ? dh_last[(b * Dn + d) * N + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    const int64_t e = (b * L + t) * Dn + d;
                    const double v = delta_raw[e] + (delta_bias ? delta_bias[d] : 0.0);
                    const double dt = softplus ? sp_softplus(v) : v;
                    const double* Bt = B + (b * L + t) * N;
                    const double* Ct = C + (b * L + t) * N;
                    const double* ht = hs + (t + 1) * N;
                    const double* hp = hs + t * N;
                    double ypre = D ? D[d] * u[e] : 0.0;
                    for (int64_t n = 0; n < N; ++n) ypre += Ct[n] * ht[n];
                    double g = dy[e];
                    if (z) {
                        const double sg = 1.0 / (1.0 + exp(-z[e]));
                        g = dy[e] * z[e] * sg;
                        dz[e] = dy[e] * ypre * sg * (1.0 + z[e] * (1.0 - sg));
                    }
                    double du_e = D ? g * D[d] : 0.0;
                    if (D) pD[d] += g * u[e];
                    double ddt = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        double abar, f, dab_dt, dab_da, df_dt, df_da;
                        disc_parts(dt, Arow[n], disc, &abar, &f, &dab_dt, &dab_da, &df_dt, &df_da);
                        const double l = Ct[n] * g + lam[n];      /* lambda_t */
                        pC[t * N + n] += g * ht[n];
                        const double dab = l * hp[n];               /* dL/dA_bar */
                        const double dfac = l * Bt[n] * u[e];       /* dL/df */
                        pB[t * N + n] += l * f * u[e];
                        du_e += l * f * Bt[n];
                        ddt += dab * dab_dt + dfac * df_dt;
                        pA[d * N + n] += dab * dab_da + dfac * df_da;
                        lam[n] = abar * l;                          /* to step t-1 */
                    }
                    du[e] = du_e;
                    const double dv = softplus ? ddt / (1.0 + exp(-v)) : ddt;
                    ddelta[e] = dv;
                    pbias[d] += dv;
                }
                if (dh0)
                    for (int64_t n = 0; n < N; ++n) dh0[(b * Dn + d) * N + n] = lam[n];
            }
            free(hs);
            free(lam);
        }
        /* reduce the row's dB, dC partials in thread order */
        for (int th = 0; th < nt; ++th) {
            double* pB = part + (size_t)th * (size_t)(2 * L * N + Dn * N + 2 * Dn);
            for (int64_t i = 0; i < L * N; ++i) {
                dB[b * L * N + i] += pB[i];
                dC[b * L * N + i] += pB[L * N + i];
            }
        }
    }
    for (int th = 0; th < nt; ++th) {
        double* pA = part + (size_t)th * (size_t)(2 * L * N + Dn * N + 2 * Dn) + 2 * L * N;
        for (int64_t i = 0; i < Dn * N; ++i) dA[i] += pA[i];
        for (int64_t i = 0; i < Dn; ++i) {
            if (dD) dD[i] += pA[Dn * N + i];
            if (dbias) dbias[i] += pA[Dn * N + Dn + i];
        }
    }
    free(part);
    return failed ? -2 : 0;
}

/* Causal depthwise conv1d, optionally followed by silu: the step that turns
 * the x branch of the block input into the scan input u (lmnt page,
 * section 3.1: a depthwise 1D convolution of width about 4 on x_ssm before
 * the SSM; section 3.2: groups = d_inner, padding = width - 1, output cut to
 * the first L steps, then silu).  For every (b, t, d):
 *   pre = bias[d] + sum_{k=0}^{width-1} w[d][k] * x[b, t - (width-1) + k, d]
 * where a time index below 0 reads x_prev[b][width-1 + index][d] when x_prev
 * is given (the width-1 inputs before t = 0, oldest first) and 0 otherwise;
 * u = silu(pre) when silu is set, else pre.
 * Layouts: x, u [batch][L][Dn]; w [Dn][width]; bias [Dn];
 * x_prev [batch][width-1][Dn]. */
int oracle_conv1d(const double* x, const double* w, const double* bias, const double* x_prev,
                  int64_t width, int silu, int64_t batch, int64_t L, int64_t Dn, double* u,
                  int nthreads) {
    if (width < 1 || batch < 0 || L < 0 || Dn < 0) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for collapse(2) schedule(static)
#endif
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            for (int64_t t = 0; t < L; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k) {
                    const int64_t ti = t - (width - 1) + k;
                    double xv = 0.0;
                    if (ti >= 0)
                        xv = x[(b * L + ti) * Dn + d];
                    else if (x_prev)
                        xv = x_prev[(b * (width - 1) + (width - 1) + ti) * Dn + d];
                    pre += w[d * width + k] * xv;
                }
                u[(b * L + t) * Dn + d] = silu ? sp_silu(pre) : pre;
            }
        }
    }
    return 0;
}

/* Number of threads OpenMP would use (for reporting the CPU baseline). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
