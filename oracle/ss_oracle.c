/*
 * Plain fp64 CPU oracle of the selective scan (S6): forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
 * baseline load this library; the GPU library shares no code with it.
 *
 * Same definition as oracle/ss_ref.py, in C for the large workloads:
 *   u_t = dt_bias[d] + dt_raw[b,d,t];  δ_t = softplus(u_t)      ("3.2 선택적 스캔 알고리즘…" page, §1.2)
 *   Ā_{t,n} = exp(δ_t A[d,n])                                  (same page, §2.1; A diagonal)
 *   h_t = Ā_t ⊙ h_{t-1} + δ_t B_t x_t                          (same page, §2.2; first-order B̄ as in §4.1)
 *     or, with zoh, + (exp(δ_t A) - 1)/A · B_t x_t               (the exact zero-order hold of §2.1)
 *   y_t = (Σ_n C_{t,n} h_{t,n} + D[d] x_t) · silu(z_t)         (readout §1.1; gate: "상태공간 모델(SSM)과
 *                                                               Mamba 아키텍처" note, §3 flowchart)
 * One channel (b,d) at a time, t in order, every operation in double.  OpenMP
 * parallelises over independent channels only; backward reductions over
 * channels go to per-thread buffers summed afterwards in thread order.
 *
 * Inputs are float32 arrays (bf16 workloads pass bf16-exact values), widened
 * to double on load.  Layouts: x, dt_raw, z, dy [B,D,L]; Bm, Cm [B,N,L];
 * A [D,N]; dt_bias, Dskip [D]; h0, dh_final [B,D,N].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_d(double u) { return (u > 0 ? u : 0.0) + log1p(exp(-fabs(u))); }

static double sigmoid_d(double z) {
    double e = exp(-fabs(z));
    return z >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

int s6o_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Forward over a list of channels.  chans[i] = b*D + d (NULL: all B*D channels
 * in order, nchan must then be B*D).  y is [nchan, L]; h_final (nullable) is
 * [nchan, N].  z and h0 are nullable.  zoh = 1: exact zero-order-hold B̄ (expm1(δA)/A;
 * δ where A = 0).  Returns 0, or -1 on bad sizes.
 */
int s6o_fwd(int64_t B, int64_t L, int64_t D, int64_t N,
            const float* x, const float* dt_raw, const float* dt_bias, const float* A,
            const float* Bm, const float* Cm, const float* Dskip, const float* z, const float* h0,
            const int64_t* chans, int64_t nchan, double* y, double* h_final, int zoh) {
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0 || nchan <= 0) return -1;
    if (!chans && nchan != B * D) return -1;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nchan; ++i) {
        int64_t c = chans ? chans[i] : i;
        int64_t b = c / D, d = c % D;
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? (double)h0[c * N + n] : 0.0;
        const float* xr = x + c * L;
        const float* dr = dt_raw + c * L;
        const float* zr = z ? z + c * L : NULL;
        const float* Br = Bm + b * N * L;
        const float* Cr = Cm + b * N * L;
        double bias = dt_bias[d], Dd = Dskip[d];
        for (int64_t t = 0; t < L; ++t) {
            double xt = xr[t];
            double delta = softplus_d(bias + (double)dr[t]);
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double an = (double)A[d * N + n];
                double abar = exp(delta * an);
                double fb = (zoh && an != 0.0) ? expm1(delta * an) / an : delta;
                h[n] = abar * h[n] + fb * (double)Br[n * L + t] * xt;
                s += (double)Cr[n * L + t] * h[n];
            }
            s += Dd * xt;
            if (zr) {
                double zt = zr[t];
                s = s * zt * sigmoid_d(zt);
            }
            y[i * L + t] = s;
        }
        if (h_final)
            for (int64_t n = 0; n < N; ++n) h_final[i * N + n] = h[n];
        free(h);
    }
    return 0;
}

/*
 * Backward over all channels: gradients of sum(dy*y) + sum(dh_final*h_final).
 * Outputs (double): dx, ddt_raw [B,D,L]; dz [B,D,L] (required iff z); ddt_bias [D];
 * dA [D,N]; dB, dC [B,N,L]; dD [D]; dh0 [B,D,N] (required iff h0).
 * Forward states are stored for the whole sequence of the channel, then the
 * adjoint g = ∂/∂h_t is swept from t = L-1 to 0 (see oracle/ss_ref.py).
 * zoh = 1: gradients of the exact zero-order-hold forward, whose input factor
 * f = expm1(δA)/A has ∂f/∂δ = Ā and ∂f/∂A = (δĀ - f)/A (series below |δA| = 1e-2).
 */
/* ∂f/∂A of the exact-hold factor: δ² Σ_k (k+1) u^k/(k+2)!, u = δA, for |u| < 1e-2
 * (ten terms), else the closed form (δ e^u - expm1(u)/A)/A. */
static double zoh_dfda(double delta, double an) {
    double u = delta * an;
    if (fabs(u) < 1e-2) {
        double sum = 0.0, fact = 2.0, pw = 1.0;
        for (int k = 0; k < 10; ++k) {
            sum += (k + 1) * pw / fact;
            pw *= u;
            fact *= k + 3;
        }
        return delta * delta * sum;
    }
    return (delta * exp(u) - expm1(u) / an) / an;
}

int s6o_bwd(int64_t B, int64_t L, int64_t D, int64_t N,
            const float* x, const float* dt_raw, const float* dt_bias, const float* A,
            const float* Bm, const float* Cm, const float* Dskip, const float* z, const float* h0,
            const float* dy, const float* dh_final,
            double* dx, double* ddt_raw, double* dz, double* ddt_bias, double* dA,
            double* dB, double* dC, double* dD, double* dh0, int zoh) {
    if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return -1;
    if ((z && !dz) || (h0 && !dh0)) return -1;
    int nth = 1;
#ifdef _OPENMP
    nth = omp_get_max_threads();
#endif
    size_t nBC = (size_t)(B * N * L);
    double* pB = (double*)calloc((size_t)nth * nBC, sizeof(double));
    double* pC = (double*)calloc((size_t)nth * nBC, sizeof(double));
    double* pA = (double*)calloc((size_t)nth * (size_t)(D * N), sizeof(double));
    double* pD = (double*)calloc((size_t)nth * (size_t)D, sizeof(double));
    double* pT = (double*)calloc((size_t)nth * (size_t)D, sizeof(double));
    if (!pB || !pC || !pA || !pD || !pT) {
        free(pB); free(pC); free(pA); free(pD); free(pT);
        return -2;
    }
    int64_t c;
#pragma omp parallel for schedule(dynamic, 1)
    for (c = 0; c < B * D; ++c) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        int64_t b = c / D, d = c % D;
        double* myB = pB + (size_t)tid * nBC + (size_t)(b * N * L);
        double* myC = pC + (size_t)tid * nBC + (size_t)(b * N * L);
        double* myA = pA + (size_t)tid * (size_t)(D * N) + (size_t)(d * N);
        double* myD = pD + (size_t)tid * (size_t)D + d;
        double* myT = pT + (size_t)tid * (size_t)D + d;
        const float* xr = x + c * L;
        const float* dr = dt_raw + c * L;
        const float* zr = z ? z + c * L : NULL;
        const float* gr = dy + c * L;
        const float* Br = Bm + b * N * L;
        const float* Cr = Cm + b * N * L;
        double bias = dt_bias[d], Dd = Dskip[d];
        /* hs[(t+1)*N + n] = h_{t,n}; hs[n] = h_{-1,n} */
        double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
        double* sv = (double*)malloc(sizeof(double) * (size_t)L);
        double* g = (double*)malloc(sizeof(double) * (size_t)N);
        for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? (double)h0[c * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double xt = xr[t];
            double delta = softplus_d(bias + (double)dr[t]);
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double an = (double)A[d * N + n];
                double abar = exp(delta * an);
                double fb = (zoh && an != 0.0) ? expm1(delta * an) / an : delta;
                double hn = abar * hs[t * N + n] + fb * (double)Br[n * L + t] * xt;
                hs[(t + 1) * N + n] = hn;
                s += (double)Cr[n * L + t] * hn;
            }
            sv[t] = s + Dd * xt;
        }
        for (int64_t n = 0; n < N; ++n) g[n] = dh_final ? (double)dh_final[c * N + n] : 0.0;
        double accT = 0.0, accD = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            double xt = xr[t];
            double u = bias + (double)dr[t];
            double delta = softplus_d(u);
            double ds;
            if (zr) {
                double zt = zr[t], sz = sigmoid_d(zt);
                ds = (double)gr[t] * zt * sz;
                dz[c * L + t] = (double)gr[t] * sv[t] * sz * (1.0 + zt * (1.0 - sz));
            } else {
                ds = (double)gr[t];
            }
            double dxt = ds * Dd, ddel = 0.0;
            accD += ds * xt;
            for (int64_t n = 0; n < N; ++n) {
                double Bt = Br[n * L + t], Ct = Cr[n * L + t];
                double an = (double)A[d * N + n];
                double abar = exp(delta * an);
                double hprev = hs[t * N + n];
                /* input factor f and its partials: (δ, 1, 0) first order */
                double fb = delta, dfd = 1.0, dfa = 0.0;
                if (zoh) {
                    fb = an != 0.0 ? expm1(delta * an) / an : delta;
                    dfd = abar;
                    dfa = zoh_dfda(delta, an);
                }
                g[n] += ds * Ct;
                myC[n * L + t] += ds * hs[(t + 1) * N + n];
                myB[n * L + t] += g[n] * fb * xt;
                dxt += g[n] * fb * Bt;
                ddel += g[n] * (an * abar * hprev + dfd * Bt * xt);
                myA[n] += g[n] * (delta * abar * hprev + dfa * Bt * xt);
                g[n] *= abar;
            }
            dx[c * L + t] = dxt;
            double dr_t = ddel * sigmoid_d(u);
            ddt_raw[c * L + t] = dr_t;
            accT += dr_t;
        }
        *myD += accD;
        *myT += accT;
        if (h0)
            for (int64_t n = 0; n < N; ++n) dh0[c * N + n] = g[n];
        free(hs); free(sv); free(g);
    }
    memset(dB, 0, sizeof(double) * nBC);
    memset(dC, 0, sizeof(double) * nBC);
    memset(dA, 0, sizeof(double) * (size_t)(D * N));
    memset(dD, 0, sizeof(double) * (size_t)D);
    memset(ddt_bias, 0, sizeof(double) * (size_t)D);
    for (int k = 0; k < nth; ++k) {
        for (size_t i = 0; i < nBC; ++i) {
            dB[i] += pB[(size_t)k * nBC + i];
            dC[i] += pC[(size_t)k * nBC + i];
        }
        for (int64_t i = 0; i < D * N; ++i) dA[i] += pA[(size_t)k * (size_t)(D * N) + (size_t)i];
        for (int64_t i = 0; i < D; ++i) {
            dD[i] += pD[(size_t)k * (size_t)D + (size_t)i];
            ddt_bias[i] += pT[(size_t)k * (size_t)D + (size_t)i];
        }
    }
    free(pB); free(pC); free(pA); free(pD); free(pT);
    return 0;
}
