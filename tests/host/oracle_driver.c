/*
 * Driver of the C fp64 oracle (oracle/ss_oracle.c) for its sanitized build
 * (tests/test_sanitize.py: -fsanitize=address,undefined, OpenMP on two threads).
 *
 * Runs the forward (all channels and a subset, first-order and exact hold, with and
 * without gate and initial state) and the backward (every optional input on and off) on
 * small seeded shapes, including N = 1 and N = 64, L = 1 and ragged sizes, and checks that
 * every output is finite.  The sanitizers report any out-of-range access in the oracle's
 * hand-indexed loops and per-thread partial buffers.  Prints "oracle ok <count>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int s6o_threads(int nthreads);
int s6o_fwd(int64_t B, int64_t L, int64_t D, int64_t N, const float* x, const float* dt_raw,
            const float* dt_bias, const float* A, const float* Bm, const float* Cm,
            const float* Dskip, const float* z, const float* h0, const int64_t* chans,
            int64_t nchan, double* y, double* h_final, int zoh);
int s6o_bwd(int64_t B, int64_t L, int64_t D, int64_t N, const float* x, const float* dt_raw,
            const float* dt_bias, const float* A, const float* Bm, const float* Cm,
            const float* Dskip, const float* z, const float* h0, const float* dy,
            const float* dh_final, double* dx, double* ddt_raw, double* dz, double* ddt_bias,
            double* dA, double* dB, double* dC, double* dD, double* dh0, int zoh);

static uint64_t rng = 12345;
static float unif(void) {   /* in [-1, 1) */
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((rng >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}
static float* arr(int64_t n, float scale, float shift) {
    float* a = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) a[i] = shift + scale * unif();
    return a;
}
static int finite_all(const double* a, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    s6o_threads(2);
    const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 9, 3, 4}, {1, 33, 5, 16}, {3, 17, 2, 2},
                                 {1, 40, 7, 64}, {2, 64, 64, 8}, {1, 5, 130, 32}};
    int count = 0;
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int64_t B = shapes[s][0], L = shapes[s][1], D = shapes[s][2], N = shapes[s][3];
        const int64_t BDL = B * D * L, BNL = B * N * L, DN = D * N, BDN = B * D * N;
        float *x = arr(BDL, 1, 0), *dtr = arr(BDL, 1, 0), *z = arr(BDL, 2, 0);
        float *dtb = arr(D, 1, -3), *A = arr(DN, 0.5f, -1.5f), *Bm = arr(BNL, 1, 0);
        float *Cm = arr(BNL, 1, 0), *Dk = arr(D, 1, 0), *h0 = arr(BDN, 1, 0);
        float *dy = arr(BDL, 1, 0), *dhf = arr(BDN, 1, 0);
        /* the channel-subset calls write 3 rows whatever B·D is */
        const int64_t ny = BDL > 3 * L ? BDL : 3 * L, nh = BDN > 3 * N ? BDN : 3 * N;
        double *y = malloc((size_t)ny * 8), *hf = malloc((size_t)nh * 8);
        double *dx = malloc((size_t)BDL * 8), *ddt = malloc((size_t)BDL * 8), *dz = malloc((size_t)BDL * 8);
        double *ddtb = malloc((size_t)D * 8), *dA = malloc((size_t)DN * 8), *dB = malloc((size_t)BNL * 8);
        double *dC = malloc((size_t)BNL * 8), *dD = malloc((size_t)D * 8), *dh0 = malloc((size_t)BDN * 8);
        int64_t chans[3] = {0, B * D - 1, (B * D) / 2};
        for (int zoh = 0; zoh < 2; ++zoh)
            for (int opt = 0; opt < 4; ++opt) {
                const float* zz = (opt & 1) ? z : NULL;
                const float* hh = (opt & 2) ? h0 : NULL;
                if (s6o_fwd(B, L, D, N, x, dtr, dtb, A, Bm, Cm, Dk, zz, hh, NULL, B * D, y, hf, zoh) ||
                    !finite_all(y, BDL) || !finite_all(hf, BDN)) {
                    printf("FAIL fwd shape %zu zoh %d opt %d\n", s, zoh, opt);
                    return 1;
                }
                if (s6o_fwd(B, L, D, N, x, dtr, dtb, A, Bm, Cm, Dk, zz, hh, chans, 3, y, hf, zoh) ||
                    !finite_all(y, 3 * L) || !finite_all(hf, 3 * N)) {
                    printf("FAIL fwd chans shape %zu zoh %d opt %d\n", s, zoh, opt);
                    return 1;
                }
                const float* dd = (opt & 1) ? dhf : NULL;
                if (s6o_bwd(B, L, D, N, x, dtr, dtb, A, Bm, Cm, Dk, zz, hh, dy, dd, dx, ddt,
                            zz ? dz : NULL, ddtb, dA, dB, dC, dD, hh ? dh0 : NULL, zoh) ||
                    !finite_all(dx, BDL) || !finite_all(ddt, BDL) || !finite_all(dA, DN) ||
                    !finite_all(dB, BNL) || !finite_all(dC, BNL) || !finite_all(dD, D) ||
                    !finite_all(ddtb, D) || (zz && !finite_all(dz, BDL)) || (hh && !finite_all(dh0, BDN))) {
                    printf("FAIL bwd shape %zu zoh %d opt %d\n", s, zoh, opt);
                    return 1;
                }
                count += 3;
            }
        free(x); free(dtr); free(z); free(dtb); free(A); free(Bm); free(Cm); free(Dk); free(h0);
        free(dy); free(dhf); free(y); free(hf); free(dx); free(ddt); free(dz); free(ddtb);
        free(dA); free(dB); free(dC); free(dD); free(dh0);
    }
    printf("oracle ok %d\n", count);
    return 0;
}
