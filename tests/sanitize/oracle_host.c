/* The C oracle run under AddressSanitizer and UndefinedBehaviorSanitizer on small odd-sized
 * problems: packed sequences with an empty one, a head selection in reverse order, fp32 and bf16
 * inputs, with and without initial states, several worker threads.  Every buffer is allocated at
 * its exact size, so a read or write past an end is reported.  Also checks that a head selection
 * reproduces the same heads of a full run, and that bad arguments are refused.
 * Exit status 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_fwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                   int io_bf16, double scale, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *s0, int nsel, const int32_t *heads, double *o,
                   double *s_final, int nthreads);
int kda_oracle_bwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                   int io_bf16, double scale, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *s0, const void *d_o, const float *d_sf, int nsel,
                   const int32_t *heads, double *dq, double *dk_out, double *dv_out, double *dg, double *dbeta,
                   double *ds0, int nthreads);
int kda_oracle_dplr_fwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                        int io_bf16, double scale, const void *q, const void *k, const void *v, const void *a,
                        const void *b, const float *g, const float *s0, double *o, double *s_final, int nthreads);

static int failures = 0, checks = 0;
#define EXPECT(c)                                                        \
    do {                                                                 \
        ++checks;                                                        \
        if (!(c)) {                                                      \
            ++failures;                                                  \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);       \
        }                                                                \
    } while (0)

static uint64_t rng = 0x243F6A8885A308D3ull;
static double uniform(void) { /* xorshift64*, [-1, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static float *floats(size_t n, double lo, double hi) {
    float *x = (float *)malloc(n * sizeof(float) + 1);
    for (size_t i = 0; i < n; ++i) x[i] = (float)(lo + (hi - lo) * 0.5 * (uniform() + 1.0));
    return x;
}
static uint16_t *bf16_of(const float *x, size_t n) { /* truncation: any bf16 values will do */
    uint16_t *y = (uint16_t *)malloc(n * sizeof(uint16_t) + 1);
    for (size_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        y[i] = (uint16_t)(u >> 16);
    }
    return y;
}
static double *zeros(size_t n) { return (double *)calloc(n ? n : 1, sizeof(double)); }
static int all_finite(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    enum { N = 4, H = 3, DK = 5, DV = 7 };
    const int64_t lens[N] = {3, 0, 1, 6};
    int64_t starts[N];
    int64_t T = 0;
    for (int n = 0; n < N; ++n) {
        starts[n] = T;
        T += lens[n];
    }
    const size_t nk = (size_t)T * H * DK, nv = (size_t)T * H * DV, ns = (size_t)N * H * DK * DV;
    float *q = floats(nk, -0.5, 0.5), *k = floats(nk, -0.5, 0.5), *v = floats(nv, -1, 1);
    float *g = floats(nk, -2.0, -0.01), *beta = floats((size_t)T * H, 0.05, 0.95), *s0 = floats(ns, -0.1, 0.1);
    float *a = floats(nk, -0.3, 0.3), *b = floats(nk, -0.3, 0.3), *d_o = floats(nv, -1, 1);
    float *dsf = floats(ns, -0.1, 0.1);
    uint16_t *qb = bf16_of(q, nk), *kb = bf16_of(k, nk), *vb = bf16_of(v, nv), *dob = bf16_of(d_o, nv);
    uint16_t *ab = bf16_of(a, nk), *bb = bf16_of(b, nk);
    const int32_t all[H] = {0, 1, 2}, sel[2] = {2, 0};

    for (int io = 0; io < 2; ++io) {
        const void *Q = io ? (const void *)qb : q, *K = io ? (const void *)kb : k, *V = io ? (const void *)vb : v;
        const void *DO = io ? (const void *)dob : d_o;
        const void *A = io ? (const void *)ab : a, *B = io ? (const void *)bb : b;
        for (int with_s0 = 0; with_s0 < 2; ++with_s0) {
            const float *S0 = with_s0 ? s0 : NULL;
            double *o_all = zeros((size_t)T * H * DV), *f_all = zeros(ns);
            EXPECT(kda_oracle_fwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, g, beta, S0, H, all, o_all, f_all,
                                  3) == 0);
            EXPECT(all_finite(o_all, (size_t)T * H * DV) && all_finite(f_all, ns));
            double *o_sel = zeros((size_t)T * 2 * DV), *f_sel = zeros((size_t)N * 2 * DK * DV);
            EXPECT(kda_oracle_fwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, g, beta, S0, 2, sel, o_sel, NULL,
                                  2) == 0);
            EXPECT(kda_oracle_fwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, g, beta, S0, 2, sel, o_sel, f_sel,
                                  5) == 0);
            int same = 1;
            for (int64_t t = 0; t < T; ++t)
                for (int s = 0; s < 2; ++s)
                    for (int j = 0; j < DV; ++j)
                        same &= o_sel[(t * 2 + s) * DV + j] == o_all[(t * H + sel[s]) * DV + j];
            for (int n = 0; n < N; ++n)
                for (int s = 0; s < 2; ++s)
                    for (int e = 0; e < DK * DV; ++e)
                        same &= f_sel[((size_t)n * 2 + s) * DK * DV + e] == f_all[((size_t)n * H + sel[s]) * DK * DV + e];
            EXPECT(same);
            /* the empty sequence passes its initial state through */
            int passthrough = 1;
            for (int h = 0; h < H; ++h)
                for (int e = 0; e < DK * DV; ++e)
                    passthrough &= f_all[((size_t)1 * H + h) * DK * DV + e] ==
                                   (S0 ? (double)S0[((size_t)1 * H + h) * DK * DV + e] : 0.0);
            EXPECT(passthrough);

            double *dq = zeros(nk), *dk = zeros(nk), *dv = zeros(nv), *dg = zeros(nk), *db = zeros((size_t)T * H);
            double *ds0 = zeros(ns);
            EXPECT(kda_oracle_bwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, g, beta, S0, DO, dsf, H, all, dq, dk,
                                  dv, dg, db, ds0, 3) == 0);
            EXPECT(all_finite(dq, nk) && all_finite(dk, nk) && all_finite(dv, nv) && all_finite(dg, nk) &&
                   all_finite(db, (size_t)T * H) && all_finite(ds0, ns));
            double *dq2 = zeros((size_t)T * 2 * DK), *dk2 = zeros((size_t)T * 2 * DK), *dv2 = zeros((size_t)T * 2 * DV);
            double *dg2 = zeros((size_t)T * 2 * DK), *db2 = zeros((size_t)T * 2);
            EXPECT(kda_oracle_bwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, g, beta, S0, DO, NULL, 2, sel, dq2,
                                  dk2, dv2, dg2, db2, NULL, 4) == 0);

            double *od = zeros((size_t)T * H * DV), *fd = zeros(ns);
            EXPECT(kda_oracle_dplr_fwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, A, B, g, S0, od, fd, 3) == 0);
            EXPECT(all_finite(od, (size_t)T * H * DV) && all_finite(fd, ns));
            EXPECT(kda_oracle_dplr_fwd(N, starts, lens, H, DK, DV, io, 0.7, Q, K, V, A, B, g, S0, od, NULL, 1) == 0);

            free(o_all), free(f_all), free(o_sel), free(f_sel), free(dq), free(dk), free(dv), free(dg), free(db);
            free(ds0), free(dq2), free(dk2), free(dv2), free(dg2), free(db2), free(od), free(fd);
        }
    }
    /* refused arguments */
    double *o = zeros((size_t)T * H * DV);
    EXPECT(kda_oracle_fwd(-1, starts, lens, H, DK, DV, 0, 1.0, q, k, v, g, beta, NULL, H, all, o, NULL, 1) == -1);
    EXPECT(kda_oracle_fwd(N, starts, lens, 0, DK, DV, 0, 1.0, q, k, v, g, beta, NULL, H, all, o, NULL, 1) == -1);
    EXPECT(kda_oracle_fwd(N, starts, lens, H, DK, DV, 0, 1.0, NULL, k, v, g, beta, NULL, H, all, o, NULL, 1) == -1);
    EXPECT(kda_oracle_fwd(N, starts, lens, H, DK, DV, 0, 1.0, q, k, v, g, beta, NULL, 0, all, o, NULL, 1) == -1);
    EXPECT(kda_oracle_fwd(0, starts, lens, H, DK, DV, 0, 1.0, NULL, NULL, NULL, NULL, NULL, NULL, H, all, o, NULL,
                          8) == 0);
    EXPECT(kda_oracle_dplr_fwd(N, starts, lens, H, DK, DV, 0, 1.0, q, k, v, NULL, b, g, NULL, o, NULL, 1) == -1);
    free(o);
    free(q), free(k), free(v), free(g), free(beta), free(s0), free(a), free(b), free(d_o), free(dsf);
    free(qb), free(kb), free(vb), free(dob), free(ab), free(bb);
    printf("%d checks, %d failed\n", checks, failures);
    return failures ? 1 : 0;
}
