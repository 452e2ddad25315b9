/*
 * Drives every entry point of the fp64 oracle (oracle/ssm_oracle.c) over small
 * inputs in each element type, both discretisations and every option, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure: tests/test_sanitize_cpu.py compiles and runs it). Any
 * out-of-bounds access, use of freed memory, leak or undefined operation
 * aborts the run; the driver itself checks that the valid calls succeed with
 * finite outputs and that bad arguments are refused with -1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's entry points (declared here: the driver shares no header with it). */
int oracle_selective_scan(int64_t batch, int64_t L, int64_t dim, int64_t N, int type, int disc, int conv_width,
                          const double *conv_weight, const double *conv_bias, const void *u, const void *delta,
                          const double *delta_bias, int delta_softplus, const double *A, const void *B,
                          const void *C, const double *D, const void *z, const double *h0, int64_t nsel,
                          const int64_t *sel, double *y, double *h_last, int nthreads);
int oracle_state_update(int64_t batch, int64_t dim, int64_t N, int type, int disc, const void *x,
                        const void *delta, const double *delta_bias, int delta_softplus, const double *A,
                        const void *B, const void *C, const double *D, const void *z, double *h, double *y,
                        int nthreads);
int oracle_selective_scan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N, int type, int disc, int conv_width,
                              const double *conv_weight, const double *conv_bias, const void *u, const void *delta,
                              const double *delta_bias, int delta_softplus, const double *A, const void *B,
                              const void *C, const double *D, const void *z, const double *h0, const double *dy,
                              const double *dh_last, int64_t nsel, const int64_t *sel, double *du, double *ddelta,
                              double *dz, double *dA_c, double *dD_c, double *dDb_c, double *dcw_c, double *dcb_c,
                              double *dh0, double *dB, double *dC, int nthreads);
int oracle_ssd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int type, int disc,
               const void *x, const void *dt, const double *dt_bias, int dt_softplus, const double *A, const void *B,
               const void *C, const double *D, const void *z, const double *h0, int64_t nsel, const int64_t *sel,
               double *y, double *h_last, int nthreads);

enum { F64 = 0, F32 = 1, BF16 = 2 };
static const int elem_bytes[3] = {8, 4, 2};

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) /* in [-1, 1) */
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static int failures = 0;
#define CHECK(cond, what)                                           \
    do {                                                            \
        if (!(cond)) {                                              \
            fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
            ++failures;                                             \
        }                                                           \
    } while (0)

/* n elements of the given type, values lo + (hi - lo) * U[0, 1) (bf16: truncated bit pattern). */
static void *tensor(int type, int64_t n, double lo, double hi)
{
    void *p = malloc((size_t)(n > 0 ? n : 1) * (size_t)elem_bytes[type]);
    for (int64_t i = 0; i < n; ++i) {
        const double v = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
        if (type == F64) {
            ((double *)p)[i] = v;
        } else {
            const float f = (float)v;
            if (type == F32) {
                ((float *)p)[i] = f;
            } else {
                uint32_t bits;
                memcpy(&bits, &f, 4);
                ((uint16_t *)p)[i] = (uint16_t)(bits >> 16);
            }
        }
    }
    return p;
}

static double *dtensor(int64_t n, double lo, double hi) { return (double *)tensor(F64, n, lo, hi); }

static int finite_all(const double *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i]))
            return 0;
    return 1;
}

static void scan_cases(void)
{
    const int64_t dims[][4] = {{2, 37, 5, 16}, {1, 1, 3, 1}, {3, 0, 4, 5}, {1, 19, 2, 64}};
    for (size_t s = 0; s < sizeof dims / sizeof dims[0]; ++s)
        for (int type = 0; type < 3; ++type)
            for (int disc = 0; disc < 2; ++disc)
                for (int opt = 0; opt < 4; ++opt) {
                    const int64_t b = dims[s][0], L = dims[s][1], d = dims[s][2], N = dims[s][3];
                    const int conv = (opt & 1) ? 4 : 0, sp = (opt & 2) != 0;
                    void *u = tensor(type, b * L * d, -1, 1), *dt = tensor(type, b * L * d, 0.01, 0.5);
                    void *B = tensor(type, b * L * N, -1, 1), *C = tensor(type, b * L * N, -1, 1);
                    void *z = tensor(type, b * L * d, -2, 2);
                    double *A = dtensor(d * N, -3, -0.1), *D = dtensor(d, 0.5, 1.5), *h0 = dtensor(b * d * N, -1, 1);
                    double *bias = dtensor(d, -2, 0), *cw = dtensor(d * 4, -0.5, 0.5), *cb = dtensor(d, -0.1, 0.1);
                    double *y = malloc(sizeof(double) * (size_t)(b * d * L + 1));
                    double *hl = malloc(sizeof(double) * (size_t)(b * d * N));
                    int rc = oracle_selective_scan(b, L, d, N, type, disc, conv, cw, cb, u, dt, sp ? bias : NULL, sp,
                                                   A, B, C, opt & 1 ? D : NULL, opt & 2 ? z : NULL,
                                                   opt & 1 ? h0 : NULL, 0, NULL, y, hl, 1);
                    CHECK(rc == 0, "selective_scan");
                    CHECK(finite_all(y, b * d * L) && finite_all(hl, b * d * N), "selective_scan finite");
                    /* a subset of channels, in another order, without y */
                    const int64_t sel[2] = {b * d - 1, 0};
                    rc = oracle_selective_scan(b, L, d, N, type, disc, conv, cw, cb, u, dt, bias, sp, A, B, C, D, z,
                                               h0, 2, sel, NULL, hl, 1);
                    CHECK(rc == 0, "selective_scan subset");
                    /* its backward, every gradient */
                    double *dy = dtensor(b * L * d, -1, 1), *dhl = dtensor(b * d * N, -1, 1);
                    const int64_t nc = b * d;
                    double *du = malloc(sizeof(double) * (size_t)(b * L * d + 1));
                    double *ddt = malloc(sizeof(double) * (size_t)(b * L * d + 1));
                    double *dz = malloc(sizeof(double) * (size_t)(b * L * d + 1));
                    double *dA = malloc(sizeof(double) * (size_t)(nc * N)), *dD = malloc(sizeof(double) * (size_t)nc);
                    double *ddb = malloc(sizeof(double) * (size_t)nc), *dcw = malloc(sizeof(double) * (size_t)(nc * 4));
                    double *dcb = malloc(sizeof(double) * (size_t)nc), *dh0 = malloc(sizeof(double) * (size_t)(nc * N));
                    double *dB = malloc(sizeof(double) * (size_t)(b * L * N + 1));
                    double *dC = malloc(sizeof(double) * (size_t)(b * L * N + 1));
                    rc = oracle_selective_scan_bwd(b, L, d, N, type, disc, conv, cw, cb, u, dt, sp ? bias : NULL, sp,
                                                   A, B, C, D, opt & 2 ? z : NULL, h0, dy, dhl, 0, NULL, du, ddt, dz,
                                                   dA, dD, ddb, dcw, dcb, dh0, dB, dC, 1);
                    CHECK(rc == 0, "selective_scan_bwd");
                    CHECK(finite_all(du, b * L * d) && finite_all(ddt, b * L * d) && finite_all(dA, nc * N) &&
                              finite_all(dB, b * L * N) && finite_all(dC, b * L * N) && finite_all(dh0, nc * N),
                          "selective_scan_bwd finite");
                    free(dy); free(dhl); free(du); free(ddt); free(dz); free(dA); free(dD); free(ddb); free(dcw);
                    free(dcb); free(dh0); free(dB); free(dC);
                    free(u); free(dt); free(B); free(C); free(z); free(A); free(D); free(h0); free(bias); free(cw);
                    free(cb); free(y); free(hl);
                }
}

static void decode_cases(void)
{
    for (int type = 0; type < 3; ++type)
        for (int disc = 0; disc < 2; ++disc) {
            const int64_t b = 3, d = 7, N = 16;
            void *x = tensor(type, b * d, -1, 1), *dt = tensor(type, b * d, 0.01, 0.5), *z = tensor(type, b * d, -2, 2);
            void *B = tensor(type, b * N, -1, 1), *C = tensor(type, b * N, -1, 1);
            double *A = dtensor(d * N, -3, -0.1), *D = dtensor(d, 0.5, 1.5), *h = dtensor(b * d * N, -1, 1);
            double *bias = dtensor(d, -2, 0), *y = malloc(sizeof(double) * (size_t)(b * d));
            for (int step = 0; step < 3; ++step) {
                const int rc = oracle_state_update(b, d, N, type, disc, x, dt, step ? bias : NULL, step == 2, A, B,
                                                   C, step ? D : NULL, step ? z : NULL, h, y, 1);
                CHECK(rc == 0 && finite_all(y, b * d) && finite_all(h, b * d * N), "state_update");
            }
            free(x); free(dt); free(z); free(B); free(C); free(A); free(D); free(h); free(bias); free(y);
        }
}

static void ssd_cases(void)
{
    const int64_t shapes[][6] = {{2, 70, 4, 8, 2, 16}, {1, 1, 2, 4, 1, 8}, {1, 0, 2, 4, 1, 8}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int type = 0; type < 3; ++type)
            for (int disc = 0; disc < 2; ++disc) {
                const int64_t b = shapes[s][0], L = shapes[s][1], H = shapes[s][2], P = shapes[s][3];
                const int64_t G = shapes[s][4], N = shapes[s][5];
                void *x = tensor(type, b * L * H * P, -1, 1), *dt = tensor(type, b * L * H, 0.01, 0.5);
                void *B = tensor(type, b * L * G * N, -1, 1), *C = tensor(type, b * L * G * N, -1, 1);
                void *z = tensor(type, b * L * H * P, -2, 2);
                double *A = dtensor(H, -4, -0.5), *D = dtensor(H, 0.5, 1.5), *bias = dtensor(H, -2, 0);
                double *h0 = dtensor(b * H * P * N, -1, 1);
                double *y = malloc(sizeof(double) * (size_t)(b * H * L * P + 1));
                double *hl = malloc(sizeof(double) * (size_t)(b * H * P * N));
                int rc = oracle_ssd(b, L, H, P, G, N, type, disc, x, dt, bias, 1, A, B, C, D, z, h0, 0, NULL, y, hl, 1);
                CHECK(rc == 0 && finite_all(y, b * H * L * P) && finite_all(hl, b * H * P * N), "ssd");
                const int64_t sel[1] = {b * H - 1};
                rc = oracle_ssd(b, L, H, P, G, N, type, disc, x, dt, NULL, 0, A, B, C, NULL, NULL, NULL, 1, sel, y,
                                NULL, 1);
                CHECK(rc == 0, "ssd subset");
                free(x); free(dt); free(B); free(C); free(z); free(A); free(D); free(bias); free(h0); free(y);
                free(hl);
            }
}

static void refusals(void)
{
    double A[4] = {-1, -1, -1, -1}, y[4], hl[4];
    float u[4] = {0};
    CHECK(oracle_selective_scan(-1, 2, 1, 1, F32, 0, 0, NULL, NULL, u, u, NULL, 0, A, u, u, NULL, NULL, NULL, 0,
                                NULL, y, hl, 1) == -1, "negative batch refused");
    CHECK(oracle_selective_scan(1, 2, 1, 1, 7, 0, 0, NULL, NULL, u, u, NULL, 0, A, u, u, NULL, NULL, NULL, 0, NULL, y,
                                hl, 1) == -1, "bad type refused");
    CHECK(oracle_selective_scan(1, 2, 1, 1, F32, 5, 0, NULL, NULL, u, u, NULL, 0, A, u, u, NULL, NULL, NULL, 0, NULL,
                                y, hl, 1) == -1, "bad discretisation refused");
    const int64_t bad_sel[1] = {5};
    CHECK(oracle_selective_scan(1, 2, 1, 1, F32, 0, 0, NULL, NULL, u, u, NULL, 0, A, u, u, NULL, NULL, NULL, 1,
                                bad_sel, y, hl, 1) == -1, "channel out of range refused");
    CHECK(oracle_state_update(1, 1, 1, F32, 0, NULL, u, NULL, 0, A, u, u, NULL, NULL, hl, y, 1) == -1,
          "decode without x refused");
    CHECK(oracle_ssd(1, 2, 3, 1, 2, 1, F32, 0, u, u, NULL, 0, A, u, u, NULL, NULL, NULL, 0, NULL, y, hl, 1) == -1,
          "heads not divisible by groups refused");
}

int main(void)
{
    scan_cases();
    decode_cases();
    ssd_cases();
    refusals();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all calls clean\n");
    return 0;
}
