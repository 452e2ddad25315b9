/*
 * Plain fp64 CPU oracle for the Mamba selective scan (S6) and its one-token
 * decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library. The product path (the HIP library and
 * its Python binding) never links, loads or calls it, and the two share no
 * source: no header, helper, table or constant.
 *
 * What it computes, for every batch row b and channel d independently (each
 * channel is its own single-input single-output SSM: itwiki "상태 공간 모델",
 * section "제어 이론의 상태 공간 표현과의 관계"):
 *
 *   h[n]  = h0[b,d,n], or 0 when no initial state is given
 *           (eommydocs "State Space Models (SSM)", §3.2 pseudo-code and §5.1
 *            SelectiveSSM._selective_scan start from a zero state)
 *   for t = 0 .. L-1:
 *     a[n]  = exp(delta[b,t,d] * A[d,n])                  (discretised A)
 *     bu[n] = delta * B[b,t,n] * u[b,t,d]                  (simplified B, default)
 *           = (exp(delta*A)-1)/A * B[b,t,n] * u[b,t,d]     (zero-order hold)
 *     h[n]  = a[n]*h[n] + bu[n]                            (recurrence)
 *     y     = sum_n C[b,t,n]*h[n] + D[d]*u[b,t,d]          (readout + skip)
 *     y     = y * z/(1+exp(-z))     when a gate z is given (SiLU gate)
 *   h_last[b,d,:] = h
 *
 * Sources for each line: the discretisation exp(ΔA) and the simplified
 * B̄ = ΔB follow eommydocs §3.2 (deltaA / deltaB_u), youngju.dev
 * SelectiveSSM.selective_scan ("A 이산화", "B 이산화") and doyouknow.kr §3-1; the
 * zero-order-hold B̄ = (ΔA)^-1 (exp(ΔA) - I) ΔB is itwiki "동작 원리 › 이산화",
 * taken elementwise because A is diagonal; the recurrence and readout are the
 * same three sources' loop bodies; the skip D·u and the SiLU gate follow
 * youngju.dev MambaBlock.forward (y + D * x_conv, then y * silu(z)).
 * The decode step is the same body for a single token with the state carried
 * in and out (itwiki "순환 형태와 합성곱 형태"; ricepunchb "Mamba" §4.2).
 *
 * Everything is evaluated in double precision, inputs widened exactly, the sum
 * over n taken in ascending order, with libm exp / expm1 (no fast-math).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Element types the oracle reads. bf16 is passed as its raw 16-bit pattern. */
enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };
/* Discretisation of B. */
enum { ORACLE_EULER = 0, ORACLE_ZOH = 1 };

/* Read element i of a buffer of the given type, widened exactly to double. */
static double load(const void *p, int type, int64_t i)
{
    if (type == ORACLE_F64)
        return ((const double *)p)[i];
    if (type == ORACLE_F32)
        return (double)((const float *)p)[i];
    /* bf16: the pattern is the upper half of an IEEE binary32. */
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Input part of one state's update for one token: the B̄·u term. */
static double input_term(int disc, double delta, double a_dn, double b_tn, double u)
{
    if (disc == ORACLE_ZOH) {
        /* (ΔA)^-1 (exp(ΔA) - 1) ΔB = expm1(ΔA)/A · B; the A -> 0 limit is ΔB. */
        double coef = (a_dn != 0.0) ? expm1(delta * a_dn) / a_dn : delta;
        return coef * b_tn * u;
    }
    return delta * b_tn * u;
}

/* SiLU(z) = z * sigmoid(z). */
static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

/*
 * Scan one channel (b, d) over L tokens.
 *   x_*  : the buffers of u, delta, z (batch, L, dim) and B, C (batch, L, N)
 *   y    : L outputs for this channel (contiguous), may be NULL
 *   hl   : N final states (contiguous), may be NULL
 */
static void scan_channel(int64_t b, int64_t d, int64_t L, int64_t dim, int64_t N,
                         int type, int disc,
                         const void *u, const void *delta,
                         const double *A, const void *B, const void *C,
                         const double *D, const void *z, const double *h0,
                         double *h, double *y, double *hl)
{
    for (int64_t n = 0; n < N; ++n)
        h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
    const double dskip = D ? D[d] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = b * L + t;        /* token index (b, t) */
        const double ut = load(u, type, row * dim + d);
        const double dt = load(delta, type, row * dim + d);
        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a_dn = A[d * N + n];
            const double abar = exp(dt * a_dn);
            const double bu = input_term(disc, dt, a_dn, load(B, type, row * N + n), ut);
            h[n] = abar * h[n] + bu;
            yt += load(C, type, row * N + n) * h[n];
        }
        yt += dskip * ut;
        if (z)
            yt *= silu(load(z, type, row * dim + d));
        if (y)
            y[t] = yt;
    }
    if (hl)
        for (int64_t n = 0; n < N; ++n)
            hl[n] = h[n];
}

/*
 * Selective scan over a set of channels.
 *
 *   batch, L, dim, N : sizes; u, delta, z are (batch, L, dim), B and C are
 *                      (batch, L, N), all row-major, of element type `type`
 *   A                : (dim, N) doubles;  D: (dim) doubles or NULL (no skip)
 *   z                : gate or NULL;  h0: (batch, dim, N) doubles or NULL (zeros)
 *   nsel, sel        : channels to compute, each c = b*dim + d; sel == NULL
 *                      means all batch*dim channels in order c = 0, 1, ...
 *   y                : (nsel, L) doubles, row k = channel sel[k]; may be NULL
 *   h_last           : (nsel, N) doubles; may be NULL
 *   nthreads         : OpenMP threads (<= 0: the runtime's default)
 * Returns 0, or -1 for a bad argument.
 */
int oracle_selective_scan(int64_t batch, int64_t L, int64_t dim, int64_t N,
                          int type, int disc,
                          const void *u, const void *delta, const double *A,
                          const void *B, const void *C, const double *D,
                          const void *z, const double *h0,
                          int64_t nsel, const int64_t *sel,
                          double *y, double *h_last, int nthreads)
{
    if (batch < 0 || L < 0 || dim < 0 || N < 1 || N > 4096)
        return -1;
    if (type != ORACLE_F64 && type != ORACLE_F32 && type != ORACLE_BF16)
        return -1;
    if (disc != ORACLE_EULER && disc != ORACLE_ZOH)
        return -1;
    if ((L > 0 && (!u || !delta || !B || !C)) || !A)
        return -1;
    if (!sel)
        nsel = batch * dim;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double h[4096];
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t k = 0; k < nsel; ++k) {
            const int64_t c = sel ? sel[k] : k;
            if (c < 0 || c >= batch * dim) {
                bad = 1;
                continue;
            }
            scan_channel(c / dim, c % dim, L, dim, N, type, disc, u, delta, A, B, C,
                         D, z, h0, h, y ? y + k * L : NULL, h_last ? h_last + k * N : NULL);
        }
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/*
 * One decode step for every (b, d): the recurrence body for a single token,
 * with the state updated in place.
 *   x, delta, z : (batch, dim) of element type `type` (z may be NULL)
 *   A           : (dim, N) doubles;  B, C: (batch, N) of type `type`
 *   D           : (dim) doubles or NULL
 *   h           : (batch, dim, N) doubles, read and overwritten
 *   y           : (batch, dim) doubles
 */
int oracle_state_update(int64_t batch, int64_t dim, int64_t N, int type, int disc,
                        const void *x, const void *delta, const double *A,
                        const void *B, const void *C, const double *D,
                        const void *z, double *h, double *y, int nthreads)
{
    if (batch < 0 || dim < 0 || N < 1)
        return -1;
    if (type != ORACLE_F64 && type != ORACLE_F32 && type != ORACLE_BF16)
        return -1;
    if (disc != ORACLE_EULER && disc != ORACLE_ZOH)
        return -1;
    if (!x || !delta || !A || !B || !C || !h || !y)
        return -1;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t c = 0; c < batch * dim; ++c) {
        const int64_t b = c / dim, d = c % dim;
        const double xt = load(x, type, c);
        const double dt = load(delta, type, c);
        double *hc = h + c * N;
        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a_dn = A[d * N + n];
            hc[n] = exp(dt * a_dn) * hc[n] + input_term(disc, dt, a_dn, load(B, type, b * N + n), xt);
            yt += load(C, type, b * N + n) * hc[n];
        }
        yt += (D ? D[d] : 0.0) * xt;
        if (z)
            yt *= silu(load(z, type, c));
        y[c] = yt;
    }
    (void)nthreads;
    return 0;
}
