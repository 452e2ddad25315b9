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
 *   with a causal depthwise convolution of width W (the prologue of the Mamba
 *   block: youngju.dev MambaBlock.forward, x_conv = silu(conv1d(x)) with
 *   left padding W-1 and the first L outputs kept), the scan input is
 *     u[b,t,d] = silu(cb[d] + sum_{k<W} cw[d,k] * x[b, t-(W-1)+k, d]),  x[t<0] = 0
 *   and the buffer passed as u holds x; otherwise u is used as given.
 *   for t = 0 .. L-1:
 *     delta = delta[b,t,d] (+ delta_bias[d]), through softplus when asked
 *     a[n]  = exp(delta * A[d,n])                          (discretised A)
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
 * The backward pass (oracle_selective_scan_bwd) returns the gradients of
 *   loss = sum_{b,t,d} dy[b,t,d] * y[b,t,d] + sum_{b,d,n} dh_last[b,d,n] * h_last[b,d,n]
 * with respect to every input, by the chain rule applied to the recurrence
 * above, walked in reverse time with the adjoint state lam[n] = dloss/dh_t[n]
 * (the backward of the selective scan that recomputes the states instead of
 * storing them: doyouknow.kr "Mamba와 상태 공간 모델(SSM)의 부상 완벽 가이드"
 * §3-3; here the oracle simply keeps every state of the channel in memory).
 * With g(z) = z*sigmoid(z) and s_t the readout before the gate:
 *   ds_t   = dy_t * g(z_t)                 dz_t = dy_t * s_t * g'(z_t)
 *   lam_t  = C_t * ds_t + a_{t+1} * lam_{t+1}   (lam_{L-1} gets dh_last added)
 *   dh_{t-1} path:  dA   += lam_t * h_{t-1} * a_t * delta_t
 *                   ddelta_t += lam_t * h_{t-1} * a_t * A
 *   input term:     simplified  bu = delta*B*u:   ddelta += lam*B*u, du += lam*delta*B, dB += lam*delta*u
 *                   hold        bu = f*B*u, f = expm1(delta*A)/A, df/ddelta = a,
 *                               df/dA = (delta*a - f)/A (A -> 0: delta^2/2):
 *                               ddelta += lam*a*B*u, du += lam*f*B, dB += lam*f*u, dA += lam*df/dA*B*u
 *   readout:        dC_t += ds_t * h_t,  dD += ds_t * u_t,  du_t += D * ds_t
 *   With the convolution prologue, du above is the gradient of u = silu(pre);
 *   dpre_t = du_t * silu'(pre_t) gives dx[t-(W-1)+k] += cw[k] dpre_t,
 *   dcw[k] += dpre_t x[t-(W-1)+k] and dcb += dpre_t, and the returned du is dx.
 *   dh0 = a_0 * lam_0; with a bias / softplus on delta, ddelta is taken with
 *   respect to the raw delta (times sigmoid of the softplus argument) and
 *   ddelta_bias[d] is its sum over batch and time.
 *
 * Everything is evaluated in double precision, inputs widened exactly, the sum
 * over n taken in ascending order, with libm exp / expm1 (no fast-math).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <stdlib.h>

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

/* The causal depthwise convolution (width W, weights cw (dim, W), bias cb)
 * and SiLU of x, for token t of channel (b, d); *pre receives the
 * convolution before the SiLU. Without a convolution (W == 0): x itself. */
static double scan_input(const void *x, int type, int64_t b, int64_t t, int64_t L, int64_t dim, int64_t d,
                         int W, const double *cw, const double *cb, double *pre)
{
    if (W == 0) {
        const double v = load(x, type, (b * L + t) * dim + d);
        if (pre)
            *pre = v;
        return v;
    }
    double acc = cb ? cb[d] : 0.0;
    for (int k = 0; k < W; ++k) {
        const int64_t s = t - (W - 1) + k;
        if (s >= 0)
            acc += cw[d * W + k] * load(x, type, (b * L + s) * dim + d);
    }
    if (pre)
        *pre = acc;
    return acc / (1.0 + exp(-acc));
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

/* softplus(x) = log(1 + exp(x)), written so that neither branch overflows. */
static double softplus(double x)
{
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/*
 * The step size used by the recurrence: delta as given, plus the channel's
 * bias when one is given, through softplus when asked (the projection output
 * becomes a positive step: youngju.dev SelectiveSSM.forward, dt = softplus(...)).
 * *dgrad receives d(step)/d(delta), the sigmoid of the softplus argument (1
 * without softplus).
 */
static double step_size(const void *delta, int type, int64_t i, int64_t d,
                        const double *bias, int sp, double *dgrad)
{
    double x = load(delta, type, i) + (bias ? bias[d] : 0.0);
    if (!sp) {
        if (dgrad)
            *dgrad = 1.0;
        return x;
    }
    if (dgrad)
        *dgrad = 1.0 / (1.0 + exp(-x));
    return softplus(x);
}

/*
 * Scan one channel (b, d) over L tokens.
 *   x_*  : the buffers of u, delta, z (batch, L, dim) and B, C (batch, L, N)
 *   y    : L outputs for this channel (contiguous), may be NULL
 *   hl   : N final states (contiguous), may be NULL
 */
static void scan_channel(int64_t b, int64_t d, int64_t L, int64_t dim, int64_t N,
                         int type, int disc, int W, const double *cw, const double *cb,
                         const void *u, const void *delta, const double *dbias, int sp,
                         const double *A, const void *B, const void *C,
                         const double *D, const void *z, const double *h0,
                         double *h, double *y, double *hl)
{
    for (int64_t n = 0; n < N; ++n)
        h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
    const double dskip = D ? D[d] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = b * L + t;        /* token index (b, t) */
        const double ut = scan_input(u, type, b, t, L, dim, d, W, cw, cb, NULL);
        const double dt = step_size(delta, type, row * dim + d, d, dbias, sp, NULL);
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
                          int type, int disc, int conv_width, const double *conv_weight,
                          const double *conv_bias,
                          const void *u, const void *delta, const double *delta_bias, int delta_softplus,
                          const double *A,
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
    if (conv_width < 0 || conv_width > 64 || (conv_width > 0 && !conv_weight))
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
            scan_channel(c / dim, c % dim, L, dim, N, type, disc, conv_width, conv_weight, conv_bias,
                         u, delta, delta_bias, delta_softplus, A, B, C,
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
                        const void *x, const void *delta, const double *delta_bias, int delta_softplus,
                        const double *A,
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
        const double dt = step_size(delta, type, c, d, delta_bias, delta_softplus, NULL);
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

/* d/dz of z*sigmoid(z) = sigmoid(z) * (1 + z*(1 - sigmoid(z))). */
static double silu_grad(double z)
{
    const double sg = 1.0 / (1.0 + exp(-z));
    return sg * (1.0 + z * (1.0 - sg));
}

/*
 * Backward of one channel (b, d). hs: (L+1)*N scratch for the states h_{-1..L-1};
 * ss: L scratch for the readouts before the gate. Per-channel results go to
 * du, dde, dz (L each, may be NULL), dA_c (N), dD_c (1), dh0_c (N, may be
 * NULL); dB and dC (batch, L, N) are accumulated into (may be NULL).
 */
static void bwd_channel(int64_t b, int64_t d, int64_t L, int64_t dim, int64_t N,
                        int type, int disc, int W, const double *cw, const double *cb,
                        const void *u, const void *delta, const double *dbias, int sp,
                        const double *A, const void *B, const void *C,
                        const double *D, const void *z, const double *h0,
                        const double *dy, const double *dh_last,
                        double *hs, double *ss, double *lam, double *gu, double *pre,
                        double *du, double *dde, double *dz, double *dA_c, double *dD_c,
                        double *dDb_c, double *dcw_c, double *dcb_c, double *dh0_c, double *dB, double *dC)
{
    const double dskip = D ? D[d] : 0.0;
    /* forward, keeping every state: hs[(t+1)*N + n] = h_t[n] */
    for (int64_t n = 0; n < N; ++n)
        hs[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = b * L + t;
        const double ut = scan_input(u, type, b, t, L, dim, d, W, cw, cb, &pre[t]);
        const double dt = step_size(delta, type, row * dim + d, d, dbias, sp, NULL);
        double st = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a_dn = A[d * N + n];
            const double hn = exp(dt * a_dn) * hs[t * N + n] +
                              input_term(disc, dt, a_dn, load(B, type, row * N + n), ut);
            hs[(t + 1) * N + n] = hn;
            st += load(C, type, row * N + n) * hn;
        }
        ss[t] = st + dskip * ut;
    }
    /* reverse */
    for (int64_t n = 0; n < N; ++n) {
        lam[n] = dh_last ? dh_last[(b * dim + d) * N + n] : 0.0;   /* a_{t+1} lam_{t+1} carried */
        dA_c[n] = 0.0;
    }
    double dDacc = 0.0, dDbacc = 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t row = b * L + t;
        const double ut = W ? pre[t] / (1.0 + exp(-pre[t])) : load(u, type, row * dim + d);
        double dstep;                                                 /* d(step)/d(delta) */
        const double dt = step_size(delta, type, row * dim + d, d, dbias, sp, &dstep);
        const double dyt = dy[row * dim + d];
        double ds = dyt;
        if (z) {
            const double zt = load(z, type, row * dim + d);
            ds = dyt * silu(zt);
            if (dz)
                dz[t] = dyt * ss[t] * silu_grad(zt);
        }
        dDacc += ds * ut;
        double dut = dskip * ds;
        double ddt = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a_dn = A[d * N + n];
            const double Bt = load(B, type, row * N + n);
            const double Ct = load(C, type, row * N + n);
            const double abar = exp(dt * a_dn);
            const double l = lam[n] + Ct * ds;                       /* lam_t */
            const double hprev = hs[t * N + n];                      /* h_{t-1} */
            const double da = l * hprev;                             /* dloss/dabar_t */
            ddt += da * abar * a_dn;
            dA_c[n] += da * abar * dt;
            if (disc == ORACLE_ZOH) {
                const double f = (a_dn != 0.0) ? expm1(dt * a_dn) / a_dn : dt;
                const double dfdA = (a_dn != 0.0) ? (dt * abar - f) / a_dn : 0.5 * dt * dt;
                ddt += l * abar * Bt * ut;
                dut += l * f * Bt;
                dA_c[n] += l * dfdA * Bt * ut;
                if (dB)
                    dB[row * N + n] += l * f * ut;
            } else {
                ddt += l * Bt * ut;
                dut += l * dt * Bt;
                if (dB)
                    dB[row * N + n] += l * dt * ut;
            }
            if (dC)
                dC[row * N + n] += ds * hs[(t + 1) * N + n];
            lam[n] = abar * l;                                       /* a_t lam_t for t-1 */
        }
        ddt *= dstep;                               /* through the bias and softplus */
        dDbacc += ddt;
        gu[t] = dut;
        if (dde)
            dde[t] = ddt;
    }
    *dD_c = dDacc;
    *dDb_c = dDbacc;
    if (W == 0) {
        if (du)
            for (int64_t t = 0; t < L; ++t)
                du[t] = gu[t];
    } else {
        /* through the SiLU and the convolution: du becomes the gradient of x */
        for (int k = 0; k < W; ++k)
            dcw_c[k] = 0.0;
        double dcb = 0.0;
        if (du)
            for (int64_t t = 0; t < L; ++t)
                du[t] = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double p = pre[t];
            const double sg = 1.0 / (1.0 + exp(-p));
            const double dp = gu[t] * sg * (1.0 + p * (1.0 - sg));
            dcb += dp;
            for (int k = 0; k < W; ++k) {
                const int64_t s = t - (W - 1) + k;
                if (s < 0)
                    continue;
                dcw_c[k] += dp * load(u, type, (b * L + s) * dim + d);
                if (du)
                    du[s] += cw[d * W + k] * dp;
            }
        }
        *dcb_c = dcb;
    }
    if (dh0_c)
        for (int64_t n = 0; n < N; ++n)
            dh0_c[n] = lam[n];
}

/*
 * Backward of the selective scan over a set of channels.
 *
 *   inputs as oracle_selective_scan; dy: (batch, L, dim) doubles;
 *   dh_last: (batch, dim, N) doubles or NULL (no gradient on the final state)
 *   nsel, sel        : channels, each c = b*dim + d (sel == NULL: all, in order)
 *   du, ddelta, dz   : (nsel, L) doubles, row k = channel sel[k]; each may be NULL
 *                      (dz is written only when z is given)
 *   dA_c             : (nsel, N) doubles, this channel's part of dA[d, :]
 *   dD_c             : (nsel) doubles, this channel's part of dD[d]
 *   dh0              : (nsel, N) doubles or NULL
 *   dB, dC           : (batch, L, N) doubles or NULL, set to the sum over the
 *                      selected channels (all channels give the full gradient)
 * Returns 0, or -1 for a bad argument or an allocation failure.
 */
int oracle_selective_scan_bwd(int64_t batch, int64_t L, int64_t dim, int64_t N,
                              int type, int disc, int conv_width, const double *conv_weight,
                              const double *conv_bias,
                              const void *u, const void *delta, const double *delta_bias,
                              int delta_softplus, const double *A,
                              const void *B, const void *C, const double *D,
                              const void *z, const double *h0,
                              const double *dy, const double *dh_last,
                              int64_t nsel, const int64_t *sel,
                              double *du, double *ddelta, double *dz,
                              double *dA_c, double *dD_c, double *dDb_c, double *dcw_c, double *dcb_c,
                              double *dh0, double *dB, double *dC, int nthreads)
{
    if (batch < 0 || L < 0 || dim < 0 || N < 1 || N > 4096)
        return -1;
    if (type != ORACLE_F64 && type != ORACLE_F32 && type != ORACLE_BF16)
        return -1;
    if (disc != ORACLE_EULER && disc != ORACLE_ZOH)
        return -1;
    if ((L > 0 && (!u || !delta || !B || !C || !dy)) || !A || !dA_c || !dD_c || !dDb_c)
        return -1;
    if (conv_width < 0 || conv_width > 64 || (conv_width > 0 && (!conv_weight || !dcw_c || !dcb_c)))
        return -1;
    if (!sel)
        nsel = batch * dim;
    const int64_t bln = batch * L * N;
    if (dB)
        for (int64_t i = 0; i < bln; ++i)
            dB[i] = 0.0;
    if (dC)
        for (int64_t i = 0; i < bln; ++i)
            dC[i] = 0.0;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    /* per-thread dB / dC sums, added in thread order afterwards */
    double *acc = NULL;
    if (dB || dC) {
        acc = (double *)calloc((size_t)nthreads * 2 * (size_t)(bln > 0 ? bln : 1), sizeof(double));
        if (!acc)
            return -1;
    }
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *lam = (double *)malloc(sizeof(double) * (size_t)N);
        double *gu = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *pre = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double *myB = acc && dB ? acc + (size_t)tid * 2 * bln : NULL;
        double *myC = acc && dC ? acc + (size_t)tid * 2 * bln + bln : NULL;
        if (!hs || !ss || !lam || !gu || !pre)
            bad = 1;
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t k = 0; k < nsel; ++k) {
            const int64_t c = sel ? sel[k] : k;
            if (bad || c < 0 || c >= batch * dim) {
                bad = 1;
                continue;
            }
            bwd_channel(c / dim, c % dim, L, dim, N, type, disc, conv_width, conv_weight, conv_bias,
                        u, delta, delta_bias, delta_softplus,
                        A, B, C, D, z, h0, dy, dh_last, hs, ss, lam, gu, pre,
                        du ? du + k * L : NULL, ddelta ? ddelta + k * L : NULL,
                        (dz && z) ? dz + k * L : NULL, dA_c + k * N, dD_c + k, dDb_c + k,
                        conv_width ? dcw_c + k * conv_width : NULL, conv_width ? dcb_c + k : NULL,
                        dh0 ? dh0 + k * N : NULL, myB, myC);
        }
        free(hs);
        free(ss);
        free(lam);
        free(gu);
        free(pre);
    }
    if (acc) {
        for (int th = 0; th < nthreads; ++th) {
            const double *tb = acc + (size_t)th * 2 * bln;
            for (int64_t i = 0; i < bln; ++i) {
                if (dB)
                    dB[i] += tb[i];
                if (dC)
                    dC[i] += tb[bln + i];
            }
        }
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Mamba-2 structured state-space duality (SSD) layer, sequential form.
 *
 * Restricting the state matrix of each head to a scalar times the identity
 * (itwiki "상태 공간 모델", section "Mamba-2와 상태 공간 쌍대성"; eommydocs
 * "State Space Models (SSM)", §2.4 "Mamba-2") gives, per batch row b and
 * head h with scalar a = A[h] and head dimension P:
 *
 *   H[p][n] = h0[b,h,p,n], or 0 when no initial state is given
 *   for t = 0 .. L-1:
 *     dt    = dt[b,t,h] (+ dt_bias[h]), through softplus when asked
 *     abar  = exp(dt * a)                              (one decay per head)
 *     wbar  = dt, or expm1(dt*a)/a (zero-order hold; dt when a == 0)
 *     H[p][n] = abar * H[p][n] + wbar * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * H[p][n] + D[h] * x[b,t,h,p]
 *     y *= silu(z[b,t,h,p])     when a gate is given
 *   h_last[b,h,:,:] = H
 * with g = h / (H_heads / G) the group whose B and C the head reads (B, C
 * shared by the heads of a group, as the key projection of youngju.dev
 * SSDBlock is shared by the head dimension of each head). Every channel p of
 * a head is the selective-scan recurrence above with A[d,n] = a for all n;
 * the chunked, attention-like evaluation of youngju.dev SSDBlock._chunk_scan
 * reaches the same y and is pinned against this form.
 *
 *   x, z : (batch, L, H, P);  dt: (batch, L, H);  B, C: (batch, L, G, N),
 *          row-major, element type `type`
 *   A    : (H) doubles; D: (H) doubles or NULL; dt_bias: (H) doubles or NULL
 *   h0   : (batch, H, P, N) doubles or NULL
 *   nsel, sel : heads to compute, each c = b*H + h (sel == NULL: all, in order)
 *   y    : (nsel, L, P) doubles or NULL;  h_last: (nsel, P, N) doubles or NULL
 * Returns 0, or -1 for a bad argument.
 */
static void ssd_head(int64_t b, int64_t hh, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                     int type, int disc, const void *x, const void *dt, const double *dt_bias, int sp,
                     const double *A, const void *B, const void *C, const double *D, const void *z,
                     const double *h0, double *st, double *y, double *hl)
{
    const int64_t g = hh / (H / G);
    const double a = A[hh];
    for (int64_t i = 0; i < P * N; ++i)
        st[i] = h0 ? h0[(b * H + hh) * P * N + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = b * L + t;
        const double step = step_size(dt, type, row * H + hh, hh, dt_bias, sp, NULL);
        const double abar = exp(step * a);
        const double wbar = (disc == ORACLE_ZOH && a != 0.0) ? expm1(step * a) / a : step;
        const int64_t bc = (row * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
            const double xv = load(x, type, (row * H + hh) * P + p);
            double yt = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double *s = &st[p * N + n];
                *s = abar * *s + wbar * xv * load(B, type, bc + n);
                yt += load(C, type, bc + n) * *s;
            }
            yt += (D ? D[hh] : 0.0) * xv;
            if (z)
                yt *= silu(load(z, type, (row * H + hh) * P + p));
            if (y)
                y[t * P + p] = yt;
        }
    }
    if (hl)
        for (int64_t i = 0; i < P * N; ++i)
            hl[i] = st[i];
}

int oracle_ssd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
               int type, int disc, const void *x, const void *dt, const double *dt_bias, int dt_softplus,
               const double *A, const void *B, const void *C, const double *D, const void *z,
               const double *h0, int64_t nsel, const int64_t *sel, double *y, double *h_last,
               int nthreads)
{
    if (batch < 0 || L < 0 || H < 1 || P < 1 || G < 1 || N < 1 || H % G != 0)
        return -1;
    if (type != ORACLE_F64 && type != ORACLE_F32 && type != ORACLE_BF16)
        return -1;
    if (disc != ORACLE_EULER && disc != ORACLE_ZOH)
        return -1;
    if ((L > 0 && (!x || !dt || !B || !C)) || !A)
        return -1;
    if (!sel)
        nsel = batch * H;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double *st = malloc(sizeof(double) * (size_t)(P * N));
        if (!st)
            bad = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t k = 0; k < nsel; ++k) {
            const int64_t c = sel ? sel[k] : k;
            if (!st || c < 0 || c >= batch * H) {
                bad = 1;
                continue;
            }
            ssd_head(c / H, c % H, L, H, P, G, N, type, disc, x, dt, dt_bias, dt_softplus, A, B, C, D, z,
                     h0, st, y ? y + k * L * P : NULL, h_last ? h_last + k * P * N : NULL);
        }
        free(st);
    }
    return bad ? -1 : 0;
}
