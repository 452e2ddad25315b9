// Selective scan (S6) and decode step for MI355X (gfx950, CDNA4).
//
// What is computed is stated in include/ssm_scan.h. This file holds the C ABI
// (argument validation, launch planning, dispatch) and the decode kernel; the
// scan kernels live in scan_kernels.hpp.
//
// Decode: one thread per (channel, 4 states); h moves as 16-byte vectors, the
// readout is reduced across the lanes of a channel with cross-lane shuffles.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssm_scan.h"
#include "scan_kernels.hpp"

namespace {

using namespace ssm_detail;

// ---------------------------------------------------------------------------
// seqlen == 0: h_last = h0 (or zeros)

__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *h_last, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) h_last[i] = h0 != nullptr ? h0[i] : 0.0f;
}

// ---------------------------------------------------------------------------
// Decode step

struct DecodeParams {
    const void *x, *delta, *z, *B, *C;
    const float *A, *D;
    float *h;
    void *y;
    int64_t channels;     // batch * dim
    int dim, N, lpc_log2; // lanes per channel = 1 << lpc_log2, 4 states per lane
    int vec4;             // N % 4 == 0 and h, A 16-byte aligned
    int bc4;              // N % 4 == 0 and B, C aligned to 4 elements
};

template <typename T, bool ZOH>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lpc = 1 << p.lpc_log2;
    const int64_t c = gid >> p.lpc_log2;      // channel = b * dim + d
    const int q = (int)(gid & (lpc - 1));
    const bool cval = c < p.channels;
    const int64_t cc = cval ? c : p.channels - 1;
    const int64_t b = cc / p.dim;
    const int d = (int)(cc % p.dim);
    const T *x = static_cast<const T *>(p.x);
    const T *dt = static_cast<const T *>(p.delta);
    const T *Bp = static_cast<const T *>(p.B);
    const T *Cp = static_cast<const T *>(p.C);
    const float xv = Elem<T>::widen(x[cc]);
    const float dv = Elem<T>::widen(dt[cc]);
    const int n0 = q * 4;

    float hv[4], av[4];
    float *hp = p.h + cc * p.N + n0;
    const float *ap = p.A + (int64_t)d * p.N + n0;
    // with N % 4 == 0 a lane's four states are either all inside the channel
    // (n0 < N) or all past it (lanes added to round lanes-per-channel up to a
    // power of two); those lanes must not touch memory
    const bool qv = n0 < p.N;
    if (p.vec4) {
        float4 h4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), a4 = h4;
        if (qv) {
            h4 = *reinterpret_cast<const float4 *>(hp);
            a4 = *reinterpret_cast<const float4 *>(ap);
        }
        hv[0] = h4.x; hv[1] = h4.y; hv[2] = h4.z; hv[3] = h4.w;
        av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool ok = n0 + k < p.N;
            hv[k] = ok ? hp[k] : 0.0f;
            av[k] = ok ? ap[k] : 0.0f;
        }
    }
    // this lane's four B and C values: one 8- or 16-byte load each when aligned
    float bv[4], cv[4];
    if (p.bc4) {
        if (qv) {
            if constexpr (sizeof(T) == 2) {
                const uint2 rb = *reinterpret_cast<const uint2 *>(Bp + b * p.N + n0);
                const uint2 rc = *reinterpret_cast<const uint2 *>(Cp + b * p.N + n0);
                bv[0] = __uint_as_float(rb.x << 16); bv[1] = __uint_as_float(rb.x & 0xffff0000u);
                bv[2] = __uint_as_float(rb.y << 16); bv[3] = __uint_as_float(rb.y & 0xffff0000u);
                cv[0] = __uint_as_float(rc.x << 16); cv[1] = __uint_as_float(rc.x & 0xffff0000u);
                cv[2] = __uint_as_float(rc.y << 16); cv[3] = __uint_as_float(rc.y & 0xffff0000u);
            } else {
                const float4 fb = *reinterpret_cast<const float4 *>(Bp + b * p.N + n0);
                const float4 fc = *reinterpret_cast<const float4 *>(Cp + b * p.N + n0);
                bv[0] = fb.x; bv[1] = fb.y; bv[2] = fb.z; bv[3] = fb.w;
                cv[0] = fc.x; cv[1] = fc.y; cv[2] = fc.z; cv[3] = fc.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) bv[k] = cv[k] = 0.0f;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool ok = n0 + k < p.N;
            bv[k] = ok ? Elem<T>::widen(Bp[b * p.N + n0 + k]) : 0.0f;
            cv[k] = ok ? Elem<T>::widen(Cp[b * p.N + n0 + k]) : 0.0f;
        }
    }
    const float du = dv * xv;
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float bk = bv[k], ck = cv[k];
        if constexpr (ZOH) {
            const float em1 = expm1f(dv * av[k]);
            const float coef = (av[k] != 0.0f) ? em1 / av[k] : dv;
            hv[k] = fmaf(1.0f + em1, hv[k], coef * bk * xv);
        } else {
            hv[k] = fmaf(__builtin_amdgcn_exp2f(dv * av[k] * kLog2e), hv[k], du * bk);
        }
        part = fmaf(ck, hv[k], part);
    }
    // sum the partial readouts of the lpc lanes of this channel (in state order)
    for (int m = lpc >> 1; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
    if (!cval) return;
    if (p.vec4) {
        if (qv) *reinterpret_cast<float4 *>(hp) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (n0 + k < p.N) hp[k] = hv[k];
    }
    if (q == 0) {
        float yv = part + (p.D != nullptr ? p.D[d] : 0.0f) * xv;
        if (p.z != nullptr) yv *= silu(Elem<T>::widen(static_cast<const T *>(p.z)[cc]));
        if constexpr (sizeof(T) == 2)
            static_cast<uint16_t *>(p.y)[cc] = Elem<uint16_t>::to_bits(yv);
        else
            static_cast<float *>(p.y)[cc] = yv;
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, dispatch

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void *p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + (uintptr_t)bytes};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a * b without overflow, both >= 0
bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a == 0 || b == 0) { *out = 0; return true; }
    if (a > INT64_MAX / b) return false;
    *out = a * b;
    return true;
}

int padded_states(int64_t N) {
    if (N <= 4) return 4;
    if (N <= 8) return 8;
    if (N <= 16) return 16;
    if (N <= 32) return 32;
    return 64;
}

// Launch shape: enough waves to keep every SIMD of the 256 CUs busy, preferring
// to split states over waves (cheap) before splitting time (a second pass).
Plan make_plan(const ssm_scan_desc &d, const ssm_scan_tuning *t) {
    Plan pl{};
    pl.npad = padded_states(d.dstate);
    const int64_t tiles = d.batch * ((d.dim + kTile - 1) / kTile);
    // waves wanted in flight: 4 per SIMD of 256 CUs (measured: the 1.4B-shaped
    // layer runs fastest with 8 waves per tile, 4096 waves)
    const int64_t want_waves = 4096;
    int G = (t && t->state_groups > 0) ? t->state_groups : 0;
    if (G == 0) {
        G = pl.npad > 16 ? pl.npad / 16 : 1;     // at most 16 states per wave
        while (G < 8 && G < pl.npad && tiles * G < want_waves) G *= 2;
    }
    pl.G = G;
    pl.npw = pl.npad / G;
    int S = (t && t->segments > 0) ? t->segments : 0;
    if (S == 0) {
        S = 1;
        // segments cost a second (aggregate) pass over their tokens: add them
        // only while the waves are too few, and keep them >= 256 tokens
        // (measured: 16 segments for L 131072 x 5120 channels, 8 for
        // L 2048 x 6144 channels)
        if (tiles * G < want_waves)
            while (S < kMaxSegments && tiles * G * S < 2 * want_waves && d.seqlen / (2 * S) >= 256) S *= 2;
    }
    if (d.seqlen > 0 && S > d.seqlen) S = (int)d.seqlen;
    if (S < 1) S = 1;
    pl.S = S;
    // segments start on 16-token boundaries (whole chunks, aligned runs of B and C)
    const int64_t seg_len = d.seqlen > 0 ? ((d.seqlen + S - 1) / S + 15) / 16 * 16 : 0;
    pl.seg_len = seg_len > INT32_MAX ? 0 : (int)seg_len;
    if (d.seqlen > 0) pl.S = (int)((d.seqlen + pl.seg_len - 1) / pl.seg_len);   // drop empty segments
    return pl;
}

bool plan_supported(const Plan &pl) {
    if (pl.G < 1 || pl.G > 16 || (pl.G & (pl.G - 1)) != 0) return false;
    if (pl.npad % pl.G != 0) return false;
    if (pl.npw < 1 || pl.npw > 16) return false;
    if (pl.S < 1 || pl.S > kMaxSegments) return false;
    return pl.seg_len > 0 || pl.S == 1;
}

size_t workspace_bytes_for(const ssm_scan_desc &d, const Plan &pl) {
    if (d.batch == 0 || d.dim == 0 || d.seqlen == 0) return 0;
    return workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, pl).total;
}

bool shape_compiled(const Plan &pl) {
    static const int table[][2] = {{4, 1}, {4, 2}, {4, 4}, {8, 1}, {8, 2}, {8, 4}, {8, 8},
                                   {16, 1}, {16, 2}, {16, 4}, {16, 8}, {16, 16},
                                   {32, 2}, {32, 4}, {32, 8}, {32, 16},
                                   {64, 4}, {64, 8}, {64, 16}};
    for (const auto &e : table)
        if (e[0] == pl.npad && e[1] == pl.G) return true;
    return false;
}

int validate_desc(const ssm_scan_desc *d) {
    if (d == nullptr) return SSM_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->dim < 0) return SSM_ERR_SHAPE;
    if (d->dtype != SSM_F32 && d->dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d->disc != SSM_DISC_EULER && d->disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d->dstate < 1 || d->dstate > 64) return SSM_ERR_UNSUPPORTED;
    // byte counts of the largest tensors must fit; kernel indices are 32-bit
    // for batch, dim and segment lengths
    int64_t bl, bld, bytes;
    if (!mul_ok(d->batch, d->seqlen, &bl) || !mul_ok(bl, d->dim, &bld) || !mul_ok(bld, 4, &bytes))
        return SSM_ERR_SHAPE;
    int64_t bdn;
    if (!mul_ok(d->batch, d->dim, &bdn) || !mul_ok(bdn, d->dstate * 4 * kMaxSegments * 3, &bytes))
        return SSM_ERR_SHAPE;
    if (d->batch > INT32_MAX || d->dim > INT32_MAX) return SSM_ERR_SHAPE;
    return SSM_OK;
}

int scan_impl(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
              const void *B, const void *C, const float *D, const void *z, const float *h0,
              void *y, float *h_last, void *workspace, size_t workspace_bytes,
              const ssm_scan_tuning *tuning, hipStream_t stream) {
    if (int rc = validate_desc(desc); rc != SSM_OK) return rc;
    const ssm_scan_desc d = *desc;
    if (d.batch == 0 || d.dim == 0) return SSM_OK;
    if (tuning && (tuning->state_groups < 0 || tuning->state_groups > 16 || tuning->segments < 0 ||
                   tuning->segments > kMaxSegments))
        return SSM_ERR_UNSUPPORTED;
    const Plan pl = make_plan(d, tuning);
    if (!plan_supported(pl) || !shape_compiled(pl)) return SSM_ERR_UNSUPPORTED;

    const int es = d.dtype == SSM_BF16 ? 2 : 4;
    const int64_t tok = d.batch * d.seqlen * d.dim;
    const int64_t bn = d.batch * d.seqlen * d.dstate;
    const int64_t state = d.batch * d.dim * d.dstate;
    if (A == nullptr) return SSM_ERR_NULL;
    if (d.seqlen > 0 && (u == nullptr || delta == nullptr || B == nullptr || C == nullptr || y == nullptr))
        return SSM_ERR_NULL;
    const void *in_ptrs[] = {u, delta, B, C, z};
    for (const void *q : in_ptrs)
        if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
    if ((y && !aligned(y, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) || (h0 && !aligned(h0, 4)) ||
        (h_last && !aligned(h_last, 4)) || (workspace && !aligned(workspace, 256)))
        return SSM_ERR_ALIGN;

    const size_t need = workspace_bytes_for(d, pl);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SSM_ERR_WORKSPACE;

    const Range r_y = range_of(y, d.seqlen > 0 ? tok * es : 0);
    const Range r_hl = range_of(h_last, state * 4);
    const Range r_ws = range_of(workspace, (int64_t)need);
    const Range inputs[] = {range_of(u, tok * es), range_of(delta, tok * es), range_of(z, z ? tok * es : 0),
                            range_of(B, bn * es), range_of(C, bn * es), range_of(A, d.dim * d.dstate * 4),
                            range_of(D, D ? d.dim * 4 : 0), range_of(h0, h0 ? state * 4 : 0)};
    for (const Range &r : inputs) {
        if (overlaps(r_y, r) || overlaps(r_ws, r)) return SSM_ERR_ALIAS;
        // h_last may be exactly h0 (in-place resume), nothing else
        if (overlaps(r_hl, r) && !(r.lo == r_hl.lo && r.hi == r_hl.hi && h0 == h_last)) return SSM_ERR_ALIAS;
    }
    if (overlaps(r_y, r_hl) || overlaps(r_y, r_ws) || overlaps(r_hl, r_ws)) return SSM_ERR_ALIAS;

    if (d.seqlen == 0) {
        if (h_last == nullptr) return SSM_OK;
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((state + 255) / 256)), dim3(256), 0, stream,
                           h0, h_last, state);
        return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }

    ScanParams p{};
    p.u = u; p.delta = delta; p.z = z; p.B = B; p.C = C;
    p.A = A; p.D = D; p.h0 = h0;
    p.y = y; p.h_last = h_last;
    p.L = d.seqlen;
    p.batch = (int)d.batch;
    p.dim = (int)d.dim;
    p.N = (int)d.dstate;
    p.seg_len = pl.seg_len;
    p.nseg = pl.S;
    p.ntiles = (int)((d.dim + kTile - 1) / kTile);
    // 4-channel pieces move as single 8-byte (bf16) or 16-byte (fp32) accesses
    p.vec = (d.dim % 4 == 0) && aligned(u, 4 * es) && aligned(delta, 4 * es) && (!z || aligned(z, 4 * es)) &&
            aligned(y, 4 * es);
    {
        const WorkspaceLayout wl = workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, pl);
        char *ws = static_cast<char *>(workspace);
        p.Bf = reinterpret_cast<float *>(ws + wl.bf);
        p.Cf = reinterpret_cast<float *>(ws + wl.cf);
        if (pl.S > 1) {
            p.agg_P = reinterpret_cast<float *>(ws + wl.agg_p);
            p.agg_H = reinterpret_cast<float *>(ws + wl.agg_h);
            p.seg_h = reinterpret_cast<float *>(ws + wl.seg_h);
        }
    }
    const int64_t blocks_per_seg = (int64_t)p.ntiles * d.batch;
    const int64_t nm = blocks_per_seg * pl.S;
    const int64_t na = pl.S > 1 ? blocks_per_seg * (pl.S - 1) : 0;
    if (nm > INT32_MAX) return SSM_ERR_SHAPE;

    hipError_t e;
    const bool zoh = d.disc == SSM_DISC_ZOH;
    if (d.dtype == SSM_BF16)
        e = zoh ? launch_scan_bf16_zoh(pl, p, (int)nm, (int)na, stream)
                : launch_scan_bf16_euler(pl, p, (int)nm, (int)na, stream);
    else
        e = zoh ? launch_scan_f32_zoh(pl, p, (int)nm, (int)na, stream)
                : launch_scan_f32_euler(pl, p, (int)nm, (int)na, stream);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" size_t ssm_scan_workspace_size_tuned(const ssm_scan_desc *desc, const ssm_scan_tuning *tuning) {
    if (validate_desc(desc) != SSM_OK) return 0;
    if (desc->batch == 0 || desc->dim == 0 || desc->seqlen == 0) return 0;
    return workspace_bytes_for(*desc, make_plan(*desc, tuning));
}

extern "C" size_t ssm_scan_workspace_size(const ssm_scan_desc *desc) {
    return ssm_scan_workspace_size_tuned(desc, nullptr);
}

extern "C" int ssm_scan_plan(const ssm_scan_desc *desc, ssm_scan_tuning *out) {
    if (int rc = validate_desc(desc); rc != SSM_OK) return rc;
    if (out == nullptr) return SSM_ERR_NULL;
    const Plan pl = make_plan(*desc, nullptr);
    out->state_groups = pl.G;
    out->segments = pl.S;
    return SSM_OK;
}

extern "C" int ssm_scan_fwd_tuned(const ssm_scan_desc *desc, const void *u, const void *delta,
                                  const float *A, const void *B, const void *C, const float *D,
                                  const void *z, const float *h0, void *y, float *h_last,
                                  void *workspace, size_t workspace_bytes,
                                  const ssm_scan_tuning *tuning, hipStream_t stream) {
    return scan_impl(desc, u, delta, A, B, C, D, z, h0, y, h_last, workspace, workspace_bytes, tuning, stream);
}

extern "C" int ssm_scan_fwd(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
                            const void *B, const void *C, const float *D, const void *z, const float *h0,
                            void *y, float *h_last, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    return scan_impl(desc, u, delta, A, B, C, D, z, h0, y, h_last, workspace, workspace_bytes, nullptr, stream);
}

extern "C" int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int32_t dtype, int32_t disc,
                                const void *x, const void *delta, const float *A, const void *B,
                                const void *C, const float *D, const void *z, float *h, void *y,
                                hipStream_t stream) {
    if (batch < 0 || dim < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (disc != SSM_DISC_EULER && disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (dstate < 1 || dstate > 64) return SSM_ERR_UNSUPPORTED;
    if (batch > INT32_MAX || dim > INT32_MAX) return SSM_ERR_SHAPE;
    int64_t ch, st, bytes;
    if (!mul_ok(batch, dim, &ch) || !mul_ok(ch, dstate * 4 * 16, &bytes)) return SSM_ERR_SHAPE;
    st = ch * dstate;
    if (ch == 0) return SSM_OK;
    if (x == nullptr || delta == nullptr || A == nullptr || B == nullptr || C == nullptr || h == nullptr ||
        y == nullptr)
        return SSM_ERR_NULL;
    const int es = dtype == SSM_BF16 ? 2 : 4;
    const void *in_ptrs[] = {x, delta, B, C, z, y};
    for (const void *q : in_ptrs)
        if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
    if (!aligned(A, 4) || !aligned(h, 4) || (D && !aligned(D, 4))) return SSM_ERR_ALIGN;
    const Range r_y = range_of(y, ch * es);
    const Range r_h = range_of(h, st * 4);
    const Range inputs[] = {range_of(x, ch * es), range_of(delta, ch * es), range_of(z, z ? ch * es : 0),
                            range_of(B, batch * dstate * es), range_of(C, batch * dstate * es),
                            range_of(A, dim * dstate * 4), range_of(D, D ? dim * 4 : 0)};
    for (const Range &r : inputs)
        if (overlaps(r_y, r) || overlaps(r_h, r)) return SSM_ERR_ALIAS;
    if (overlaps(r_y, r_h)) return SSM_ERR_ALIAS;

    DecodeParams p{};
    p.x = x; p.delta = delta; p.z = z; p.B = B; p.C = C;
    p.A = A; p.D = D; p.h = h; p.y = y;
    p.channels = ch;
    p.dim = (int)dim;
    p.N = (int)dstate;
    p.lpc_log2 = ilog2((int)((dstate + 3) / 4));
    p.vec4 = (dstate % 4 == 0) && aligned(h, 16) && aligned(A, 16);
    p.bc4 = (dstate % 4 == 0) && aligned(B, 4 * es) && aligned(C, 4 * es);
    const int64_t threads = ch << p.lpc_log2;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) return SSM_ERR_SHAPE;
    if (dtype == SSM_BF16) {
        if (disc == SSM_DISC_ZOH)
            hipLaunchKernelGGL((decode_kernel<uint16_t, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((decode_kernel<uint16_t, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    } else {
        if (disc == SSM_DISC_ZOH)
            hipLaunchKernelGGL((decode_kernel<float, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((decode_kernel<float, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" const char *ssm_status_string(int status) {
    switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid or too large sizes";
    case SSM_ERR_DTYPE: return "unknown element type";
    case SSM_ERR_UNSUPPORTED: return "unsupported dstate, discretisation or launch shape";
    case SSM_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "the HIP runtime refused a kernel launch";
    case SSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    default: return "unknown status";
    }
}
