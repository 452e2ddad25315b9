// Selective scan (S6) and decode step for MI355X (gfx950, CDNA4).
//
// What is computed is stated in include/ssm_scan.h. This file holds the C ABI
// (argument validation, launch planning, dispatch) and the decode kernel; the
// scan kernels live in scan_kernels.hpp.
//
// Decode: one thread per (channel, 4 states); the state moves as 16-byte
// vectors and a thread walks a few batch rows.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "ssm_scan.h"
#include "scan_kernels.hpp"
#include "bwd_kernels.hpp"
#include "ssd_kernels.hpp"

namespace ssm_detail {
hipError_t launch_bwd_reduce(const BwdReduceParams &p, hipStream_t st);
}

namespace {

using namespace ssm_detail;

// ---------------------------------------------------------------------------
// seqlen == 0: h_last = h0 (or zeros)

__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *h_last, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) h_last[i] = h0 != nullptr ? h0[i] : 0.0f;
}

// ---------------------------------------------------------------------------
// Backward of the convolution prologue. The backward scan runs on the
// prologue's output u = silu(cb + sum_k w[k] x[t-(W-1)+k]) (x before t = 0
// is zero), materialised by conv_silu_kernel; conv_bwd_kernel then turns the
// scan's du (kept in fp32) into
//   dpre_t  = du_t * silu'(pre_t),   silu'(p) = s (1 + p (1 - s)), s = sigmoid(p)
//   dx_s    = sum_k w[k] dpre_{s+(W-1)-k}
//   dw[k]  += dpre_t x_{t-(W-1)+k},  dcb += dpre_t
// Both kernels give a thread CPT consecutive channels (4 when dim % 4 == 0 and
// the tensors are aligned: one 8- or 16-byte access per token) of one batch
// row and walk a run of tokens with a window of the last W values in
// registers, so every element of x, u and du moves once. With the taps taken
// by lag j (wr[j] = w[W-1-j] multiplies x_{t-j}) every register index is a
// compile-time constant. conv_bwd_kernel writes per-run partial sums of dw
// and dcb, added in a fixed order by conv_reduce_kernel.
constexpr int kConvBlock = 256;

struct ConvParams {
    const void *x;            // (batch, L, dim)
    const float *w, *cb;      // (dim, W), (dim) or null
    void *u;                  // conv_silu_kernel output (batch, L, dim), fp32
    const float *du;          // gradient of u (fp32)
    void *dx;                 // gradient of x
    float *part_w, *part_b;   // (batch, nblk, dim, W), (batch, nblk, dim)
    float *dw, *db;           // (dim, W), (dim) or null
    int64_t L;
    int batch, dim, W, nblk;
    int run;                  // tokens per thread of conv_silu_kernel
    int b0;                   // first batch row of this launch (grid z: at most 65535 rows)
};

template <typename T>
__device__ __forceinline__ float conv_ld(const void *p, int64_t i) {
    if constexpr (sizeof(T) == 2)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    else
        return static_cast<const float *>(p)[i];
}

// CPT consecutive values of a T tensor at element offset i
template <typename T, int CPT>
__device__ __forceinline__ void conv_ld_piece(const void *p, int64_t i, float (&v)[CPT]) {
    if constexpr (CPT == 1) {
        v[0] = conv_ld<T>(p, i);
    } else if constexpr (sizeof(T) == 2) {
        const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        v[0] = __uint_as_float(r.x << 16);
        v[1] = __uint_as_float(r.x & 0xffff0000u);
        v[2] = __uint_as_float(r.y << 16);
        v[3] = __uint_as_float(r.y & 0xffff0000u);
    } else {
        const float4 r = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        v[0] = r.x, v[1] = r.y, v[2] = r.z, v[3] = r.w;
    }
}

template <int CPT>
__device__ __forceinline__ void conv_ld_f32(const float *p, int64_t i, float (&v)[CPT]) {
    if constexpr (CPT == 1) {
        v[0] = p[i];
    } else {
        const float4 r = *reinterpret_cast<const float4 *>(p + i);
        v[0] = r.x, v[1] = r.y, v[2] = r.z, v[3] = r.w;
    }
}

template <typename T>
__device__ __forceinline__ uint16_t conv_bf(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

template <typename T, int CPT>
__device__ __forceinline__ void conv_st_piece(void *p, int64_t i, const float (&v)[CPT]) {
    if constexpr (CPT == 1) {
        if constexpr (sizeof(T) == 2)
            static_cast<uint16_t *>(p)[i] = conv_bf<T>(v[0]);
        else
            static_cast<float *>(p)[i] = v[0];
    } else if constexpr (sizeof(T) == 2) {
        const uint2 r = {(uint32_t)conv_bf<T>(v[0]) | ((uint32_t)conv_bf<T>(v[1]) << 16),
                         (uint32_t)conv_bf<T>(v[2]) | ((uint32_t)conv_bf<T>(v[3]) << 16)};
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p) + i) = r;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Taps by lag (wr[c][j] multiplies x_{t-j}; zero past W) and the bias of the
// thread's channels
template <int CPT>
__device__ __forceinline__ void conv_taps(const ConvParams &p, int d0, float (&wr)[CPT][kConvMax], float (&cb)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        cb[c] = p.cb ? p.cb[d0 + c] : 0.0f;
#pragma unroll
        for (int j = 0; j < kConvMax; ++j)
            wr[c][j] = j < p.W ? p.w[(int64_t)(d0 + c) * p.W + (p.W - 1 - j)] : 0.0f;
    }
}

// pre_t = cb + sum_{j < W} wr[j] x_{t-j}, with xs[j] = x_{t-j}
template <int CPT>
__device__ __forceinline__ void conv_pre(const float (&wr)[CPT][kConvMax], const float (&cb)[CPT],
                                         const float (&xs)[kConvMax][CPT], int W, float (&pre)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float acc = cb[c];
#pragma unroll
        for (int j = 0; j < kConvMax; ++j)
            if (j < W) acc = fmaf(wr[c][j], xs[j][c], acc);
        pre[c] = acc;
    }
}

template <typename T, int CPT, typename UT = float>
__global__ __launch_bounds__(256) void conv_silu_kernel(const ConvParams p) {
    const int d0 = (blockIdx.x * blockDim.x + threadIdx.x) * CPT;
    if (d0 >= p.dim) return;
    const int64_t row = (int64_t)(p.b0 + (int)blockIdx.z) * p.L;
    const int64_t t0 = (int64_t)blockIdx.y * p.run;
    if (t0 >= p.L) return;
    const int64_t t1 = min(p.L, t0 + p.run);
    float wr[CPT][kConvMax], cb[CPT];
    conv_taps<CPT>(p, d0, wr, cb);
    // xs[j] holds x_{t0-1-j} before the first shift (zero before the sequence)
    float xs[kConvMax][CPT];
#pragma unroll
    for (int j = 0; j < kConvMax; ++j) {
        const int64_t s = t0 - 1 - j;
        if (j + 1 < p.W && s >= 0) {
            conv_ld_piece<T, CPT>(p.x, (row + s) * p.dim + d0, xs[j]);
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) xs[j][c] = 0.0f;
        }
    }
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
#pragma unroll
        for (int j = kConvMax - 1; j > 0; --j)
#pragma unroll
            for (int c = 0; c < CPT; ++c) xs[j][c] = xs[j - 1][c];
        const int64_t i = (row + t) * p.dim + d0;
        conv_ld_piece<T, CPT>(p.x, i, xs[0]);
        float u[CPT];
        conv_pre<CPT>(wr, cb, xs, p.W, u);
#pragma unroll
        for (int c = 0; c < CPT; ++c) u[c] = silu(u[c]);
        conv_st_piece<UT, CPT>(p.u, i, u);
    }
}

template <typename T, int CPT>
__global__ __launch_bounds__(256) void conv_bwd_kernel(const ConvParams p) {
    const int d0 = (blockIdx.x * blockDim.x + threadIdx.x) * CPT;
    if (d0 >= p.dim) return;
    const int blk = blockIdx.y;
    const int b = p.b0 + (int)blockIdx.z;
    const int W = p.W;
    float wr[CPT][kConvMax], cb[CPT];
    conv_taps<CPT>(p, d0, wr, cb);
    const int64_t t0 = (int64_t)blk * kConvBlock;
    const int64_t t1 = min(p.L, t0 + kConvBlock);
    const int64_t row = (int64_t)b * p.L;
    // xs[j]: x_{t-j}, ds[j]: dpre_{t-j} (zero outside the sequence)
    float xs[kConvMax][CPT], ds[kConvMax][CPT], gw[CPT][kConvMax], gb[CPT];
#pragma unroll
    for (int j = 0; j < kConvMax; ++j) {
        const int64_t s = t0 - 1 - j;        // slot j + 1 after the shift at t0
        if (j + 1 < W && s >= 0) {
            conv_ld_piece<T, CPT>(p.x, (row + s) * p.dim + d0, xs[j]);
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) xs[j][c] = 0.0f;
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            ds[j][c] = 0.0f;
            gw[c][j] = 0.0f;
        }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) gb[c] = 0.0f;
    // dx_s = sum_{j < W} wr[j] dpre_{s+j}: emitted at t = s + kConvMax - 1, when
    // ds[kConvMax-1-j] holds dpre_{s+j}; the walk runs kConvMax - 1 tokens past
    // the block, with zero x and dpre past the sequence
    auto step = [&](int64_t t, auto load) {
#pragma unroll
        for (int j = kConvMax - 1; j > 0; --j)
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                xs[j][c] = xs[j - 1][c];
                ds[j][c] = ds[j - 1][c];
            }
        if constexpr (decltype(load)::value) {
            const int64_t i = (row + t) * p.dim + d0;
            float du[CPT], pre[CPT];
            conv_ld_piece<T, CPT>(p.x, i, xs[0]);
            conv_ld_f32<CPT>(p.du, i, du);
            conv_pre<CPT>(wr, cb, xs, W, pre);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float sg = 1.0f / (1.0f + __expf(-pre[c]));
                ds[0][c] = du[c] * sg * (1.0f + pre[c] * (1.0f - sg));
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) xs[0][c] = ds[0][c] = 0.0f;
        }
        if (t < t1) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                gb[c] += ds[0][c];
#pragma unroll
                for (int j = 0; j < kConvMax; ++j)
                    if (j < W) gw[c][j] = fmaf(ds[0][c], xs[j][c], gw[c][j]);
            }
        }
        const int64_t s = t - (kConvMax - 1);
        if (s >= t0) {
            float g[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < kConvMax; ++j)
                    if (j < W) acc = fmaf(wr[c][j], ds[kConvMax - 1 - j][c], acc);
                g[c] = acc;
            }
            conv_st_piece<T, CPT>(p.dx, (row + s) * p.dim + d0, g);
        }
    };
    const int64_t tw = t1 + kConvMax - 1;        // end of the walk
    const int64_t tl = min(p.L, tw);             // end of the tokens that exist
    int64_t t = t0;
#pragma unroll 4
    for (; t < tl; ++t) step(t, std::true_type{});
    for (; t < tw; ++t) step(t, std::false_type{});
    // per-block partials: dw[k] of the lag j = W - 1 - k
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float *pw = p.part_w + (((int64_t)b * p.nblk + blk) * p.dim + d0 + c) * W;
#pragma unroll
        for (int j = 0; j < kConvMax; ++j)
            if (j < W) pw[W - 1 - j] = gw[c][j];
        p.part_b[((int64_t)b * p.nblk + blk) * p.dim + d0 + c] = gb[c];
    }
}

__global__ __launch_bounds__(256) void conv_reduce_kernel(const ConvParams p) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (d, k), then d for the bias
    const int64_t nw = (int64_t)p.dim * p.W;
    if (i < nw) {
        float acc = 0.0f;
        for (int b = 0; b < p.batch; ++b)
#pragma unroll 8
            for (int k = 0; k < p.nblk; ++k) acc += p.part_w[((int64_t)b * p.nblk + k) * nw + i];
        p.dw[i] = acc;
    } else if (i < nw + p.dim && p.db != nullptr) {
        const int64_t d = i - nw;
        float acc = 0.0f;
        for (int b = 0; b < p.batch; ++b)
#pragma unroll 8
            for (int k = 0; k < p.nblk; ++k) acc += p.part_b[((int64_t)b * p.nblk + k) * p.dim + d];
        p.db[d] = acc;
    }
}

// Both prologue passes run over every batch row in launches of at most 65535
// rows, the grid's z extent.
constexpr int64_t kMaxGridZ = 65535;

// u = silu(conv(x)) in fp32. cpt: channels per thread (4 for whole, aligned
// 4-channel pieces, else 1).
hipError_t launch_conv_silu(ConvParams cp, bool bf16, int cpt, hipStream_t stream) {
    // runs of at least 64 tokens, at most 65535 of them per batch row
    const int64_t runs = std::min<int64_t>((cp.L + 63) / 64, 65535);
    cp.run = (int)((cp.L + runs - 1) / runs);
    for (int64_t b0 = 0; b0 < cp.batch; b0 += kMaxGridZ) {
        cp.b0 = (int)b0;
        const dim3 grid((unsigned)((cp.dim / cpt + 255) / 256), (unsigned)runs,
                        (unsigned)std::min<int64_t>(kMaxGridZ, cp.batch - b0));
        if (bf16) {
            if (cpt == 4)
                hipLaunchKernelGGL((conv_silu_kernel<uint16_t, 4, float>), grid, dim3(256), 0, stream, cp);
            else
                hipLaunchKernelGGL((conv_silu_kernel<uint16_t, 1, float>), grid, dim3(256), 0, stream, cp);
        } else {
            if (cpt == 4)
                hipLaunchKernelGGL((conv_silu_kernel<float, 4, float>), grid, dim3(256), 0, stream, cp);
            else
                hipLaunchKernelGGL((conv_silu_kernel<float, 1, float>), grid, dim3(256), 0, stream, cp);
        }
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

// dx and the per-block tap and bias partials, then their fixed-order sums.
hipError_t launch_conv_bwd(ConvParams cp, bool bf16, int cpt, hipStream_t stream) {
    for (int64_t b0 = 0; b0 < cp.batch; b0 += kMaxGridZ) {
        cp.b0 = (int)b0;
        const dim3 grid((unsigned)((cp.dim / cpt + 255) / 256), (unsigned)cp.nblk,
                        (unsigned)std::min<int64_t>(kMaxGridZ, cp.batch - b0));
        if (bf16) {
            if (cpt == 4)
                hipLaunchKernelGGL((conv_bwd_kernel<uint16_t, 4>), grid, dim3(256), 0, stream, cp);
            else
                hipLaunchKernelGGL((conv_bwd_kernel<uint16_t, 1>), grid, dim3(256), 0, stream, cp);
        } else {
            if (cpt == 4)
                hipLaunchKernelGGL((conv_bwd_kernel<float, 4>), grid, dim3(256), 0, stream, cp);
            else
                hipLaunchKernelGGL((conv_bwd_kernel<float, 1>), grid, dim3(256), 0, stream, cp);
        }
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    cp.b0 = 0;
    const int64_t nr = (int64_t)cp.dim * cp.W + cp.dim;
    hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, stream, cp);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode step

// Decode: one thread per (channel, 4 states), so that a wave's 16-byte state
// accesses are contiguous; the LPC lanes of a channel add their partial
// readouts with DPP quad permutes (and cross-lane shuffles beyond 4 lanes). A
// workgroup covers consecutive channels d of kDecodeRows batch rows; a thread
// keeps its A values in registers for all its rows and issues the state loads
// of its rows before the arithmetic. The state is read and written once.
// (Measured on b256 d5120 N16: 1 row per thread 34.2 us, 2 rows 31.6 us,
// 4 rows 31.9 us, 8 rows 36.3 us.)
constexpr int kDecodeRows = 2;

struct DecodeParams {
    const void *x, *delta, *z, *B, *C;
    const float *delta_bias;   // (dim) or null
    int delta_softplus;
    const float *A, *D;
    float *h;
    void *y;
    int batch, dim, N;
    int vec4;             // N % 4 == 0 and h, A 16-byte aligned
    int bc4;              // N % 4 == 0 and B, C aligned to 4 elements
};

// v + (v of the lane whose index differs in bit m), for m = 1, 2 (inside
// groups of 4 lanes) by DPP, else by a cross-lane shuffle
template <int M> __device__ __forceinline__ float add_xor(float v) {
    if constexpr (M == 1 || M == 2) {
        constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;      // quad_perm [1,0,3,2] / [2,3,0,1]
        return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true));
    } else {
        return v + __shfl_xor(v, M, 64);
    }
}

template <typename T, bool ZOH, int LPC>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    typedef typename std::conditional<sizeof(T) == 2, uint2, uint4>::type RawBC;   // 4 values of B or C
    constexpr int kCPB = 256 / LPC;                // channels per workgroup
    const int d = blockIdx.x * kCPB + (int)(threadIdx.x / LPC);
    const int q = (int)(threadIdx.x % LPC);
    const bool dvalid = d < p.dim;
    const int dc = dvalid ? d : p.dim - 1;
    const int n0 = q * 4;
    // with N % 4 == 0 a lane's four states are either all inside the channel
    // (n0 < N) or all past it (lanes added to round lanes-per-channel up to a
    // power of two); those lanes must not touch memory
    const bool qv = n0 < p.N;
    const T *x = static_cast<const T *>(p.x);
    const T *dt = static_cast<const T *>(p.delta);
    const T *zp = static_cast<const T *>(p.z);
    const T *Bp = static_cast<const T *>(p.B);
    const T *Cp = static_cast<const T *>(p.C);

    float av[4];
    const float *ap = p.A + (int64_t)dc * p.N + n0;
    if (p.vec4) {
        const float4 a4 = qv ? *reinterpret_cast<const float4 *>(ap) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) av[k] = n0 + k < p.N ? ap[k] : 0.0f;
    }
    const float Dd = p.D != nullptr ? p.D[dc] : 0.0f;
    const float dbias = p.delta_bias != nullptr ? p.delta_bias[dc] : 0.0f;

    // groups of kDecodeRows rows, strided over the grid's y extent; a thread
    // with more than one group loads its next group while it updates the
    // current one
    const int ngroups = (p.batch + kDecodeRows - 1) / kDecodeRows;
    struct Group {
        float hv[kDecodeRows][4];
        T xr[kDecodeRows], dr[kDecodeRows], zr[kDecodeRows];
        RawBC br[kDecodeRows], cr[kDecodeRows];
    };
    auto load = [&](int grp, Group &g) {
#pragma unroll
        for (int r = 0; r < kDecodeRows; ++r) {
            const int64_t b = min(grp * kDecodeRows + r, p.batch - 1);
            const int64_t cc = b * p.dim + dc;
            const float *hp = p.h + cc * p.N + n0;
            if (p.vec4) {
                const float4 h4 = qv ? *reinterpret_cast<const float4 *>(hp) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                g.hv[r][0] = h4.x; g.hv[r][1] = h4.y; g.hv[r][2] = h4.z; g.hv[r][3] = h4.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) g.hv[r][k] = n0 + k < p.N ? hp[k] : 0.0f;
            }
            g.xr[r] = x[cc];
            g.dr[r] = dt[cc];
            g.zr[r] = zp != nullptr ? zp[cc] : T(0);
            if (p.bc4 && qv) {
                g.br[r] = *reinterpret_cast<const RawBC *>(Bp + b * p.N + n0);
                g.cr[r] = *reinterpret_cast<const RawBC *>(Cp + b * p.N + n0);
            }
        }
    };
    Group cur, nxt;
    int grp = blockIdx.y;
    if (grp < ngroups) load(grp, cur);
    for (; grp < ngroups; grp += gridDim.y) {
        if (grp + (int)gridDim.y < ngroups) load(grp + gridDim.y, nxt);
        float (&hv)[kDecodeRows][4] = cur.hv;
        const T (&xr)[kDecodeRows] = cur.xr;
        const T (&dr)[kDecodeRows] = cur.dr;
        const T (&zr)[kDecodeRows] = cur.zr;
        const RawBC (&br)[kDecodeRows] = cur.br;
        const RawBC (&cr)[kDecodeRows] = cur.cr;
#pragma unroll
        for (int r = 0; r < kDecodeRows; ++r) {
            const int64_t b = grp * kDecodeRows + r;
            const int64_t bl = min(b, (int64_t)p.batch - 1);
            float bv[4], cv[4];
            if (p.bc4) {
                if (qv) {
                    if constexpr (sizeof(T) == 2) {
                        const uint2 rb = br[r], rc = cr[r];
                        bv[0] = __uint_as_float(rb.x << 16); bv[1] = __uint_as_float(rb.x & 0xffff0000u);
                        bv[2] = __uint_as_float(rb.y << 16); bv[3] = __uint_as_float(rb.y & 0xffff0000u);
                        cv[0] = __uint_as_float(rc.x << 16); cv[1] = __uint_as_float(rc.x & 0xffff0000u);
                        cv[2] = __uint_as_float(rc.y << 16); cv[3] = __uint_as_float(rc.y & 0xffff0000u);
                    } else {
                        const uint4 rb = br[r], rc = cr[r];
                        bv[0] = __uint_as_float(rb.x); bv[1] = __uint_as_float(rb.y);
                        bv[2] = __uint_as_float(rb.z); bv[3] = __uint_as_float(rb.w);
                        cv[0] = __uint_as_float(rc.x); cv[1] = __uint_as_float(rc.y);
                        cv[2] = __uint_as_float(rc.z); cv[3] = __uint_as_float(rc.w);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) bv[k] = cv[k] = 0.0f;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool ok = n0 + k < p.N;
                    bv[k] = ok ? Elem<T>::widen(Bp[bl * p.N + n0 + k]) : 0.0f;
                    cv[k] = ok ? Elem<T>::widen(Cp[bl * p.N + n0 + k]) : 0.0f;
                }
            }
            const float xv = Elem<T>::widen(xr[r]);
            float dv = Elem<T>::widen(dr[r]) + dbias;
            if (p.delta_softplus) dv = softplus_f(dv);
            const float du = dv * xv;
            float part = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (ZOH) {
                    const float a = __builtin_amdgcn_exp2f(dv * av[k] * kLog2e);
                    hv[r][k] = fmaf(a, hv[r][k], dv * expm1_over_x(dv * av[k], a) * bv[k] * xv);
                } else {
                    hv[r][k] = fmaf(__builtin_amdgcn_exp2f(dv * av[k] * kLog2e), hv[r][k], du * bv[k]);
                }
                part = fmaf(cv[k], hv[r][k], part);
            }
            // sum the partial readouts of the LPC lanes of this channel
            if constexpr (LPC >= 2) part = add_xor<1>(part);
            if constexpr (LPC >= 4) part = add_xor<2>(part);
            if constexpr (LPC >= 8) part = add_xor<4>(part);
            if constexpr (LPC >= 16) part = add_xor<8>(part);
            if (!dvalid || b >= p.batch) continue;
            const int64_t cc = b * p.dim + d;
            float *hp = p.h + cc * p.N + n0;
            if (p.vec4) {
                if (qv) *reinterpret_cast<float4 *>(hp) = make_float4(hv[r][0], hv[r][1], hv[r][2], hv[r][3]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (n0 + k < p.N) hp[k] = hv[r][k];
            }
            if (q == 0) {
                float yv = part + Dd * xv;
                if (zp != nullptr) yv *= silu(Elem<T>::widen(zr[r]));
                if constexpr (sizeof(T) == 2)
                    static_cast<uint16_t *>(p.y)[cc] = Elem<uint16_t>::to_bits(yv);
                else
                    static_cast<float *>(p.y)[cc] = yv;
            }
        }
        cur = nxt;
    }
}

template <typename T, bool ZOH>
hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
    // lanes per channel: 4 states per lane, rounded up to a power of two
    const int lpc = p.N <= 4 ? 1 : p.N <= 8 ? 2 : p.N <= 16 ? 4 : p.N <= 32 ? 8 : 16;
    const int cpb = 256 / lpc;
    const int ngroups = (p.batch + kDecodeRows - 1) / kDecodeRows;
    // up to about 32K waves; past that, threads take several groups each
    // (b256 d5120 N16: 38.40 us per step against 39.09 with one group per
    // thread; 41.07 with the grid cut to the ~8K waves the GPU keeps resident)
    const int gx = (p.dim + cpb - 1) / cpb;
    const int gy = max(1, min(ngroups, min(65535, 8192 / max(gx, 1))));
    const dim3 grid((unsigned)gx, (unsigned)gy);
    switch (lpc) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, ZOH, 1>), grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, ZOH, 2>), grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, ZOH, 4>), grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<T, ZOH, 8>), grid, dim3(256), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<T, ZOH, 16>), grid, dim3(256), 0, stream, p); break;
    }
    return hipGetLastError();
}

// One decode step of the SSD layer (ssm_ssd_fwd with one token): per batch row
// and head, the (P x N) state is updated in place and y written for the token.
// One thread per (batch row, head, p, 4 consecutive n): a state row of N fp32
// values moves as N/4 16-byte pieces over N/4 consecutive lanes, which sum the
// readout C . h over the row by lane exchanges.
struct SsdDecodeParams {
    const uint16_t *x, *dt, *B, *C, *z;   // bf16 bit patterns
    const float *dt_bias, *A, *D;
    float *h;
    uint16_t *y;
    int64_t rows;                         // batch * nheads * headdim
    int H, G, hpg, P, N;
    int dt_softplus;
};

template <bool ZOH>
__global__ __launch_bounds__(256) void ssd_decode_kernel(const SsdDecodeParams p) {
    const int lpr = p.N / 4;                              // lanes per state row (16 or 32)
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = tid / lpr;                        // (b, h, p)
    const int q = (int)(tid % lpr);
    const bool valid = row < p.rows;
    const int64_t r = valid ? row : 0;
    const int64_t bh = r / p.P;                           // b * H + h
    const int hd = (int)(bh % p.H);
    const int64_t b = bh / p.H;
    const int g = hd / p.hpg;
    auto bf = [](uint16_t v) { return __uint_as_float((uint32_t)v << 16); };

    float part = 0.0f, xv = 0.0f;
    if (valid) {
        float dtv = bf(p.dt[bh]) + (p.dt_bias ? p.dt_bias[hd] : 0.0f);
        if (p.dt_softplus) dtv = softplus_f(dtv);
        const float Ah = p.A[hd];
        const float a = __builtin_amdgcn_exp2f(dtv * Ah * kLog2e);
        const float wbar = ZOH ? dtv * expm1_over_x(dtv * Ah, a) : dtv;
        xv = bf(p.x[r]);
        const float wx = wbar * xv;
        const int64_t bc = (b * p.G + g) * p.N + 4 * q;
        const uint2 bw = *reinterpret_cast<const uint2 *>(p.B + bc);
        const uint2 cw = *reinterpret_cast<const uint2 *>(p.C + bc);
        const float bv[4] = {bf(bw.x & 0xffffu), bf(bw.x >> 16), bf(bw.y & 0xffffu), bf(bw.y >> 16)};
        const float cv[4] = {bf(cw.x & 0xffffu), bf(cw.x >> 16), bf(cw.y & 0xffffu), bf(cw.y >> 16)};
        float4 *hp = reinterpret_cast<float4 *>(p.h + r * p.N + 4 * q);
        float4 hv = *hp;
        hv.x = fmaf(a, hv.x, wx * bv[0]);
        hv.y = fmaf(a, hv.y, wx * bv[1]);
        hv.z = fmaf(a, hv.z, wx * bv[2]);
        hv.w = fmaf(a, hv.w, wx * bv[3]);
        *hp = hv;
        part = fmaf(cv[3], hv.w, fmaf(cv[2], hv.z, fmaf(cv[1], hv.y, cv[0] * hv.x)));
    }
    // the row's lanes are lpr consecutive lanes starting at a multiple of lpr
    for (int o = lpr / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (valid && q == 0) {
        float yv = part + (p.D ? p.D[hd] * xv : 0.0f);
        if (p.z) yv *= silu(bf(p.z[r]));
        p.y[r] = __builtin_bit_cast(uint16_t, (__bf16)yv);
    }
}

// ---------------------------------------------------------------------------
// Backward: sums of the per-tile dB, dC and per-row dA, dD partials, in a fixed
// order (tiles, then batch rows), so that the result does not depend on timing.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const BwdReduceParams p) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nbc = (int64_t)p.batch * p.L * p.N;
    const int64_t na = (int64_t)p.dim * p.N;
    if (i < nbc) {
        const int n = (int)(i % p.N);
        const int64_t bt = i / p.N;
        const int64_t t = bt % p.L, b = bt / p.L;
        float sb = 0.0f, sc = 0.0f;
        for (int tile = 0; tile < p.ntiles; ++tile) {
            const float2 v = *reinterpret_cast<const float2 *>(
                p.part_bc + ((((int64_t)b * p.ntiles + tile) * p.L + t) * p.npad + n) * 2);
            sb += v.x;
            sc += v.y;
        }
        p.dB[i] = sb;
        p.dC[i] = sc;
    } else if (i < nbc + na) {
        const int64_t k = i - nbc;
        const int n = (int)(k % p.N);
        const int64_t d = k / p.N;
        float sa = 0.0f;
        for (int b = 0; b < p.batch; ++b) sa += p.part_a[((int64_t)b * p.dim + d) * p.npad + n];
        p.dA[k] = sa;
    } else if (i < nbc + na + p.dim) {
        const int64_t d = i - nbc - na;
        float sd = 0.0f;
        for (int b = 0; b < p.batch; ++b) sd += p.part_d[(int64_t)b * p.dim + d];
        if (p.dD != nullptr) p.dD[d] = sd;
        if (p.ddelta_bias != nullptr) {
            float sb = 0.0f;
            for (int b = 0; b < p.batch; ++b) sb += p.part_db[(int64_t)b * p.dim + d];
            p.ddelta_bias[d] = sb;
        }
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
    // segments cost a second (aggregate) pass over their tokens: add them only
    // while the waves are too few, and keep them >= 256 tokens
    auto segments_for = [&](int g) {
        int s = 1;
        if (tiles * g < want_waves)
            while (s < kMaxSegments && tiles * g * s < 2 * want_waves && d.seqlen / (2 * s) >= 256) s *= 2;
        return s;
    };
    bool long_ctx = false;
    if (G == 0) {
        G = pl.npad > 16 ? pl.npad / 16 : 1;     // at most 16 states per wave
        while (G < 8 && G < pl.npad && tiles * G < want_waves) G *= 2;
        // Too few channels for 8 waves per tile and long segments: 4 waves of
        // 4 states per tile, whose smaller workgroups fit more per CU and add
        // 3 instead of 7 partial readouts per output (measured on L 131072 x
        // 5120 channels, 16 states: 4 waves x 32 segments 3.80 ms against 8 x
        // 16 4.24 ms; on L 2048 x 6144 channels the segments are short and
        // 8 waves x 8 segments stay faster, 0.105 against 0.106 ms)
        if (G == 8 && pl.npad == 16 && tiles * G < want_waves && (t == nullptr || t->segments == 0) &&
            d.seqlen / segments_for(4) >= 2048) {
            G = 4;
            long_ctx = true;
        }
    }
    pl.G = G;
    pl.npw = pl.npad / G;
    int S = (t && t->segments > 0) ? t->segments : 0;
    if (S == 0) {
        S = segments_for(G);
        // Long context at 4 waves per tile: half as many segments again
        // (measured on L 131072 x 5120 channels, 16 states: 48 segments 3.55
        // and 3.65 ms on two boxes, against 3.65 and 3.80 for 32 and 3.81
        // for 64)
        if (long_ctx) S = std::min(kMaxSegments, S + S / 2);
    }
    if (d.seqlen > 0 && S > d.seqlen) S = (int)d.seqlen;
    if (S < 1) S = 1;
    pl.S = S;
    // segments start on 16-token boundaries (whole chunks, aligned runs of B and C)
    const int64_t seg_len = d.seqlen > 0 ? ((d.seqlen + S - 1) / S + 15) / 16 * 16 : 0;
    // a segment longer than an int is not supported (-1): the kernels count a
    // segment's tokens in 32 bits
    pl.seg_len = seg_len > INT32_MAX ? -1 : (int)seg_len;
    if (d.seqlen > 0 && pl.seg_len > 0)
        pl.S = (int)((d.seqlen + pl.seg_len - 1) / pl.seg_len);   // drop empty segments
    return pl;
}

bool plan_supported(const Plan &pl) {
    if (pl.G < 1 || pl.G > 16 || (pl.G & (pl.G - 1)) != 0) return false;
    if (pl.npad % pl.G != 0) return false;
    if (pl.npw < 1 || pl.npw > 16) return false;
    if (pl.S < 1 || pl.S > kMaxSegments) return false;
    return pl.seg_len > 0 || (pl.seg_len == 0 && pl.S == 1);   // 0: an empty sequence
}

// The scan's passes for the descriptor's element type and rule; bf16 tensors
// whose u is the convolution pass's fp32 output take the units reading u so.
hipError_t launch_scan(const ssm_scan_desc &d, const Plan &pl, const ScanParams &p, int nm, int na,
                       hipStream_t stream) {
    const bool zoh = d.disc == SSM_DISC_ZOH;
    if (d.dtype == SSM_BF16 && p.u_f32)
        return zoh ? launch_scan_bf16_zoh_u32(pl, p, nm, na, stream) : launch_scan_bf16_euler_u32(pl, p, nm, na, stream);
    if (d.dtype == SSM_BF16)
        return zoh ? launch_scan_bf16_zoh(pl, p, nm, na, stream) : launch_scan_bf16_euler(pl, p, nm, na, stream);
    return zoh ? launch_scan_f32_zoh(pl, p, nm, na, stream) : launch_scan_f32_euler(pl, p, nm, na, stream);
}

// The forward runs the convolution prologue as a pass of its own: u =
// silu(conv(x)) in fp32, in the workspace after the scan's own part. The scan
// is ALU-bound, so the prologue's instructions inside it cost it more than this
// pass's memory traffic. u stays fp32 for bf16 tensors too: the scan sums many
// products of it, which can cancel, and a bf16 rounding of u then shows in y
// well beyond one rounding of y.
size_t conv_u_bytes(const ssm_scan_desc &d) { return align256((size_t)d.batch * d.seqlen * d.dim * 4); }

size_t workspace_bytes_for(const ssm_scan_desc &d, const Plan &pl) {
    if (d.batch == 0 || d.dim == 0 || d.seqlen == 0) return 0;
    const size_t scan = align256(workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, pl).total);
    return scan + (d.conv_width > 0 ? conv_u_bytes(d) : 0);
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

constexpr int64_t kMaxDim = int64_t(1) << 26;

int validate_desc(const ssm_scan_desc *d) {
    if (d == nullptr) return SSM_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->dim < 0) return SSM_ERR_SHAPE;
    if (d->dtype != SSM_F32 && d->dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d->disc != SSM_DISC_EULER && d->disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d->dstate < 1 || d->dstate > 64) return SSM_ERR_UNSUPPORTED;
    if (d->delta_softplus != 0 && d->delta_softplus != 1) return SSM_ERR_UNSUPPORTED;
    if (d->conv_width < 0 || d->conv_width > kConvMax) return SSM_ERR_UNSUPPORTED;
    if (d->conv_width > 0 && d->conv_weight == nullptr) return SSM_ERR_NULL;
    if ((d->delta_bias != nullptr && !aligned(d->delta_bias, 4)) ||
        (d->conv_width > 0 && !aligned(d->conv_weight, 4)) || (d->conv_bias != nullptr && !aligned(d->conv_bias, 4)))
        return SSM_ERR_ALIGN;
    // byte counts of the largest tensors must fit; kernel indices are 32-bit
    // for batch, dim and segment lengths
    int64_t bl, bld, bytes;
    if (!mul_ok(d->batch, d->seqlen, &bl) || !mul_ok(bl, d->dim, &bld) || !mul_ok(bld, 4, &bytes))
        return SSM_ERR_SHAPE;
    int64_t bdn;
    if (!mul_ok(d->batch, d->dim, &bdn) || !mul_ok(bdn, d->dstate * 4 * kMaxSegments * 3, &bytes))
        return SSM_ERR_SHAPE;
    if (d->batch > INT32_MAX || d->dim > INT32_MAX) return SSM_ERR_SHAPE;
    // a chunk of up to 16 token rows of fp32 channels spans less than 4 GiB,
    // so the kernels address it with 32-bit offsets
    if (d->dim > kMaxDim) return SSM_ERR_SHAPE;
    return SSM_OK;
}

// What a forward that keeps the backward's checkpoints adds: the backward's
// workspace size, and where in it the checkpoints go (the forward's own
// workspace, regrouped B and C and segment arrays, comes first in both)
struct SaveForBwd {
    size_t need, ckpt;
    int nck;
    size_t conv_u;   // where the convolution pass's u goes (where the backward reads it)
};

int scan_impl(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
              const void *B, const void *C, const float *D, const void *z, const float *h0,
              void *y, float *h_last, void *workspace, size_t workspace_bytes,
              const ssm_scan_tuning *tuning, hipStream_t stream, const SaveForBwd *save = nullptr) {
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

    const size_t need = save ? save->need : workspace_bytes_for(d, pl);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SSM_ERR_WORKSPACE;

    const Range r_y = range_of(y, d.seqlen > 0 ? tok * es : 0);
    const Range r_hl = range_of(h_last, state * 4);
    const Range r_ws = range_of(workspace, (int64_t)need);
    const Range inputs[] = {range_of(u, tok * es), range_of(delta, tok * es), range_of(z, z ? tok * es : 0),
                            range_of(B, bn * es), range_of(C, bn * es), range_of(A, d.dim * d.dstate * 4),
                            range_of(D, D ? d.dim * 4 : 0), range_of(h0, h0 ? state * 4 : 0),
                            range_of(d.delta_bias, d.delta_bias ? d.dim * 4 : 0),
                            range_of(d.conv_width ? d.conv_weight : nullptr, d.dim * d.conv_width * 4),
                            range_of(d.conv_width ? d.conv_bias : nullptr, d.dim * 4)};
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

    // the main pass's grid (checked before anything is launched)
    if ((d.dim + kTile - 1) / kTile * d.batch * pl.S > INT32_MAX) return SSM_ERR_SHAPE;

    // the convolution prologue as a pass of its own, writing u in fp32; the scan
    // then reads that u. Keeping the checkpoints, it writes u where the backward
    // reads it, so that the backward need not form it again
    const void *us = u;
    if (d.conv_width > 0) {
        char *ws = static_cast<char *>(workspace);
        void *uw = ws + (save ? save->conv_u : align256(workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, pl).total));
        ConvParams cp{};
        cp.x = u;
        cp.w = d.conv_weight;
        cp.cb = d.conv_bias;
        cp.u = uw;
        cp.L = d.seqlen;
        cp.batch = (int)d.batch;
        cp.dim = (int)d.dim;
        cp.W = d.conv_width;
        const int cpt = (d.dim % 4 == 0 && aligned(u, 4 * es)) ? 4 : 1;
        if (launch_conv_silu(cp, d.dtype == SSM_BF16, cpt, stream) != hipSuccess) return SSM_ERR_HIP;
        us = uw;
    }

    ScanParams p{};
    p.u = us; p.delta = delta; p.z = z; p.B = B; p.C = C;
    p.u_f32 = us != u && d.dtype == SSM_BF16;
    p.delta_bias = d.delta_bias; p.delta_softplus = d.delta_softplus;
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
    p.vec = (d.dim % 4 == 0) && aligned(us, 4 * es) && aligned(delta, 4 * es) && (!z || aligned(z, 4 * es)) &&
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
        if (save) {
            p.ckpt = reinterpret_cast<float *>(ws + save->ckpt);
            p.nck = save->nck;
        }
    }
    const int64_t blocks_per_seg = (int64_t)p.ntiles * d.batch;
    const int64_t nm = blocks_per_seg * pl.S;
    const int64_t na = pl.S > 1 ? blocks_per_seg * (pl.S - 1) : 0;
    return launch_scan(d, pl, p, (int)nm, (int)na, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// Backward workspace: the checkpoint pass's forward workspace (regrouped B, C
// and segment arrays), then the checkpoints, the per-tile dB/dC partials and
// the per-row dA, dD partials.
struct BwdLayout {
    Plan pl;
    BwdShape sh;
    int nck, ntiles, nblk;
    size_t ckpt, part_bc, part_a, part_d, part_db, conv_u, conv_du, conv_pw, conv_pb, total;
};

BwdLayout bwd_layout(const ssm_scan_desc &d) {
    BwdLayout w{};
    w.sh = bwd_shape(padded_states(d.dstate));
    ssm_scan_tuning t{w.sh.G, 0};
    w.pl = make_plan(d, &t);
    w.nck = (int)((d.seqlen + w.sh.TC - 1) / w.sh.TC);
    w.ntiles = (int)((d.dim + kTile - 1) / kTile);
    const size_t fwd = workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, w.pl).total;
    const size_t np = (size_t)w.sh.npad;
    w.ckpt = fwd;
    w.part_bc = w.ckpt + align256((size_t)d.batch * w.nck * np * d.dim * 4);
    w.part_a = w.part_bc + align256((size_t)d.batch * w.ntiles * d.seqlen * np * 2 * 4);
    w.part_d = w.part_a + align256((size_t)d.batch * d.dim * np * 4);
    w.part_db = w.part_d + align256((size_t)d.batch * d.dim * 4);
    w.conv_u = w.part_db + (d.delta_bias != nullptr ? align256((size_t)d.batch * d.dim * 4) : 0);
    w.total = w.conv_u;
    if (d.conv_width > 0) {
        // the prologue's output u and the gradient of u, per-block sums of the tap and bias gradients
        const size_t tok = (size_t)d.batch * d.seqlen * d.dim;
        w.nblk = (int)((d.seqlen + kConvBlock - 1) / kConvBlock);
        w.conv_du = w.conv_u + align256(tok * 4);
        w.conv_pw = w.conv_du + align256(tok * 4);
        w.conv_pb = w.conv_pw + align256((size_t)d.batch * w.nblk * d.dim * d.conv_width * 4);
        w.total = w.conv_pb + align256((size_t)d.batch * w.nblk * d.dim * 4);
    }
    return w;
}

size_t bwd_workspace_bytes(const ssm_scan_desc &d) {
    if (d.batch == 0 || d.dim == 0 || d.seqlen == 0) return 0;
    return bwd_layout(d).total;
}

int bwd_impl(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A, const void *B,
             const void *C, const float *D, const void *z, const float *h0, const void *dy, const float *dh_last,
             void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz, float *dh0,
             float *ddelta_bias, float *dconv_weight, float *dconv_bias, void *workspace, size_t workspace_bytes,
             hipStream_t stream, bool saved = false) {
    if (int rc = validate_desc(desc); rc != SSM_OK) return rc;
    const ssm_scan_desc d = *desc;
    const int cw = d.conv_width;
    if (cw > 0 && dconv_weight == nullptr) return SSM_ERR_NULL;
    if (cw == 0) dconv_weight = dconv_bias = nullptr;
    if (d.batch == 0 || d.dim == 0) return SSM_OK;
    const int es = d.dtype == SSM_BF16 ? 2 : 4;
    const int64_t tok = d.batch * d.seqlen * d.dim;
    const int64_t bn = d.batch * d.seqlen * d.dstate;
    const int64_t state = d.batch * d.dim * d.dstate;
    const int64_t adn = d.dim * d.dstate;
    if (A == nullptr || dA == nullptr) return SSM_ERR_NULL;
    if (D != nullptr && dD == nullptr) return SSM_ERR_NULL;
    const float *dbias = d.delta_bias;
    if (dbias != nullptr && ddelta_bias == nullptr) return SSM_ERR_NULL;
    if (dbias == nullptr) ddelta_bias = nullptr;
    if (d.seqlen > 0 && (u == nullptr || delta == nullptr || B == nullptr || C == nullptr || dy == nullptr ||
                         du == nullptr || ddelta == nullptr || dB == nullptr || dC == nullptr ||
                         (z != nullptr && dz == nullptr)))
        return SSM_ERR_NULL;
    const void *tok_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, z ? dz : nullptr};
    for (const void *q : tok_ptrs)
        if (q && !aligned(q, es)) return SSM_ERR_ALIGN;
    const void *f32_ptrs[] = {A, D, h0, dh_last, dA, dB, dC, dD, dh0, ddelta_bias, dconv_weight, dconv_bias};
    for (const void *q : f32_ptrs)
        if (q && !aligned(q, 4)) return SSM_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return SSM_ERR_ALIGN;

    const BwdLayout wl = bwd_layout(d);
    if (!plan_supported(wl.pl)) return SSM_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace_bytes(d);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SSM_ERR_WORKSPACE;

    const int64_t tk = d.seqlen > 0 ? tok : 0;
    const Range outs[] = {range_of(du, tk * es), range_of(ddelta, tk * es), range_of(z ? dz : nullptr, tk * es),
                          range_of(dA, adn * 4), range_of(dB, d.seqlen > 0 ? bn * 4 : 0),
                          range_of(dC, d.seqlen > 0 ? bn * 4 : 0), range_of(D ? dD : nullptr, d.dim * 4),
                          range_of(dh0, state * 4), range_of(ddelta_bias, d.dim * 4),
                          range_of(dconv_weight, (int64_t)d.dim * cw * 4), range_of(dconv_bias, d.dim * 4),
                          range_of(workspace, (int64_t)need)};
    const Range ins[] = {range_of(u, tok * es), range_of(delta, tok * es), range_of(z, z ? tok * es : 0),
                         range_of(B, bn * es), range_of(C, bn * es), range_of(A, adn * 4),
                         range_of(D, D ? d.dim * 4 : 0), range_of(h0, h0 ? state * 4 : 0),
                         range_of(dy, tok * es), range_of(dh_last, dh_last ? state * 4 : 0),
                         range_of(dbias, dbias ? d.dim * 4 : 0),
                         range_of(d.conv_weight, (int64_t)d.dim * cw * 4),
                         range_of(d.conv_bias, cw > 0 && d.conv_bias ? d.dim * 4 : 0)};
    const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int i = 0; i < nout; ++i) {
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return SSM_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
    }

    if (d.seqlen == 0) {
        // no tokens: dA = dD = 0, dh0 = dh_last (or 0)
        hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((adn + 255) / 256)), dim3(256), 0, stream,
                           nullptr, dA, adn);
        if (D != nullptr)
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((d.dim + 255) / 256)), dim3(256), 0, stream,
                               nullptr, dD, d.dim);
        if (dh0 != nullptr)
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((state + 255) / 256)), dim3(256), 0, stream,
                               dh_last, dh0, state);
        if (ddelta_bias != nullptr)
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((d.dim + 255) / 256)), dim3(256), 0, stream,
                               nullptr, ddelta_bias, d.dim);
        if (dconv_weight != nullptr)
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((d.dim * cw + 255) / 256)), dim3(256), 0, stream,
                               nullptr, dconv_weight, d.dim * cw);
        if (dconv_bias != nullptr)
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((d.dim + 255) / 256)), dim3(256), 0, stream,
                               nullptr, dconv_bias, d.dim);
        return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }

    char *ws = static_cast<char *>(workspace);
    // with the convolution prologue the scan's backward runs on its output u,
    // materialised in the workspace, and writes the gradient of u there; the
    // caller's u holds x and its du receives the gradient of x
    const void *x_in = u;
    void *dx_out = du;
    // channels per thread of the convolution kernels: 4-channel pieces when
    // they are whole and aligned (the workspace's u and du always are)
    const int cpt = (d.dim % 4 == 0 && aligned(x_in, 4 * es) && aligned(dx_out, 4 * es)) ? 4 : 1;
    ConvParams cp{};
    // a forward that kept the checkpoints has left u in fp32 here
    const bool u_saved = saved && cw > 0;
    // grids, checked before anything is launched: the checkpoint pass's blocks,
    // conv_bwd_kernel's 256-token blocks (grid y)
    if ((int64_t)wl.ntiles * d.batch * wl.pl.S > INT32_MAX) return SSM_ERR_SHAPE;
    if (cw > 0 && wl.nblk > 65535) return SSM_ERR_SHAPE;
    if (cw > 0) {
        cp.x = x_in;
        cp.w = d.conv_weight;
        cp.cb = d.conv_bias;
        cp.u = ws + wl.conv_u;
        cp.du = reinterpret_cast<const float *>(ws + wl.conv_du);
        cp.dx = dx_out;
        cp.part_w = reinterpret_cast<float *>(ws + wl.conv_pw);
        cp.part_b = reinterpret_cast<float *>(ws + wl.conv_pb);
        cp.dw = dconv_weight;
        cp.db = dconv_bias;
        cp.L = d.seqlen;
        cp.batch = (int)d.batch;
        cp.dim = (int)d.dim;
        cp.W = cw;
        cp.nblk = wl.nblk;
        if (!u_saved && launch_conv_silu(cp, d.dtype == SSM_BF16, cpt, stream) != hipSuccess) return SSM_ERR_HIP;
    }
    const bool vec = (d.dim % 4 == 0) && aligned(u, 4 * es) && aligned(delta, 4 * es) && (!z || aligned(z, 4 * es)) &&
                     aligned(dy, 4 * es) && aligned(du, 4 * es) && aligned(ddelta, 4 * es) &&
                     (!z || aligned(dz, 4 * es));
    // 1. checkpoints: the forward scan in its checkpoint mode (segment-parallel).
    // With the prologue it reads the u materialised above (fp32)
    ScanParams p{};
    p.u = cw > 0 ? cp.u : u; p.delta = delta; p.z = z; p.B = B; p.C = C;
    p.u_f32 = cw > 0 && d.dtype == SSM_BF16;
    p.delta_bias = dbias; p.delta_softplus = d.delta_softplus;
    p.A = A; p.D = D; p.h0 = h0;
    p.L = d.seqlen;
    p.batch = (int)d.batch;
    p.dim = (int)d.dim;
    p.N = (int)d.dstate;
    p.seg_len = wl.pl.seg_len;
    p.nseg = wl.pl.S;
    p.ntiles = wl.ntiles;
    p.vec = vec;
    p.ckpt = reinterpret_cast<float *>(ws + wl.ckpt);
    p.nck = wl.nck;
    {
        const WorkspaceLayout fl = workspace_layout(d.batch, d.seqlen, d.dim, d.dstate, wl.pl);
        p.Bf = reinterpret_cast<float *>(ws + fl.bf);
        p.Cf = reinterpret_cast<float *>(ws + fl.cf);
        if (wl.pl.S > 1) {
            p.agg_P = reinterpret_cast<float *>(ws + fl.agg_p);
            p.agg_H = reinterpret_cast<float *>(ws + fl.agg_h);
            p.seg_h = reinterpret_cast<float *>(ws + fl.seg_h);
        }
    }
    const int64_t blocks_per_seg = (int64_t)wl.ntiles * d.batch;
    const int64_t nm = blocks_per_seg * wl.pl.S;
    const int64_t na = wl.pl.S > 1 ? blocks_per_seg * (wl.pl.S - 1) : 0;
    const bool zoh = d.disc == SSM_DISC_ZOH;
    hipError_t e = hipSuccess;
    // (a forward that kept the checkpoints has left them, and the regrouped B
    // and C, in this workspace)
    if (!saved && launch_scan(d, wl.pl, p, (int)nm, (int)na, stream) != hipSuccess) return SSM_ERR_HIP;

    // 2. the reverse pass
    BwdParams bp{};
    bp.u = cw > 0 ? cp.u : u; bp.delta = delta; bp.z = z; bp.dy = dy;
    bp.u_f32 = cw > 0;
    bp.delta_bias = dbias; bp.delta_softplus = d.delta_softplus;
    bp.A = A; bp.D = D; bp.dh_last = dh_last;
    bp.Bf = p.Bf; bp.Cf = p.Cf; bp.ckpt = p.ckpt;
    bp.du = du; bp.ddelta = ddelta; bp.dz = dz; bp.dh0 = dh0;
    // with the prologue the gradient of u stays fp32 for the prologue's backward:
    // dx sums W products of it, which cancel, so its bf16 rounding would show
    bp.du_f32 = cw > 0 ? reinterpret_cast<float *>(ws + wl.conv_du) : nullptr;
    bp.part_bc = reinterpret_cast<float *>(ws + wl.part_bc);
    bp.part_a = reinterpret_cast<float *>(ws + wl.part_a);
    bp.part_d = reinterpret_cast<float *>(ws + wl.part_d);
    bp.part_db = dbias ? reinterpret_cast<float *>(ws + wl.part_db) : nullptr;
    bp.L = d.seqlen;
    bp.batch = (int)d.batch;
    bp.dim = (int)d.dim;
    bp.N = (int)d.dstate;
    bp.ntiles = wl.ntiles;
    bp.nck = wl.nck;
    bp.vec = vec;
    if (d.dtype == SSM_BF16)
        e = zoh ? launch_bwd_bf16_zoh(wl.sh, bp, stream) : launch_bwd_bf16_euler(wl.sh, bp, stream);
    else
        e = zoh ? launch_bwd_f32_zoh(wl.sh, bp, stream) : launch_bwd_f32_euler(wl.sh, bp, stream);
    if (e != hipSuccess) return SSM_ERR_HIP;

    // 3. sums of the partials
    BwdReduceParams rp{};
    rp.part_bc = bp.part_bc; rp.part_a = bp.part_a; rp.part_d = bp.part_d; rp.part_db = bp.part_db;
    rp.dB = dB; rp.dC = dC; rp.dA = dA; rp.dD = D ? dD : nullptr; rp.ddelta_bias = ddelta_bias;
    rp.L = d.seqlen;
    rp.batch = (int)d.batch;
    rp.dim = (int)d.dim;
    rp.N = (int)d.dstate;
    rp.npad = wl.sh.npad;
    rp.ntiles = wl.ntiles;
    e = launch_bwd_reduce(rp, stream);
    if (e != hipSuccess) return SSM_ERR_HIP;

    // 4. the convolution prologue: dx, and the sums of the tap and bias gradients
    if (cw > 0 && launch_conv_bwd(cp, d.dtype == SSM_BF16, cpt, stream) != hipSuccess) return SSM_ERR_HIP;
    return SSM_OK;
}

// ---------------------------------------------------------------------------
// The no-allocation forward's scratch: one fixed device array, held by every
// GPU the library's module is loaded on until the process ends. Host code never
// passes `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol); it passes the device address looked up once per GPU below.

static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

// The device address of `scratch` on the GPU that owns `stream` (the current
// device for the null stream), looked up with that GPU current on the first
// call for it.
int scratch_address(hipStream_t stream, void **out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SSM_ERR_HIP;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return SSM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return SSM_ERR_HIP;
        void *addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return SSM_ERR_HIP;
        if (e != hipSuccess || addr == nullptr) return SSM_ERR_HIP;
        g_scratch_addr[dev] = addr;
    }
    *out = g_scratch_addr[dev];
    return SSM_OK;
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

extern "C" int ssm_scan_fwd_noalloc(const ssm_scan_desc *desc, const void *u, const void *delta,
                                    const float *A, const void *B, const void *C, const float *D,
                                    const void *z, const float *h0, void *y, float *h_last, hipStream_t stream) {
    if (int rc = validate_desc(desc); rc != SSM_OK) return rc;
    if (desc->batch == 0 || desc->dim == 0) return SSM_OK;
    // the size check comes before any HIP call
    const size_t need = workspace_bytes_for(*desc, make_plan(*desc, nullptr));
    if (need > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0)
        if (int rc = scratch_address(stream, &ws); rc != SSM_OK) return rc;
    return scan_impl(desc, u, delta, A, B, C, D, z, h0, y, h_last, ws, ws ? SSM_NOALLOC_SCRATCH_BYTES : 0, nullptr,
                     stream);
}

extern "C" int ssm_scan_fwd_save(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
                                 const void *B, const void *C, const float *D, const void *z, const float *h0,
                                 void *y, float *h_last, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (int rc = validate_desc(desc); rc != SSM_OK) return rc;
    if (desc->batch == 0 || desc->dim == 0 || desc->seqlen == 0)   // nothing for a backward to reuse
        return scan_impl(desc, u, delta, A, B, C, D, z, h0, y, h_last, workspace, workspace_bytes, nullptr, stream);
    // the backward's launch shape, so that its checkpoints are the ones this pass passes through
    const BwdLayout wl = bwd_layout(*desc);
    const ssm_scan_tuning t{wl.sh.G, 0};
    const SaveForBwd sv{wl.total, wl.ckpt, wl.nck, wl.conv_u};
    return scan_impl(desc, u, delta, A, B, C, D, z, h0, y, h_last, workspace, workspace_bytes, &t, stream, &sv);
}

extern "C" int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int32_t dtype, int32_t disc,
                                const void *x, const void *delta, const float *delta_bias,
                                int32_t delta_softplus, const float *A, const void *B,
                                const void *C, const float *D, const void *z, float *h, void *y,
                                hipStream_t stream) {
    if (batch < 0 || dim < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (disc != SSM_DISC_EULER && disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (dstate < 1 || dstate > 64) return SSM_ERR_UNSUPPORTED;
    if (delta_softplus != 0 && delta_softplus != 1) return SSM_ERR_UNSUPPORTED;
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
    if (!aligned(A, 4) || !aligned(h, 4) || (D && !aligned(D, 4)) || (delta_bias && !aligned(delta_bias, 4)))
        return SSM_ERR_ALIGN;
    const Range r_y = range_of(y, ch * es);
    const Range r_h = range_of(h, st * 4);
    const Range inputs[] = {range_of(x, ch * es), range_of(delta, ch * es), range_of(z, z ? ch * es : 0),
                            range_of(B, batch * dstate * es), range_of(C, batch * dstate * es),
                            range_of(A, dim * dstate * 4), range_of(D, D ? dim * 4 : 0),
                            range_of(delta_bias, delta_bias ? dim * 4 : 0)};
    for (const Range &r : inputs)
        if (overlaps(r_y, r) || overlaps(r_h, r)) return SSM_ERR_ALIAS;
    if (overlaps(r_y, r_h)) return SSM_ERR_ALIAS;

    DecodeParams p{};
    p.x = x; p.delta = delta; p.z = z; p.B = B; p.C = C;
    p.delta_bias = delta_bias; p.delta_softplus = delta_softplus;
    p.A = A; p.D = D; p.h = h; p.y = y;
    p.batch = (int)batch;
    p.dim = (int)dim;
    p.N = (int)dstate;
    p.vec4 = (dstate % 4 == 0) && aligned(h, 16) && aligned(A, 16);
    p.bc4 = (dstate % 4 == 0) && aligned(B, 4 * es) && aligned(C, 4 * es);
    hipError_t e;
    if (dtype == SSM_BF16)
        e = disc == SSM_DISC_ZOH ? launch_decode<uint16_t, true>(p, stream) : launch_decode<uint16_t, false>(p, stream);
    else
        e = disc == SSM_DISC_ZOH ? launch_decode<float, true>(p, stream) : launch_decode<float, false>(p, stream);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" size_t ssm_scan_bwd_workspace_size(const ssm_scan_desc *desc) {
    if (validate_desc(desc) != SSM_OK) return 0;
    return bwd_workspace_bytes(*desc);
}

extern "C" int ssm_scan_bwd(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
                            const void *B, const void *C, const float *D, const void *z, const float *h0,
                            const void *dy, const float *dh_last, void *du, void *ddelta, float *dA, float *dB,
                            float *dC, float *dD, void *dz, float *dh0, float *ddelta_bias, float *dconv_weight,
                            float *dconv_bias, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(desc, u, delta, A, B, C, D, z, h0, dy, dh_last, du, ddelta, dA, dB, dC, dD, dz, dh0,
                    ddelta_bias, dconv_weight, dconv_bias, workspace, workspace_bytes, stream);
}

extern "C" int ssm_scan_bwd_saved(const ssm_scan_desc *desc, const void *u, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z, const float *h0,
                                  const void *dy, const float *dh_last, void *du, void *ddelta, float *dA, float *dB,
                                  float *dC, float *dD, void *dz, float *dh0, float *ddelta_bias, float *dconv_weight,
                                  float *dconv_bias, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(desc, u, delta, A, B, C, D, z, h0, dy, dh_last, du, ddelta, dA, dB, dC, dD, dz, dh0,
                    ddelta_bias, dconv_weight, dconv_bias, workspace, workspace_bytes, stream, true);
}

extern "C" int ssm_ssd_fwd(const ssm_ssd_desc *desc, const void *x, const void *dt, const float *A,
                           const void *B, const void *C, const float *D, const void *z, const float *h0,
                           void *y, float *h_last, hipStream_t stream) {
    if (desc == nullptr) return SSM_ERR_NULL;
    const ssm_ssd_desc &d = *desc;
    if (d.batch < 0 || d.seqlen < 0 || d.nheads < 1 || d.ngroups < 1 || d.nheads % d.ngroups != 0)
        return SSM_ERR_SHAPE;
    if (d.dtype != SSM_F32 && d.dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d.dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
    if (d.disc != SSM_DISC_EULER && d.disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d.dt_softplus != 0 && d.dt_softplus != 1) return SSM_ERR_UNSUPPORTED;
    if (!ssd_shape_supported(d.headdim, d.dstate)) return SSM_ERR_UNSUPPORTED;
    const int64_t P = d.headdim, N = d.dstate, H = d.nheads, G = d.ngroups;
    int64_t bl, heads, tok_elems, bc_elems, st_elems;
    if (!mul_ok(d.batch, d.seqlen, &bl) || !mul_ok(d.batch, H, &heads) || !mul_ok(bl, H * P, &tok_elems) ||
        !mul_ok(bl, G * N, &bc_elems) || !mul_ok(heads, P * N * 4, &st_elems) || tok_elems > INT64_MAX / 4 ||
        heads > INT32_MAX || 64 * H * P > INT32_MAX || 64 * G * N > INT32_MAX)
        return SSM_ERR_SHAPE;
    st_elems /= 4;
    if (heads == 0) return SSM_OK;
    if (A == nullptr) return SSM_ERR_NULL;
    if (bl > 0 && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || y == nullptr))
        return SSM_ERR_NULL;
    // x, z, y, B, C move in 8- and 16-byte pieces, states in 16-byte pieces
    const void *wide[] = {x, z, y, B, C, h0, h_last};
    for (const void *q : wide)
        if (q && !aligned(q, 16)) return SSM_ERR_ALIGN;
    if (!aligned(dt, 2) || !aligned(A, 4) || (D && !aligned(D, 4)) || (d.dt_bias && !aligned(d.dt_bias, 4)))
        return SSM_ERR_ALIGN;
    const Range r_y = range_of(y, tok_elems * 2);
    const Range r_hl = range_of(h_last, h_last ? st_elems * 4 : 0);
    const Range inputs[] = {range_of(x, tok_elems * 2), range_of(z, z ? tok_elems * 2 : 0),
                            range_of(dt, bl * H * 2), range_of(B, bc_elems * 2), range_of(C, bc_elems * 2),
                            range_of(A, H * 4), range_of(D, D ? H * 4 : 0),
                            range_of(d.dt_bias, d.dt_bias ? H * 4 : 0), range_of(h0, h0 ? st_elems * 4 : 0)};
    const int n_in = (int)(sizeof(inputs) / sizeof(inputs[0]));
    for (int k = 0; k < n_in; ++k) {
        const Range &r = inputs[k];
        if (overlaps(r_y, r)) return SSM_ERR_ALIAS;
        // h_last may be h0 itself (the state continued in place): the last input
        const bool in_place = k == n_in - 1 && h_last == h0;
        if (overlaps(r_hl, r) && !in_place) return SSM_ERR_ALIAS;
    }
    if (overlaps(r_y, r_hl)) return SSM_ERR_ALIAS;
    if (bl == 0 && h_last == nullptr) return SSM_OK;

    SsdParams p{};
    p.x = static_cast<const uint16_t *>(x);
    p.dt = static_cast<const uint16_t *>(dt);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<const uint16_t *>(C);
    p.z = static_cast<const uint16_t *>(z);
    p.dt_bias = d.dt_bias;
    p.A = A;
    p.D = D;
    p.h0 = h0;
    p.y = static_cast<uint16_t *>(y);
    p.h_last = h_last;
    p.L = d.seqlen;
    p.batch = (int)d.batch;
    p.H = (int)H;
    p.G = (int)G;
    p.hpg = (int)(H / G);
    p.dt_softplus = d.dt_softplus;
    const hipError_t e = d.disc == SSM_DISC_ZOH ? launch_ssd_zoh(p, (int)P, (int)N, stream)
                                                : launch_ssd_euler(p, (int)P, (int)N, stream);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" int ssm_ssd_state_update(const ssm_ssd_desc *desc, const void *x, const void *dt, const float *A,
                                    const void *B, const void *C, const float *D, const void *z, float *h,
                                    void *y, hipStream_t stream) {
    if (desc == nullptr) return SSM_ERR_NULL;
    const ssm_ssd_desc &d = *desc;
    if (d.batch < 0 || d.seqlen != 1 || d.nheads < 1 || d.ngroups < 1 || d.nheads % d.ngroups != 0)
        return SSM_ERR_SHAPE;
    if (d.dtype != SSM_F32 && d.dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d.dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
    if (d.disc != SSM_DISC_EULER && d.disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
    if (d.dt_softplus != 0 && d.dt_softplus != 1) return SSM_ERR_UNSUPPORTED;
    if (!ssd_shape_supported(d.headdim, d.dstate)) return SSM_ERR_UNSUPPORTED;
    const int64_t P = d.headdim, N = d.dstate, H = d.nheads, G = d.ngroups;
    int64_t heads, rows, st_elems;
    if (!mul_ok(d.batch, H, &heads) || !mul_ok(heads, P, &rows) || !mul_ok(rows, N * 4, &st_elems) ||
        heads > INT32_MAX)
        return SSM_ERR_SHAPE;
    st_elems /= 4;
    if (heads == 0) return SSM_OK;
    if (A == nullptr || x == nullptr || dt == nullptr || B == nullptr || C == nullptr || h == nullptr ||
        y == nullptr)
        return SSM_ERR_NULL;
    // states move in 16-byte pieces, B and C in 8-byte ones
    if (!aligned(h, 16) || !aligned(B, 8) || !aligned(C, 8) || !aligned(x, 2) || (z && !aligned(z, 2)) ||
        !aligned(y, 2) || !aligned(dt, 2) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
        (d.dt_bias && !aligned(d.dt_bias, 4)))
        return SSM_ERR_ALIGN;
    const int64_t bcn = d.batch * G * N;
    const Range r_y = range_of(y, rows * 2);
    const Range r_h = range_of(h, st_elems * 4);
    const Range inputs[] = {range_of(x, rows * 2), range_of(z, z ? rows * 2 : 0), range_of(dt, heads * 2),
                            range_of(B, bcn * 2), range_of(C, bcn * 2), range_of(A, H * 4),
                            range_of(D, D ? H * 4 : 0), range_of(d.dt_bias, d.dt_bias ? H * 4 : 0)};
    for (const Range &r : inputs)
        if (overlaps(r_y, r) || overlaps(r_h, r)) return SSM_ERR_ALIAS;
    if (overlaps(r_y, r_h)) return SSM_ERR_ALIAS;

    SsdDecodeParams p{};
    p.x = static_cast<const uint16_t *>(x);
    p.dt = static_cast<const uint16_t *>(dt);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<const uint16_t *>(C);
    p.z = static_cast<const uint16_t *>(z);
    p.dt_bias = d.dt_bias;
    p.A = A;
    p.D = D;
    p.h = h;
    p.y = static_cast<uint16_t *>(y);
    p.rows = rows;
    p.H = (int)H;
    p.G = (int)G;
    p.hpg = (int)(H / G);
    p.P = (int)P;
    p.N = (int)N;
    p.dt_softplus = d.dt_softplus;
    const int64_t threads = rows * (N / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) return SSM_ERR_SHAPE;
    if (d.disc == SSM_DISC_ZOH)
        hipLaunchKernelGGL((ssd_decode_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((ssd_decode_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" const char *ssm_status_string(int status) {
    switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid or too large sizes";
    case SSM_ERR_DTYPE: return "unknown element type";
    case SSM_ERR_UNSUPPORTED: return "unsupported dstate, head size, element type, discretisation or launch shape";
    case SSM_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "the HIP runtime refused a kernel launch";
    case SSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SSM_ERR_SCRATCH: return "the problem needs more scratch than the no-allocation forward's fixed buffer "
                                 "(SSM_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
    }
}

namespace ssm_detail {
hipError_t launch_bwd_reduce(const BwdReduceParams &p, hipStream_t st) {
    const int64_t n = (int64_t)p.batch * p.L * p.N + (int64_t)p.dim * p.N + p.dim;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}
}  // namespace ssm_detail
