// Backward of the selective scan on gfx950: the reverse pass that turns the
// gradient of y (and of the final state) into gradients of u, delta, A, B, C,
// D, z and h0, recomputing the states instead of reading stored ones.
//
// Math (per channel; lam_t = dloss/dh_t, the adjoint state, walked backwards;
// g(z) = z*sigmoid(z); s_t = sum_n C_t[n] h_t[n] + D u_t):
//   ds_t  = dy_t g(z_t),  dz_t = dy_t s_t g'(z_t),  dD += ds_t u_t,  du_t += D ds_t
//   lam_t = C_t ds_t + a_{t+1} lam_{t+1}     (dh_last joins at t = L-1)
//   da_t  = lam_t h_{t-1}:  ddelta_t += da_t a_t A,  dA += da_t a_t delta_t
//   simplified input term delta B u: ddelta_t += u sum_n lam B, du_t += delta sum_n lam B,
//                                    dB_t[n] += sum_d lam delta u
//   hold input term f B u, f = expm1(delta A)/A: ddelta_t += sum_n lam a B u,
//                    du_t += sum_n lam f B, dB_t[n] += sum_d lam f u,
//                    dA += lam (delta a - f)/A B u   (A -> 0: delta^2/2)
//   dC_t[n] = sum_d ds_t h_t[n],  dh0 = a_0 lam_0.
// (The backward that recomputes the discretised states on chip rather than
// storing them: doyouknow.kr "Mamba와 상태 공간 모델(SSM)의 부상 완벽 가이드"
// §3-3.)
//
// Kernel design:
//  * A checkpoint pass (the forward scan kernel in its checkpoint mode, with
//    the usual segment carry) writes the state at the start of every chunk of
//    TC tokens: (batch, chunks, Npad, dim) fp32.
//  * The reverse kernel keeps the forward's layout: a workgroup is a 64-channel
//    tile of one batch row with G waves, wave w owning NPW states; lane =
//    channel. It walks the chunks from last to first. Per chunk:
//      1. every thread stages a piece of the chunk into LDS: (delta, x) pairs
//         (x = delta*u, or u for the hold rule) and ds = dy g(z); it keeps
//         delta, u, ds and dy g'(z) in registers for its outputs;
//      2. each wave recomputes its states over the chunk from the checkpoint
//         (h_t, and the decay a_t when NPW <= 2, in registers) and writes its
//         part of s_t to an LDS plane;
//      3. each thread sums the planes of its piece: dz = dy g'(z) s;
//      4. each wave runs the adjoint over the chunk in reverse, writing its
//         parts of sum_n lam B (or lam f B) and of the delta gradient to two
//         planes, and the chunk's dB, dC terms reduced over its 64 channels
//         (DPP row shifts and row broadcasts) to LDS;
//      5. each thread finalizes du and ddelta of its piece; the tile's dB, dC
//         sums of the chunk go to a per-tile partial buffer.
//    dA and dD are accumulated per lane and written per batch row at the end.
//  * A reduction kernel adds the per-tile dB, dC partials and the per-row dA,
//    dD partials in a fixed order, so the result does not depend on timing.
#pragma once

#include <type_traits>

#include "scan_kernels.hpp"

namespace ssm_detail {

struct BwdParams {
    const void *u, *delta, *z, *dy;
    const float *delta_bias;   // as in ScanParams
    int delta_softplus;
    const float *A, *D, *dh_last;
    const float *Bf, *Cf;      // the checkpoint pass's regrouped B and C (same groups as here)
    const float *ckpt;         // (batch, nck, Npad, dim)
    void *du, *ddelta, *dz;
    float *du_f32;             // if set, du is written here in fp32 instead (the convolution prologue's input)
    int u_f32;                 // u is fp32 (the convolution prologue's output) whatever the tensors' type
    float *dh0;
    float *part_bc;            // (batch, ntiles, L, Npad, 2): per-tile sums over channels of dB, dC terms
    float *part_a;             // (batch, dim, Npad): per-row dA
    float *part_d;             // (batch, dim): per-row dD
    float *part_db;            // (batch, dim): per-row delta-bias gradient (with a bias)
    int64_t L;
    int batch, dim, N, ntiles, nck;
    int vec;                   // u, delta, z, dy, du, ddelta, dz move 2 or 4 channels per aligned access
};

struct BwdReduceParams {
    const float *part_bc, *part_a, *part_d, *part_db;
    float *dB, *dC, *dA, *dD, *ddelta_bias;
    int64_t L;
    int batch, dim, N, npad, ntiles;
};

// Backward launch shape: (padded states, waves per tile, chunk length); the
// checkpoint pass uses the same (npad, G), so its regrouped B and C serve both.
struct BwdShape {
    int npad, G, TC;
};

inline BwdShape bwd_shape(int npad) {
    switch (npad) {
    case 4: return {4, 2, 16};
    case 8: return {8, 8, 16};
    case 16: return {16, 8, 16};
    case 32: return {32, 16, 8};
    default: return {64, 16, 8};
    }
}

hipError_t launch_bwd_bf16_euler(const BwdShape &sh, const BwdParams &p, hipStream_t st);
hipError_t launch_bwd_bf16_zoh(const BwdShape &sh, const BwdParams &p, hipStream_t st);
hipError_t launch_bwd_f32_euler(const BwdShape &sh, const BwdParams &p, hipStream_t st);
hipError_t launch_bwd_f32_zoh(const BwdShape &sh, const BwdParams &p, hipStream_t st);
hipError_t launch_bwd_reduce(const BwdReduceParams &p, hipStream_t st);

}  // namespace ssm_detail

#ifdef SSM_BWD_INSTANTIATE
namespace ssm_detail {
namespace {

// Sums of four values a, b, c, d over the 64 lanes of the wave, as a
// transposing reduction in which gfx950's lane swaps do the exchanges:
//  * v_permlane32_swap of (a, c) and of (b, d), then an add: the lower half of
//    the wave holds a (b) summed over both halves, the upper half c (d);
//  * v_permlane16_swap of those two, then an add: row k of the wave (16 lanes)
//    holds value k (a, b, c, d) summed over all four rows;
//  * an inclusive scan inside each row (DPP row shifts by 1, 2, 4, 8) leaves
//    the row's total in its last lane.
// The sums end in lanes 15 (a), 31 (b), 47 (c) and 63 (d): 10 VALU
// instructions, no LDS. The s_nops give every DPP read the two wait states
// it needs after the write it depends on.
__device__ __forceinline__ float wave_sum4_transposed(float a, float b, float c, float d) {
    const auto ac = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
    const auto bd = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(d), false, false);
    const float x = __uint_as_float(ac[0]) + __uint_as_float(ac[1]);   // lower half: a, upper half: c
    const float y = __uint_as_float(bd[0]) + __uint_as_float(bd[1]);   // lower half: b, upper half: d
    const auto xy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    float s = __uint_as_float(xy[0]) + __uint_as_float(xy[1]);          // row k: value k
    asm volatile(
        "s_nop 1\n\t"
        "v_add_f32_dpp %[s], %[s], %[s] row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %[s], %[s], %[s] row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %[s], %[s], %[s] row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %[s], %[s], %[s] row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        : [s] "+v"(s));
    return s;
}

template <int KV> struct BwdFloats;
template <> struct BwdFloats<2> { typedef float2 type; };
template <> struct BwdFloats<4> { typedef float4 type; };

// UF: u is read as fp32 whatever T is (the convolution prologue's output,
// formed in fp32 like the forward forms it)
// FEAT: the step options (delta bias, softplus) are compiled in; without it
// the kernel carries none of their registers
template <typename T, int NPW, int G, int TC, bool ZOH, bool UF = false, bool FEAT = true>
struct BwdKernel {
    static constexpr int kThreads = kTile * G;
    static constexpr int kNP = NPW * G;
    static constexpr int kV = TC * kTile >= 4 * kThreads ? 4 : 2;   // channels per staged piece
    static constexpr int kWords = kV * (int)sizeof(T) / 4;
    static constexpr int kRowPieces = kTile / kV;
    static constexpr int kPieces = TC * kRowPieces;
    static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
    static constexpr int kRowStep = kThreads / kRowPieces;
    static_assert(kThreads % kRowPieces == 0, "a thread keeps the same channels in every piece");
    static_assert(TC <= kPadRows, "spare rows of the regrouped B and C");
    static constexpr bool kPacked = sizeof(T) == 2;
    static constexpr int kWPS = kPacked ? 1 : 2;
    static constexpr bool kKeepA = NPW == 1;
    // Otherwise the first state's decay of each token goes through the wave's
    // own slot of the second plane set, which holds nothing from the
    // recomputation until the reverse step overwrites it, token by token,
    // with that token's delta-gradient part (after reading the decay there).
    static constexpr bool kPlaneA = !kKeepA;
    // the hold rule's phi(delta A) of the chunk, kept from the recomputation for
    // the reverse step: the 8-wave hold-rule kernels run at 2 waves per SIMD
    // and have the registers for it
    static constexpr bool kKeepF = ZOH && G == 8;
    static constexpr int kRed = (2 * NPW + 3) / 4 * 4;             // reduced values per step, in 4s
    // bf16 B/C words of the whole chunk fit in 32 scalar registers: they are
    // requested before the barrier that opens the chunk, so that their
    // latency overlaps it, and held for both passes over the chunk
    static constexpr bool kPreBC = kPacked && TC * NPW <= 32;
    typedef typename Words<kWords>::type Raw;
    typedef typename BwdFloats<kV>::type VecF;

    struct __align__(16) Smem {
        float2 dx[TC][kTile];          // (delta, x)
        float ds[TC][kTile];           // dy g(z)
        float pl[2][G][TC][kTile];     // planes: s parts, then (lam B parts, delta-gradient parts)
        float red[TC][kNP][2];         // the tile's sums over channels of the dB and dC terms
    };
    static_assert(sizeof(Smem) <= 81920, "two workgroups per CU in 160 KiB of LDS");

    struct Prefetch {
        typename std::conditional<UF, VecF, Raw>::type u[kPPT];
        Raw dt[kPPT], z[kPPT], dy[kPPT];
    };
    struct Held {
        float dt[kPPT][kV], u[kPPT][kV], ds[kPPT][kV], gz[kPPT][kV];   // gz = dy g'(z)
        float sg[FEAT ? kPPT : 1][FEAT ? kV : 1];   // d step / d delta (sigmoid of the softplus argument, or 1)
    };

    __device__ static int piece_row(int j) { return threadIdx.x / kRowPieces + j * kRowStep; }
    __device__ static bool piece_in_chunk(int j) { return kPieces % kThreads == 0 || piece_row(j) < TC; }

    __device__ static Raw gather(const T *src, int c0, int dim, bool on) {
        uint32_t w[kWords];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                const uint32_t lo = (on && c0 + 2 * i < dim) ? src[2 * i] : 0u;
                const uint32_t hi = (on && c0 + 2 * i + 1 < dim) ? src[2 * i + 1] : 0u;
                w[i] = lo | (hi << 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kWords; ++i) w[i] = (on && c0 + i < dim) ? __float_as_uint(src[i]) : 0u;
        }
        Raw r;
        make_words(r, w);
        return r;
    }

    __device__ static void unpack(const Raw &r, float (&v)[kV]) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) {
            const uint32_t x = word<kWords>(r, i);
            if constexpr (sizeof(T) == 2) {
                v[2 * i] = __uint_as_float(x << 16);
                v[2 * i + 1] = __uint_as_float(x & 0xffff0000u);
            } else {
                v[i] = __uint_as_float(x);
            }
        }
    }

    __device__ static void store(T *dst, const float (&o)[kV], int c0, int dim, bool vec) {
        if constexpr (sizeof(T) == 2) {
            typedef float f2v __attribute__((ext_vector_type(2)));
            typedef __bf16 b2v __attribute__((ext_vector_type(2)));
            uint32_t w[kWords];
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                const f2v pr = {o[2 * i], o[2 * i + 1]};
                w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2v));
            }
            if (vec) {
                Raw r;
                make_words(r, w);
                *reinterpret_cast<Raw *>(dst) = r;
            } else {
#pragma unroll
                for (int e = 0; e < kV; ++e)
                    if (c0 + e < dim) dst[e] = (uint16_t)(e & 1 ? w[e / 2] >> 16 : w[e / 2] & 0xffffu);
            }
        } else {
            if (vec) {
                VecF v;
                float *pv = reinterpret_cast<float *>(&v);
#pragma unroll
                for (int e = 0; e < kV; ++e) pv[e] = o[e];
                *reinterpret_cast<VecF *>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < kV; ++e)
                    if (c0 + e < dim) dst[e] = o[e];
            }
        }
    }

    template <typename PP>
    __device__ static void load(const PP &p, Prefetch &pf, int64_t base, int tval, int col, int d0, bool colv) {
        const T *u = static_cast<const T *>(p.u) + base;
        const T *dt = static_cast<const T *>(p.delta) + base;
        const T *z = static_cast<const T *>(p.z) + base;
        const T *dy = static_cast<const T *>(p.dy) + base;
        const bool gate = p.z != nullptr;
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int row = piece_row(j);
            if (!piece_in_chunk(j) || row >= tval || !colv) continue;
            const uint32_t off = (uint32_t)row * (uint32_t)p.dim + (uint32_t)col;
            if constexpr (UF) {
                const float *uf = static_cast<const float *>(p.u) + base + off;
                if (p.vec) {
                    pf.u[j] = *reinterpret_cast<const VecF *>(uf);
                } else {
                    float *pv = reinterpret_cast<float *>(&pf.u[j]);
#pragma unroll
                    for (int e = 0; e < kV; ++e) pv[e] = d0 + col + e < p.dim ? uf[e] : 0.0f;
                }
            }
            if (p.vec) {
                if constexpr (!UF) pf.u[j] = *reinterpret_cast<const Raw *>(u + off);
                pf.dt[j] = *reinterpret_cast<const Raw *>(dt + off);
                pf.dy[j] = *reinterpret_cast<const Raw *>(dy + off);
                if (gate) pf.z[j] = *reinterpret_cast<const Raw *>(z + off);
            } else {
                if constexpr (!UF) pf.u[j] = gather(u + off, d0 + col, p.dim, true);
                pf.dt[j] = gather(dt + off, d0 + col, p.dim, true);
                pf.dy[j] = gather(dy + off, d0 + col, p.dim, true);
                pf.z[j] = gather(z + off, d0 + col, p.dim, gate);
            }
        }
    }

    // Stage one chunk; rows past tval (and channels past dim) become delta = 0,
    // x = 0, ds = 0: a step that changes neither the state nor any stored
    // gradient.
    __device__ static void commit(const Prefetch &pf, Smem &s, Held &held, float (&dDacc)[kPPT][kV], int tval,
                                  int col, bool colv, bool gate, const float (&dbk)[kV], int prep) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int row = piece_row(j);
            if (!piece_in_chunk(j)) continue;
            float4 *dxp = reinterpret_cast<float4 *>(&s.dx[row][col]);
            VecF *dsp = reinterpret_cast<VecF *>(&s.ds[row][col]);
            float dsv[kV];
            if (row < tval && colv) {
                float u[kV], d[kV], g[kV];
                if constexpr (UF) {
                    const float *pv = reinterpret_cast<const float *>(&pf.u[j]);
#pragma unroll
                    for (int e = 0; e < kV; ++e) u[e] = pv[e];
                } else {
                    unpack(pf.u[j], u);
                }
                unpack(pf.dt[j], d);
                unpack(pf.dy[j], g);
#pragma unroll
                for (int e = 0; e < kV; ++e) {
                    if constexpr (!FEAT) continue;
                    held.sg[j][e] = 1.0f;
                    if (prep == 2) {
                        const float xs = d[e] + dbk[e];
                        d[e] = softplus_f(xs);
                        held.sg[j][e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-xs * kLog2e));
                    } else if (prep == 1) {
                        d[e] += dbk[e];
                    }
                }
                if (gate) {
                    float z[kV];
                    unpack(pf.z[j], z);
#pragma unroll
                    for (int e = 0; e < kV; ++e) {
                        // sigmoid, silu and its derivative sigmoid (1 + z (1 - sigmoid))
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z[e] * kLog2e));
                        held.gz[j][e] = g[e] * sg * (1.0f + z[e] * (1.0f - sg));
                        dsv[e] = g[e] * z[e] * sg;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < kV; ++e) {
                        held.gz[j][e] = 0.0f;
                        dsv[e] = g[e];
                    }
                }
#pragma unroll
                for (int e = 0; e < kV; e += 2)
                    dxp[e / 2] = make_float4(d[e], ZOH ? u[e] : d[e] * u[e], d[e + 1], ZOH ? u[e + 1] : d[e + 1] * u[e + 1]);
#pragma unroll
                for (int e = 0; e < kV; ++e) {
                    held.dt[j][e] = d[e];
                    held.u[j][e] = u[e];
                    held.ds[j][e] = dsv[e];
                    dDacc[j][e] = fmaf(dsv[e], u[e], dDacc[j][e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < kV; e += 2) dxp[e / 2] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                for (int e = 0; e < kV; ++e) dsv[e] = 0.0f;
            }
            VecF v;
            float *pv = reinterpret_cast<float *>(&v);
#pragma unroll
            for (int e = 0; e < kV; ++e) pv[e] = dsv[e];
            *dsp = v;
        }
    }

    // sum over the G planes of plane set `k` at (row, col .. col + kV)
    // (from the first plane on, not from 0.0f + the first: the compiler keeps
    // that add, since it turns a -0.0f into +0.0f)
    __device__ static void plane_sum(const Smem &s, int k, int row, int col, float (&acc)[kV]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const VecF v = *reinterpret_cast<const VecF *>(&s.pl[k][g][row][col]);
            const float *pv = reinterpret_cast<const float *>(&v);
#pragma unroll
            for (int e = 0; e < kV; ++e) acc[e] = g == 0 ? pv[e] : acc[e] + pv[e];
        }
    }

    // The same kernel arguments through an address the compiler cannot see
    // through: what is read from it is loaded again where it is used (one
    // scalar load from the argument segment) instead of being held in scalar
    // registers across the chunk loop, which would spill them.
    typedef const __attribute__((address_space(4))) BwdParams KernArgs;
    __device__ static KernArgs &fresh() {
        KernArgs *q = (KernArgs *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(q));
        return *q;
    }

    __device__ static void run(const BwdParams &p) {
        __shared__ Smem s;
        // workgroup -> (batch row, tile); the tiles of a batch row run on one XCD
        int b, tile;
        {
            const int nb = gridDim.x;
            const int bid = blockIdx.x;
            const int q = nb / kXcds, r = nb % kXcds;
            const int x = bid % kXcds;
            const int logical = x * q + min(x, r) + bid / kXcds;
            tile = logical % p.ntiles;
            b = logical / p.ntiles;
        }
        const int lane = threadIdx.x & (kTile - 1);
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kTile);
        const int d0 = tile * kTile;
        const int d = d0 + lane;
        const bool dval = d < p.dim;
        const int dc = dval ? d : p.dim - 1;
        const bool gate = p.z != nullptr;

        float A[NPW], A2[NPW], Ainv[NPW], mu[NPW], dA[NPW];
#pragma unroll
        for (int q = 0; q < NPW; ++q) {
            const int n = w * NPW + q;
            const bool nv = n < p.N;
            A[q] = nv ? p.A[(int64_t)dc * p.N + n] : 0.0f;
            A2[q] = A[q] * kLog2e;
            Ainv[q] = A[q] != 0.0f ? 1.0f / A[q] : 0.0f;
            mu[q] = (nv && p.dh_last != nullptr) ? p.dh_last[((int64_t)b * p.dim + dc) * p.N + n] : 0.0f;
            dA[q] = 0.0f;
        }
        const int col = (threadIdx.x % kRowPieces) * kV;
        const bool colv = d0 + col < p.dim;
        float Dk[kV], dbk[kV], dDacc[kPPT][kV], dbacc[kPPT][kV];
#pragma unroll
        for (int e = 0; e < kV; ++e) {
            Dk[e] = (p.D != nullptr && d0 + col + e < p.dim) ? p.D[d0 + col + e] : 0.0f;
            dbk[e] = (FEAT && p.delta_bias != nullptr && d0 + col + e < p.dim) ? p.delta_bias[d0 + col + e] : 0.0f;
        }
        const int prep = !FEAT ? 0 : p.delta_softplus ? 2 : (p.delta_bias != nullptr ? 1 : 0);
#pragma unroll
        for (int j = 0; j < kPPT; ++j)
#pragma unroll
            for (int e = 0; e < kV; ++e) dDacc[j][e] = dbacc[j][e] = 0.0f;

        const int nck = p.nck;                                  // chunks of this row, walked last to first
        const int64_t row0 = (int64_t)b * p.L;
        // every chunk but the last holds TC rows (a 32-bit compare on the
        // scalar unit, not a 64-bit one per chunk on the vector unit)
        const int last_rows = nck > 0 ? (int)(p.L - (int64_t)(nck - 1) * TC) : 0;
        auto rows_of = [&](int c) { return c == nck - 1 ? last_rows : TC; };
        const int64_t Lp = padded_len(p.L);
        cword *bw0 = (cword *)(p.Bf) + ((int64_t)b * G + w) * Lp * NPW;
        cword *cw0 = (cword *)(p.Cf) + ((int64_t)b * G + w) * Lp * NPW;
        auto ckpt_at = [&](int c, int q) {
            return fresh().ckpt[(((int64_t)b * nck + c) * kNP + w * NPW + q) * p.dim + dc];
        };

        Prefetch pf;
        Held held;
        float hnext[NPW];
        if (nck > 0) {
            const int c = nck - 1;
            load(p, pf, (row0 + (int64_t)c * TC) * p.dim + d0, rows_of(c), col, d0, colv);
#pragma unroll
            for (int q = 0; q < NPW; ++q) hnext[q] = ckpt_at(c, q);
        }

        for (int c = nck - 1; c >= 0; --c) {
            const int tval = rows_of(c);
            const int64_t t0 = (int64_t)c * TC;
            // 1. stage this chunk; prefetch the previous one and its checkpoint
            commit(pf, s, held, dDacc, tval, col, colv, gate, dbk, prep);
            float hstart[NPW];
#pragma unroll
            for (int q = 0; q < NPW; ++q) hstart[q] = hnext[q];
            if (c > 0) {
                load(fresh(), pf, (row0 + (int64_t)(c - 1) * TC) * p.dim + d0, rows_of(c - 1), col, d0, colv);
#pragma unroll
                for (int q = 0; q < NPW; ++q) hnext[q] = ckpt_at(c - 1, q);
            }
            cword *bw = bw0 + t0 * NPW;
            cword *cw = cw0 + t0 * NPW;
            uint32_t bcw[kPreBC ? TC : 1][kPreBC ? NPW : 1];
            if constexpr (kPreBC) {
                // the barrier, as __syncthreads() is, with the chunk's B and C
                // requested after the LDS writes have completed
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
#pragma unroll
                for (int t = 0; t < TC; ++t)
#pragma unroll
                    for (int q = 0; q < NPW; ++q) bcw[t][q] = bw[t * NPW + q];
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            } else {
                __syncthreads();
            }
            auto bc_word = [&](int t, int q) { return kPreBC ? bcw[kPreBC ? t : 0][kPreBC ? q : 0] : bw[t * NPW + q]; };

            // 2. recompute the chunk's states of this wave; parts of s_t. The
            // two arithmetic phases (this and 4) run at a higher issue
            // priority than the staging, dz and finalize phases, so that a
            // SIMD's VALU is fed from them first when its waves are in
            // different phases.
            __builtin_amdgcn_s_setprio(2);
            float hs[TC][NPW];
            float as[kKeepA ? TC : 1][NPW];
            float fs[kKeepF ? TC : 1][NPW];
            {
                float h[NPW];
#pragma unroll
                for (int q = 0; q < NPW; ++q) h[q] = hstart[q];
#pragma unroll
                for (int t = 0; t < TC; ++t) {
                    const float2 v = s.dx[t][lane];
                    float part = 0.0f;
#pragma unroll
                    for (int q = 0; q < NPW; ++q) {
                        const uint32_t wb = bc_word(t, q);
                        const float bq = __uint_as_float(kPacked ? wb << 16 : wb);
                        const float cq = __uint_as_float(kPacked ? wb & 0xffff0000u : cw[t * NPW + q]);
                        if constexpr (ZOH) {
                            const float a = __builtin_amdgcn_exp2f(v.x * A2[q]);
                            const float ph = expm1_over_x(v.x * A[q], a);
                            h[q] = fmaf(a, h[q], ph * (v.x * v.y * bq));
                            if constexpr (kKeepA) as[t][q] = a;
                            if constexpr (kPlaneA) if (q == 0) s.pl[1][w][t][lane] = a;
                            if constexpr (kKeepF) fs[t][q] = ph;
                        } else {
                            const float a = __builtin_amdgcn_exp2f(v.x * A2[q]);
                            h[q] = fmaf(a, h[q], v.y * bq);
                            if constexpr (kKeepA) as[t][q] = a;
                            if constexpr (kPlaneA) if (q == 0) s.pl[1][w][t][lane] = a;
                        }
                        hs[t][q] = h[q];
                        part = fmaf(cq, h[q], part);
                    }
                    s.pl[0][w][t][lane] = part;
                }
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();

            // 3. dz of this thread's pieces
#pragma unroll
            for (int j = 0; j < kPPT; ++j) {
                const int row = piece_row(j);
                if (!gate || !piece_in_chunk(j) || row >= tval || !colv) continue;
                float acc[kV], o[kV];
                plane_sum(s, 0, row, col, acc);
#pragma unroll
                for (int e = 0; e < kV; ++e) o[e] = held.gz[j][e] * (acc[e] + Dk[e] * held.u[j][e]);
                T *dst = static_cast<T *>(fresh().dz) + (row0 + t0 + row) * p.dim + d0 + col;
                store(dst, o, d0 + col, p.dim, p.vec);
            }
            __syncthreads();

            // 4. adjoint over the chunk in reverse
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int t = TC - 1; t >= 0; --t) {
                const float2 v = s.dx[t][lane];
                const float dsv = s.ds[t][lane];
                float pU = 0.0f, pD = 0.0f;
                float vr[kRed];                  // (dB term, dC term) per state, zero padded to 4s
#pragma unroll
                for (int i = 2 * NPW; i < kRed; ++i) vr[i] = 0.0f;
#pragma unroll
                for (int q = 0; q < NPW; ++q) {
                    const uint32_t wb = bc_word(t, q);
                    const float bq = __uint_as_float(kPacked ? wb << 16 : wb);
                    const float cq = __uint_as_float(kPacked ? wb & 0xffff0000u : cw[t * NPW + q]);
                    const float a = kKeepA                 ? as[t][q]
                                    : (kPlaneA && q == 0) ? s.pl[1][w][t][lane]
                                                          : __builtin_amdgcn_exp2f(v.x * A2[q]);
                    const float l = fmaf(cq, dsv, mu[q]);
                    const float al = a * l;                 // the adjoint passed back to t - 1
                    const float hp = t > 0 ? hs[t - 1][q] : hstart[q];
                    const float daa = al * hp;
                    pD = fmaf(daa, A[q], pD);
                    dA[q] = fmaf(daa, v.x, dA[q]);
                    float vb;
                    if constexpr (ZOH) {
                        // f = expm1(delta A)/A = delta phi(delta A)
                        const float xa = v.x * A[q];
                        const float f = v.x * (kKeepF ? fs[t][q] : expm1_over_x(xa, a));
                        // d f / d A = (delta a - f) / A, by its series near 0 (cancellation)
                        float dfdA;
                        if (fabsf(xa) < 0.125f)
                            dfdA = v.x * v.x *
                                   (0.5f + xa * (1.0f / 3.0f + xa * (0.125f + xa * (1.0f / 30.0f + xa * (1.0f / 144.0f)))));
                        else
                            dfdA = (v.x * a - f) * Ainv[q];
                        const float lbu = l * bq * v.y;
                        pU = fmaf(l * f, bq, pU);
                        pD = fmaf(lbu, a, pD);
                        dA[q] = fmaf(lbu, dfdA, dA[q]);
                        vb = l * f * v.y;
                    } else {
                        pU = fmaf(l, bq, pU);
                        vb = l * v.y;
                    }
                    vr[2 * q] = vb;
                    vr[2 * q + 1] = dsv * hs[t][q];
                    mu[q] = al;
                }
                // the chunk's dB, dC terms of this wave's states, summed over the 64
                // channels: values (dB q, dC q, dB q+1, dC q+1) land in lanes 15
                // (dB q), 31 (dC q), 47 (dB q+1), 63 (dC q+1)
#pragma unroll
                for (int i = 0; i < kRed; i += 4) {
                    const float sum = wave_sum4_transposed(vr[i], vr[i + 1], vr[i + 2], vr[i + 3]);
                    const int v = lane >> 4;
                    const int q = i / 2 + (v >> 1);
                    if ((lane & 15) == 15 && q < NPW) s.red[t][w * NPW + q][v & 1] = sum;
                }
                s.pl[0][w][t][lane] = pU;
                s.pl[1][w][t][lane] = pD;
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();

            // 5. du, ddelta of this thread's pieces; the tile's dB, dC sums
            KernArgs &po = fresh();
#pragma unroll
            for (int j = 0; j < kPPT; ++j) {
                const int row = piece_row(j);
                if (!piece_in_chunk(j) || row >= tval || !colv) continue;
                float su[kV], sd[kV], ou[kV], od[kV];
                plane_sum(s, 0, row, col, su);
                plane_sum(s, 1, row, col, sd);
#pragma unroll
                for (int e = 0; e < kV; ++e) {
                    if constexpr (ZOH) {
                        ou[e] = fmaf(Dk[e], held.ds[j][e], su[e]);
                        od[e] = sd[e];
                    } else {
                        ou[e] = fmaf(held.dt[j][e], su[e], Dk[e] * held.ds[j][e]);
                        od[e] = fmaf(held.u[j][e], su[e], sd[e]);
                    }
                    if constexpr (FEAT) {
                        od[e] *= held.sg[j][e];      // gradient of the raw delta
                        dbacc[j][e] += od[e];
                    }
                }
                const int64_t off = (row0 + t0 + row) * p.dim + d0 + col;
                if (po.du_f32 != nullptr) {
#pragma unroll
                    for (int e = 0; e < kV; ++e)
                        if (d0 + col + e < p.dim) po.du_f32[off + e] = ou[e];
                } else {
                    store(static_cast<T *>(po.du) + off, ou, d0 + col, p.dim, p.vec);
                }
                store(static_cast<T *>(po.ddelta) + off, od, d0 + col, p.dim, p.vec);
            }
            {
                float *dst = po.part_bc + (((int64_t)b * p.ntiles + tile) * p.L + t0) * (kNP * 2);
                const float *src = &s.red[0][0][0];
                for (int i = threadIdx.x; i < tval * kNP * 2; i += kThreads) dst[i] = src[i];
            }
            // No barrier here: the next chunk's staging writes only the staged
            // pairs and ds, which this phase does not read, and its first
            // barrier keeps the planes and sums read here from being
            // overwritten before every wave is done with them.
        }
        __syncthreads();   // the planes, reused below, are free once every wave is past the last chunk

        // dA, dD of this batch row; dh0 = a_0 lam_0
        if (dval) {
#pragma unroll
            for (int q = 0; q < NPW; ++q) {
                const int n = w * NPW + q;
                p.part_a[((int64_t)b * p.dim + d) * kNP + n] = dA[q];
                if (p.dh0 != nullptr && n < p.N) p.dh0[((int64_t)b * p.dim + d) * p.N + n] = mu[q];
            }
        }
        // dD: the threads sharing a channel column hold different rows' sums;
        // add them through LDS (the planes are free after the barrier above)
        float (*dsum)[kTile] = s.pl[0][0];
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            if (!piece_in_chunk(j)) continue;
#pragma unroll
            for (int e = 0; e < kV; ++e) dsum[piece_row(j)][col + e] = dDacc[j][e];
        }
        __syncthreads();
        if (threadIdx.x < kTile && d0 + (int)threadIdx.x < p.dim) {
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < TC; ++r) acc += dsum[r][threadIdx.x];
            p.part_d[(int64_t)b * p.dim + d0 + threadIdx.x] = acc;
        }
        if (FEAT && p.part_db != nullptr) {
            // the same for the delta-bias gradient, through the second plane set
            float (*bsum)[kTile] = s.pl[1][0];
#pragma unroll
            for (int j = 0; j < kPPT; ++j) {
                if (!piece_in_chunk(j)) continue;
#pragma unroll
                for (int e = 0; e < kV; ++e) bsum[piece_row(j)][col + e] = dbacc[j][e];
            }
            __syncthreads();
            if (threadIdx.x < kTile && d0 + (int)threadIdx.x < p.dim) {
                float acc = 0.0f;
#pragma unroll
                for (int r = 0; r < TC; ++r) acc += bsum[r][threadIdx.x];
                p.part_db[(int64_t)b * p.dim + d0 + threadIdx.x] = acc;
            }
        }
    }
};

// the simplified rule fits 128 VGPRs: at least 4 waves per SIMD (two 8-wave
// workgroups, or one 16-wave one, per CU); the hold rule's reverse step needs
// more registers, and capping it at 128 spilled 80-170 of them to scratch.
// With 2 waves per workgroup (up to 4 states) the staged chunk and planes take
// 28.5 KB of LDS per workgroup, so at most 5 workgroups (2.5 waves per SIMD)
// fit a CU whatever the registers: the target there is 2.
template <int G, bool ZOH> constexpr int bwd_waves_per_simd() { return (ZOH || G == 2) ? 2 : 4; }
template <typename T, int NPW, int G, int TC, bool ZOH, bool UF, bool FEAT>
__global__ __launch_bounds__(kTile * G, (bwd_waves_per_simd<G, ZOH>())) void bwd_kernel(const BwdParams p) {
    BwdKernel<T, NPW, G, TC, ZOH, UF, FEAT>::run(p);
}

template <typename T, bool ZOH>
hipError_t launch_bwd_shape(const BwdShape &sh, const BwdParams &p, hipStream_t st) {
    const int64_t blocks = (int64_t)p.batch * p.ntiles;
    // fp32 u with bf16 tensors: the UF variant (fp32 tensors read u as fp32 anyway)
    const bool uf = sizeof(T) == 2 && p.u_f32;
    // the step options' instance only when one is on
    const bool feat = p.delta_bias != nullptr || p.delta_softplus;
#define SSM_BWD_LAUNCH(NP, GG, TCC, UFV, FV) \
    hipLaunchKernelGGL((bwd_kernel<T, NP / GG, GG, TCC, ZOH, UFV, FV>), dim3((unsigned)blocks), dim3(kTile * GG), 0, \
                       st, p)
#define SSM_BWD_CASE(NP, GG, TCC) \
    if (sh.npad == NP && sh.G == GG && sh.TC == TCC) { \
        if (uf && feat) SSM_BWD_LAUNCH(NP, GG, TCC, sizeof(T) == 2, true); \
        else if (uf) SSM_BWD_LAUNCH(NP, GG, TCC, sizeof(T) == 2, false); \
        else if (feat) SSM_BWD_LAUNCH(NP, GG, TCC, false, true); \
        else SSM_BWD_LAUNCH(NP, GG, TCC, false, false); \
        return hipGetLastError(); \
    }
    SSM_BWD_CASE(4, 2, 16) SSM_BWD_CASE(8, 8, 16) SSM_BWD_CASE(16, 8, 16) SSM_BWD_CASE(32, 16, 8)
    SSM_BWD_CASE(64, 16, 8)
#undef SSM_BWD_CASE
#undef SSM_BWD_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ssm_detail
#endif  // SSM_BWD_INSTANTIATE
