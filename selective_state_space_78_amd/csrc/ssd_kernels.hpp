// Mamba-2 SSD (state-space duality) layer on gfx950 matrix cores.
//
// With the state matrix of a head restricted to a scalar a times the identity
// (itwiki "상태 공간 모델", section "Mamba-2와 상태 공간 쌍대성"), the layer
// is, per batch row and head, h_t = exp(a dt_t) h_{t-1} + wbar_t x_t B_t^T and
// y_t = h_t C_t (+ D x_t, * silu(z_t)), with a (P x N) state. Inside a chunk
// of Q tokens that is a causally masked product plus the state carried in
// (youngju.dev "mamba-state-space-model-selective-ssm", SSDBlock._chunk_scan,
// for the chunk-internal part); with S_i = sum_{c0<=r<=i} a dt_r:
//
//   y_i   = sum_{j<=i} (C_i . B_j) exp(S_i - S_j) wbar_j x_j  +  exp(S_i) C_i . H
//   H_out = exp(S_last) H + sum_j exp(S_last - S_j) wbar_j x_j B_j^T
//
// Kernel design:
//  * A workgroup takes HPW heads of one batch row and group: two when the head
//    size is 64 and the group's head count is even (their LDS then fits),
//    otherwise one. Per head, four compute waves and four helper waves.
//  * Compute wave WL of a head holds the state tiles h^T[n][p] of p tiles WL,
//    WL + 4, ... for every n as MFMA accumulators (lane = p column, 4
//    consecutive n); the fp32 state never leaves registers. Every product is
//    a 16x16x32 bf16 MFMA with fp32 accumulation.
//  * Each chunk of Q = 64 tokens takes two phases, each closed by a barrier:
//      1. compute waves: the readout of the state entering the chunk,
//         Y^T[p][i] = H[p][:] . C_i for every token i, whose A operand is the
//         wave's own state split hi + lo in registers (K runs over n in the
//         order in which the lane holds its accumulators), times exp(S_i).
//         Helpers: they write the next chunk's x, B and C rows (loaded during
//         the previous chunk) into the other half of double-buffered LDS,
//         form its step tables (S_t, wbar_t, wbar_t exp(S_last - S_t)), and
//         issue the loads of the chunk after it.
//      2. compute waves: the masked product Y^T[p][i] += sum_j x^T[p][j]
//         M^T[j][i] (x by transposing LDS reads, M from the exchange buffer);
//         skip, gate, bf16 rounding and stores; then the state update
//         h^T[n][p] = exp(S_last) h^T[n][p] + sum_j B_j[n] wbar_j
//         exp(S_last - S_j) x_j[p] (B by transposing reads, the weighted x
//         split hi + lo in registers).
//         Helpers: the next chunk's score tiles G^T[j][i] = B_j . C_i (j and
//         i blocks J <= T), formed once for the workgroup's heads, then per
//         head decayed, weighted, masked to j <= i and split hi + lo into the
//         exchange buffer, in the lane order of the compute waves' operand.
//         With a pair of heads, two of the ten tiles are instead scored in
//         phase 1 of their own chunk by two helpers with no step table to
//         form, so that each helper scores at most one tile in phase 2.
//  * The computed operands (the state for its readout, the scores, the
//    weighted x) are split into hi + lo bf16 pairs; x, B and C are exact in
//    bf16.
//  * Global accesses are raw buffer accesses sized to the chunk's valid rows:
//    rows past the end of the sequence load as zero (step 0: they neither
//    decay nor feed the state) and their outputs are dropped.
//  * The gate is a compile-time option (GATE), the skip a run-time one.
//  * Workgroup ids are remapped so that the heads of one batch row, which read
//    the same B and C rows, run on the same XCD and share its L2.
#pragma once

#include "scan_kernels.hpp"

namespace ssm_detail {

struct SsdParams {
    const uint16_t *x, *dt, *B, *C, *z;   // bf16 bit patterns
    const float *dt_bias, *A, *D, *h0;
    uint16_t *y;
    float *h_last;
    int64_t L;
    int batch, H, G, hpg;   // heads, groups, heads per group
    int dt_softplus;
};

// Head dimensions 64, 96, 128 and state sizes 64, 128.
#define SSM_SSD_SHAPES(X) X(64, 64) X(64, 128) X(96, 64) X(96, 128) X(128, 64) X(128, 128)

inline bool ssd_shape_supported(int P, int N) {
#define SSM_SSD_IS(PP, NN) if (P == PP && N == NN) return true;
    SSM_SSD_SHAPES(SSM_SSD_IS)
#undef SSM_SSD_IS
    return false;
}

hipError_t launch_ssd_euler(const SsdParams &p, int P, int N, hipStream_t st);
hipError_t launch_ssd_zoh(const SsdParams &p, int P, int N, hipStream_t st);

#ifdef SSM_SSD_INSTANTIATE

typedef __bf16 ssd_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 ssd_bf16x2 __attribute__((ext_vector_type(2)));
typedef float ssd_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSsdQ = 64;        // tokens per chunk

// LDS row padding (elements) of the token-row tiles of x and of B and C. With
// N + 8 (4 banks mod 64 per row) the score and readout row reads of B and C
// are conflict-free; N + 16 measured 10% slower, P + 16 about 1% faster than
// P + 8 (a pair of heads then takes 159 KB of the 160 KB).
constexpr int kSsdXPad = 16;
constexpr int kSsdHPad = 8;

constexpr int kSsdThreads = 256; // 4 waves

__device__ __forceinline__ float ssd_bf(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t ssd_to_bf(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

__device__ __forceinline__ uint32_t ssd_pack(float lo, float hi) {
    const ssd_bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ ssd_f32x4 ssd_mfma(const ssd_bf16x8 &a, const ssd_bf16x8 &b, const ssd_f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ ssd_bf16x8 ssd_ld16(const uint16_t *p) {
    return __builtin_bit_cast(ssd_bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit values V_s[0..3], and
// lane 4q + c receives V_q[c], V_{q+4}[c], V_{q+8}[c], V_{q+12}[c]. With lane s
// pointing at row r0 + (s >> 2), columns c0 + 4 (s & 3) of a row-major tile,
// lane 4q + c gets column c0 + 4q + c of rows r0 .. r0 + 3: a column of the
// tile, as a matrix-core operand whose K runs along the rows needs it.
__device__ __forceinline__ uint2 ssd_ld_tr(const uint16_t *p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// Two transposing reads (K positions 0..3 and 4..7) as one operand.
__device__ __forceinline__ ssd_bf16x8 ssd_ld_tr2(const uint16_t *p0, const uint16_t *p1) {
    const uint2 a = ssd_ld_tr(p0);
    const uint2 b = ssd_ld_tr(p1);
    const uint4 v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(ssd_bf16x8, v);
}

// Inclusive prefix sum over the 64 lanes of a wave: Kogge-Stone steps within
// rows of 16 (DPP row shifts), then the row totals carried across rows (DPP
// row broadcasts of lanes 15 and 31). Lanes without a source add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float ssd_dpp_add(float v, bool take) {
    const float u = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                          ROW_MASK, 0xF, false));
    return take ? v + u : v;
}

__device__ __forceinline__ float ssd_prefix_sum(float v, int lane) {
    const int r = lane & 15;
    v = ssd_dpp_add<0x111, 0xF>(v, r >= 1);              // row_shr:1
    v = ssd_dpp_add<0x112, 0xF>(v, r >= 2);              // row_shr:2
    v = ssd_dpp_add<0x114, 0xF>(v, r >= 4);              // row_shr:4
    v = ssd_dpp_add<0x118, 0xF>(v, r >= 8);              // row_shr:8
    v = ssd_dpp_add<0x142, 0xA>(v, (lane & 16) != 0);    // row_bcast:15 -> rows 1, 3
    v = ssd_dpp_add<0x143, 0xC>(v, (lane & 32) != 0);    // row_bcast:31 -> rows 2, 3
    return v;
}

// Two floats as the hi and lo words of packed bf16 pairs whose sums carry 16
// significant bits: hi is the pair rounded to bf16, lo the two remainders
// rounded to bf16.
__device__ __forceinline__ void ssd_split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = ssd_pack(a, b);
    const float ra = a - __uint_as_float(hi << 16);
    const float rb = b - __uint_as_float(hi & 0xffff0000u);
    lo = ssd_pack(ra, rb);
}

typedef unsigned int ssd_u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer of `bytes` bytes at `base` (dword 3: 32-bit data format, the
// setting for untyped access on gfx9). Buffer instructions check every access
// against that size: loads past it return zero and stores past it are
// dropped. Rows past the end of the sequence then need no branch, and the
// compiler's wait counts, which must assume the shortest path through a
// branch, stay exact.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ssd_buffer(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ssd_bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const ssd_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void ssd_bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4 &v) {
    __builtin_amdgcn_raw_buffer_store_b128(ssd_u32x4{v.x, v.y, v.z, v.w}, r, (int)off, 0, 0);
}

typedef unsigned int ssd_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 ssd_bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const ssd_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return uint2{v.x, v.y};
}

__device__ __forceinline__ void ssd_bstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint2 &v) {
    __builtin_amdgcn_raw_buffer_store_b64(ssd_u32x2{v.x, v.y}, r, (int)off, 0, 0);
}

// The chunk's causal score tiles (output token tile T, key token tile J <= T),
// dealt round-robin to the helper waves.
constexpr int kSsdTiles = 10;
constexpr int kSsdTileT[kSsdTiles] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int kSsdTileJ[kSsdTiles] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
// Slot of the masked scores of (T, key half Jp) in the exchange buffer
__host__ __device__ constexpr int ssd_slot(int T, int Jp) { return T < 2 ? T : 2 + 2 * (T - 2) + Jp; }
constexpr int kSsdSlots = 6;
// With a pair of heads (8 helpers) tiles 0..7 are scored one per helper in
// the second phase of the chunk before theirs; the last two in the first
// phase of their own chunk, by helpers 2 and 3 (the helpers that form no step
// table and whose staging is done by then). One head (4 helpers): every tile
// in the second phase, dealt round-robin.
template <int HPW> constexpr int ssd_early_tiles() { return HPW == 2 ? 8 : kSsdTiles; }
template <int HPW> constexpr int ssd_tile_owner(int q) {
    return q < ssd_early_tiles<HPW>() ? q % (4 * HPW) : 2 + (q - ssd_early_tiles<HPW>());
}

// HPW heads of one group per workgroup. Per head four compute waves hold the
// state (wave WL: p tiles WL, WL + 4, ...; every n) and make the chunk's
// outputs and state update; 4 HPW helper waves prepare the next chunk
// meanwhile: they stage its x, B and C rows, its step tables and its masked
// scores into the other half of double-buffered LDS.
template <int P, int N, bool ZOH, int HPW, bool GATE>
__global__ __launch_bounds__(2 * kSsdThreads * HPW) void ssd_fwd_kernel(const SsdParams p) {
    constexpr int Q = kSsdQ;
    constexpr int PT = P / 16;     // p tiles
    constexpr int NT = N / 16;     // n tiles
    constexpr int NK = N / 32;     // MFMA steps over n
    constexpr int XS = P + kSsdXPad;   // LDS row stride of the x token rows
    constexpr int HS = N + kSsdHPad;   // LDS row stride of the B and C token rows
    constexpr int NH = kSsdThreads * HPW;   // helper threads
    // staging: 16-byte pieces of the token rows, numbered (head,) token-major;
    // helper thread ut takes pieces k NH + ut, so that one load instruction
    // covers whole rows of one head
    constexpr int XPR = P / 8, BPR = N / 8;                  // pieces per token row
    constexpr int XI = HPW * Q * XPR / NH;                   // x loads per helper thread
    constexpr int BI = Q * BPR / NH;                         // B (and C) loads per helper thread
    static_assert(P % 32 == 0 && N % 64 == 0, "tile shape");
    static_assert(XI * NH == HPW * Q * XPR && BI * NH == Q * BPR, "staging pieces cover the chunk");
    static_assert(HPW == 1 || (Q * XPR) % NH == 0, "one head per x load instruction");

    __shared__ __attribute__((aligned(16))) uint16_t sX[2][HPW][Q * XS];   // x, token rows
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][Q * HS];        // B, token rows
    __shared__ __attribute__((aligned(16))) uint16_t sC[2][Q * HS];        // C, token rows
    __shared__ __attribute__((aligned(16))) uint4 sM[2][HPW][kSsdSlots][2][64];   // masked scores, hi and lo
    __shared__ __attribute__((aligned(16))) float sS[2][HPW][Q];   // S_t: prefix sums of a dt (log2)
    __shared__ __attribute__((aligned(16))) float sW[2][HPW][Q];   // wbar_t
    __shared__ __attribute__((aligned(16))) float sF[2][HPW][Q];   // wbar_t exp(S_last - S_t)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;

    const int nb = gridDim.x, bid = blockIdx.x;
    const int qx = nb / kXcds, rx = nb % kXcds, xcd = bid % kXcds;
    const int logical = xcd * qx + min(xcd, rx) + bid / kXcds;
    const int hpb = p.H / HPW;
    const int b = logical / hpb;
    const int hbase = (logical % hpb) * HPW;
    const int grp = hbase / p.hpg;
    const int64_t L = p.L;
    const int64_t xs = (int64_t)p.H * P;   // token stride of x, z, y
    const int64_t bs = (int64_t)p.G * N;   // token stride of B, C
    // (64 token rows of x and of B fit 32-bit element offsets: the library checks it)
    const uint32_t xs32 = (uint32_t)xs, bs32 = (uint32_t)bs, H32 = (uint32_t)p.H;
    const int nchunks = (int)((L + Q - 1) / Q);
    auto valid_tokens = [&](int64_t c) { return (uint32_t)max<int64_t>(0, min<int64_t>(Q, L - c)); };

    if (w >= 4 * HPW) {
        // ================= helper waves =================
        const int ut = tid - kSsdThreads * HPW;   // 0 .. NH - 1 (after the 4 HPW compute waves)
        const int u = w - 4 * HPW;
        const uint16_t *Bb = p.B + (int64_t)b * L * bs + (int64_t)grp * N;
        const uint16_t *Cb = p.C + (int64_t)b * L * bs + (int64_t)grp * N;
        uint32_t xoff[XI], boff[BI];
#pragma unroll
        for (int k = 0; k < XI; ++k) {
            const int rem = (k * NH + ut) % (Q * XPR);
            xoff[k] = 2u * ((uint32_t)(rem / XPR) * xs32 + 8u * (rem % XPR));
        }
#pragma unroll
        for (int k = 0; k < BI; ++k) {
            const int piece = k * NH + ut;
            boff[k] = 2u * ((uint32_t)(piece / BPR) * bs32 + 8u * (piece % BPR));
        }
        uint4 xr[XI], br[BI], cr[BI];
        // the last HPW helpers also form the step tables, helper 4 HPW - HPW + hs
        // those of head hs: its dt (token `lane`), and the head's constants
        const int th = u - 3 * HPW;              // head of the tables this helper forms, or < 0
        const int hth = hbase + (th >= 0 ? th : 0);
        const uint16_t *dtb = p.dt + (int64_t)b * L * p.H + hth;
        const float a = p.A[hth];
        const float a2 = a * kLog2e;
        const float bias = p.dt_bias ? p.dt_bias[hth] : 0.0f;
        uint16_t dtr = 0;
        // loads of the chunk starting at c (rows past the end read zero)
        auto load = [&](int64_t c) {
            const uint32_t nv = valid_tokens(c);
            if (th >= 0)
                dtr = __builtin_amdgcn_raw_buffer_load_b16(ssd_buffer(dtb + c * p.H, 2u * nv * H32),
                                                           (int)(2u * (uint32_t)lane * H32), 0, 0);
#pragma unroll
            for (int k = 0; k < XI; ++k) {
                const int hs = k * NH / (Q * XPR);
                const uint16_t *xb = p.x + ((int64_t)b * L + c) * xs + (int64_t)(hbase + hs) * P;
                xr[k] = ssd_bload16(ssd_buffer(xb, 2u * nv * xs32), xoff[k]);
            }
            const __amdgpu_buffer_rsrc_t rb = ssd_buffer(Bb + c * bs, 2u * nv * bs32);
            const __amdgpu_buffer_rsrc_t rc = ssd_buffer(Cb + c * bs, 2u * nv * bs32);
#pragma unroll
            for (int k = 0; k < BI; ++k) {
                br[k] = ssd_bload16(rb, boff[k]);
                cr[k] = ssd_bload16(rc, boff[k]);
            }
        };
        // Scores of the chunk staged in buffer `buf`, decayed, weighted and
        // masked for each head, as hi + lo bf16: the lane of tile (T, J) holds
        // M^T[16 J + 4 g4 + r][16 T + r16], element 4 (J % 2) + r of the same
        // lane's operand of the compute waves' (T, J / 2) product. The tiles
        // are dealt round-robin to the helpers; each forms its tile's scores
        // C_i . B_j once for the workgroup's heads (they share B and C). U, the
        // helper, is a constant, so that a helper's tiles form one
        // straight-line block whose loads, products and exponentials overlap.
        auto score_jobs = [&](auto uc, auto latec, int buf) {
            constexpr int U = decltype(uc)::value;
            constexpr bool LATE = decltype(latec)::value;
#pragma unroll
            for (int q = 0; q < kSsdTiles; ++q) {
                if (ssd_tile_owner<HPW>(q) != U || (q >= ssd_early_tiles<HPW>()) != LATE) continue;
                const int T = kSsdTileT[q], J = kSsdTileJ[q];
                ssd_f32x4 gt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < NK; ++s)
                    gt = ssd_mfma(ssd_ld16(&sB[buf][(16 * J + r16) * HS + 32 * s + 8 * g4]),
                                  ssd_ld16(&sC[buf][(16 * T + r16) * HS + 32 * s + 8 * g4]), gt);
#pragma unroll
                for (int hs = 0; hs < HPW; ++hs) {
                    const float Si = sS[buf][hs][16 * T + r16];
                    const float4 Sj = *reinterpret_cast<const float4 *>(&sS[buf][hs][16 * J + 4 * g4]);
                    const float4 Wj = *reinterpret_cast<const float4 *>(&sW[buf][hs][16 * J + 4 * g4]);
                    const float sj[4] = {Sj.x, Sj.y, Sj.z, Sj.w}, wj[4] = {Wj.x, Wj.y, Wj.z, Wj.w};
                    float m[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool keep = J < T || 4 * g4 + r <= r16;
                        m[r] = keep ? gt[r] * __builtin_amdgcn_exp2f(Si - sj[r]) * wj[r] : 0.0f;
                    }
                    uint2 hi, lo;
                    ssd_split2(m[0], m[1], hi.x, lo.x);
                    ssd_split2(m[2], m[3], hi.y, lo.y);
                    uint2 *mh = reinterpret_cast<uint2 *>(&sM[buf][hs][ssd_slot(T, J >> 1)][0][lane]);
                    uint2 *ml = reinterpret_cast<uint2 *>(&sM[buf][hs][ssd_slot(T, J >> 1)][1][lane]);
                    mh[J & 1] = hi;
                    ml[J & 1] = lo;
                    if (J == T && (T & 1) == 0) {
                        // the key tile past the diagonal that shares this slot: zeros
                        mh[1] = uint2{0u, 0u};
                        ml[1] = uint2{0u, 0u};
                    }
                }
            }
        };
        load(0);
        for (int k = -1; k < nchunks; ++k) {
            const int buf = k & 1;   // the compute waves' buffer; this loop fills the other
            const bool work = k + 1 < nchunks;
            if (work) {
                // staged rows of chunk k + 1, into the other buffer
#pragma unroll
                for (int q = 0; q < XI; ++q) {
                    const int piece = q * NH + ut;
                    const int hs = piece / (Q * XPR), rem = piece % (Q * XPR);
                    *reinterpret_cast<uint4 *>(&sX[buf ^ 1][hs][(rem / XPR) * XS + 8 * (rem % XPR)]) = xr[q];
                }
#pragma unroll
                for (int q = 0; q < BI; ++q) {
                    const int piece = q * NH + ut;
                    const int o = (piece / BPR) * HS + 8 * (piece % BPR);
                    *reinterpret_cast<uint4 *>(&sB[buf ^ 1][o]) = br[q];
                    *reinterpret_cast<uint4 *>(&sC[buf ^ 1][o]) = cr[q];
                }
                if (th >= 0) {
                    // step, decay and input weight of token `lane` of chunk k + 1
                    float step = 0.0f;
                    if (lane < (int)valid_tokens((int64_t)(k + 1) * Q)) {
                        step = ssd_bf(dtr) + bias;
                        if (p.dt_softplus)
                            step = softplus_f(step);
                    }
                    const float la = step * a2;
                    float wbar = step;
                    if (ZOH)
                        wbar = step * expm1_over_x(step * a, __builtin_amdgcn_exp2f(la));
                    const float S = ssd_prefix_sum(la, lane);
                    const float Slast =
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, S), 63));
                    sS[buf ^ 1][th][lane] = S;
                    sW[buf ^ 1][th][lane] = wbar;
                    sF[buf ^ 1][th][lane] = wbar * __builtin_amdgcn_exp2f(Slast - S);
                }
                if (k + 2 < nchunks) load((int64_t)(k + 2) * Q);
            }
            if constexpr (ssd_early_tiles<HPW>() < kSsdTiles) {
                // the late tiles of chunk k, whose rows and tables are in buffer buf
                if (k >= 0) {
                    if (u == 2) score_jobs(std::integral_constant<int, 2>{}, std::true_type{}, buf);
                    if (u == 3) score_jobs(std::integral_constant<int, 3>{}, std::true_type{}, buf);
                }
            }
            __syncthreads();
            if (work) {
                switch (u) {
                case 0: score_jobs(std::integral_constant<int, 0>{}, std::false_type{}, buf ^ 1); break;
                case 1: score_jobs(std::integral_constant<int, 1>{}, std::false_type{}, buf ^ 1); break;
                case 2: score_jobs(std::integral_constant<int, 2>{}, std::false_type{}, buf ^ 1); break;
                case 3: score_jobs(std::integral_constant<int, 3>{}, std::false_type{}, buf ^ 1); break;
                case 4: if constexpr (HPW > 1) score_jobs(std::integral_constant<int, 4>{}, std::false_type{}, buf ^ 1); break;
                case 5: if constexpr (HPW > 1) score_jobs(std::integral_constant<int, 5>{}, std::false_type{}, buf ^ 1); break;
                case 6: if constexpr (HPW > 1) score_jobs(std::integral_constant<int, 6>{}, std::false_type{}, buf ^ 1); break;
                default: if constexpr (HPW > 1) score_jobs(std::integral_constant<int, 7>{}, std::false_type{}, buf ^ 1); break;
                }
            }
            __syncthreads();
        }
        return;
    }

    // ================= compute waves =================
    const int hs = w >> 2;
    const int h = hbase + hs;
    const float dskip = p.D ? p.D[h] : 0.0f;
    const uint16_t *zb = GATE ? p.z + (int64_t)b * L * xs + (int64_t)h * P : nullptr;
    uint16_t *yb = p.y + (int64_t)b * L * xs + (int64_t)h * P;
    const float *h0b = p.h0 ? p.h0 + ((int64_t)b * p.H + h) * P * N : nullptr;
    float *hlb = p.h_last ? p.h_last + ((int64_t)b * p.H + h) * P * N : nullptr;

    // The role WL (p tiles WL, WL + 4, ...) is a compile-time constant, so
    // each role's loop is straight-line code.
    auto run = [&](auto role) {
        constexpr int WL = decltype(role)::value;
        constexpr int NPT = (PT - WL + 3) / 4;   // p tiles of this wave
        // State: hacc[k][nt][r] = h[p = 16 (WL + 4 k) + r16][n = 16 nt + 4 g4 + r]
        // (an h^T tile: lane = p column, 4 consecutive n)
        ssd_f32x4 hacc[NPT][NT];
#pragma unroll
        for (int k = 0; k < NPT; ++k)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                hacc[k][nt] = h0b ? *reinterpret_cast<const ssd_f32x4 *>(h0b + (16 * (WL + 4 * k) + r16) * N +
                                                                          16 * nt + 4 * g4)
                                  : ssd_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        ssd_f32x4 yacc[NPT][4];
        uint2 zop[NPT][4];
        for (int k = -1; k < nchunks; ++k) {
            const int buf = k & 1;
            const int64_t c0 = (int64_t)k * Q;
            const uint32_t nvu = k >= 0 ? valid_tokens(c0) : 0u;
            if (k >= 0) {
                // gate values of this wave's outputs (token 16 T + r16, channels
                // 16 pt + 4 g4 .. + 3)
                if constexpr (GATE) {
                    const __amdgpu_buffer_rsrc_t rz = ssd_buffer(zb + c0 * xs, 2u * nvu * xs32);
#pragma unroll
                    for (int q = 0; q < NPT; ++q)
#pragma unroll
                        for (int T = 0; T < 4; ++T)
                            zop[q][T] =
                                ssd_bload8(rz, 2u * ((uint32_t)(16 * T + r16) * xs32 + 16 * (WL + 4 * q) + 4 * g4));
                }

                // ---- readout of the state entering the chunk, for every output
                // token: Y^T[p][i] = sum_n H[p][n] C_i[n], with K running over n
                // in the order n = 32 s + 16 (e / 4) + 4 g4 + e % 4 (e = the
                // operand element), the order in which the lane holds its state
#pragma unroll
                for (int q = 0; q < NPT; ++q)
#pragma unroll
                    for (int T = 0; T < 4; ++T)
                        yacc[q][T] = ssd_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < NK; ++s) {
                    ssd_bf16x8 ah[NPT], al[NPT];
#pragma unroll
                    for (int q = 0; q < NPT; ++q) {
                        uint32_t hw[4], lw[4];
                        ssd_split2(hacc[q][2 * s][0], hacc[q][2 * s][1], hw[0], lw[0]);
                        ssd_split2(hacc[q][2 * s][2], hacc[q][2 * s][3], hw[1], lw[1]);
                        ssd_split2(hacc[q][2 * s + 1][0], hacc[q][2 * s + 1][1], hw[2], lw[2]);
                        ssd_split2(hacc[q][2 * s + 1][2], hacc[q][2 * s + 1][3], hw[3], lw[3]);
                        ah[q] = __builtin_bit_cast(ssd_bf16x8, uint4{hw[0], hw[1], hw[2], hw[3]});
                        al[q] = __builtin_bit_cast(ssd_bf16x8, uint4{lw[0], lw[1], lw[2], lw[3]});
                    }
#pragma unroll
                    for (int T = 0; T < 4; ++T) {
                        const uint16_t *cp = &sC[buf][(16 * T + r16) * HS + 32 * s + 4 * g4];
                        const uint2 c0v = *reinterpret_cast<const uint2 *>(cp);
                        const uint2 c1v = *reinterpret_cast<const uint2 *>(cp + 16);
                        const ssd_bf16x8 cop = __builtin_bit_cast(ssd_bf16x8, uint4{c0v.x, c0v.y, c1v.x, c1v.y});
#pragma unroll
                        for (int q = 0; q < NPT; ++q) {
                            yacc[q][T] = ssd_mfma(ah[q], cop, yacc[q][T]);
                            yacc[q][T] = ssd_mfma(al[q], cop, yacc[q][T]);
                        }
                    }
                }
                // decay from the chunk's start to each output token
#pragma unroll
                for (int T = 0; T < 4; ++T) {
                    const float ei = __builtin_amdgcn_exp2f(sS[buf][hs][16 * T + r16]);
#pragma unroll
                    for (int q = 0; q < NPT; ++q)
                        yacc[q][T] *= ei;
                }
            }
            __syncthreads();
            if (k >= 0) {
                // ---- masked product: Y^T[p][i] += sum_j x[j][p] M^T[j][i], K over
                // j in the order j = 32 Jp + 16 (e / 4) + 4 g4 + e % 4
                const uint16_t *X = sX[buf][hs];
#pragma unroll
                for (int Jp = 0; Jp < 2; ++Jp) {
                    ssd_bf16x8 xop[NPT];
#pragma unroll
                    for (int q = 0; q < NPT; ++q) {
                        const uint16_t *src = &X[(32 * Jp + 4 * g4 + (r16 >> 2)) * XS + 16 * (WL + 4 * q) + 4 * (r16 & 3)];
                        xop[q] = ssd_ld_tr2(src, src + 16 * XS);
                    }
#pragma unroll
                    for (int T = 2 * Jp; T < 4; ++T) {
                        const ssd_bf16x8 mh = __builtin_bit_cast(ssd_bf16x8, sM[buf][hs][ssd_slot(T, Jp)][0][lane]);
                        const ssd_bf16x8 ml = __builtin_bit_cast(ssd_bf16x8, sM[buf][hs][ssd_slot(T, Jp)][1][lane]);
#pragma unroll
                        for (int q = 0; q < NPT; ++q) {
                            yacc[q][T] = ssd_mfma(xop[q], mh, yacc[q][T]);
                            yacc[q][T] = ssd_mfma(xop[q], ml, yacc[q][T]);
                        }
                    }
                }

                // ---- skip, gate, store: yacc[q][T][r] = y[i = 16 T + r16][p = 16 pt + 4 g4 + r];
                // rows past the end are dropped by the buffer's range
                {
                    const __amdgpu_buffer_rsrc_t ry = ssd_buffer(yb + c0 * xs, 2u * nvu * xs32);
#pragma unroll
                    for (int q = 0; q < NPT; ++q)
#pragma unroll
                        for (int T = 0; T < 4; ++T) {
                            const int pc = 16 * (WL + 4 * q) + 4 * g4;
                            float v[4] = {yacc[q][T][0], yacc[q][T][1], yacc[q][T][2], yacc[q][T][3]};
                            if (p.D) {
                                const uint2 xw = *reinterpret_cast<const uint2 *>(&X[(16 * T + r16) * XS + pc]);
                                v[0] += dskip * ssd_bf(xw.x & 0xffffu);
                                v[1] += dskip * ssd_bf(xw.x >> 16);
                                v[2] += dskip * ssd_bf(xw.y & 0xffffu);
                                v[3] += dskip * ssd_bf(xw.y >> 16);
                            }
                            if constexpr (GATE) {
                                const uint2 zw = zop[q][T];
                                v[0] *= silu(ssd_bf(zw.x & 0xffffu));
                                v[1] *= silu(ssd_bf(zw.x >> 16));
                                v[2] *= silu(ssd_bf(zw.y & 0xffffu));
                                v[3] *= silu(ssd_bf(zw.y >> 16));
                            }
                            ssd_bstore8(ry, 2u * ((uint32_t)(16 * T + r16) * xs32 + pc),
                                        uint2{ssd_pack(v[0], v[1]), ssd_pack(v[2], v[3])});
                        }
                }

                // ---- state update: h^T[n][p] = exp(S_last) h^T[n][p] + sum_j B_j[n] fd_j x[j][p],
                // K over j = 32 ks + 8 g4 + e
                {
                    const uint16_t *X = sX[buf][hs];
                    const float dec = __builtin_amdgcn_exp2f(sS[buf][hs][Q - 1]);
#pragma unroll
                    for (int q = 0; q < NPT; ++q)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            hacc[q][nt] *= dec;
#pragma unroll
                    for (int ks = 0; ks < Q / 32; ++ks) {
                        const int j0 = 32 * ks + 8 * g4;
                        const float4 f0 = *reinterpret_cast<const float4 *>(&sF[buf][hs][j0]);
                        const float4 f1 = *reinterpret_cast<const float4 *>(&sF[buf][hs][j0 + 4]);
                        const float fj[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
                        ssd_bf16x8 xh[NPT], xl[NPT];
#pragma unroll
                        for (int q = 0; q < NPT; ++q) {
                            const uint16_t *src = &X[(j0 + (r16 >> 2)) * XS + 16 * (WL + 4 * q) + 4 * (r16 & 3)];
                            const uint4 xv = __builtin_bit_cast(uint4, ssd_ld_tr2(src, src + 4 * XS));
                            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
                            uint32_t hw[4], lw[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                ssd_split2(ssd_bf(xw[e] & 0xffffu) * fj[2 * e], ssd_bf(xw[e] >> 16) * fj[2 * e + 1],
                                           hw[e], lw[e]);
                            xh[q] = __builtin_bit_cast(ssd_bf16x8, uint4{hw[0], hw[1], hw[2], hw[3]});
                            xl[q] = __builtin_bit_cast(ssd_bf16x8, uint4{lw[0], lw[1], lw[2], lw[3]});
                        }
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const uint16_t *src = &sB[buf][(j0 + (r16 >> 2)) * HS + 16 * nt + 4 * (r16 & 3)];
                            const ssd_bf16x8 bop = ssd_ld_tr2(src, src + 4 * HS);
#pragma unroll
                            for (int q = 0; q < NPT; ++q) {
                                hacc[q][nt] = ssd_mfma(bop, xh[q], hacc[q][nt]);
                                hacc[q][nt] = ssd_mfma(bop, xl[q], hacc[q][nt]);
                            }
                        }
                    }
                }

            }
            __syncthreads();
        }

        if (hlb) {
#pragma unroll
            for (int q = 0; q < NPT; ++q)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *reinterpret_cast<ssd_f32x4 *>(hlb + (16 * (WL + 4 * q) + r16) * N + 16 * nt + 4 * g4) =
                        hacc[q][nt];
        }
    };
    switch (w & 3) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
    }
}

// Two heads per workgroup when they share a group and their LDS fits (head
// size 64); otherwise one.
template <int P, int N, bool ZOH>
hipError_t launch_ssd_pn(const SsdParams &p, hipStream_t st) {
    // the gate is a compile-time option: the instance without it carries none
    // of its loads or registers (4% faster on the Mamba-2-shaped layer). The
    // skip stays a run-time branch: as a compile-time option it measured 3%
    // slower than this, the compiler then scheduling the epilogue differently.
    constexpr int kPair = P == 64 ? 2 : 1;
    const bool pair = P == 64 && p.hpg % 2 == 0;
    const dim3 grid((unsigned)((int64_t)p.batch * (pair ? p.H / 2 : p.H)));
    if (pair && p.z)
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, kPair, true>), grid, dim3(2 * kSsdThreads * kPair), 0, st, p);
    else if (pair)
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, kPair, false>), grid, dim3(2 * kSsdThreads * kPair), 0, st, p);
    else if (p.z)
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, 1, true>), grid, dim3(2 * kSsdThreads), 0, st, p);
    else
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, 1, false>), grid, dim3(2 * kSsdThreads), 0, st, p);
    return hipGetLastError();
}

template <bool ZOH>
hipError_t launch_ssd_t(const SsdParams &p, int P, int N, hipStream_t st) {
#define SSM_SSD_CASE(PP, NN) \
    if (P == PP && N == NN)  \
        return launch_ssd_pn<PP, NN, ZOH>(p, st);
    SSM_SSD_SHAPES(SSM_SSD_CASE)
#undef SSM_SSD_CASE
    return hipErrorInvalidValue;
}

#endif  // SSM_SSD_INSTANTIATE

}  // namespace ssm_detail
