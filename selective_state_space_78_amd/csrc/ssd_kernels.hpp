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
//  * Four waves own one (batch row, head) and walk its chunks of Q = 64
//    tokens in order; the fp32 state never leaves registers. Wave w holds the
//    state rows n in [w N/4, (w+1) N/4) for every p, as MFMA accumulators
//    (h^T tiles: lane = p column, 4 consecutive n). A workgroup of 8 waves
//    takes two heads of one group, which share the staged B rows, when head
//    size 64 lets their LDS fit; otherwise a workgroup is one head, 4 waves.
//  * Every product is a 16x16x32 bf16 MFMA with fp32 accumulation:
//      scores  G^T[j][i] = B_j . C_i        (K = n; operands straight from L2)
//      readout Y^T[p][i] = H[p][:] . C_i    (K = n; H from LDS as bf16)
//      intra   Y^T[p][i] += sum_j X~[j][p] M^T[j][i]   (K = j)
//      update  h^T[n][p] += sum_j B[j][n] X~d[j][p]    (K = j)
//    Y^T rather than Y makes the score tile's accumulator layout (lane = i,
//    4 consecutive j) usable as the next product's operand without a trip
//    through LDS: the K order of that product is permuted to match, and the
//    X~ operand is read in the same order.
//  * Products over tokens need token-contiguous operands, so each chunk is
//    staged into LDS transposed: X~ = wbar x, X~d = wbar exp(S_last - S_j) x
//    (both P x Q) and B^T (N x Q); and the state as bf16 (P x N) for the
//    readout. Waves split the staging (lane = token) and then the work: wave w
//    computes the outputs of tokens [16w, 16w+16) and its state rows.
//  * Tokens past the end of the sequence enter with step 0 and zero x and B,
//    so they neither decay nor feed the state; their outputs are not stored.
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

// LDS row padding (elements) of the token-row tiles of x and of the
// n-contiguous tiles (B rows), and of the state copy (read as 16-byte row
// pieces); the mask of the row bits that swizzle the state copy's 64-byte
// column blocks. A sweep of the pads over {8, 16, 24} and of the swizzle
// (off, one bit, two bits) found these fastest.
constexpr int kSsdXPad = 16;
constexpr int kSsdHPad = 16;
constexpr int kSsdSPad = 8;
constexpr int kSsdSwizzle = 1;

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

// One chunk's global inputs as a lane (= token) of each wave loads them, one
// chunk ahead of their use.
template <int P, int N, int HPW>
struct SsdStage {
    // 16-byte pieces of a chunk's x rows (this head's P values per token) and
    // B rows (N values per token), numbered token-major; consecutive lanes
    // take consecutive pieces, so a load instruction covers whole rows.
    static constexpr int XPR = P / 8;                        // x pieces per token row
    static constexpr int XI = kSsdQ * XPR / (4 * 64);        // x loads per wave (four waves per head)
    static constexpr int BPR = N / 8;                        // B pieces per token row
    static constexpr int BI = kSsdQ * BPR / (4 * HPW * 64);  // B loads per wave (all waves)
    uint16_t dt;                 // bf16 step of token `lane` for this wave's head
    uint4 x[XI];                 // x piece wl XI 64 + 64 k + lane
    uint4 b[BI];                 // B piece w BI 64 + 64 k + lane
};

// HPW heads of one group per workgroup, four waves per head; the heads share
// the staged B tiles.
template <int P, int N, bool ZOH, int HPW>
__global__ __launch_bounds__(kSsdThreads * HPW, 1) void ssd_fwd_kernel(const SsdParams p) {
    constexpr int Q = kSsdQ;
    constexpr int PT = P / 16;     // p tiles
    constexpr int NK = N / 32;     // MFMA steps over n
    constexpr int NW = N / 4;      // state rows per wave
    constexpr int NTW = NW / 16;   // state row tiles per wave
    constexpr int XS = P + kSsdXPad;   // LDS row stride of token rows of x (conflict-free transposing reads)
    constexpr int HS = N + kSsdHPad;   // LDS row stride of the B token rows (likewise)
    constexpr int HSH = N + kSsdSPad;  // LDS row stride of the state copy (16-byte row reads)
    typedef SsdStage<P, N, HPW> Stage;
    static_assert(P % 32 == 0 && N % 64 == 0, "tile shape");
    static_assert(Stage::XI * 4 * 64 == Q * Stage::XPR && Stage::BI * 4 * HPW * 64 == Q * Stage::BPR,
                  "staging pieces cover the chunk");

    __shared__ __attribute__((aligned(16))) uint16_t sBR[Q * HS];         // B, token rows
    __shared__ __attribute__((aligned(16))) uint16_t sXT[HPW][Q * XS];    // x, token rows, output channel order
    __shared__ __attribute__((aligned(16))) uint16_t sXh[HPW][Q * XS];    // wbar exp(S_last - S_j) x, hi
    __shared__ __attribute__((aligned(16))) uint16_t sXl[HPW][Q * XS];    // ... lo
    __shared__ __attribute__((aligned(16))) uint16_t sHh[HPW][P * HSH];   // state entering the chunk, hi
    __shared__ __attribute__((aligned(16))) uint16_t sHl[HPW][P * HSH];   // ... lo

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hs = w >> 2;               // head slot
    // role within the head: the second head takes the roles in reverse, so
    // that the two waves sharing a SIMD (w and w + 4) pair a short and a long
    // causal triangle
    const int wl = hs ? 3 - (w & 3) : (w & 3);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int I0 = 16 * wl;              // this wave's output tokens within a chunk
    // Output channel order: row m of p tile pt of the readout's and the
    // masked product's outputs is channel PW (m / 4) + 4 pt + m % 4, so that
    // the output accumulator rows 4 g4 .. 4 g4 + 3 of all tiles are the PW
    // contiguous channels PW g4 .. PW g4 + PW - 1. The state and its update
    // keep the natural order (row m of tile pt is channel 16 pt + m). The raw
    // x rows in LDS hold channel PW a + 4 pt + r in column xcol = 16 pt + 4 a + r,
    // and the state's bf16 copy puts channel c in row hrow(c): both are then
    // read in the output order with natural addressing.
    constexpr int PW = P / 4;
    auto hrow = [](int c) { return 16 * ((c % PW) >> 2) + 4 * (c / PW) + (c & 3); };
    // column swizzle of the state copy: the 64-byte column blocks of a row
    // are permuted by bits of its row index / 16, which spreads the writes
    // of a wave (rows 16 apart) over the banks
    constexpr int SWZ = kSsdSwizzle & (N / 32 - 1);
    auto hcol = [](int R, int col) { return col ^ (32 * ((R >> 4) & SWZ)); };

    const int nb = gridDim.x, bid = blockIdx.x;
    const int qx = nb / kXcds, rx = nb % kXcds, xcd = bid % kXcds;
    const int logical = xcd * qx + min(xcd, rx) + bid / kXcds;
    const int hpb = p.H / HPW;
    const int b = logical / hpb;
    const int h = (logical % hpb) * HPW + hs;
    const int grp = h / p.hpg;

    const float a = p.A[h];
    const float a2 = a * kLog2e;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float dskip = p.D ? p.D[h] : 0.0f;
    const int64_t L = p.L;
    const int64_t xs = (int64_t)p.H * P;   // token stride of x, z, y
    const int64_t bs = (int64_t)p.G * N;   // token stride of B, C
    // (64 token rows of x and of B fit 32-bit element offsets: the library checks it)
    const uint32_t xs32 = (uint32_t)xs, bs32 = (uint32_t)bs, H32 = (uint32_t)p.H;
    const uint16_t *xb = p.x + (int64_t)b * L * xs + (int64_t)h * P;
    const uint16_t *zb = p.z ? p.z + (int64_t)b * L * xs + (int64_t)h * P : nullptr;
    uint16_t *yb = p.y + (int64_t)b * L * xs + (int64_t)h * P;
    const uint16_t *Bb = p.B + (int64_t)b * L * bs + (int64_t)grp * N;
    const uint16_t *Cb = p.C + (int64_t)b * L * bs + (int64_t)grp * N;
    const uint16_t *db = p.dt + (int64_t)b * L * p.H + h;
    uint16_t *const XT = sXT[hs];
    uint16_t *const Xh = sXh[hs];
    uint16_t *const Xl = sXl[hs];
    uint16_t *const Hh = sHh[hs];
    uint16_t *const Hl = sHl[hs];

    // byte offsets of the lane's staging pieces within a chunk; the same for
    // every chunk, whose buffers start at its first token
    uint32_t xoff[Stage::XI], boff[Stage::BI];
#pragma unroll
    for (int k = 0; k < Stage::XI; ++k) {
        const int piece = (wl * Stage::XI + k) * 64 + lane;
        xoff[k] = 2u * ((uint32_t)(piece / Stage::XPR) * xs32 + 8u * (piece % Stage::XPR));
    }
#pragma unroll
    for (int k = 0; k < Stage::BI; ++k) {
        const int piece = (w * Stage::BI + k) * 64 + lane;
        boff[k] = 2u * ((uint32_t)(piece / Stage::BPR) * bs32 + 8u * (piece % Stage::BPR));
    }
    // Valid tokens of the chunk starting at c (0 past the end)
    auto valid_tokens = [&](int64_t c) { return (uint32_t)max<int64_t>(0, min<int64_t>(Q, L - c)); };
    // Staging loads of the chunk starting at c, one chunk ahead: the buffers
    // end at the chunk's last valid token, so rows past the end read as zero
    // and a chunk past the end loads nothing.
    auto load_stage = [&](int64_t c, Stage &st) {
        const uint32_t nv = valid_tokens(c);
        const __amdgpu_buffer_rsrc_t rd = ssd_buffer(db + c * p.H, 2u * nv * H32);
        const __amdgpu_buffer_rsrc_t rxb = ssd_buffer(xb + c * xs, 2u * nv * xs32);
        const __amdgpu_buffer_rsrc_t rbb = ssd_buffer(Bb + c * bs, 2u * nv * bs32);
        st.dt = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)(2u * (uint32_t)lane * H32), 0, 0);
#pragma unroll
        for (int k = 0; k < Stage::XI; ++k)
            st.x[k] = ssd_bload16(rxb, xoff[k]);
#pragma unroll
        for (int k = 0; k < Stage::BI; ++k)
            st.b[k] = ssd_bload16(rbb, boff[k]);
    };

    // State: hacc[i][pt][r] = h[p = 16 pt + r16][n = 16 (wl NTW + i) + 4 g4 + r]; its
    // bf16 copy in LDS is written to rows hrow(p), the order in which the
    // readout's A operand takes its rows.
    ssd_f32x4 hacc[NTW][PT];
    const float *h0b = p.h0 ? p.h0 + ((int64_t)b * p.H + h) * P * N : nullptr;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int n = 16 * (wl * NTW + i) + 4 * g4;
            hacc[i][pt] = h0b ? *reinterpret_cast<const ssd_f32x4 *>(h0b + (16 * pt + r16) * N + n)
                              : ssd_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

    Stage st;
    load_stage(0, st);
    // nothing of the prologue stays in flight into the loop (the loop's wait
    // counts then only see its own loads)
    __builtin_amdgcn_s_waitcnt(0);

    for (int64_t c0 = 0; c0 < L; c0 += Q) {
        const uint32_t nvu = valid_tokens(c0);
        const int nv = (int)nvu;                         // valid tokens in this chunk
        const bool valid = lane < nv;

        // this wave's C rows (operands of the readout and the scores) and
        // gate values, issued before the next chunk's staging loads, so that
        // waiting for them never waits for those; rows past the end read zero
        const __amdgpu_buffer_rsrc_t rc = ssd_buffer(Cb + c0 * bs, 2u * nvu * bs32);
        ssd_bf16x8 cop[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s)
            cop[s] = __builtin_bit_cast(ssd_bf16x8,
                                        ssd_bload16(rc, 2u * ((uint32_t)(I0 + r16) * bs32 + 32 * s + 8 * g4)));
        const __amdgpu_buffer_rsrc_t rz = ssd_buffer(zb ? zb + c0 * xs : xb, zb ? 2u * nvu * xs32 : 0u);
        uint4 zop[PT / 2];
#pragma unroll
        for (int k = 0; k < PT / 2; ++k)
            zop[k] = ssd_bload16(rz, 2u * ((uint32_t)(I0 + r16) * xs32 + PW * g4 + 8 * k));

        // the state entering this chunk, as hi + lo bf16 (every wave has
        // finished reading the previous one: barrier at the end of the last chunk)
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                uint2 hi, lo;
                ssd_split2(hacc[i][pt][0], hacc[i][pt][1], hi.x, lo.x);
                ssd_split2(hacc[i][pt][2], hacc[i][pt][3], hi.y, lo.y);
                const int R = hrow(16 * pt + r16);
                const int o = R * HSH + hcol(R, 16 * (wl * NTW + i) + 4 * g4);
                *reinterpret_cast<uint2 *>(&Hh[o]) = hi;
                *reinterpret_cast<uint2 *>(&Hl[o]) = lo;
            }

        // step, decay and input weight of token `lane` (every wave of a head computes all 64)
        float step = 0.0f;
        if (valid) {
            step = ssd_bf(st.dt) + bias;
            if (p.dt_softplus)
                step = softplus_f(step);
        }
        const float la = step * a2;                 // log2 of the token's decay
        float wbar = step;
        if (ZOH)
            wbar = step * expm1_over_x(step * a, __builtin_amdgcn_exp2f(la));
        const float S = ssd_prefix_sum(la, lane);    // inclusive prefix sum over the chunk
        const float Slast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, S), 63));
        const float fd = wbar * __builtin_amdgcn_exp2f(Slast - S);

        // stage x (raw, in the output channel order, and weighted for the
        // state update as hi + lo) and B as token rows, one 16-byte piece per
        // lane and load. Products over tokens read these rows with
        // transposing LDS reads.
#pragma unroll
        for (int k = 0; k < Stage::XI; ++k) {
            const int piece = (wl * Stage::XI + k) * 64 + lane;
            const int t = piece / Stage::XPR;
            const int col = 8 * (piece % Stage::XPR);
            const float f = __shfl(fd, t);        // the piece's token's weight
            const uint4 v = st.x[k];
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ssd_split2(ssd_bf(wd[e] & 0xffffu) * f, ssd_bf(wd[e] >> 16) * f, hw[e], lw[e]);
            const int o = t * XS + col;
            // channels col .. col + 3 and col + 4 .. col + 7 of the output order
            const int xo = t * XS + 16 * ((col % PW) >> 2) + 4 * (col / PW);
            *reinterpret_cast<uint2 *>(&XT[xo]) = uint2{v.x, v.y};
            *reinterpret_cast<uint2 *>(&XT[xo + 16]) = uint2{v.z, v.w};
            *reinterpret_cast<uint4 *>(&Xh[o]) = uint4{hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<uint4 *>(&Xl[o]) = uint4{lw[0], lw[1], lw[2], lw[3]};
        }
#pragma unroll
        for (int k = 0; k < Stage::BI; ++k) {
            const int piece = (w * Stage::BI + k) * 64 + lane;
            *reinterpret_cast<uint4 *>(&sBR[(piece / Stage::BPR) * HS + 8 * (piece % Stage::BPR)]) = st.b[k];
        }
        // the next chunk's staging loads (nothing past the end)
        load_stage(c0 + Q, st);
        __syncthreads();

        // The rest of the chunk, specialised on the wave's role so that each
        // role is straight-line code the scheduler can interleave.
        auto compute = [&](auto role) {
            constexpr int WL = decltype(role)::value;
            constexpr int IW = 16 * WL;
            // ---- outputs of tokens [IW, IW + 16): lane column i = IW + r16
            const float Si = __shfl(S, IW + r16);

            // readout of the state entering the chunk (hi + lo)
            ssd_f32x4 yacc[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                yacc[pt] = ssd_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < NK; ++s) {
                    const int R = 16 * pt + r16;
                    const int o = R * HSH + hcol(R, 32 * s + 8 * g4);
                    yacc[pt] = ssd_mfma(ssd_ld16(&Hh[o]), cop[s], yacc[pt]);
                    yacc[pt] = ssd_mfma(ssd_ld16(&Hl[o]), cop[s], yacc[pt]);
                }
            }
            {
                const float ei = __builtin_amdgcn_exp2f(Si);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    yacc[pt] *= ei;
            }

            // scheduling fence: keeps the scheduler from hoisting this phase's
            // operand loads into the previous one past the register budget
            __builtin_amdgcn_sched_barrier(0);
            // scores of key tiles J <= WL, decayed, weighted, masked, as hi + lo
            // operands: element 4 (J%2) + r of m*[J/2] is M^T[16 J + 4 g4 + r][i]
            // (packed two to a word)
            uint32_t mh[2][4], ml[2][4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J <= WL) {
                    ssd_f32x4 gt = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < NK; ++s)
                        gt = ssd_mfma(ssd_ld16(&sBR[(16 * J + r16) * HS + 32 * s + 8 * g4]), cop[s], gt);
                    float m[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int jj = 16 * J + 4 * g4 + r;
                        const float Sj = __shfl(S, jj);
                        const float wj = __shfl(wbar, jj);
                        const bool keep = J < WL || 4 * g4 + r <= r16;
                        m[r] = keep ? gt[r] * __builtin_amdgcn_exp2f(Si - Sj) * wj : 0.0f;
                    }
                    ssd_split2(m[0], m[1], mh[J >> 1][2 * (J & 1)], ml[J >> 1][2 * (J & 1)]);
                    ssd_split2(m[2], m[3], mh[J >> 1][2 * (J & 1) + 1], ml[J >> 1][2 * (J & 1) + 1]);
                } else if ((J & 1) && J - 1 <= WL) {
                    // odd key tile past the diagonal, paired with a computed one: zeros
                    mh[J >> 1][2] = mh[J >> 1][3] = 0u;
                    ml[J >> 1][2] = ml[J >> 1][3] = 0u;
                }
            }
#pragma unroll
            for (int Jp = 0; Jp < 2; ++Jp) {
                if (2 * Jp <= WL) {
                    const ssd_bf16x8 mhv = __builtin_bit_cast(ssd_bf16x8, uint4{mh[Jp][0], mh[Jp][1], mh[Jp][2], mh[Jp][3]});
                    const ssd_bf16x8 mlv = __builtin_bit_cast(ssd_bf16x8, uint4{ml[Jp][0], ml[Jp][1], ml[Jp][2], ml[Jp][3]});
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        // x^T operand in the K order of mh / ml: tokens
                        // 32 Jp + 4 g4 + e, then 32 Jp + 16 + 4 g4 + e
                        const uint16_t *src = &XT[(32 * Jp + 4 * g4 + (r16 >> 2)) * XS + 16 * pt + 4 * (r16 & 3)];
                        const ssd_bf16x8 xo = ssd_ld_tr2(src, src + 16 * XS);
                        yacc[pt] = ssd_mfma(xo, mhv, yacc[pt]);
                        yacc[pt] = ssd_mfma(xo, mlv, yacc[pt]);
                    }
                }
            }

            // skip, gate, store: yacc[pt][r] = y[i][p = PW g4 + 4 pt + r], so
            // the lane's PW outputs are contiguous and leave in 16-byte
            // pieces; rows past the end are dropped by the buffer's range
            const __amdgpu_buffer_rsrc_t ry = ssd_buffer(yb + c0 * xs, 2u * nvu * xs32);
#pragma unroll
            for (int k = 0; k < PT / 2; ++k) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = yacc[2 * k + (e >> 2)][e & 3];
                if (p.D) {
                    // x of channels PW g4 + 8 k + e from the raw rows (output order)
                    const uint16_t *xr = &XT[(IW + r16) * XS + 32 * k + 4 * g4];
                    const uint2 x0 = *reinterpret_cast<const uint2 *>(xr);
                    const uint2 x1 = *reinterpret_cast<const uint2 *>(xr + 16);
                    const uint32_t xw[4] = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] += dskip * ssd_bf(e & 1 ? xw[e >> 1] >> 16 : xw[e >> 1] & 0xffffu);
                }
                if (zb) {
                    const uint32_t zw[4] = {zop[k].x, zop[k].y, zop[k].z, zop[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] *= silu(ssd_bf(e & 1 ? zw[e >> 1] >> 16 : zw[e >> 1] & 0xffffu));
                }
                const uint4 o = {ssd_pack(v[0], v[1]), ssd_pack(v[2], v[3]), ssd_pack(v[4], v[5]),
                                 ssd_pack(v[6], v[7])};
                ssd_bstore16(ry, 2u * ((uint32_t)(IW + r16) * xs32 + PW * g4 + 8 * k), o);
            }

            __builtin_amdgcn_sched_barrier(0);   // (likewise)
            // ---- state update of rows [WL NW, (WL+1) NW)
            {
                const float dec = __builtin_amdgcn_exp2f(Slast);
#pragma unroll
                for (int i = 0; i < NTW; ++i)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
                        hacc[i][pt] *= dec;
#pragma unroll
                for (int ks = 0; ks < Q / 32; ++ks) {
                    ssd_bf16x8 bop[NTW];
#pragma unroll
                    for (int i = 0; i < NTW; ++i)
                        bop[i] = ssd_ld_tr2(&sBR[(32 * ks + 8 * g4 + (r16 >> 2)) * HS + 16 * (WL * NTW + i) + 4 * (r16 & 3)],
                                            &sBR[(32 * ks + 8 * g4 + 4 + (r16 >> 2)) * HS + 16 * (WL * NTW + i) + 4 * (r16 & 3)]);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const int o = (32 * ks + 8 * g4 + (r16 >> 2)) * XS + 16 * pt + 4 * (r16 & 3);
                        const ssd_bf16x8 xh = ssd_ld_tr2(&Xh[o], &Xh[o + 4 * XS]);
                        const ssd_bf16x8 xl = ssd_ld_tr2(&Xl[o], &Xl[o + 4 * XS]);
#pragma unroll
                        for (int i = 0; i < NTW; ++i) {
                            hacc[i][pt] = ssd_mfma(bop[i], xh, hacc[i][pt]);
                            hacc[i][pt] = ssd_mfma(bop[i], xl, hacc[i][pt]);
                        }
                    }
                }
            }
        };
        switch (wl) {
        case 0: compute(std::integral_constant<int, 0>{}); break;
        case 1: compute(std::integral_constant<int, 1>{}); break;
        case 2: compute(std::integral_constant<int, 2>{}); break;
        default: compute(std::integral_constant<int, 3>{}); break;
        }
        __syncthreads();
    }

    if (p.h_last) {
        float *hl = p.h_last + ((int64_t)b * p.H + h) * P * N;
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
                *reinterpret_cast<ssd_f32x4 *>(hl + (16 * pt + r16) * N + 16 * (wl * NTW + i) + 4 * g4) = hacc[i][pt];
    }
}

// Two heads per workgroup when the LDS of two fits (head size 64) and they
// share a group; otherwise one.
template <int P, int N, bool ZOH>
hipError_t launch_ssd_pn(const SsdParams &p, hipStream_t st) {
    if (P == 64 && p.hpg % 2 == 0) {
        const int64_t blocks = (int64_t)p.batch * (p.H / 2);
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, (P == 64 ? 2 : 1)>), dim3((unsigned)blocks),
                           dim3(kSsdThreads * (P == 64 ? 2 : 1)), 0, st, p);
    } else {
        const int64_t blocks = (int64_t)p.batch * p.H;
        hipLaunchKernelGGL((ssd_fwd_kernel<P, N, ZOH, 1>), dim3((unsigned)blocks), dim3(kSsdThreads), 0, st, p);
    }
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
