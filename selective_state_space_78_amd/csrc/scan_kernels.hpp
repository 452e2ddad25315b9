// Scan kernels of the gfx950 selective-scan library, shared by the
// translation units that instantiate them (one per element type and
// discretisation, compiled in parallel) and by the ABI unit.
//
// Kernel design (the scan):
//  * One workgroup owns a tile of 64 consecutive channels of one batch row and
//    one time segment. Lane = channel. The workgroup has G waves; wave w owns
//    NPW = Npad/G of the states of all 64 channels, so a lane keeps its NPW
//    states h[n] in VGPRs for the whole segment, and B_t[n], C_t[n] are the
//    same for every lane of the wave: they are read with scalar loads into
//    SGPRs and used directly as instruction operands. Splitting states over
//    waves multiplies the parallelism of a channel tile by G at the cost of a
//    few per-token instructions, instead of splitting time, which would cost
//    a second pass of the recurrence.
//  * A prologue copies B and C once into the workspace, regrouped so that one
//    wave's values are contiguous in time (and padded with zero rows and
//    states), so that a few wide scalar loads fetch a batch of steps and are
//    waited for once: scalar and LDS reads share one wait counter, and a
//    scalar load per step would expose its latency at every LDS wait. bf16
//    B_t[n] and C_t[n] share one 32-bit word (the scalar unit splits it), so a
//    chunk's values fit in 32 SGPRs; fp32 values take a word each.
//  * Time is walked in chunks of TC tokens with one barrier per chunk. While
//    the waves scan chunk k, every thread of the workgroup also stages a
//    piece (2 or 4 channels) of chunk k+1: it loads u, delta and z two chunks
//    ahead into registers, writes (delta, delta*u) pairs into LDS for all
//    waves, and keeps D*u and silu(z) in registers; and it finalizes its
//    piece of chunk k-1. Every per-token product shared by the states is so
//    formed once. The expanded (t, d, n) decay and input terms exist only in
//    registers and are never written.
//  * Each wave writes its partial readout sum_{n in wave} C_t[n] h_t[n] per
//    (t, channel) to its own LDS plane; one chunk later every thread adds the
//    G planes of its piece and the skip, applies the gate, rounds to the
//    output type and stores its channels at once. Pairs and planes are
//    double-buffered by chunk parity. (Sharing planes through LDS float
//    atomics was measured several times slower.)
//  * Long sequences with few channels are split into S segments. An
//    aggregate pass computes, per segment, the affine map h -> P*h + H that
//    the segment applies to its incoming state (P = exp(A * sum delta),
//    H = end state from zero); a carry pass composes those maps with a
//    wave-level Kogge-Stone scan over (P, H) pairs built from DPP row shifts
//    and row broadcasts; the main pass then scans every segment from its true
//    initial state. Associativity of (a1,b1).(a2,b2) = (a2 a1, a2 b1 + b2) is
//    what makes this exact up to rounding (ricepunchb "Mamba" §5.1 Parallel
//    Scan).
//  * Workgroup ids are remapped so that the tiles of one batch row (which
//    share the B and C rows) run on the same XCD and hit the same L2.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "ssm_scan.h"

namespace ssm_detail {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;        // channels per workgroup tile = lanes per wave
constexpr int kXcds = 8;         // MI355X: 8 accelerator complex dies
constexpr int kMaxSegments = 64;
constexpr int kPadRows = 32;     // spare zero rows after the widened B and C (>= every TC, the aggregate pass's too)
constexpr int kConvMax = 4;      // widest convolution prologue

// ---------------------------------------------------------------------------
// Element access. bf16 travels as its 16-bit pattern.

template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    __device__ static float widen(float v) { return v; }
};

template <> struct Elem<uint16_t> {
    static constexpr int kBytes = 2;
    __device__ static float widen(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
    // round to bf16 (nearest even, v_cvt_pk_bf16_f32)
    __device__ static uint16_t to_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
};

__device__ __forceinline__ float silu(float z) {
    // z * sigmoid(z) = z / (1 + 2^(-z log2 e))
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// softplus(x) = log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|)). log1p(e) is
// taken as log(u) * e / (u - 1) with u = 1 + e, which cancels the rounding of
// 1 + e, so a tiny e keeps its relative precision.
__device__ __forceinline__ float softplus_f(float x) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float u = 1.0f + e;
    const float dd = u - 1.0f;
    const float l = dd == 0.0f ? e : __builtin_amdgcn_logf(u) * 0.69314718055994531f * (e * __builtin_amdgcn_rcpf(dd));
    return fmaxf(x, 0.0f) + l;
}

// The zero-order-hold input coefficient (exp(x) - 1)/x for x = delta*A (so the
// held input term is phi * delta * B * u), given a = exp(x) as the decay
// already computes it. |x| < 0.1: Taylor series to x^3 (truncation below
// 8.4e-7 relative; x = 0, i.e. A = 0, gives 1, the limit); otherwise
// (a - 1)/x, where the rounding of a costs at most 6.8e-7 relative (2.7e-7
// at |x| = 0.25, growing as 1/|x|). The threshold balances the two.
__device__ __forceinline__ float expm1_over_x(float x, float a) {
    float p = fmaf(x, 1.0f / 24.0f, 1.0f / 6.0f);
    p = fmaf(x, p, 0.5f);
    p = fmaf(x, p, 1.0f);
    const float q = (a - 1.0f) * __builtin_amdgcn_rcpf(x);
    return fabsf(x) < 0.1f ? p : q;
}

struct ScanParams {
    const void *u, *delta, *z, *B, *C;
    const float *delta_bias;  // (dim) added to delta before the recurrence uses it, or null
    int delta_softplus;       // the step is softplus(delta + bias)
    const float *A, *D, *h0;
    float *Bf, *Cf;       // (batch, G, padded_len(L), Npad/G) fp32 widened B and C (workspace)
    const float *seg_h;   // (batch, nseg, dim, N) initial state of each segment, or null
    void *y;
    float *h_last;
    float *agg_P, *agg_H; // (batch, nseg, dim, N) segment maps (aggregate pass)
    float *ckpt;          // (batch, nck, Npad, dim) state at the start of every chunk (checkpoint pass)
    int nck;
    int64_t L;
    int batch, dim, N;
    int seg_len, nseg;
    int ntiles;
    int vec;              // u, delta, z, y move 4 channels per aligned access
    int u_f32;            // u is fp32 whatever T is (the convolution prologue's output,
                          // materialised by its own pass): the scan_bf16_*_u32 units
};

struct Plan {
    int npad, G, npw, S, seg_len;
};

// Workspace layout for a plan: widened B and C, then (segments > 1) the
// segment maps and segment initial states. Offsets in bytes, 256-aligned.
struct WorkspaceLayout {
    size_t bf, cf, agg_p, agg_h, seg_h, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Tokens per batch row in the widened B and C: L rounded up to 16, plus
// kPadRows spare zero rows (keeps every chunk's run 64-byte aligned).
__host__ __device__ inline int64_t padded_len(int64_t L) { return (L + 15) / 16 * 16 + kPadRows; }

inline WorkspaceLayout workspace_layout(int64_t batch, int64_t L, int64_t dim, int64_t N, const Plan &pl) {
    WorkspaceLayout w{};
    const size_t bc = align256((size_t)batch * padded_len(L) * pl.npad * sizeof(float));
    const size_t seg = pl.S > 1 ? align256((size_t)batch * pl.S * dim * N * sizeof(float)) : 0;
    w.bf = 0;
    w.cf = bc;
    w.agg_p = 2 * bc;
    w.agg_h = w.agg_p + seg;
    w.seg_h = w.agg_h + seg;
    w.total = w.seg_h + seg;
    return w;
}

// Launches the prologue, aggregate, carry and main passes for one element
// type and discretisation (defined in the scan_<type>_<disc>.hip units; with
// bf16 tensors and an fp32 u, the scan_bf16_<disc>_u32.hip units).
hipError_t launch_scan_bf16_euler(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_bf16_zoh(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_bf16_euler_u32(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_bf16_zoh_u32(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_f32_euler(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_f32_zoh(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);

inline int ilog2(int v) { int r = 0; while ((1 << r) < v) ++r; return r; }

}  // namespace ssm_detail

#ifdef SSM_SCAN_INSTANTIATE
namespace ssm_detail {
namespace {

typedef const __attribute__((address_space(4))) uint32_t cword;   // scalar-load view

// ---------------------------------------------------------------------------
// Prologue: B and C widened to fp32 and regrouped so that the values one wave
// needs are contiguous in time: (batch, group, t, state-in-group) with Npad
// states split into G groups of NPW, and kPadRows zero rows after each batch
// row's L tokens (and zeros for padded states).

template <typename T>
__global__ __launch_bounds__(256) void widen_bc_kernel(const T *__restrict__ B, const T *__restrict__ C,
                                                       float *__restrict__ Bf, float *__restrict__ Cf,
                                                       int batch, int64_t L, int N, int groups, int npw) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t Lp = padded_len(L);
    const int64_t total = (int64_t)batch * groups * Lp * npw;
    if (i >= total) return;
    const int q = (int)(i % npw);
    int64_t r = i / npw;
    const int64_t t = r % Lp;
    r /= Lp;
    const int g = (int)(r % groups);
    const int64_t b = r / groups;
    const int n = g * npw + q;
    const bool on = t < L && n < N;
    const int64_t src = (b * L + t) * N + n;
    if constexpr (sizeof(T) == 2) {
        // bf16: B and C stay bf16, packed into one word (C in the high half)
        const uint32_t vb = on ? (uint32_t)B[src] : 0u;
        const uint32_t vc = on ? (uint32_t)C[src] : 0u;
        reinterpret_cast<uint32_t *>(Bf)[i] = vb | (vc << 16);
    } else {
        Bf[i] = on ? B[src] : 0.0f;
        Cf[i] = on ? C[src] : 0.0f;
    }
}

// Linear workgroup id -> (segment, batch row, channel tile). Consecutive ids
// go round-robin over the XCDs; undo that so that each XCD receives a
// contiguous range of logical ids (tile fastest, then batch row).
__device__ __forceinline__ void map_block(const ScanParams &p, int &seg, int &b, int &tile) {
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int q = nb / kXcds, r = nb % kXcds;
    const int x = bid % kXcds;
    const int logical = x * q + min(x, r) + bid / kXcds;
    tile = logical % p.ntiles;
    const int rest = logical / p.ntiles;
    b = rest % p.batch;
    seg = rest / p.batch;
}

// Raw bits of KV consecutive elements of a per-token tensor (one 4, 8 or
// 16-byte access).
template <int W> struct Words;
template <> struct Words<1> { typedef uint32_t type; };
template <> struct Words<2> { typedef uint2 type; };
template <> struct Words<4> { typedef uint4 type; };

template <int W> __device__ __forceinline__ uint32_t word(const typename Words<W>::type &r, int i);
template <> __device__ __forceinline__ uint32_t word<1>(const uint32_t &r, int) { return r; }
template <> __device__ __forceinline__ uint32_t word<2>(const uint2 &r, int i) { return i == 0 ? r.x : r.y; }
template <> __device__ __forceinline__ uint32_t word<4>(const uint4 &r, int i) {
    return i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w;
}
__device__ __forceinline__ void make_words(uint32_t &r, const uint32_t *w) { r = w[0]; }
__device__ __forceinline__ void make_words(uint2 &r, const uint32_t *w) { r = make_uint2(w[0], w[1]); }
__device__ __forceinline__ void make_words(uint4 &r, const uint32_t *w) { r = make_uint4(w[0], w[1], w[2], w[3]); }

// a < b for values every lane of the wave shares, compared as 32-bit scalars
// right where the branch takes it: a boolean kept across divergent blocks
// would be rebuilt as a lane mask with vector instructions.
__device__ __forceinline__ bool uniform_less(int a, int b) {
    return __builtin_amdgcn_readfirstlane(b - a) > 0;
}

template <int KV> struct FloatsOf;
template <> struct FloatsOf<2> { typedef float2 type; };
template <> struct FloatsOf<4> { typedef float4 type; };

// What a pass of the scan kernel produces.
enum ScanMode { kModeMain = 0, kModeAggregate = 1, kModeCheckpoint = 2, kModeMainCheckpoint = 3 };

// The aggregate and checkpoint-only passes stage no readout planes, so their
// chunks can be longer than the main pass's within the same LDS, for fewer
// barriers per token: twice as long with 4 waves or more (fewer waves would
// hold several times the staged pieces in registers).
template <int G> constexpr int long_chunk_factor() { return G >= 4 ? 2 : 1; }

// With segments (few channels, so few workgroups per segment), the main pass
// of an 8-wave tile runs in chunks half as long: a quarter of the LDS, so four
// workgroups fit per CU instead of two, and a segmented plan's workgroups are
// resident at once rather than in one and a half rounds.
template <int G, int TC> constexpr int seg_main_tc() { return G == 8 ? TC / 2 : TC; }

// FEAT: the step options (delta bias, softplus) are compiled in; without it
// the kernel carries none of their state (their uniform values alone pushed
// the scalar registers into spills).
template <typename T, int NPW, int G, int TC, bool ZOH, int MODE, bool FEAT, bool UF = false>
struct ScanKernel {
    // main: y and h_last; aggregate: each segment's map h -> P h + H;
    // checkpoint: the state at the start of every chunk (for the backward);
    // main with checkpoints: both y, h_last and those states
    static constexpr bool kMain = MODE == kModeMain || MODE == kModeMainCheckpoint;
    static constexpr bool kCkpt = MODE == kModeCheckpoint || MODE == kModeMainCheckpoint;
    static constexpr bool AGG = !kMain;                       // no readout and no y
    static constexpr bool kSum = MODE == kModeAggregate;
    // Checkpoint spacing in tokens: the backward's chunk, which is the main
    // pass's; the checkpoint-only pass runs in longer chunks (see
    // long_chunk_factor) and stores that many checkpoints per chunk.
    static constexpr int kCkEvery = MODE == kModeCheckpoint ? TC / long_chunk_factor<G>() : TC;
    static constexpr int kThreads = kTile * G;
    static constexpr int kNP = NPW * G;                       // padded state count
    // channels per staged piece: 2 when that gives every thread of the
    // workgroup a piece of the chunk, else 4
    static constexpr int kV = TC * kTile >= 4 * kThreads ? 4 : 2;
    static constexpr int kWords = kV * (int)sizeof(T) / 4;
    static constexpr int kRowPieces = kTile / kV;              // pieces per 64-channel row
    static constexpr int kPieces = TC * kRowPieces;            // pieces per chunk per tensor
    static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
    static constexpr int kRowStep = kThreads / kRowPieces;      // rows between a thread's pieces
    static_assert(kThreads % kRowPieces == 0, "a thread keeps the same channels in every piece");
    static_assert(TC <= kPadRows, "spare rows of the widened B and C");
    typedef typename Words<kWords>::type Raw;
    // a piece of u: T words, or kV fp32 words when u is fp32 (UF)
    typedef typename Words<UF ? kV : kWords>::type URaw;
    typedef typename FloatsOf<kV>::type VecF;

    // LDS: the staged chunk as (delta, delta*u) pairs (u instead of delta*u
    // for the hold rule), and one partial-readout plane per wave, both
    // double-buffered by chunk parity: while the waves scan chunk k, the
    // staging threads read chunk k-1's planes and write chunk k+1's pairs,
    // so one barrier per chunk orders everything.
    struct __align__(16) Smem {
        union {
            float2 dx[2][TC][kTile];
            // aggregate pass, after the last chunk: the staging threads' step sums
            double dred[kSum ? kRowStep : 1][kSum ? kTile : 1];
        };
        float y[AGG ? 1 : 2][AGG ? 1 : G][AGG ? 1 : TC][AGG ? 1 : kTile];
    };
    static_assert(sizeof(Smem) <= 81920, "two workgroups per CU in 160 KiB of LDS");

    struct Prefetch {
        URaw u[kPPT];
        Raw dt[kPPT], z[kPPT];
    };

    // D*u and silu(z) of the thread's staged pieces, kept in registers until
    // the same thread finalizes those outputs
    struct Held {
        float sk[kPPT][kV], g[kPPT][kV];
    };

    __device__ static int piece_row(int j) { return threadIdx.x / kRowPieces + j * kRowStep; }
    __device__ static bool piece_in_chunk(int j) { return kPieces % kThreads == 0 || piece_row(j) < TC; }

    // Element-wise load of one piece (unaligned tensors), zero past dim.
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

    // Element-wise load of one fp32 piece of u (UF), zero past dim.
    __device__ static URaw gather_f32(const float *src, int c0, int dim) {
        uint32_t w[kV];
#pragma unroll
        for (int i = 0; i < kV; ++i) w[i] = c0 + i < dim ? __float_as_uint(src[i]) : 0u;
        URaw r;
        make_words(r, w);
        return r;
    }

    __device__ static void unpack_u(const URaw &r, float (&v)[kV]) {
        if constexpr (UF) {
#pragma unroll
            for (int i = 0; i < kV; ++i) v[i] = __uint_as_float(word<kV>(r, i));
        } else {
            unpack(r, v);
        }
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

    // Issue the global loads of one chunk: `base` is the element offset of
    // (the chunk's first token row, the tile's first channel); rows [0, tval).
    __device__ static void load(const ScanParams &p, Prefetch &pf, int64_t base, int tval, int col, int d0,
                                bool colv) {
        const T *u = static_cast<const T *>(p.u) + base;
        const T *dt = static_cast<const T *>(p.delta) + base;
        const bool gate = !AGG && p.z != nullptr;
        // without a gate the z slot reloads delta (its value is not used), so
        // that the aligned path loads unconditionally
        const T *z = static_cast<const T *>(gate ? p.z : p.delta) + base;
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int row = piece_row(j);
            if (!piece_in_chunk(j) || row >= tval || !colv) continue;
            const uint32_t off = (uint32_t)row * (uint32_t)p.dim + (uint32_t)col;
            if (p.vec) {
                if constexpr (UF)
                    pf.u[j] = *reinterpret_cast<const URaw *>(static_cast<const float *>(p.u) + base + off);
                else
                    pf.u[j] = *reinterpret_cast<const Raw *>(u + off);
                pf.dt[j] = *reinterpret_cast<const Raw *>(dt + off);
                pf.z[j] = *reinterpret_cast<const Raw *>(z + off);
            } else {
                if constexpr (UF)
                    pf.u[j] = gather_f32(static_cast<const float *>(p.u) + base + off, d0 + col, p.dim);
                else
                    pf.u[j] = gather(u + off, d0 + col, p.dim, true);
                pf.dt[j] = gather(dt + off, d0 + col, p.dim, true);
                pf.z[j] = gather(z + off, d0 + col, p.dim, gate);
            }
        }
    }

    // Stage the prefetched chunk into LDS buffer `dx`, forming the per-token
    // products once for all states, and keep D*u and silu(z) in `held`. Rows
    // past tval (and channels past dim) are staged as delta = 0, x = 0: a step
    // that leaves the state unchanged.
    __device__ static void commit(const Prefetch &pf, float2 (*dx)[kTile], Held &held, int tval, int col,
                                  bool colv, const float (&Dk)[kV], bool gate, const float (&dbk)[kV], int prep,
                                  double (&dsum)[kV]) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int row = piece_row(j);
            if (!piece_in_chunk(j)) continue;
            float4 *dst = reinterpret_cast<float4 *>(&dx[row][col]);
            if (row < tval && colv) {
                float u[kV], d[kV];
                unpack_u(pf.u[j], u);
                unpack(pf.dt[j], d);
                if (FEAT && prep) {
                    // the step: delta + bias, through softplus when asked
#pragma unroll
                    for (int e = 0; e < kV; ++e) d[e] = prep == 2 ? softplus_f(d[e] + dbk[e]) : d[e] + dbk[e];
                }
#pragma unroll
                for (int e = 0; e < kV; e += 2)
                    dst[e / 2] = make_float4(d[e], ZOH ? u[e] : d[e] * u[e], d[e + 1], ZOH ? u[e + 1] : d[e + 1] * u[e + 1]);
                if constexpr (kSum) {
                    // the segment's sum of steps, once per (token, channel), in fp64
#pragma unroll
                    for (int e = 0; e < kV; ++e) dsum[e] += (double)d[e];
                }
                if constexpr (!AGG) {
#pragma unroll
                    for (int e = 0; e < kV; ++e) held.sk[j][e] = Dk[e] * u[e];
                    if (gate) {
                        float z[kV];
                        unpack(pf.z[j], z);
#pragma unroll
                        for (int e = 0; e < kV; ++e) held.g[j][e] = silu(z[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < kV; ++e) held.g[j][e] = 1.0f;
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < kV; e += 2) dst[e / 2] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }

    // For the thread's pieces of one chunk: add the G partial-readout planes
    // and the skip, apply the gate, round and store y (one access per piece).
    // yb points at (the chunk's first token row, the tile's first channel).
    __device__ static void finalize(const ScanParams &p, const float (*planes)[TC][kTile], const Held &held,
                                    T *yb, int tval, int col, int d0) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int row = piece_row(j);
            if (!piece_in_chunk(j) || row >= tval || d0 + col >= p.dim) continue;
            float acc[kV];
            {
                const VecF v = *reinterpret_cast<const VecF *>(&planes[0][row][col]);
                const float *pv = reinterpret_cast<const float *>(&v);
#pragma unroll
                for (int e = 0; e < kV; ++e) acc[e] = pv[e];
            }
#pragma unroll
            for (int g = 1; g < G; ++g) {
                const VecF v = *reinterpret_cast<const VecF *>(&planes[g][row][col]);
                const float *pv = reinterpret_cast<const float *>(&v);
#pragma unroll
                for (int e = 0; e < kV; ++e) acc[e] += pv[e];
            }
            float o[kV];
#pragma unroll
            for (int e = 0; e < kV; ++e) o[e] = (acc[e] + held.sk[j][e]) * held.g[j][e];
            T *dst = yb + (uint32_t)row * (uint32_t)p.dim + col;
            if constexpr (sizeof(T) == 2) {
                typedef float f2v __attribute__((ext_vector_type(2)));
                typedef __bf16 b2v __attribute__((ext_vector_type(2)));
                uint32_t w[kWords];
#pragma unroll
                for (int i = 0; i < kWords; ++i) {
                    const f2v pr = {o[2 * i], o[2 * i + 1]};
                    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2v));
                }
                if (p.vec) {
                    Raw r;
                    make_words(r, w);
                    *reinterpret_cast<Raw *>(dst) = r;
                } else {
#pragma unroll
                    for (int e = 0; e < kV; ++e)
                        if (d0 + col + e < p.dim) dst[e] = (uint16_t)(e & 1 ? w[e / 2] >> 16 : w[e / 2] & 0xffffu);
                }
            } else {
                if (p.vec) {
                    VecF v;
                    float *pv = reinterpret_cast<float *>(&v);
#pragma unroll
                    for (int e = 0; e < kV; ++e) pv[e] = o[e];
                    *reinterpret_cast<VecF *>(dst) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < kV; ++e)
                        if (d0 + col + e < p.dim) dst[e] = o[e];
                }
            }
        }
    }

    struct Lane {
        float A2[NPW], h[NPW];
        float Az[ZOH ? NPW : 1];
    };

    // B_t[n] and C_t[n] reach the wave as scalar words: for bf16 inputs one
    // word holds both (B low, C high) and the scalar unit splits them; fp32
    // inputs take a word each.
    static constexpr bool kPacked = sizeof(T) == 2;
    static constexpr int kWPS = kPacked ? 1 : 2;               // words per state and step
    // Steps whose B and C words are fetched together: at most 32 scalar
    // registers for packed words (which leaves room for most of the rest of
    // the kernel's scalars), 64 for fp32 words. With the step options 16 would
    // avoid a few scalar spills, but fetching twice per chunk measured slower
    // (1.20 against 1.16 ms on the 1.4B-shaped layer with the softplus step).
    static constexpr int kBudget = kPacked ? 32 : 64;
    static constexpr int kTBMax = kBudget / (kWPS * NPW) > 0 ? kBudget / (kWPS * NPW) : 1;
    static constexpr int kTB = kTBMax < TC ? kTBMax : TC;
    static_assert(TC % kTB == 0, "batches of steps tile the chunk");

    __device__ static __forceinline__ float b_of(const uint32_t (&w)[kWPS]) {
        return __uint_as_float(kPacked ? w[0] << 16 : w[0]);
    }
    __device__ static __forceinline__ float c_of(const uint32_t (&w)[kWPS]) {
        return __uint_as_float(kPacked ? w[0] & 0xffff0000u : w[kWPS - 1]);
    }

    // One token of this wave's states: update, and return the partial readout.
    // bc: the wave's B_t and C_t words (uniform, in scalar registers).
    __device__ static __forceinline__ float step(Lane &l, const float2 (*dx)[kTile], int t, int lane,
                                                 const uint32_t (&bc)[NPW][kWPS]) {
        const float2 v = dx[t][lane];
        const float dd = v.x;
        const float xx = v.y;
        const float du = ZOH ? dd * xx : 0.0f;       // hold rule: xx is u
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < NPW; ++q) {
            const float bq = b_of(bc[q]);
            if constexpr (ZOH) {
                const float a = __builtin_amdgcn_exp2f(dd * l.A2[q]);
                const float ph = expm1_over_x(dd * l.Az[q], a);
                l.h[q] = fmaf(a, l.h[q], ph * (du * bq));
            } else {
                const float a = __builtin_amdgcn_exp2f(dd * l.A2[q]);
                l.h[q] = fmaf(a, l.h[q], xx * bq);
            }
            if (!AGG) part = q == 0 ? c_of(bc[q]) * l.h[q] : fmaf(c_of(bc[q]), l.h[q], part);
        }
        return part;
    }

    __device__ static void run(const ScanParams &p) {
        __shared__ Smem s;
        int seg, b, tile;
        map_block(p, seg, b, tile);
        const int lane = threadIdx.x & (kTile - 1);
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kTile);
        const int d0 = tile * kTile;
        const int d = d0 + lane;
        const bool dval = d < p.dim;
        const int dc = dval ? d : p.dim - 1;
        const int64_t t_begin = (int64_t)seg * p.seg_len;
        const int64_t t_end = min(p.L, t_begin + (int64_t)p.seg_len);
        const bool gate = !AGG && p.z != nullptr;

        // Per-lane constants and initial state of this wave's states.
        Lane l;
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int n = w * NPW + k;
            const bool nv = n < p.N;
            const float a = nv ? p.A[(int64_t)dc * p.N + n] : 0.0f;
            l.A2[k] = a * kLog2e;
            if constexpr (ZOH) l.Az[k] = a;
            float h_init = 0.0f;
            if (MODE != kModeAggregate && nv) {
                // with segments, every segment (also the first) starts from the
                // carry pass's output, so that h_last may alias h0
                if (p.seg_h != nullptr)
                    h_init = p.seg_h[(((int64_t)b * p.nseg + seg) * p.dim + dc) * p.N + n];
                else if (p.h0 != nullptr)
                    h_init = p.h0[((int64_t)b * p.dim + dc) * p.N + n];
            }
            l.h[k] = h_init;
        }
        // This thread stages (and finalizes) channels [col, col + kV) of the tile.
        const int col = (threadIdx.x % kRowPieces) * kV;
        const bool colv = d0 + col < p.dim;
        float Dk[kV], dbk[kV];
#pragma unroll
        for (int e = 0; e < kV; ++e) {
            Dk[e] = (!AGG && p.D != nullptr && d0 + col + e < p.dim) ? p.D[d0 + col + e] : 0.0f;
            dbk[e] = (FEAT && p.delta_bias != nullptr && d0 + col + e < p.dim) ? p.delta_bias[d0 + col + e] : 0.0f;
        }
        // 0: delta as given; 1: plus the bias; 2: softplus of that
        const int prep = !FEAT ? 0 : p.delta_softplus ? 2 : (p.delta_bias != nullptr ? 1 : 0);

        // the segment's tokens: at most seg_len, an int (32-bit arithmetic
        // keeps the per-chunk row counts on the scalar unit)
        const int seg_rows = (int)(t_end - t_begin);
        const int nchunks = (seg_rows + TC - 1) / TC;
        const int64_t row0 = (int64_t)b * p.L + t_begin;        // token row of (b, t_begin)
        auto rows_of = [&](int k) { return min(TC, seg_rows - k * TC); };
        Prefetch pf;
        Held held[2];                                            // by chunk parity
        double dsum[kV];                                         // aggregate pass: this thread's staged steps
#pragma unroll
        for (int e = 0; e < kV; ++e) dsum[e] = 0.0;
        auto load_chunk = [&](int k) {
            load(p, pf, (row0 + (int64_t)k * TC) * p.dim + d0, rows_of(k), col, d0, colv);
        };
        if (nchunks > 0) {
            load_chunk(0);
            commit(pf, s.dx[0], held[0], rows_of(0), col, colv, Dk, gate, dbk, prep, dsum);
        }
        if (nchunks > 1) load_chunk(1);
        __syncthreads();

        // this wave's B and C words: NPW (x kWPS) per token, contiguous in time
        const int64_t grp = ((int64_t)b * G + w) * padded_len(p.L) + t_begin;
        cword *bw = (cword *)(p.Bf) + grp * NPW;
        cword *cw = (cword *)(p.Cf) + grp * NPW;
        T *yb = AGG ? nullptr : static_cast<T *>(p.y) + row0 * p.dim + d0;

        // B and C of a batch of kTB steps, fetched with a few wide scalar loads
        // and waited for once. Scalar and LDS reads share one wait counter, so
        // the first batch of a chunk is requested between the LDS wait and the
        // barrier that close the chunk before it: its latency then overlaps the
        // barrier, and it lands before the first LDS wait of its chunk.
        uint32_t bc[kTB][NPW][kWPS];
        auto fetch = [&](int t0b) {
#pragma unroll
            for (int i = 0; i < kTB; ++i)
#pragma unroll
                for (int q = 0; q < NPW; ++q) {
                    bc[i][q][0] = bw[(t0b + i) * NPW + q];
                    if constexpr (!kPacked) bc[i][q][kWPS - 1] = AGG ? 0u : cw[(t0b + i) * NPW + q];
                }
        };

        // Chunk k (parity P): stage chunk k+1's inputs, store chunk k-1's
        // outputs, scan chunk k, then one barrier (with chunk k+1's first B and
        // C requested just before it).
        if (nchunks > 0) fetch(0);
        auto chunk = [&](auto parity, int k) {
            constexpr int P = decltype(parity)::value;
            if constexpr (!AGG) {
                // chunk k-1's outputs first: its skip and gate then make room
                // for chunk k+1's in the same registers
                if (k > 0) {
                    finalize(p, s.y[P ^ 1], held[P ^ 1], yb, TC, col, d0);
                    yb += (int64_t)TC * p.dim;
                }
            }
            if (uniform_less(k + 1, nchunks))
                commit(pf, s.dx[P ^ 1], held[P ^ 1], rows_of(k + 1), col, colv, Dk, gate, dbk, prep, dsum);
            if (uniform_less(k + 2, nchunks)) load_chunk(k + 2);
            const int tval = rows_of(k);
            const float2 (*dx)[kTile] = s.dx[P];
            // The recurrence runs at a higher issue priority than the staging
            // work: where a SIMD holds waves in both phases (its two
            // workgroups are rarely in step), the arbiter then feeds the VALU
            // from the recurrence's long dependent chains first, and the
            // staging's loads, LDS traffic and stores fill the gaps.
            __builtin_amdgcn_s_setprio(2);
            // the state before token j of the chunk, where a checkpoint falls
            // (j is a compile-time constant once the loops are unrolled)
            auto checkpoint = [&](int j) {
                if constexpr (kCkpt) {
                    if (j % kCkEvery == 0 && dval) {
                        const int64_t c = (t_begin + (int64_t)k * TC + j) / kCkEvery;
#pragma unroll
                        for (int q = 0; q < NPW; ++q)
                            p.ckpt[(((int64_t)b * p.nck + c) * kNP + w * NPW + q) * p.dim + d] = l.h[q];
                    }
                }
            };
#pragma unroll
            for (int t0b = 0; t0b < TC; t0b += kTB) {
                if (t0b > 0) fetch(t0b);
                if (tval == TC) {
#pragma unroll
                    for (int i = 0; i < kTB; ++i) {
                        checkpoint(t0b + i);
                        const float part = step(l, dx, t0b + i, lane, bc[i]);
                        if constexpr (!AGG) s.y[P][w][t0b + i][lane] = part;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kTB; ++i) {
                        if (t0b + i < tval) {
                            checkpoint(t0b + i);
                            const float part = step(l, dx, t0b + i, lane, bc[i]);
                            if constexpr (!AGG) s.y[P][w][t0b + i][lane] = part;
                        }
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
            bw += TC * NPW;
            cw += TC * NPW;
            // the barrier, as __syncthreads() is, with the next chunk's first
            // fetch after the LDS writes have completed
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            if (uniform_less(k + 1, nchunks)) fetch(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        };
        for (int k = 0; k < nchunks; k += 2) {
            chunk(std::integral_constant<int, 0>(), k);
            if (k + 1 < nchunks) chunk(std::integral_constant<int, 1>(), k + 1);
        }
        if constexpr (!AGG) {
            if (nchunks > 0) {
                const int tl = rows_of(nchunks - 1);
                if ((nchunks - 1) & 1)
                    finalize(p, s.y[1], held[1], yb, tl, col, d0);
                else
                    finalize(p, s.y[0], held[0], yb, tl, col, d0);
            }
        }

        float dtot = 0.0f;
        if constexpr (kSum) {
            // the staging threads' sums of this segment's steps: thread
            // (row group r, channels col..) holds rows r, r + kRowStep, ... of
            // every chunk; every lane adds the groups of its channel in order.
            // (dred aliases dx, which no wave reads after the last chunk's barrier.)
#pragma unroll
            for (int e = 0; e < kV; ++e) s.dred[threadIdx.x / kRowPieces][col + e] = dsum[e];
            __syncthreads();
            double acc = 0.0;
            for (int r = 0; r < kRowStep; ++r) acc += s.dred[r][lane];
            dtot = (float)acc;
        }
        if (!dval) return;
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int n = w * NPW + k;
            if (n >= p.N) continue;
            if (kSum) {
                const int64_t o = (((int64_t)b * p.nseg + seg) * p.dim + d) * p.N + n;
                p.agg_P[o] = __builtin_amdgcn_exp2f(l.A2[k] * dtot);
                p.agg_H[o] = l.h[k];
            } else if (kMain && p.h_last != nullptr && seg == p.nseg - 1) {
                p.h_last[((int64_t)b * p.dim + d) * p.N + n] = l.h[k];
            }
        }
    }
};

template <typename T, int NPW, int G, int TC, bool ZOH, int MODE, bool FEAT, bool UF = false>
__global__ __launch_bounds__(kTile * G) void scan_kernel(const ScanParams p) {
    ScanKernel<T, NPW, G, TC, ZOH, MODE, FEAT, UF>::run(p);
}

// ---------------------------------------------------------------------------
// Carry pass: for each (b, d, n), the initial state of segment s is the
// composition of the maps of segments 0..s-1 applied to h0. Lanes hold
// consecutive segments of one (b, d, n) item in groups of SP lanes (SP =
// segments rounded up to a power of two, <= 64), and an inclusive
// Kogge-Stone scan over the affine pairs runs with DPP: row shifts by 1, 2, 4,
// 8 inside 16-lane rows, then row broadcasts of lanes 15 and 31 to cross rows.
// With up to kCarryDirect segments every lane reads its pair from global
// memory directly (a wave then touches runs of at least 32 bytes); with more,
// a workgroup stages a block of kCarryItems consecutive items of one batch
// row through LDS, so that it reads and writes every segment's rows of the
// block as 256-byte runs.

struct CarryParams {
    const float *P, *H, *h0;
    float *seg_h;
    int batch, dim, N, nseg, sp_log2;
    int64_t total;    // batch * dim * N
    int b0;           // staged form: first batch row of this launch (grid.y covers at most 65535)
};

constexpr int kCarryDirect = 8;
constexpr int kCarryItems = 64;      // staged form: (d, n) items per workgroup
constexpr int kCarryThreads = 256;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void affine_step(float &P, float &H, bool take) {
    // Fetch (P, H) of the lane CTRL points at; lanes without a source keep the
    // identity (1, 0) because bound_ctrl is off and `old` is the identity.
    const float Pp = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, P), CTRL, ROW_MASK, 0xF, false));
    const float Hp = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 0.0f), __builtin_bit_cast(int, H), CTRL, ROW_MASK, 0xF, false));
    if (take) {
        // (Pp, Hp) comes first, then (P, H)
        H = fmaf(P, Hp, H);
        P = P * Pp;
    }
}

// Inclusive scan of the affine pairs inside groups of sp = 2^sp_log2 lanes
// (s: the lane's position in its group).
__device__ __forceinline__ void affine_scan(float &P, float &H, int lane, int sp, int s) {
    if (sp > 1)  affine_step<0x111, 0xF>(P, H, s >= 1);    // row_shr:1
    if (sp > 2)  affine_step<0x112, 0xF>(P, H, s >= 2);    // row_shr:2
    if (sp > 4)  affine_step<0x114, 0xF>(P, H, s >= 4);    // row_shr:4
    if (sp > 8)  affine_step<0x118, 0xF>(P, H, s >= 8);    // row_shr:8
    if (sp > 16) affine_step<0x142, 0xA>(P, H, (lane & 16) != 0);   // row_bcast:15 -> rows 1, 3
    if (sp > 32) affine_step<0x143, 0xC>(P, H, (lane & 32) != 0);   // row_bcast:31 -> rows 2, 3
}

__global__ __launch_bounds__(kCarryThreads) __attribute__((unused)) void carry_direct_kernel(const CarryParams p) {
    const int lane = threadIdx.x & 63;
    const int sp = 1 << p.sp_log2;
    const int s = lane & (sp - 1);                                  // segment
    const int64_t item = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> p.sp_log2;  // (b, d, n)
    const bool valid = item < p.total && s < p.nseg;
    int64_t b = 0, dn = 0;
    if (item < p.total) {
        b = item / ((int64_t)p.dim * p.N);
        dn = item % ((int64_t)p.dim * p.N);
    }
    // The map of segment s-1 feeds segment s: lane s holds map(s-1), lane 0 the identity.
    float P = 1.0f, H = 0.0f;
    if (valid && s > 0) {
        const int64_t o = ((b * p.nseg + (s - 1)) * p.dim * p.N) + dn;
        P = p.P[o];
        H = p.H[o];
    }
    affine_scan(P, H, lane, sp, s);
    if (!valid) return;
    const float hin = p.h0 != nullptr ? p.h0[b * (int64_t)p.dim * p.N + dn] : 0.0f;
    p.seg_h[((b * p.nseg + s) * p.dim * p.N) + dn] = fmaf(P, hin, H);
}

// grid: (blocks of kCarryItems items per batch row, batch rows from b0)
__global__ __launch_bounds__(kCarryThreads) __attribute__((unused)) void carry_staged_kernel(const CarryParams p) {
    // one row of the block's items per segment, padded by one against bank conflicts
    __shared__ float sP[kMaxSegments][kCarryItems + 1], sH[kMaxSegments][kCarryItems + 1];
    const int64_t per_row = (int64_t)p.dim * p.N;
    const int64_t b = p.b0 + (int64_t)blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kCarryItems;
    const int items = (int)min((int64_t)kCarryItems, per_row - i0);
    // Row s of the block holds the map of segment s-1, which feeds segment s;
    // row 0 the identity.
    for (int e = threadIdx.x; e < p.nseg * kCarryItems; e += kCarryThreads) {
        const int s = e / kCarryItems, k = e % kCarryItems;
        float P = 1.0f, H = 0.0f;
        if (s > 0 && k < items) {
            const int64_t o = (b * p.nseg + (s - 1)) * per_row + i0 + k;
            P = p.P[o];
            H = p.H[o];
        }
        sP[s][k] = P;
        sH[s][k] = H;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x / 64;
    const int sp = 1 << p.sp_log2;
    const int s = lane & (sp - 1);               // segment
    const int per_wave = 64 >> p.sp_log2;        // items a wave scans at once
    for (int k0 = wave * per_wave; k0 < items; k0 += 4 * per_wave) {
        const int k = k0 + (lane >> p.sp_log2);
        const bool valid = k < items && s < p.nseg;
        float P = valid ? sP[s][k] : 1.0f;
        float H = valid ? sH[s][k] : 0.0f;
        affine_scan(P, H, lane, sp, s);
        if (valid) {
            const float hin = p.h0 != nullptr ? p.h0[b * per_row + i0 + k] : 0.0f;
            sH[s][k] = fmaf(P, hin, H);   // only this lane reads or writes (s, k)
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < p.nseg * kCarryItems; e += kCarryThreads) {
        const int s2 = e / kCarryItems, k = e % kCarryItems;
        if (k < items) p.seg_h[(b * p.nseg + s2) * per_row + i0 + k] = sH[s2][k];
    }
}

// CK: the shape also has the checkpoint pass (the launch shapes the backward
// uses). UF: u is fp32 with bf16 tensors (every pass reads it so).
template <typename T, int NPW, int G, int TC, bool ZOH, bool CK, bool FEAT, bool UF>
hipError_t launch_scan_tf(const ScanParams &p, int nblocks_main, int nblocks_agg, hipStream_t st) {
    if (!CK && p.ckpt != nullptr) return hipErrorInvalidValue;
    if ((p.u_f32 != 0) != UF) return hipErrorInvalidValue;
    constexpr int kLongTC = TC * long_chunk_factor<G>();   // aggregate and checkpoint-only passes
    constexpr int kSegTC = seg_main_tc<G, TC>();            // main pass of a plan with segments
    {
        const int64_t total = (int64_t)p.batch * padded_len(p.L) * (NPW * G);
        hipLaunchKernelGGL(widen_bc_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                           static_cast<const T *>(p.B), static_cast<const T *>(p.C), p.Bf, p.Cf, p.batch, p.L,
                           p.N, G, NPW);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (nblocks_agg > 0) {
        hipLaunchKernelGGL((scan_kernel<T, NPW, G, kLongTC, ZOH, kModeAggregate, FEAT, UF>), dim3(nblocks_agg),
                           dim3(kTile * G), 0, st, p);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        CarryParams cp{};
        cp.P = p.agg_P;
        cp.H = p.agg_H;
        cp.h0 = p.h0;
        cp.seg_h = const_cast<float *>(p.seg_h);
        cp.batch = p.batch;
        cp.dim = p.dim;
        cp.N = p.N;
        cp.nseg = p.nseg;
        cp.sp_log2 = ilog2(p.nseg);
        cp.total = (int64_t)p.batch * p.dim * p.N;
        if (p.nseg <= kCarryDirect) {
            const int64_t threads = cp.total << cp.sp_log2;
            hipLaunchKernelGGL(carry_direct_kernel, dim3((unsigned)((threads + kCarryThreads - 1) / kCarryThreads)),
                               dim3(kCarryThreads), 0, st, cp);
            if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        } else {
            const int64_t per_row = (int64_t)p.dim * p.N;
            for (int b0 = 0; b0 < p.batch; b0 += 65535) {
                cp.b0 = b0;
                const dim3 grid((unsigned)((per_row + kCarryItems - 1) / kCarryItems),
                                (unsigned)min(p.batch - b0, 65535));
                hipLaunchKernelGGL(carry_staged_kernel, grid, dim3(kCarryThreads), 0, st, cp);
                if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
            }
        }
    }
    if constexpr (CK) {
        if (p.ckpt != nullptr) {
            // the forward that also keeps the backward's checkpoints, or the
            // checkpoints alone
            if (p.y != nullptr)
                hipLaunchKernelGGL((scan_kernel<T, NPW, G, TC, ZOH, kModeMainCheckpoint, FEAT, UF>),
                                   dim3(nblocks_main), dim3(kTile * G), 0, st, p);
            else
                hipLaunchKernelGGL((scan_kernel<T, NPW, G, kLongTC, ZOH, kModeCheckpoint, FEAT, UF>),
                                   dim3(nblocks_main), dim3(kTile * G), 0, st, p);
            return hipGetLastError();
        }
    }
    if constexpr (kSegTC != TC) {
        if (nblocks_agg > 0) {
            hipLaunchKernelGGL((scan_kernel<T, NPW, G, kSegTC, ZOH, kModeMain, FEAT, UF>), dim3(nblocks_main),
                               dim3(kTile * G), 0, st, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((scan_kernel<T, NPW, G, TC, ZOH, kModeMain, FEAT, UF>), dim3(nblocks_main), dim3(kTile * G),
                       0, st, p);
    return hipGetLastError();
}

template <typename T, int NPW, int G, int TC, bool ZOH, bool CK, bool UF>
hipError_t launch_scan_t(const ScanParams &p, int nblocks_main, int nblocks_agg, hipStream_t st) {
    const bool feat = p.delta_bias != nullptr || p.delta_softplus;
    return feat ? launch_scan_tf<T, NPW, G, TC, ZOH, CK, true, UF>(p, nblocks_main, nblocks_agg, st)
                : launch_scan_tf<T, NPW, G, TC, ZOH, CK, false, UF>(p, nblocks_main, nblocks_agg, st);
}

template <typename T, bool ZOH, bool UF = false>
hipError_t launch_scan_shape(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st) {
    // (padded states, waves per tile, chunk length): LDS stays <= 80 KiB
    // (two workgroups per CU) and every thread of a workgroup of up to 8
    // waves stages a piece of each chunk
#define SSM_CASE(NP, GG, TCC, CK) \
    if (pl.npad == NP && pl.G == GG) return launch_scan_t<T, NP / GG, GG, TCC, ZOH, CK, UF>(p, nm, na, st);
    SSM_CASE(4, 1, 16, 0)  SSM_CASE(4, 2, 16, 1)  SSM_CASE(4, 4, 8, 0)
    SSM_CASE(8, 1, 16, 0)  SSM_CASE(8, 2, 16, 0)  SSM_CASE(8, 4, 8, 0)   SSM_CASE(8, 8, 16, 1)
    SSM_CASE(16, 1, 16, 0) SSM_CASE(16, 2, 16, 0) SSM_CASE(16, 4, 8, 0)  SSM_CASE(16, 8, 16, 1)
    SSM_CASE(16, 16, 8, 0)
    SSM_CASE(32, 2, 16, 0) SSM_CASE(32, 4, 8, 0)  SSM_CASE(32, 8, 16, 0) SSM_CASE(32, 16, 8, 1)
    SSM_CASE(64, 4, 8, 0)  SSM_CASE(64, 8, 16, 0) SSM_CASE(64, 16, 8, 1)
#undef SSM_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ssm_detail
#endif  // SSM_SCAN_INSTANTIATE
