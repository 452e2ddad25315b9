// Scan kernels of the gfx950 selective-scan library, shared by the
// translation units that instantiate them (one per element type and
// discretisation, compiled in parallel) and by the ABI unit.
//
// Kernel design (the scan):
//  * One workgroup owns a tile of 64 consecutive channels of one batch row and
//    one time segment. Lane = channel. The workgroup has G waves; wave w owns
//    NPW = Npad/G of the states of all 64 channels, so a lane keeps its NPW
//    states h[n] in VGPRs for the whole segment and B_t[n], C_t[n] are the same
//    for the whole wave (read from LDS as broadcasts). Splitting states over
//    waves multiplies the parallelism of a channel tile by G at the cost of a
//    few per-token instructions, instead of splitting time, which would cost
//    a second pass of the recurrence.
//  * Time is walked in chunks of TC tokens. The workgroup loads a chunk of u,
//    delta, z (TC rows x 64 channels, 16-byte coalesced loads), and of B and C,
//    into registers one chunk ahead, converts it to fp32 into LDS, and every
//    wave walks the chunk sequentially from LDS. The expanded (t, d, n) decay
//    and input terms exist only in registers and are never written.
//  * Each wave writes its partial readout sum_{n in wave} C_t[n] h_t[n] per
//    (t, channel) to LDS; after a barrier the whole workgroup adds the G
//    partials, the D skip and the SiLU gate, rounds, and stores y coalesced.
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
//
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "ssm_scan.h"

namespace ssm_detail {


constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;        // channels per workgroup tile = lanes per wave
constexpr int kXcds = 8;         // MI355X: 8 accelerator complex dies
constexpr int kMaxSegments = 64;

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
    // round to bf16 (nearest even, v_cvt_pk_bf16_f32) and keep it as a float
    __device__ static uint16_t to_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
};

__device__ __forceinline__ float silu(float z) {
    // z * sigmoid(z) = z / (1 + 2^(-z log2 e))
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

struct ScanParams {
    const void *u, *delta, *z, *B, *C;
    const float *A, *D, *h0;
    const float *seg_h;   // (batch, nseg, dim, N) initial state of each segment, or null
    void *y;
    float *h_last;
    float *agg_P, *agg_H; // (batch, nseg, dim, N) segment maps (aggregate pass)
    int64_t L;
    int batch, dim, N;
    int seg_len, nseg, nseg_launched;
    int ntiles;
    int vec;              // 16-byte loads of u/delta/z are aligned
    int pair_store;       // y can be stored as aligned channel pairs
};

struct Plan {
    int npad, G, npw, S, seg_len;
};

// Launches the aggregate, carry and main passes for one element type and
// discretisation (defined in the scan_<type>_<disc>.hip units).
hipError_t launch_scan_bf16_euler(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_bf16_zoh(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_f32_euler(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);
hipError_t launch_scan_f32_zoh(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st);

inline int ilog2(int v) { int r = 0; while ((1 << r) < v) ++r; return r; }

}  // namespace ssm_detail

#ifdef SSM_SCAN_INSTANTIATE
namespace ssm_detail {
namespace {

// ---------------------------------------------------------------------------
// Scan kernels



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

template <typename T, int NPW, int G, int TC, bool ZOH, bool AGG>
struct ScanKernel {
    static constexpr int kThreads = kTile * G;
    static constexpr int kNP = NPW * G;                       // padded state count
    static constexpr int kV = 16 / Elem<T>::kBytes;            // elements per 16-byte piece
    static constexpr int kPieces = TC * kTile / kV;            // pieces per chunk per tensor
    static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
    static constexpr int kBCE = TC * kNP;                      // B (or C) elements per chunk
    static constexpr int kBPT = (kBCE + kThreads - 1) / kThreads;

    struct Smem {
        float u[TC][kTile];
        float dt[TC][kTile];
        float z[AGG ? 1 : TC][kTile];
        float B[TC][kNP];
        float C[AGG ? 1 : TC][kNP];
        float y[AGG ? 1 : G][AGG ? 1 : TC][kTile];
    };
    static_assert(sizeof(Smem) <= 65536, "LDS per workgroup");

    struct Prefetch {
        uint4 u[kPPT], dt[kPPT], z[kPPT];
        T B[kBPT], C[kBPT];
    };

    // Issue the global loads of one chunk [t0, t0 + tval) into registers.
    __device__ static void load(const ScanParams &p, Prefetch &pf, int b, int d0, int64_t t0, int tval) {
        const T *u = static_cast<const T *>(p.u);
        const T *dt = static_cast<const T *>(p.delta);
        const T *z = static_cast<const T *>(p.z);
        const bool gate = !AGG && z != nullptr;
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int piece = threadIdx.x + j * kThreads;
            const int t = piece / (kTile / kV);
            const int c = (piece % (kTile / kV)) * kV;
            uint4 ru = {0, 0, 0, 0}, rd = {0, 0, 0, 0}, rz = {0, 0, 0, 0};
            if (piece < kPieces && t < tval && d0 + c < p.dim) {
                const int64_t off = ((int64_t)b * p.L + t0 + t) * p.dim + d0 + c;
                if (p.vec) {
                    ru = *reinterpret_cast<const uint4 *>(u + off);
                    rd = *reinterpret_cast<const uint4 *>(dt + off);
                    if (gate) rz = *reinterpret_cast<const uint4 *>(z + off);
                } else {
                    T eu[kV], ed[kV], ez[kV];
#pragma unroll
                    for (int e = 0; e < kV; ++e) {
                        const bool ok = d0 + c + e < p.dim;
                        eu[e] = ok ? u[off + e] : T(0);
                        ed[e] = ok ? dt[off + e] : T(0);
                        ez[e] = (ok && gate) ? z[off + e] : T(0);
                    }
                    memcpy(&ru, eu, 16);
                    memcpy(&rd, ed, 16);
                    memcpy(&rz, ez, 16);
                }
            }
            pf.u[j] = ru;
            pf.dt[j] = rd;
            pf.z[j] = rz;
        }
        const T *Bp = static_cast<const T *>(p.B);
        const T *Cp = static_cast<const T *>(p.C);
#pragma unroll
        for (int j = 0; j < kBPT; ++j) {
            const int e = threadIdx.x + j * kThreads;
            const int t = e / kNP, n = e % kNP;
            T vb = T(0), vc = T(0);
            if (e < kBCE && t < tval && n < p.N) {
                const int64_t off = ((int64_t)b * p.L + t0 + t) * p.N + n;
                vb = Bp[off];
                if (!AGG) vc = Cp[off];
            }
            pf.B[j] = vb;
            pf.C[j] = vc;
        }
    }

    // Widen the prefetched chunk to fp32 into LDS.
    __device__ static void commit(const Prefetch &pf, Smem &s) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {
            const int piece = threadIdx.x + j * kThreads;
            if (piece >= kPieces) continue;
            const int t = piece / (kTile / kV);
            const int c = (piece % (kTile / kV)) * kV;
            T eu[kV], ed[kV], ez[kV];
            memcpy(eu, &pf.u[j], 16);
            memcpy(ed, &pf.dt[j], 16);
            memcpy(ez, &pf.z[j], 16);
#pragma unroll
            for (int e = 0; e < kV; ++e) {
                s.u[t][c + e] = Elem<T>::widen(eu[e]);
                s.dt[t][c + e] = Elem<T>::widen(ed[e]);
                if (!AGG) s.z[t][c + e] = Elem<T>::widen(ez[e]);
            }
        }
#pragma unroll
        for (int j = 0; j < kBPT; ++j) {
            const int e = threadIdx.x + j * kThreads;
            if (e >= kBCE) continue;
            const int t = e / kNP, n = e % kNP;
            s.B[t][n] = Elem<T>::widen(pf.B[j]);
            if (!AGG) s.C[t][n] = Elem<T>::widen(pf.C[j]);
        }
    }

    // Add the G partial readouts, the D skip and the gate; round and store y.
    __device__ static void finalize(const ScanParams &p, const Smem &s, int b, int d0, int64_t t0,
                                    int tval, float D0, float D1) {
        const int c = (threadIdx.x & 31) * 2;
        const bool gate = p.z != nullptr;
        T *y = static_cast<T *>(p.y);
        for (int t = threadIdx.x >> 5; t < tval; t += kThreads / 32) {
            float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                y0 += s.y[g][t][c];
                y1 += s.y[g][t][c + 1];
            }
            y0 = fmaf(D0, s.u[t][c], y0);
            y1 = fmaf(D1, s.u[t][c + 1], y1);
            if (gate) {
                y0 *= silu(s.z[t][c]);
                y1 *= silu(s.z[t][c + 1]);
            }
            const int64_t off = ((int64_t)b * p.L + t0 + t) * p.dim + d0 + c;
            const bool ok0 = d0 + c < p.dim, ok1 = d0 + c + 1 < p.dim;
            if constexpr (sizeof(T) == 2) {
                const uint16_t r0 = Elem<uint16_t>::to_bits(y0), r1 = Elem<uint16_t>::to_bits(y1);
                if (p.pair_store && ok1) {
                    *reinterpret_cast<uint32_t *>(y + off) = (uint32_t)r0 | ((uint32_t)r1 << 16);
                } else {
                    if (ok0) y[off] = r0;
                    if (ok1) y[off + 1] = r1;
                }
            } else {
                if (p.pair_store && ok1) {
                    *reinterpret_cast<float2 *>(y + off) = make_float2(y0, y1);
                } else {
                    if (ok0) y[off] = y0;
                    if (ok1) y[off + 1] = y1;
                }
            }
        }
    }

    __device__ static void run(const ScanParams &p) {
        __shared__ Smem s;
        int seg, b, tile;
        map_block(p, seg, b, tile);
        const int lane = threadIdx.x & (kTile - 1);
        const int w = threadIdx.x / kTile;
        const int d0 = tile * kTile;
        const int d = d0 + lane;
        const bool dval = d < p.dim;
        const int dc = dval ? d : p.dim - 1;
        const int64_t t_begin = (int64_t)seg * p.seg_len;
        const int64_t t_end = min(p.L, t_begin + (int64_t)p.seg_len);

        // Per-lane constants and initial state of this wave's states.
        float A2[NPW], h[NPW];
        float Az[ZOH ? NPW : 1], Ainv[ZOH ? NPW : 1];
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int n = w * NPW + k;
            const bool nv = n < p.N;
            const float a = nv ? p.A[(int64_t)dc * p.N + n] : 0.0f;
            A2[k] = a * kLog2e;
            if constexpr (ZOH) {
                Az[k] = a;
                Ainv[k] = (a != 0.0f) ? 1.0f / a : 0.0f;
            }
            float h_init = 0.0f;
            if (!AGG && nv) {
                // with segments, every segment (also the first) starts from the
                // carry pass's output, so that h_last may alias h0
                if (p.seg_h != nullptr)
                    h_init = p.seg_h[(((int64_t)b * p.nseg + seg) * p.dim + dc) * p.N + n];
                else if (p.h0 != nullptr)
                    h_init = p.h0[((int64_t)b * p.dim + dc) * p.N + n];
            }
            h[k] = h_init;
        }
        // finalize handles the channel pair (2*(tid%32), +1) for all its rows
        float D0 = 0.0f, D1 = 0.0f;
        if (!AGG && p.D != nullptr) {
            const int c = d0 + (threadIdx.x & 31) * 2;
            D0 = c < p.dim ? p.D[c] : 0.0f;
            D1 = c + 1 < p.dim ? p.D[c + 1] : 0.0f;
        }
        float dsum = 0.0f, dcomp = 0.0f;   // compensated sum of delta (aggregate pass)

        const int nchunks = (int)((t_end - t_begin + TC - 1) / TC);
        Prefetch pf;
        if (nchunks > 0) {
            load(p, pf, b, d0, t_begin, (int)min((int64_t)TC, t_end - t_begin));
            commit(pf, s);
        }
        __syncthreads();

        for (int k = 0; k < nchunks; ++k) {
            const int64_t t0 = t_begin + (int64_t)k * TC;
            const int tval = (int)min((int64_t)TC, t_end - t0);
            if (k + 1 < nchunks)
                load(p, pf, b, d0, t0 + TC, (int)min((int64_t)TC, t_end - t0 - TC));

            for (int t = 0; t < tval; ++t) {
                const float uu = s.u[t][lane];
                const float dd = s.dt[t][lane];
                const float du = dd * uu;
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < NPW; ++q) {
                    const float bq = s.B[t][w * NPW + q];
                    if constexpr (ZOH) {
                        const float em1 = expm1f(dd * Az[q]);
                        const float coef = (Az[q] != 0.0f) ? em1 * Ainv[q] : dd;
                        h[q] = fmaf(1.0f + em1, h[q], coef * bq * uu);
                    } else {
                        const float a = __builtin_amdgcn_exp2f(dd * A2[q]);
                        h[q] = fmaf(a, h[q], du * bq);
                    }
                    if (!AGG) part = fmaf(s.C[t][w * NPW + q], h[q], part);
                }
                if (AGG) {
                    // Kahan summation of delta over the segment
                    const float yk = dd - dcomp;
                    const float tk = dsum + yk;
                    dcomp = (tk - dsum) - yk;
                    dsum = tk;
                } else {
                    s.y[w][t][lane] = part;
                }
            }
            __syncthreads();
            if (!AGG) finalize(p, s, b, d0, t0, tval, D0, D1);
            if (k + 1 < nchunks) {
                __syncthreads();
                commit(pf, s);
                __syncthreads();
            }
        }

        if (!dval) return;
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int n = w * NPW + k;
            if (n >= p.N) continue;
            if (AGG) {
                const int64_t o = (((int64_t)b * p.nseg + seg) * p.dim + d) * p.N + n;
                p.agg_P[o] = __builtin_amdgcn_exp2f(A2[k] * dsum);
                p.agg_H[o] = h[k];
            } else if (p.h_last != nullptr && seg == p.nseg - 1) {
                p.h_last[((int64_t)b * p.dim + d) * p.N + n] = h[k];
            }
        }
    }
};

template <typename T, int NPW, int G, int TC, bool ZOH, bool AGG>
__global__ __launch_bounds__(kTile * G) void scan_kernel(const ScanParams p) {
    ScanKernel<T, NPW, G, TC, ZOH, AGG>::run(p);
}

// ---------------------------------------------------------------------------
// Carry pass: for each (b, d, n), the initial state of segment s is the
// composition of the maps of segments 0..s-1 applied to h0. Lanes hold
// consecutive segments of one (b, d, n) in groups of SP lanes (SP = segments
// rounded up to a power of two, <= 64). An inclusive Kogge-Stone scan over the
// affine pairs runs with DPP: row shifts by 1, 2, 4, 8 inside 16-lane rows,
// then row broadcasts of lanes 15 and 31 to cross rows.

struct CarryParams {
    const float *P, *H, *h0;
    float *seg_h;
    int batch, dim, N, nseg, sp_log2;
    int64_t total;    // batch * dim * N
};

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

__global__ __launch_bounds__(256) void carry_kernel(const CarryParams p) {
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
    // inclusive scan inside groups of sp lanes
    if (sp > 1)  affine_step<0x111, 0xF>(P, H, s >= 1);    // row_shr:1
    if (sp > 2)  affine_step<0x112, 0xF>(P, H, s >= 2);    // row_shr:2
    if (sp > 4)  affine_step<0x114, 0xF>(P, H, s >= 4);    // row_shr:4
    if (sp > 8)  affine_step<0x118, 0xF>(P, H, s >= 8);    // row_shr:8
    if (sp > 16) affine_step<0x142, 0xA>(P, H, (lane & 16) != 0);   // row_bcast:15 -> rows 1, 3
    if (sp > 32) affine_step<0x143, 0xC>(P, H, (lane & 32) != 0);   // row_bcast:31 -> rows 2, 3
    if (!valid) return;
    const float hin = p.h0 != nullptr ? p.h0[b * (int64_t)p.dim * p.N + dn] : 0.0f;
    p.seg_h[((b * p.nseg + s) * p.dim * p.N) + dn] = fmaf(P, hin, H);
}

template <typename T, int NPW, int G, int TC, bool ZOH>
hipError_t launch_scan_t(const ScanParams &p, int nblocks_main, int nblocks_agg, hipStream_t st) {
    if (nblocks_agg > 0) {
        ScanParams pa = p;
        pa.nseg_launched = p.nseg - 1;
        hipLaunchKernelGGL((scan_kernel<T, NPW, G, TC, ZOH, true>), dim3(nblocks_agg), dim3(kTile * G), 0, st, pa);
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
        const int64_t threads = cp.total << cp.sp_log2;
        hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, cp);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((scan_kernel<T, NPW, G, TC, ZOH, false>), dim3(nblocks_main), dim3(kTile * G), 0, st, p);
    return hipGetLastError();
}

template <typename T, bool ZOH>
hipError_t launch_scan_shape(const Plan &pl, const ScanParams &p, int nm, int na, hipStream_t st) {
    // (padded states, waves per tile) -> states per wave; chunk length keeps LDS <= 64 KiB
#define SSM_CASE(NP, GG, TCC) \
    if (pl.npad == NP && pl.G == GG) return launch_scan_t<T, NP / GG, GG, TCC, ZOH>(p, nm, na, st);
    SSM_CASE(4, 1, 32)  SSM_CASE(4, 2, 32)  SSM_CASE(4, 4, 32)
    SSM_CASE(8, 1, 32)  SSM_CASE(8, 2, 32)  SSM_CASE(8, 4, 32)  SSM_CASE(8, 8, 16)
    SSM_CASE(16, 1, 32) SSM_CASE(16, 2, 32) SSM_CASE(16, 4, 32) SSM_CASE(16, 8, 16) SSM_CASE(16, 16, 8)
    SSM_CASE(32, 2, 32) SSM_CASE(32, 4, 16) SSM_CASE(32, 8, 16) SSM_CASE(32, 16, 8)
    SSM_CASE(64, 4, 16) SSM_CASE(64, 8, 16) SSM_CASE(64, 16, 8)
#undef SSM_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace ssm_detail
#endif  // SSM_SCAN_INSTANTIATE
