/*
 * ssm_scan.h — C ABI of the MI355X (gfx950) selective-scan library.
 *
 * The library computes the Mamba selective scan (S6) forward pass, its
 * backward, its one-token decode step and the Mamba-2 SSD layer with
 * hand-written HIP kernels. Every pointer that
 * names tensor data is a DEVICE pointer owned by the caller; the library
 * allocates and frees nothing. Work is enqueued asynchronously on the given
 * HIP stream: buffers must stay alive until the stream has finished with
 * them. No function prints, throws or exits; each returns an ssm_status.
 *
 * Operation (for every batch row b, channel d and state n; each channel is
 * an independent single-input single-output SSM, itwiki "상태 공간 모델",
 * section "제어 이론의 상태 공간 표현과의 관계"):
 *
 *   Abar_t = exp(delta_t * A[d,n])                 discretised decay
 *   Bu_t   = delta_t * B_t[n] * u_t                default: simplified rule
 *          = (exp(delta_t A) - 1)/A * B_t[n] * u_t zero-order hold (SSM_DISC_ZOH)
 *   h_t    = Abar_t * h_{t-1} + Bu_t               h_{-1} = h0 (or 0)
 *   y_t    = sum_n C_t[n] h_t[n] + D[d] u_t        readout after the update
 *   y_t   *= z_t * sigmoid(z_t)                    optional SiLU gate
 *
 * Passages: eommydocs "State Space Models (SSM)" §3.2 "Selective Scan
 * Algorithm" (shapes of u, delta, A, B, C and the deltaA / deltaB_u
 * discretisation); youngju.dev "Mamba와 State Space Model 논문 심층 분석",
 * SelectiveSSM.selective_scan and MambaBlock.forward (recurrence, readout,
 * y + D*x skip, y * silu(z) gate); itwiki "상태 공간 모델", "동작 원리 › 이산화"
 * (zero-order hold); doyouknow.kr "Mamba와 상태 공간 모델(SSM)의 부상 완벽
 * 가이드" §3-1 (h_t = exp(delta_t A) h_{t-1} + delta_t B_t x_t).
 *
 * Numerics: state and arithmetic in fp32; bf16 inputs are widened exactly;
 * bf16 outputs are rounded to nearest-even. NaN and Inf propagate unchecked.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Every error is detected on the host before any work is
 * enqueued, except SSM_ERR_HIP, which reports a failed kernel launch. */
typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,        /* a required pointer is NULL */
    SSM_ERR_SHAPE = -2,       /* a negative size, or sizes whose byte count overflows */
    SSM_ERR_DTYPE = -3,       /* unknown element type */
    SSM_ERR_UNSUPPORTED = -4, /* dstate outside 1..64, unknown discretisation or flag, conv_width
                                 outside 0..4, bad tuning */
    SSM_ERR_ALIAS = -5,       /* an output overlaps an input or another output */
    SSM_ERR_WORKSPACE = -6,   /* workspace missing or smaller than ssm_scan_workspace_size() */
    SSM_ERR_HIP = -7,         /* the HIP runtime refused a launch (e.g. not a gfx950 device) */
    SSM_ERR_ALIGN = -8,       /* a pointer is not aligned to its element size */
    SSM_ERR_SCRATCH = -9      /* ssm_scan_fwd_noalloc: the problem needs more than
                                 SSM_NOALLOC_SCRATCH_BYTES of scratch */
} ssm_status;

/* Element type of the per-token tensors u, delta, z, B, C and of the output y.
 * A, D and all states are always fp32. */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Discretisation of B (A is always exp(delta*A)). */
typedef enum { SSM_DISC_EULER = 0, SSM_DISC_ZOH = 1 } ssm_disc;

/* Sizes and types of one scan, and how the step size is formed.
 * The step used by the recurrence is delta[b,t,d] (+ delta_bias[d] when the
 * bias is given), passed through softplus(x) = log(1 + exp(x)) when
 * delta_softplus is nonzero: the projection output becomes a positive step
 * inside the kernel (youngju.dev SelectiveSSM.forward, dt = softplus(...)).
 * With conv_width W > 0 the Mamba block's prologue runs in the kernel (youngju.dev
 * MambaBlock.forward, x_conv = silu(conv1d(x)), a causal depthwise convolution
 * with left padding W-1): the buffer passed as u holds x, and the scan input is
 *     u[b,t,d] = silu(conv_bias[d] + sum_{k<W} conv_weight[d,k] * x[b,t-(W-1)+k,d]),
 * x before t = 0 being zero; the D skip uses this u. Forward and backward
 * form u in a pass of their own and keep it in fp32, whatever the tensors'
 * type (a bf16 rounding of u can show in y far beyond one rounding of y where
 * the scan's sums cancel).
 * Zero-initialise the struct for "delta used as given, no convolution". */
typedef struct {
    int64_t batch;   /* b  >= 0 */
    int64_t seqlen;  /* L  >= 0 */
    int64_t dim;     /* d  in 0..2^26 (channels, d_inner) */
    int64_t dstate;  /* N  in 1..64 */
    int32_t dtype;   /* ssm_dtype */
    int32_t disc;    /* ssm_disc */
    int32_t delta_softplus;   /* 0 or 1 */
    int32_t conv_width;       /* 0 (u used as given) or W in 1..4: see below */
    const float *delta_bias;  /* (dim) fp32 device pointer, or NULL */
    const float *conv_weight; /* (dim, W) fp32 device pointer when conv_width > 0 */
    const float *conv_bias;   /* (dim) fp32 device pointer, or NULL */
} ssm_scan_desc;

/* Optional launch shape, for tuning and for tests of every kernel variant.
 * Zero fields are chosen by the library. state_groups: waves that share one
 * 64-channel tile, each owning dstate/state_groups states (1,2,4,8,16);
 * segments: independent pieces of the sequence, joined by an affine carry
 * (1..64). */
typedef struct {
    int32_t state_groups;
    int32_t segments;
} ssm_scan_tuning;

/* Bytes of device workspace ssm_scan_fwd needs for `desc`: B and C widened
 * to fp32 (about 2 * batch * seqlen * dstate * 4 bytes) plus, when the
 * sequence is split into segments, three (batch, segments, dim, dstate) fp32
 * arrays, plus, with the convolution prologue, u (batch, seqlen, dim) in
 * fp32. 0 when there is nothing to compute; 0 for an invalid descriptor. */
size_t ssm_scan_workspace_size(const ssm_scan_desc *desc);

/*
 * Selective scan forward (the pages' selective_scan(u, delta, A, B, C) with
 * the D skip and SiLU gate of the Mamba block fused in).
 *
 *   u, delta  (batch, seqlen, dim)   dtype, row-major, channel fastest
 *   A         (dim, dstate)          fp32 (negative for a decaying state)
 *   B, C      (batch, seqlen, dstate) dtype, shared by all channels of a row
 *   D         (dim) fp32, or NULL for no skip term
 *   z         (batch, seqlen, dim)   dtype, or NULL for no gate
 *   h0        (batch, dim, dstate)   fp32 initial state, or NULL for zeros
 *   y         (batch, seqlen, dim)   dtype, written
 *   h_last    (batch, dim, dstate)   fp32 final state, written; may be NULL.
 *             h_last may equal h0 exactly (resume in place).
 *   workspace device scratch of at least ssm_scan_workspace_size(desc) bytes,
 *             256-byte aligned (may be NULL when that size is 0); its
 *             contents on entry do not matter and are clobbered.
 * delta is used as given (the caller applies softplus). Outputs must not
 * overlap any input, each other or the workspace. Pointers must be aligned to
 * their element size. seqlen == 0 writes h_last = h0 (or zeros) and no y.
 */
int ssm_scan_fwd(const ssm_scan_desc *desc,
                 const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *h0, void *y, float *h_last,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssm_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes
 * no workspace; the library keeps one fixed scratch buffer of
 * SSM_NOALLOC_SCRATCH_BYTES per GPU (a static device array, held from the
 * module's load on that GPU until the process ends) and runs the same kernels
 * as ssm_scan_fwd on it, so its results equal ssm_scan_fwd's bit for bit.
 *
 *   Arguments, shapes, conditions and errors: those of ssm_scan_fwd, without
 *   workspace and workspace_bytes.
 *   SSM_ERR_SCRATCH when ssm_scan_workspace_size(desc) exceeds
 *   SSM_NOALLOC_SCRATCH_BYTES (checked on the host before anything else is
 *   done; e.g. the 1.4B-shaped layer b8 L8192 d4096 N16 needs 8.4 MB, the
 *   131072-token d5120 layer about 33 MB, and the convolution prologue adds
 *   4*b*L*d bytes of fp32 u).
 *   The buffer's device address is looked up once per GPU, on the first call
 *   whose stream belongs to that GPU; that first call is best made outside
 *   graph capture. The call itself allocates nothing and frees nothing.
 *   Calls on one GPU share its buffer: calls that overlap in time on that GPU
 *   (two streams, or two host threads) race and give wrong results. Calls
 *   ordered on one stream are safe. Nothing in the buffer needs to start at
 *   zero: every pass writes what the next one reads.
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssm_scan_fwd_noalloc(const ssm_scan_desc *desc,
                         const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *h0, void *y, float *h_last, hipStream_t stream);

/* ssm_scan_workspace_size / ssm_scan_fwd with an explicit launch shape
 * (tuning == NULL is the same as the plain calls). */
size_t ssm_scan_workspace_size_tuned(const ssm_scan_desc *desc, const ssm_scan_tuning *tuning);
int ssm_scan_fwd_tuned(const ssm_scan_desc *desc,
                       const void *u, const void *delta, const float *A,
                       const void *B, const void *C, const float *D, const void *z,
                       const float *h0, void *y, float *h_last,
                       void *workspace, size_t workspace_bytes,
                       const ssm_scan_tuning *tuning, hipStream_t stream);

/* The launch shape ssm_scan_fwd would use for `desc` (written to *out). */
int ssm_scan_plan(const ssm_scan_desc *desc, ssm_scan_tuning *out);

/*
 * Backward of ssm_scan_fwd: the gradients of
 *     loss = sum_{b,t,d} dy[b,t,d] * y[b,t,d] + sum_{b,d,n} dh_last[b,d,n] * h_last[b,d,n]
 * with respect to u, delta, A, B, C, D, z and h0, for the same inputs and
 * discretisation as the forward call. The states are recomputed on the GPU
 * (a checkpoint every 16 tokens, or 8 for dstate > 16, then a reverse pass
 * per chunk) instead of being stored by the forward (doyouknow.kr "Mamba와
 * 상태 공간 모델(SSM)의 부상 완벽 가이드" §3-3: the backward recomputes the
 * intermediate states). With lam_t = dloss/dh_t:
 *     lam_t = C_t * dy_t g(z_t) + exp(delta_{t+1} A) lam_{t+1}
 * and every gradient follows by the chain rule through the recurrence,
 * readout, skip and gate stated above.
 *
 *   u .. h0       as for ssm_scan_fwd (same shapes, types, layouts)
 *   dy            (batch, seqlen, dim) dtype: gradient of y
 *   dh_last       (batch, dim, dstate) fp32 gradient of the final state, or NULL (0)
 *   du, ddelta    (batch, seqlen, dim) dtype, written
 *   dz            (batch, seqlen, dim) dtype, written; required when z is given, unused otherwise
 *   dA            (dim, dstate) fp32, written (summed over batch and time)
 *   dB, dC        (batch, seqlen, dstate) fp32, written (summed over channels)
 *   dD            (dim) fp32, written; required when D is given, unused otherwise
 *   dh0           (batch, dim, dstate) fp32, written, or NULL (not wanted)
 *   ddelta_bias   (dim) fp32, written when desc->delta_bias is given (else unused)
 *   dconv_weight  (dim, W) fp32, written; required when desc->conv_width W > 0 (else unused)
 *   dconv_bias    (dim) fp32, written when given and W > 0 (else unused); NULL: not wanted
 * With a delta bias or softplus in the descriptor, ddelta is the gradient of
 * the raw delta (the chain rule through the bias and softplus). With the
 * convolution prologue (W > 0), u holds x as for ssm_scan_fwd and du receives
 * the gradient of x: with pre_t = conv_bias + sum_k w[k] x_{t-(W-1)+k} and
 * g_t the gradient of the scan input u_t = silu(pre_t),
 *     dpre_t = g_t silu'(pre_t),  dx_s = sum_k w[k] dpre_{s+(W-1)-k},
 *     dconv_weight[k] = sum_{b,t} dpre_t x_{t-(W-1)+k},  dconv_bias = sum_{b,t} dpre_t
 * (the chain rule through youngju.dev MambaBlock.forward's x_conv =
 * silu(conv1d(x))). u is formed from x once, in fp32 in the workspace; the
 * recomputation reads it (or, when the sequence is split into segments, forms
 * it from x again as the forward does), and the reverse pass writes its
 * gradient in fp32 in the workspace.
 *   workspace     at least ssm_scan_bwd_workspace_size(desc) bytes, 256-byte
 *                 aligned; contents on entry do not matter.
 * Results do not depend on timing: every sum over channels, batch rows or
 * tiles is taken in a fixed order. Outputs must not overlap each other, any
 * input or the workspace. seqlen == 0 writes dA = 0, dD = 0, dh0 = dh_last.
 */
size_t ssm_scan_bwd_workspace_size(const ssm_scan_desc *desc);
int ssm_scan_bwd(const ssm_scan_desc *desc,
                 const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *h0, const void *dy, const float *dh_last,
                 void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD,
                 void *dz, float *dh0, float *ddelta_bias, float *dconv_weight, float *dconv_bias,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The forward and backward of one training step, sharing the recomputation
 * the backward starts with. ssm_scan_fwd_save is ssm_scan_fwd (same arguments
 * and results) run in the backward's launch shape, which also leaves in
 * `workspace` what the backward would first recompute: the state
 * at the start of every chunk of the sequence and the regrouped B and C (the
 * intermediate states of doyouknow.kr "Mamba와 상태 공간 모델(SSM)의 부상 완벽
 * 가이드" §3-3, kept at chunk granularity).
 * ssm_scan_bwd_saved is ssm_scan_bwd without that recomputation; it reads
 * them from the same workspace instead. Its gradients equal ssm_scan_bwd's
 * (the checkpoints are the states the forward passes through). h_last equals
 * ssm_scan_fwd's bit for bit; y may differ from it in the last bit where the
 * backward's launch shape splits the states over another number of waves
 * and so sums the readout in another order. With the convolution prologue the
 * saving forward leaves its fp32 u where the backward then reads it.
 *
 *   workspace  at least ssm_scan_bwd_workspace_size(desc) bytes, 256-byte
 *              aligned, for both calls. ssm_scan_bwd_saved must receive the
 *              workspace of an ssm_scan_fwd_save call with the same descriptor
 *              and the same u, delta, A, B, C, h0 (and delta bias, convolution
 *              taps), unmodified in between; nothing checks this, and other
 *              contents give wrong gradients.
 * Every other argument, condition and error is that of ssm_scan_fwd and
 * ssm_scan_bwd. The caller owns the workspace and keeps it alive from the
 * forward call until the backward call has completed on its stream.
 */
int ssm_scan_fwd_save(const ssm_scan_desc *desc,
                      const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z,
                      const float *h0, void *y, float *h_last,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);
int ssm_scan_bwd_saved(const ssm_scan_desc *desc,
                       const void *u, const void *delta, const float *A,
                       const void *B, const void *C, const float *D, const void *z,
                       const float *h0, const void *dy, const float *dh_last,
                       void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD,
                       void *dz, float *dh0, float *ddelta_bias, float *dconv_weight, float *dconv_bias,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step: the recurrence for a single new token per sequence, with
 * the fixed-size state updated in place (itwiki "상태 공간 모델", "순환 형태와
 * 합성곱 형태": generation only updates h_t; ricepunchb "Mamba" §4.2: only the
 * last hidden state is needed to produce the next token).
 *
 *   x, delta, z  (batch, dim)          dtype; z may be NULL (no gate)
 *   delta_bias   (dim) fp32 or NULL; delta_softplus 0 or 1: the step is
 *                softplus(delta + bias) as for the scan descriptor
 *   A            (dim, dstate)         fp32
 *   B, C         (batch, dstate)       dtype
 *   D            (dim) fp32 or NULL
 *   h            (batch, dim, dstate)  fp32, read and overwritten
 *   y            (batch, dim)          dtype, written; must not overlap h or an input
 * Equal to ssm_scan_fwd with seqlen 1, h0 = h and h_last = h.
 */
int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int32_t dtype, int32_t disc,
                     const void *x, const void *delta, const float *delta_bias, int32_t delta_softplus,
                     const float *A,
                     const void *B, const void *C, const float *D, const void *z,
                     float *h, void *y, hipStream_t stream);

/*
 * Mamba-2 SSD layer (structured state-space duality). Each head h has a
 * scalar decay rate A[h] (the state matrix restricted to a scalar times the
 * identity: itwiki "상태 공간 모델", section "Mamba-2와 상태 공간 쌍대성";
 * eommydocs "State Space Models (SSM)", §2.4) and a (headdim x dstate) state;
 * the heads of a group share B and C. Per batch row b, head h, p < headdim:
 *
 *   dt_t    = dt[b,t,h] (+ dt_bias[h]), through softplus when dt_softplus
 *   H_t     = exp(dt_t A[h]) H_{t-1} + wbar_t x[b,t,h,:] B[b,t,g,:]^T     H_{-1} = h0 (or 0)
 *   wbar_t  = dt_t (SSM_DISC_EULER) or (exp(dt_t A[h]) - 1)/A[h] (SSM_DISC_ZOH)
 *   y[b,t,h,p] = sum_n C[b,t,g,n] H_t[p,n] + D[h] x[b,t,h,p],  times silu(z[b,t,h,p]) with a gate
 *
 * with g = h / (nheads / ngroups). The library evaluates it chunk by chunk
 * in the attention-like form of youngju.dev "mamba-state-space-model-
 * selective-ssm", SSDBlock._chunk_scan (scores C_i . B_j times the causal
 * decay exp(A (cum dt_i - cum dt_j)), applied to wbar x), with the state
 * carried from chunk to chunk, on bf16 matrix cores with fp32 accumulation;
 * the state is kept in fp32 and rounded to bf16 only as a matrix operand.
 */
typedef struct {
    int64_t batch;     /* >= 0 */
    int64_t seqlen;    /* >= 0 */
    int32_t nheads;    /* H >= 1 */
    int32_t headdim;   /* P: 64, 96 or 128 */
    int32_t ngroups;   /* G >= 1, dividing nheads */
    int32_t dstate;    /* N: 64 or 128 */
    int32_t dtype;     /* SSM_BF16 (SSM_F32 is reported as SSM_ERR_UNSUPPORTED) */
    int32_t disc;      /* ssm_disc */
    int32_t dt_softplus;    /* 0 or 1 */
    int32_t reserved;       /* 0 */
    const float *dt_bias;   /* (nheads) fp32 device pointer, or NULL */
} ssm_ssd_desc;

/*
 *   x, z      (batch, seqlen, nheads, headdim)  bf16, row-major; z may be NULL (no gate)
 *   dt        (batch, seqlen, nheads)           bf16
 *   A         (nheads) fp32 (negative for a decaying state); D (nheads) fp32 or NULL
 *   B, C      (batch, seqlen, ngroups, dstate)  bf16
 *   h0        (batch, nheads, headdim, dstate)  fp32, or NULL for zeros
 *   y         (batch, seqlen, nheads, headdim)  bf16, written
 *   h_last    (batch, nheads, headdim, dstate)  fp32, written, or NULL; may equal h0 exactly
 * x, z, y, B, C, h0 and h_last must be 16-byte aligned (dt 2-byte, A, D,
 * dt_bias 4-byte): SSM_ERR_ALIGN otherwise. Outputs must not overlap inputs
 * or each other (SSM_ERR_ALIAS). No workspace. seqlen == 0 writes h_last = h0
 * (or zeros) and no y.
 */
int ssm_ssd_fwd(const ssm_ssd_desc *desc, const void *x, const void *dt, const float *A,
                const void *B, const void *C, const float *D, const void *z, const float *h0,
                void *y, float *h_last, hipStream_t stream);

/*
 * One decode step of the SSD layer: the recurrence above for a single new
 * token per sequence, with each head's (headdim x dstate) state updated in
 * place (itwiki "상태 공간 모델", "순환 형태와 합성곱 형태": generation only
 * updates the state; the SSD layer's state as above). desc->seqlen must be 1.
 *
 *   x, z      (batch, nheads, headdim)   bf16; z may be NULL (no gate)
 *   dt        (batch, nheads)            bf16 (desc->dt_bias, dt_softplus and disc as for ssm_ssd_fwd)
 *   A, D      (nheads) fp32; D may be NULL
 *   B, C      (batch, ngroups, dstate)   bf16, 8-byte aligned
 *   h         (batch, nheads, headdim, dstate) fp32, 16-byte aligned, read and overwritten
 *   y         (batch, nheads, headdim)   bf16, written; must not overlap h or an input
 * Equal to ssm_ssd_fwd with seqlen 1, h0 = h and h_last = h, computed
 * directly in fp32 (no matrix cores: one token is a rank-1 update).
 */
int ssm_ssd_state_update(const ssm_ssd_desc *desc, const void *x, const void *dt, const float *A,
                         const void *B, const void *C, const float *D, const void *z, float *h,
                         void *y, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *ssm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
