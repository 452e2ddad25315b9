"""Seeded synthetic inputs for the selective scan and the decode step.

Shared by the tests, the bench and the smoke check, and by both sides of
every parity comparison (the HIP path and the fp64 oracle). It holds none of
the scan's arithmetic: it only draws random tensors, shapes them like a Mamba
layer's scan inputs and rounds them to the storage type.

Recipe (one workload per entry of ``CONFIGS``):
  * u, B, C, z ~ N(0, 1); decode state h ~ N(0, 1).
  * delta = softplus(0.5 * N(0,1) + bias[d]) with one bias per channel,
    bias = inv_softplus(U[1e-3, 1e-1]), or inv_softplus of a log-uniform draw
    in [1e-4, 1e-1] for the long-context workload. delta is therefore
    positive, as after the softplus of youngju.dev SelectiveSSM.forward.
  * A[d, n] = -(n + 1): the S4D-Real values that the pages' A_log = log(1..N)
    initialisation produces (eommydocs §5.1 SelectiveSSM, youngju.dev
    MambaBlock.__init__).
  * D = 1 (tiny workload) or D ~ N(1, 0.1).
  * bf16 tensors are produced as float32 and rounded to nearest-even; they are
    returned as uint16 bit patterns, which both sides read.
Streams: numpy PCG64 children of SeedSequence(seed), one per tensor in the
fixed order [u, delta_noise, delta_bias, B, C, z, D, h0]; large tensors are
drawn in fixed 4 Mi-element blocks, each from its own grandchild seed, so the
values do not depend on the number of threads used to draw them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK = 1 << 22
STREAMS = ("u", "delta_noise", "delta_bias", "B", "C", "z", "D", "h0", "dy", "dh_last", "conv")


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str          # "f32" or "bf16": type of u, delta, B, C, z, y
    gate: bool          # z present
    d_skip: str         # "ones" or "normal"
    bias: str           # "uniform" or "loguniform"

    @property
    def tokens_ch(self) -> int:
        return self.batch * self.seqlen * self.dim


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int
    dtype: str = "bf16"
    gate: bool = True
    bias: str = "uniform"


CONFIGS = {
    "tiny": ScanConfig("tiny", 1, 64, 16, 4, "f32", False, "ones", "uniform"),
    "mamba130m": ScanConfig("mamba130m", 4, 2048, 1536, 16, "bf16", True, "normal", "uniform"),
    "mamba1.4b": ScanConfig("mamba1.4b", 8, 8192, 4096, 16, "bf16", True, "normal", "uniform"),
    "long": ScanConfig("long", 1, 131072, 5120, 16, "bf16", True, "normal", "loguniform"),
}
DECODE = DecodeConfig("decode", 256, 5120, 16, 1000)


@dataclass(frozen=True)
class SsdConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    gate: bool = False
    skip: bool = False
    dtype: str = "bf16"

    @property
    def tokens_ch(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim


# Mamba-2 SSD layers. "ssd-block" has the head shape of youngju.dev SSDBlock's
# defaults (d_model 768 as 8 heads of 96, d_state 128); "mamba2-ssd" puts the
# same layer at the scale of the Mamba-1.4B-shaped scan workload (batch 8,
# 8192 tokens, 4096 channels as 64 heads of 64, d_state 128, one group).
SSD_CONFIGS = {
    "ssd-block": SsdConfig("ssd-block", 2, 1000, 8, 96, 1, 128),
    "mamba2-ssd": SsdConfig("mamba2-ssd", 8, 8192, 64, 64, 1, 128),
}


def ssd_inputs(cfg: SsdConfig, seed: int = 0, batch=None, seqlen=None, nheads=None, headdim=None,
               ngroups=None, dstate=None, gate=None, skip=None):
    """Inputs of one SSD layer (sizes and options may be overridden):
    x, z ~ N(0, 1) (batch, L, H, P); dt = softplus(0.5 N(0,1) + bias[h])
    (batch, L, H) with the scan recipe's per-head bias; B, C ~ N(0, 1)
    (batch, L, G, N); A[h] = -(h + 1) (youngju.dev SSDBlock: A_log =
    log(1..n_heads)); D ~ N(1, 0.1) per head when the skip is on. bf16
    tensors are uint16 patterns."""
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    H = cfg.nheads if nheads is None else nheads
    P = cfg.headdim if headdim is None else headdim
    G = cfg.ngroups if ngroups is None else ngroups
    N = cfg.dstate if dstate is None else dstate
    gate = cfg.gate if gate is None else gate
    skip = cfg.skip if skip is None else skip
    bias = delta_bias(seed, H, "uniform")
    return dict(
        x=_normal(seed, "u", (b, L, H, P), cfg.dtype),
        dt=_delta(seed, (b, L, H), bias, cfg.dtype),
        A=-np.arange(1, H + 1, dtype=np.float32),
        B=_normal(seed, "B", (b, L, G, N), cfg.dtype),
        C=_normal(seed, "C", (b, L, G, N), cfg.dtype),
        D=d_skip(seed, H, "normal") if skip else None,
        z=_normal(seed, "z", (b, L, H, P), cfg.dtype) if gate else None,
        h0=None,
    )


def ssd_bytes(cfg: SsdConfig, h_last: bool = True) -> int:
    """Bytes one SSD layer must move: x, dt, B, C (and z) once, y once, A and D,
    and the final state."""
    es = 2 if cfg.dtype == "bf16" else 4
    tok = cfg.batch * cfg.seqlen
    nbytes = (2 + (1 if cfg.gate else 0)) * cfg.tokens_ch * es      # x, y (+ z)
    nbytes += tok * cfg.nheads * es                                 # dt
    nbytes += 2 * tok * cfg.ngroups * cfg.dstate * es               # B, C
    nbytes += cfg.nheads * 4 * (2 if cfg.skip else 1)               # A (+ D)
    if h_last:
        nbytes += cfg.batch * cfg.nheads * cfg.headdim * cfg.dstate * 4
    return nbytes


def ssd_flops(cfg: SsdConfig, chunk: int = 64) -> int:
    """Matrix-core flops of the chunked evaluation at chunk length Q, per
    (token, head): scores Q N / 2 and the masked product Q P / 2 (the causal
    half), the state readout N P and the state update N P, two flops each."""
    Q, N, P = chunk, cfg.dstate, cfg.headdim
    per = 2 * (Q * N // 2 + Q * P // 2 + 2 * N * P)
    return per * cfg.batch * cfg.seqlen * cfg.nheads


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(seed: int, name: str) -> np.random.SeedSequence:
    return np.random.SeedSequence(seed).spawn(len(STREAMS))[STREAMS.index(name)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def softplus(x):
    return np.logaddexp(0.0, x)


def inv_softplus(y):
    return np.log(np.expm1(y))


def _blocked(seed_seq, total, fill, out_dtype):
    """Fill a flat array of ``total`` elements block by block, in parallel."""
    out = np.empty(total, dtype=out_dtype)
    nblocks = (total + BLOCK - 1) // BLOCK
    children = seed_seq.spawn(nblocks) if nblocks else []

    def work(i):
        lo, hi = i * BLOCK, min(total, (i + 1) * BLOCK)
        rng = np.random.Generator(np.random.PCG64(children[i]))
        out[lo:hi] = fill(rng, lo, hi)

    if nblocks <= 1:
        for i in range(nblocks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblocks)))
    return out


def _normal(seed, name, shape, dtype):
    total = int(np.prod(shape))
    if dtype == "bf16":
        fill = lambda rng, lo, hi: to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))
        return _blocked(_stream(seed, name), total, fill, np.uint16).reshape(shape)
    fill = lambda rng, lo, hi: rng.standard_normal(hi - lo, dtype=np.float32)
    return _blocked(_stream(seed, name), total, fill, np.float32).reshape(shape)


def delta_bias(seed: int, dim: int, kind: str) -> np.ndarray:
    """Per-channel pre-softplus bias of delta (float64)."""
    rng = np.random.Generator(np.random.PCG64(_stream(seed, "delta_bias")))
    if kind == "loguniform":
        target = np.exp(rng.uniform(np.log(1e-4), np.log(1e-1), size=dim))
    else:
        target = rng.uniform(1e-3, 1e-1, size=dim)
    return inv_softplus(target)


def _delta(seed, shape, bias, dtype, stream="delta_noise"):
    dim = shape[-1]
    total = int(np.prod(shape))

    def fill(rng, lo, hi):
        noise = rng.standard_normal(hi - lo, dtype=np.float32).astype(np.float64)
        d_idx = np.arange(lo, hi, dtype=np.int64) % dim
        val = softplus(0.5 * noise + bias[d_idx]).astype(np.float32)
        return to_bf16_bits(val) if dtype == "bf16" else val

    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    return _blocked(_stream(seed, stream), total, fill, out_dtype).reshape(shape)


def a_matrix(dim: int, dstate: int) -> np.ndarray:
    """A[d, n] = -(n + 1), float32."""
    return np.broadcast_to(-np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)).copy()


def d_skip(seed: int, dim: int, kind: str) -> np.ndarray:
    if kind == "ones":
        return np.ones(dim, np.float32)
    rng = np.random.Generator(np.random.PCG64(_stream(seed, "D")))
    return rng.normal(1.0, 0.1, size=dim).astype(np.float32)


def scan_inputs(cfg: ScanConfig, seed: int = 0, batch: int | None = None,
                seqlen: int | None = None, dim: int | None = None, dstate: int | None = None):
    """Inputs of one scan workload (sizes may be overridden for reduced tests).

    Returns a dict with u, delta, A, B, C, D, z (None without a gate), h0 (None).
    """
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    d = cfg.dim if dim is None else dim
    N = cfg.dstate if dstate is None else dstate
    bias = delta_bias(seed, d, cfg.bias)
    return dict(
        u=_normal(seed, "u", (b, L, d), cfg.dtype),
        delta=_delta(seed, (b, L, d), bias, cfg.dtype),
        A=a_matrix(d, N),
        B=_normal(seed, "B", (b, L, N), cfg.dtype),
        C=_normal(seed, "C", (b, L, N), cfg.dtype),
        D=d_skip(seed, d, cfg.d_skip),
        z=_normal(seed, "z", (b, L, d), cfg.dtype) if cfg.gate else None,
        h0=None,
    )


def raw_delta_inputs(cfg: ScanConfig, seed: int = 0, batch: int | None = None,
                     seqlen: int | None = None, dim: int | None = None):
    """The step before its bias and softplus, for the in-kernel step option:
    delta_raw = 0.5 N(0, 1) (batch, L, dim) in the workload's element type and
    the per-channel bias (dim,) float32, so that softplus(delta_raw + bias)
    follows the same recipe as ``scan_inputs``' delta."""
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    d = cfg.dim if dim is None else dim
    total = b * L * d

    def fill(rng, lo, hi):
        val = (0.5 * rng.standard_normal(hi - lo, dtype=np.float32)).astype(np.float32)
        return to_bf16_bits(val) if cfg.dtype == "bf16" else val

    out_dtype = np.uint16 if cfg.dtype == "bf16" else np.float32
    raw = _blocked(_stream(seed, "delta_noise"), total, fill, out_dtype).reshape(b, L, d)
    return dict(delta=raw, delta_bias=delta_bias(seed, d, cfg.bias).astype(np.float32))


def conv_inputs(dim: int, width: int = 4, seed: int = 0):
    """Taps (dim, width) and bias (dim,) of the causal depthwise convolution
    prologue, float32, uniform in +-1/sqrt(width) (a depthwise convolution's
    fan-in is its width)."""
    rng = np.random.Generator(np.random.PCG64(_stream(seed, "conv")))
    bound = 1.0 / np.sqrt(width)
    w = rng.uniform(-bound, bound, (dim, width)).astype(np.float32)
    b = rng.uniform(-bound, bound, dim).astype(np.float32)
    return dict(conv_weight=w, conv_bias=b)


def grad_inputs(cfg: ScanConfig, seed: int = 0, batch: int | None = None,
                seqlen: int | None = None, dim: int | None = None, dstate: int | None = None):
    """Upstream gradients for the backward of one scan workload: dy ~ N(0, 1) in
    the workload's element type (batch, L, dim) and dh_last ~ N(0, 1) float32
    (batch, dim, N)."""
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    d = cfg.dim if dim is None else dim
    N = cfg.dstate if dstate is None else dstate
    return dict(dy=_normal(seed, "dy", (b, L, d), cfg.dtype),
                dh_last=_normal(seed, "dh_last", (b, d, N), "f32"))


def decode_static(cfg: DecodeConfig = DECODE, seed: int = 0, batch=None, dim=None, dstate=None):
    """A, D, the initial state h (fp32 N(0,1)) and the delta bias of a decode workload."""
    b = cfg.batch if batch is None else batch
    d = cfg.dim if dim is None else dim
    N = cfg.dstate if dstate is None else dstate
    return dict(A=a_matrix(d, N), D=d_skip(seed, d, "normal"),
                h=_normal(seed, "h0", (b, d, N), "f32"),
                bias=delta_bias(seed, d, cfg.bias))


def decode_step(cfg: DecodeConfig = DECODE, step_set: int = 0, seed: int = 0,
                batch=None, dim=None, dstate=None, bias=None):
    """Per-token inputs x, delta, z (batch, dim) and B, C (batch, N) of one step set."""
    b = cfg.batch if batch is None else batch
    d = cfg.dim if dim is None else dim
    N = cfg.dstate if dstate is None else dstate
    if bias is None:
        bias = delta_bias(seed, d, cfg.bias)
    s = seed + 1000003 * (step_set + 1)   # a distinct master seed per step set
    return dict(
        x=_normal(s, "u", (b, d), cfg.dtype),
        delta=_delta(s, (b, d), bias, cfg.dtype),
        B=_normal(s, "B", (b, N), cfg.dtype),
        C=_normal(s, "C", (b, N), cfg.dtype),
        z=_normal(s, "z", (b, d), cfg.dtype) if cfg.gate else None,
    )


def algorithmic_bytes(cfg: ScanConfig, h_last: bool = True, h0: bool = False) -> int:
    """Bytes the scan must move: every input once, every output once."""
    es = 4 if cfg.dtype == "f32" else 2
    per_tok = 3 if not cfg.gate else 4          # u, delta, y (+ z)
    nbytes = per_tok * cfg.tokens_ch * es
    nbytes += 2 * cfg.batch * cfg.seqlen * cfg.dstate * es      # B, C
    nbytes += cfg.dim * cfg.dstate * 4 + cfg.dim * 4            # A, D
    if h_last:
        nbytes += cfg.batch * cfg.dim * cfg.dstate * 4
    if h0:
        nbytes += cfg.batch * cfg.dim * cfg.dstate * 4
    return nbytes


def decode_bytes(cfg: DecodeConfig = DECODE) -> int:
    """Bytes one decode step must move: h read and written, x/delta/z/y, B/C, A, D."""
    es = 2 if cfg.dtype == "bf16" else 4
    bd = cfg.batch * cfg.dim
    return (2 * bd * cfg.dstate * 4 + (4 if cfg.gate else 3) * bd * es
            + 2 * cfg.batch * cfg.dstate * es + cfg.dim * cfg.dstate * 4 + cfg.dim * 4)
