"""Arbitrary-precision brute force of the selective scan, for tiny inputs.

TEST INFRASTRUCTURE ONLY (a pin for the fp64 oracle, not a second oracle of
the product). It evaluates the scan in the unrolled form instead of the
recurrence: with a_r = exp(delta_r * A) and bu_s the input term,

    h_t = (prod_{r<=t} a_r) * h0 + sum_{s<=t} (prod_{s<r<=t} a_r) * bu_s

which is the recurrence h_t = a_t h_{t-1} + bu_t written out (eommydocs
"State Space Models (SSM)" §3.2 pseudo-code; itwiki "상태 공간 모델",
"동작 원리 › 이산화"), then y_t = sum_n C_t[n] h_t[n] + D u_t, gated by SiLU(z)
(youngju.dev MambaBlock.forward). All arithmetic is mpmath at 50 digits, in
O(L^2) per state: use it for L up to a few dozen.
"""
from __future__ import annotations

import mpmath as mp
import numpy as np


def _bf16_to_float(bits):
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def _widen(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return _bf16_to_float(a)
    return a.astype(np.float64)


def selective_scan(u, delta, A, B, C, D=None, z=None, h0=None, disc="euler", dps=50):
    """Brute-force scan; returns (y (batch,L,dim), h_last (batch,dim,N)) as float64."""
    u, delta, A, B, C = (_widen(x) for x in (u, delta, A, B, C))
    D = None if D is None else _widen(D)
    z = None if z is None else _widen(z)
    h0 = None if h0 is None else _widen(h0)
    batch, L, dim = u.shape
    N = A.shape[1]
    y = np.zeros((batch, L, dim))
    hl = np.zeros((batch, dim, N))
    with mp.workdps(dps):
        for b in range(batch):
            for d in range(dim):
                abar = [[mp.e ** (mp.mpf(delta[b, t, d]) * mp.mpf(A[d, n])) for n in range(N)]
                        for t in range(L)]
                bu = [[None] * N for _ in range(L)]
                for t in range(L):
                    dt = mp.mpf(delta[b, t, d])
                    for n in range(N):
                        a = mp.mpf(A[d, n])
                        if disc == "zoh":
                            coef = mp.expm1(dt * a) / a if a != 0 else dt
                        else:
                            coef = dt
                        bu[t][n] = coef * mp.mpf(B[b, t, n]) * mp.mpf(u[b, t, d])
                h = [None] * N
                for t in range(L):
                    for n in range(N):
                        acc = mp.mpf(0)
                        if h0 is not None:
                            prod = mp.mpf(1)
                            for r in range(t + 1):
                                prod *= abar[r][n]
                            acc += prod * mp.mpf(h0[b, d, n])
                        for s in range(t + 1):
                            prod = mp.mpf(1)
                            for r in range(s + 1, t + 1):
                                prod *= abar[r][n]
                            acc += prod * bu[s][n]
                        h[n] = acc
                    yt = mp.fsum(mp.mpf(C[b, t, n]) * h[n] for n in range(N))
                    if D is not None:
                        yt += mp.mpf(D[d]) * mp.mpf(u[b, t, d])
                    if z is not None:
                        zz = mp.mpf(z[b, t, d])
                        yt *= zz / (1 + mp.e ** (-zz))
                    y[b, t, d] = float(yt)
                for n in range(N):
                    hl[b, d, n] = float(h[n]) if L > 0 else (0.0 if h0 is None else h0[b, d, n])
    return y, hl
