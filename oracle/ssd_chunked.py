"""The Mamba-2 SSD layer evaluated chunk by chunk, in numpy float64.

TEST INFRASTRUCTURE ONLY (a pin of the sequential oracle ``oracle_ssd``, not
the product). It follows the chunked algorithm of youngju.dev
"mamba-state-space-model-selective-ssm", class SSDBlock, method _chunk_scan:
split the sequence into chunks, take the cumulative sum of the per-token log
decay inside each chunk, build the causal decay matrix
exp(a * (cum_i - cum_j)) for i >= j, and evaluate the chunk like a masked
attention, scores C_i . B_j times that matrix applied to the values. The page
stops at the chunk-internal term; the terms that carry the state across
chunk boundaries are derived here from the same recurrence (itwiki "상태 공간
모델", section "Mamba-2와 상태 공간 쌍대성": the recurrent and the attention
form of one computation, mixed by chunk):

  inside a chunk with first token c0, S_i = sum_{c0 <= r <= i} a dt_r and
  the state H entering the chunk,
    y_i   = sum_{c0 <= j <= i} (C_i . B_j) exp(S_i - S_j) wbar_j x_j     (attention-like part)
          + exp(S_i) * (C_i . H)                                          (state entering the chunk)
    H_out = exp(S_last) H + sum_j exp(S_last - S_j) wbar_j x_j B_j^T     (state leaving the chunk)

Every array op is a numpy einsum, cumsum or exp; no blocking beyond the chunk
split that the page itself makes.
"""
from __future__ import annotations

import numpy as np


def _widen(a):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ssd_chunked(x, dt, A, B, C, D=None, z=None, h0=None, disc="euler", dt_bias=None,
                dt_softplus=False, chunk=256):
    """y (batch, L, H, P) and h_last (batch, H, P, N) of the SSD layer."""
    x, dt, B, C, z = (_widen(v) for v in (x, dt, B, C, z))
    A = np.asarray(A, dtype=np.float64)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    step = dt + (0.0 if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)[None, None, :])
    if dt_softplus:
        step = np.logaddexp(0.0, step)
    la = step * A[None, None, :]                       # log decay of each token, (b, L, H)
    if disc == "zoh":
        safe = np.where(A == 0.0, 1.0, A)[None, None, :]
        wbar = np.where(A[None, None, :] == 0.0, step, np.expm1(la) / safe)
    else:
        wbar = step
    group = np.arange(H) // (H // G)
    Bh = B[:, :, group, :]                             # (b, L, H, N): each head's group
    Ch = C[:, :, group, :]
    xw = x * wbar[..., None]                           # wbar_j x_j, (b, L, H, P)
    state = np.zeros((batch, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((batch, L, H, P))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        S = np.cumsum(la[:, c0:c1], axis=1)            # (b, Q, H), inclusive
        Q = c1 - c0
        causal = np.tril(np.ones((Q, Q), dtype=bool))
        decay = np.exp(S[:, :, None, :] - S[:, None, :, :])          # (b, i, j, H)
        decay = np.where(causal[None, :, :, None], decay, 0.0)
        scores = np.einsum("bihn,bjhn->bijh", Ch[:, c0:c1], Bh[:, c0:c1])
        y_in = np.einsum("bijh,bjhp->bihp", scores * decay, xw[:, c0:c1])
        y_st = np.einsum("bihn,bhpn->bihp", Ch[:, c0:c1], state) * np.exp(S)[..., None]
        y[:, c0:c1] = y_in + y_st
        to_end = np.exp(S[:, -1:, :] - S)              # exp(S_last - S_j), (b, Q, H)
        state = (state * np.exp(S[:, -1, :])[:, :, None, None]
                 + np.einsum("bjhn,bjhp->bhpn", Bh[:, c0:c1] * to_end[..., None], xw[:, c0:c1]))
    if D is not None:
        y = y + np.asarray(D, dtype=np.float64)[None, None, :, None] * x
    if z is not None:
        y = y * (z / (1.0 + np.exp(-z)))
    return y, state
