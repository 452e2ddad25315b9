"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with an independent statement of the
same quantity. They are collected by ``test_oracle_pins.py`` against the real
oracle and by ``test_oracle_mutants.py`` against deliberately broken copies of
it (to show that a plausible mistake anywhere in the oracle fails a pin).

None of these re-types the oracle's loop. The independent statements are:
  * the unrolled sum-of-products form in arbitrary precision (``oracle.brute``),
  * the LTI convolution kernel K_k = sum_n C_n Abar_n^k Bbar_n with
    Abar^k = exp(k*delta*A) in closed form (itwiki "상태 공간 모델", "순환 형태와
    합성곱 형태"), as a direct causal convolution and through numpy.fft with
    zero padding to 2L (youngju.dev S4Layer.forward),
  * delta -> 0 keeps the state (itwiki "Mamba의 선택 메커니즘";
    ricepunchb "Mamba" §3.2; doyouknow.kr §3-1),
  * large delta forgets and focuses on the input (same passages),
  * zero-order hold is the exact solution of x' = Ax + Bu with u held over the
    step (eommydocs §1.2; itwiki "이산화"), checked by RK4 integration,
  * N = 1, A = 0 reduces the scan to a prefix sum (numpy.cumsum),
  * the affine-pair composition (a1,b1).(a2,b2) = (a2 a1, a2 b1 + b2) is
    associative (ricepunchb "Mamba" §5.1),
  * resuming from the last state reproduces the tail (ricepunchb §4.2:
    only the last hidden state is needed to continue),
  * with h0 = 0 and no gate the output is linear in u and causal,
  * the SiLU gate and the D skip at points with a closed form,
  * the convolution prologue equals numpy.convolve with reversed taps and the
    SiLU (youngju.dev MambaBlock.forward), and
  * the backward pass equals central finite differences of the forward oracle
    (the gradient of sum(dy*y) + sum(dh_last*h_last) by definition), and with
    dy = 0 the state gradient reduces to the closed form exp(A*sum(delta)),
  * the Mamba-2 SSD layer is the selective scan with A a scalar per head
    (itwiki "Mamba-2와 상태 공간 쌍대성"), equals the chunked attention-like
    evaluation of youngju.dev SSDBlock._chunk_scan with the state carried
    across chunks (oracle.ssd_chunked) for every chunk size, reduces to a
    causally masked matrix product when A = 0, and to the current token alone
    when A is very negative.
"""
from __future__ import annotations

import numpy as np

from oracle import brute

RNG_SEED = 1234


def rel_err(got, ref):
    """max |g - r| / max(|r|, rms(r)) over the tensor (rms floor for cancellation)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    with np.errstate(over="ignore", invalid="ignore"):
        rms = float(np.sqrt(np.mean(ref * ref)))
        floor = np.maximum(np.abs(ref), rms if rms > 0 else 1e-300)
        e = float(np.max(np.abs(got - ref) / floor))
    return e if np.isfinite(e) else float("inf")


def _case(rng, batch, L, dim, N, with_d=True, with_z=False, with_h0=False, a_zero=False):
    u = rng.standard_normal((batch, L, dim))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (batch, L, dim)))
    A = -np.exp(rng.uniform(np.log(0.2), np.log(8.0), (dim, N)))
    if a_zero:
        A[:] = 0.0
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    D = rng.normal(1.0, 0.3, dim) if with_d else None
    z = rng.standard_normal((batch, L, dim)) if with_z else None
    h0 = rng.standard_normal((batch, dim, N)) if with_h0 else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, h0=h0)


def pin_brute_force(o):
    """P1: the oracle equals the 50-digit unrolled form on small random cases."""
    rng = np.random.default_rng(RNG_SEED)
    cases = [
        (dict(batch=2, L=7, dim=3, N=3, with_d=True, with_z=True, with_h0=True), "euler"),
        (dict(batch=1, L=9, dim=2, N=4, with_d=False, with_z=False, with_h0=False), "euler"),
        (dict(batch=2, L=6, dim=2, N=2, with_d=True, with_z=True, with_h0=True), "zoh"),
        (dict(batch=1, L=5, dim=3, N=1, with_d=True, with_z=False, with_h0=True), "zoh"),
    ]
    for shape, disc in cases:
        x = _case(rng, **shape)
        y, hl = o.selective_scan(**x, disc=disc)
        yb, hb = brute.selective_scan(**x, disc=disc)
        assert rel_err(y, yb) < 1e-12, ("y", shape, disc, rel_err(y, yb))
        assert rel_err(hl, hb) < 1e-12, ("h_last", shape, disc, rel_err(hl, hb))


def pin_brute_force_storage_types(o):
    """P1 for float32 and bf16 inputs: the oracle widens them exactly."""
    rng = np.random.default_rng(RNG_SEED + 1)
    x = _case(rng, 2, 6, 3, 4, with_d=True, with_z=True, with_h0=False)
    for name in ("u", "delta", "B", "C", "z"):
        x[name] = x[name].astype(np.float32)
    y32, h32 = o.selective_scan(**x)
    yb, hb = brute.selective_scan(**x)
    assert rel_err(y32, yb) < 1e-12 and rel_err(h32, hb) < 1e-12
    bf = dict(x)
    for name in ("u", "delta", "B", "C", "z"):
        bits = x[name].view(np.uint32) >> np.uint32(16)      # truncation: any pattern will do
        bf[name] = bits.astype(np.uint16)
    ybf, hbf = o.selective_scan(**bf)
    widened = {k: (v if k not in ("u", "delta", "B", "C", "z")
                   else (bf[k].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64))
               for k, v in bf.items()}
    yw, hw = brute.selective_scan(**widened)
    assert rel_err(ybf, yw) < 1e-12 and rel_err(hbf, hw) < 1e-12


def _lti_case(rng, batch, L, dim, N, disc, with_h0):
    """Delta per channel, B and C held constant over t (and across batch rows)."""
    dch = np.exp(rng.uniform(np.log(1e-2), np.log(0.3), dim))
    A = -np.exp(rng.uniform(np.log(0.1), np.log(4.0), (dim, N)))
    Bn = rng.standard_normal(N)
    Cn = rng.standard_normal(N)
    u = rng.standard_normal((batch, L, dim))
    D = rng.normal(1.0, 0.2, dim)
    h0 = rng.standard_normal((batch, dim, N)) if with_h0 else None
    x = dict(u=u, delta=np.broadcast_to(dch, (batch, L, dim)).copy(), A=A,
             B=np.broadcast_to(Bn, (batch, L, N)).copy(), C=np.broadcast_to(Cn, (batch, L, N)).copy(),
             D=D, z=None, h0=h0)
    dA = dch[:, None] * A                                        # (dim, N)
    if disc == "zoh":
        bbar = np.expm1(dA) / A * Bn[None, :]
    else:
        bbar = dch[:, None] * Bn[None, :]
    k = np.arange(L)
    # K[d, k] = sum_n C_n exp(k dA[d,n]) Bbar[d,n]: the closed-form kernel
    K = np.einsum("n,dnk,dn->dk", Cn, np.exp(dA[:, :, None] * k[None, None, :]), bbar)
    # initial-state response: sum_n C_n exp((t+1) dA) h0
    if h0 is not None:
        free = np.einsum("n,dnt,bdn->btd", Cn, np.exp(dA[:, :, None] * (k[None, None, :] + 1)), h0)
    else:
        free = 0.0
    return x, K, free, D


def pin_lti_direct(o):
    """P2: constant delta, B, C -> y = u * K + D u, by direct causal convolution."""
    rng = np.random.default_rng(RNG_SEED + 2)
    for disc in ("euler", "zoh"):
        batch, L, dim, N = 2, 160, 3, 5
        x, K, free, D = _lti_case(rng, batch, L, dim, N, disc, with_h0=True)
        ref = np.zeros((batch, L, dim))
        for t in range(L):
            # y_t = sum_{k<=t} K_k u_{t-k}
            ref[:, t, :] = np.einsum("dk,bkd->bd", K[:, :t + 1][:, ::-1], x["u"][:, :t + 1, :])
        ref = ref + free + D[None, None, :] * x["u"]
        y, _ = o.selective_scan(**x, disc=disc)
        assert rel_err(y, ref) < 1e-10, (disc, rel_err(y, ref))


def pin_lti_fft(o):
    """P2 at length 4096 through an FFT convolution zero-padded to 2L."""
    rng = np.random.default_rng(RNG_SEED + 3)
    batch, L, dim, N = 1, 4096, 2, 4
    x, K, _, D = _lti_case(rng, batch, L, dim, N, "euler", with_h0=False)
    uf = np.fft.rfft(x["u"].transpose(0, 2, 1), n=2 * L)
    kf = np.fft.rfft(K, n=2 * L)
    conv = np.fft.irfft(uf * kf[None], n=2 * L)[..., :L].transpose(0, 2, 1)
    ref = conv + D[None, None, :] * x["u"]
    y, _ = o.selective_scan(**x)
    assert rel_err(y, ref) < 1e-10, rel_err(y, ref)


def pin_delta_zero(o):
    """P3: delta = 0 keeps h = h0 exactly and y_t = C_t . h0 + D u_t."""
    rng = np.random.default_rng(RNG_SEED + 4)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 12, 3, 4, with_d=True, with_z=False, with_h0=True)
        x["delta"] = np.zeros_like(x["delta"])
        y, hl = o.selective_scan(**x, disc=disc)
        assert np.array_equal(hl, x["h0"]), disc
        ref = np.einsum("btn,bdn->btd", x["C"], x["h0"]) + x["D"][None, None, :] * x["u"]
        assert rel_err(y, ref) < 1e-13, disc


def pin_large_delta(o):
    """P4: with A < 0 and a huge delta, Abar -> 0, so h_t is the current input term only:
    ZOH gives -B_t u_t / A, the simplified rule gives delta B_t u_t."""
    rng = np.random.default_rng(RNG_SEED + 5)
    x = _case(rng, 1, 6, 2, 3, with_d=False, with_z=False, with_h0=True)
    big = 2.0e3
    x["delta"] = np.full_like(x["delta"], big)
    for disc in ("zoh", "euler"):
        for L1 in range(1, 7):
            sub = dict(x, u=x["u"][:, :L1], delta=x["delta"][:, :L1], B=x["B"][:, :L1], C=x["C"][:, :L1])
            _, hl = o.selective_scan(**sub, disc=disc)
            bt = x["B"][0, L1 - 1]          # (N,)
            ut = x["u"][0, L1 - 1]          # (dim,)
            if disc == "zoh":
                ref = -(ut[:, None] * bt[None, :]) / x["A"]
            else:
                ref = big * ut[:, None] * bt[None, :]
            assert rel_err(hl[0], ref) < 1e-12, (disc, L1)


def _rk4_hold(a, bcoef, u, h, dt, steps=10000):
    """Integrate h' = a h + bcoef u over [0, dt] with u held, classic RK4."""
    f = lambda hh: a * hh + bcoef * u
    s = dt / steps
    for _ in range(steps):
        k1 = f(h)
        k2 = f(h + 0.5 * s * k1)
        k3 = f(h + 0.5 * s * k2)
        k4 = f(h + s * k3)
        h = h + s / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
    return h


def pin_zoh_exact_hold(o):
    """P5: one ZOH step equals the exact continuous solution with the input held,
    and the ZOH input term tends to the simplified one as delta -> 0."""
    rng = np.random.default_rng(RNG_SEED + 6)
    dim, N = 2, 3
    A = -np.exp(rng.uniform(np.log(0.2), np.log(5.0), (dim, N)))
    B = rng.standard_normal((1, 1, N))
    C = rng.standard_normal((1, 1, N))
    u = rng.standard_normal((1, 1, dim))
    h0 = rng.standard_normal((1, dim, N))
    delta = np.array([[[0.37, 1.3]]])
    _, hl = o.selective_scan(u=u, delta=delta, A=A, B=B, C=C, h0=h0, disc="zoh")
    ref = _rk4_hold(A, B[0, 0][None, :], u[0, 0][:, None], h0[0], delta[0, 0][:, None])
    assert np.all(np.abs(hl[0] - ref) <= 1e-10 * np.maximum(1.0, np.abs(ref))), (hl[0], ref)
    tiny = np.full((1, 1, dim), 1e-7)
    _, hz = o.selective_scan(u=u, delta=tiny, A=A, B=B, C=C, disc="zoh")
    _, he = o.selective_scan(u=u, delta=tiny, A=A, B=B, C=C, disc="euler")
    assert rel_err(hz, he) < 1e-6


def pin_prefix_sum(o):
    """P6: N = 1 and A = 0 make Abar = 1, so h_t = cumsum(delta B u) (both rules)."""
    rng = np.random.default_rng(RNG_SEED + 7)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 300, 3, 1, with_d=False, a_zero=True)
        y, hl = o.selective_scan(**dict(x, C=np.ones_like(x["C"])), disc=disc)
        ref = np.cumsum(x["delta"] * x["B"][:, :, :1] * x["u"], axis=1)
        assert rel_err(y, ref) < 1e-12, disc
        assert rel_err(hl[:, :, 0], ref[:, -1, :]) < 1e-12, disc


def _aggregate(o, x, disc):
    """Segment aggregate (P, H) from the oracle: P = decay of a unit state with no input,
    H = end state from zero."""
    N = x["A"].shape[1]
    batch, _, dim = x["u"].shape
    ones = np.ones((batch, dim, N))
    _, P = o.selective_scan(**dict(x, B=np.zeros_like(x["B"]), h0=ones, z=None), disc=disc)
    _, H = o.selective_scan(**dict(x, h0=None, z=None), disc=disc)
    return P, H


def pin_affine_composition(o):
    """P7: segments compose as affine maps h -> P h + H, and the composition is
    associative: any bracketing over four segments gives the full scan's state."""
    rng = np.random.default_rng(RNG_SEED + 8)
    x = _case(rng, 2, 40, 3, 4, with_d=True, with_z=False, with_h0=True)
    cuts = [0, 7, 19, 20, 40]
    segs = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        sub = {k: (v[:, lo:hi] if k in ("u", "delta", "B", "C") else v) for k, v in x.items()}
        segs.append(_aggregate(o, sub, "euler"))

    def comp(p, q):  # apply p first, then q
        return (q[0] * p[0], q[0] * p[1] + q[1])

    left = comp(comp(comp(segs[0], segs[1]), segs[2]), segs[3])
    right = comp(segs[0], comp(segs[1], comp(segs[2], segs[3])))
    tree = comp(comp(segs[0], segs[1]), comp(segs[2], segs[3]))
    _, hl = o.selective_scan(**x)
    for P, H in (left, right, tree):
        assert rel_err(P * x["h0"] + H, hl) < 1e-12


def pin_resume(o):
    """P8: scanning [0, L) equals scanning [0, L1) then [L1, L) from its last state."""
    rng = np.random.default_rng(RNG_SEED + 9)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 50, 3, 4, with_d=True, with_z=True, with_h0=True)
        y, hl = o.selective_scan(**x, disc=disc)
        L1 = 23
        head = {k: (v[:, :L1] if k in ("u", "delta", "B", "C", "z") else v) for k, v in x.items()}
        tail = {k: (v[:, L1:] if k in ("u", "delta", "B", "C", "z") else v) for k, v in x.items()}
        y1, h1 = o.selective_scan(**head, disc=disc)
        y2, h2 = o.selective_scan(**dict(tail, h0=h1), disc=disc)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y), disc
        assert np.array_equal(h2, hl), disc


def pin_decode_is_scan(o):
    """P9: k decode steps equal a k-token scan (state in, state out, per-token y)."""
    rng = np.random.default_rng(RNG_SEED + 10)
    for disc in ("euler", "zoh"):
        x = _case(rng, 3, 5, 4, 3, with_d=True, with_z=True, with_h0=True)
        y, hl = o.selective_scan(**x, disc=disc)
        h = x["h0"].copy()
        for t in range(5):
            yt = o.state_update(x["u"][:, t], x["delta"][:, t], x["A"], x["B"][:, t], x["C"][:, t],
                                h, D=x["D"], z=x["z"][:, t], disc=disc)
            assert rel_err(yt, y[:, t]) < 1e-14, (disc, t)
        assert rel_err(h, hl) < 1e-14, disc


def pin_linear_causal(o):
    """P10: with h0 = 0 and no gate, y is linear in u; y_s ignores u_t for t > s."""
    rng = np.random.default_rng(RNG_SEED + 11)
    x = _case(rng, 2, 30, 3, 4, with_d=True)
    u1, u2 = x["u"], rng.standard_normal(x["u"].shape)
    y1, _ = o.selective_scan(**x)
    y2, _ = o.selective_scan(**dict(x, u=u2))
    y3, _ = o.selective_scan(**dict(x, u=2.5 * u1 - 0.75 * u2))
    assert rel_err(y3, 2.5 * y1 - 0.75 * y2) < 1e-12
    up = u1.copy()
    up[:, 17, :] += 1.0
    y4, _ = o.selective_scan(**dict(x, u=up))
    assert np.array_equal(y4[:, :17], y1[:, :17])
    assert np.all(np.abs(y4[:, 17] - y1[:, 17]) > 0)


def pin_gate_and_skip(o):
    """SiLU gate and D skip at points with closed forms; the readout uses h_t after
    the update (a one-token scan from zero gives C . (delta B u) + D u)."""
    # B = 0 keeps h = 0, so y = D u silu(z); silu(1) = 1/(1+e^-1), silu(-2) = -2/(1+e^2)
    u = np.array([[[1.0, 3.0]]])
    z = np.array([[[1.0, -2.0]]])
    x = dict(u=u, delta=np.full_like(u, 0.1), A=-np.ones((2, 2)), B=np.zeros((1, 1, 2)),
             C=np.ones((1, 1, 2)), D=np.array([1.0, 0.5]), z=z, h0=None)
    y, _ = o.selective_scan(**x)
    ref = np.array([1.0 / (1.0 + np.exp(-1.0)), 1.5 * (-2.0) / (1.0 + np.exp(2.0))])
    assert rel_err(y[0, 0], ref) < 1e-15
    x["z"] = np.zeros_like(z)
    y0, _ = o.selective_scan(**x)
    assert np.all(y0 == 0.0)
    # readout after update: L = 1 from zero
    rng = np.random.default_rng(RNG_SEED + 12)
    xr = _case(rng, 2, 1, 3, 4, with_d=True)
    y1, _ = o.selective_scan(**xr)
    ref1 = (np.einsum("bn,bd,bd,bn->bd", xr["C"][:, 0], xr["delta"][:, 0], xr["u"][:, 0], xr["B"][:, 0])
            + xr["D"][None, :] * xr["u"][:, 0])
    assert rel_err(y1[:, 0], ref1) < 1e-14
    # C = 0 leaves only the skip, exactly
    y2, _ = o.selective_scan(**dict(xr, C=np.zeros_like(xr["C"])))
    assert np.array_equal(y2, xr["D"][None, None, :] * xr["u"])


def pin_channel_selection(o):
    """Computing a subset of channels gives exactly the rows of the full scan."""
    rng = np.random.default_rng(RNG_SEED + 13)
    x = _case(rng, 3, 20, 5, 3, with_d=True, with_z=True, with_h0=True)
    y, hl = o.selective_scan(**x)
    chans = [(2, 4), (0, 0), (1, 3), (2, 0)]
    ys, hs = o.selective_scan(**x, channels=chans)
    for i, (b, d) in enumerate(chans):
        assert np.array_equal(ys[i], y[b, :, d]) and np.array_equal(hs[i], hl[b, d])


# ---------------------------------------------------------------------------
# Backward pass


def _loss(o, x, dy, dhl, disc):
    y, hl = o.selective_scan(**x, disc=disc)
    return float((dy * y).sum() + (dhl * hl).sum())


def _fd_grad(o, x, name, dy, dhl, disc, eps=1e-6):
    arr = x[name]
    g = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        xp = dict(x); xm = dict(x)
        ap = arr.copy(); ap[idx] += eps
        am = arr.copy(); am[idx] -= eps
        xp[name] = ap; xm[name] = am
        g[idx] = (_loss(o, xp, dy, dhl, disc) - _loss(o, xm, dy, dhl, disc)) / (2 * eps)
    return g


_GRAD_OF = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz", h0="dh0")


def pin_bwd_finite_differences(o):
    """Every gradient equals the central difference of the forward oracle's loss."""
    rng = np.random.default_rng(RNG_SEED + 20)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 6, 2, 3, with_d=True, with_z=True, with_h0=True)
        dy = rng.standard_normal(x["u"].shape)
        dhl = rng.standard_normal(x["h0"].shape)
        g = o.selective_scan_bwd(**x, dy=dy, dh_last=dhl, disc=disc)
        for name, gname in _GRAD_OF.items():
            fd = _fd_grad(o, x, name, dy, dhl, disc)
            assert rel_err(g[gname], fd) < 1e-6, (disc, name, rel_err(g[gname], fd))


def pin_bwd_zoh_at_a_zero(o):
    """The hold rule's A -> 0 branch: its gradient in A (delta^2/2 B u) and the rest
    match finite differences taken across A = 0."""
    rng = np.random.default_rng(RNG_SEED + 21)
    x = _case(rng, 1, 5, 2, 3, with_d=False, with_h0=True)
    x["A"][0, 1] = 0.0
    x["A"][1, :] = 0.0
    dy = rng.standard_normal(x["u"].shape)
    dhl = rng.standard_normal(x["h0"].shape)
    g = o.selective_scan_bwd(**x, dy=dy, dh_last=dhl, disc="zoh")
    for name in ("A", "u", "delta", "B"):
        fd = _fd_grad(o, x, name, dy, dhl, "zoh", eps=1e-5)
        assert rel_err(g[_GRAD_OF[name]], fd) < 1e-6, (name, rel_err(g[_GRAD_OF[name]], fd))


def pin_bwd_state_only(o):
    """dy = 0: the loss is dh_last . h_last, so dh0 = exp(A * sum_t delta_t) dh_last
    exactly, and (simplified rule) du_t = sum_n dh_last exp(A sum_{s>t} delta_s) delta_t B_t."""
    rng = np.random.default_rng(RNG_SEED + 22)
    x = _case(rng, 2, 7, 3, 4, with_d=True, with_z=True, with_h0=True)
    dy = np.zeros_like(x["u"])
    dhl = rng.standard_normal(x["h0"].shape)
    g = o.selective_scan_bwd(**x, dy=dy, dh_last=dhl)
    tot = x["delta"].sum(axis=1)                                   # (b, d)
    ref = np.exp(x["A"][None] * tot[:, :, None]) * dhl
    assert rel_err(g["dh0"], ref) < 1e-13
    after = np.cumsum(x["delta"][:, ::-1], axis=1)[:, ::-1] - x["delta"]   # sum_{s>t} delta_s
    du = np.einsum("bdn,btdn,btd,btn->btd", dhl, np.exp(x["A"][None, None] * after[..., None]),
                   x["delta"], x["B"])
    assert rel_err(g["du"], du) < 1e-12
    assert np.all(g["dz"] == 0) and np.all(g["dD"] == 0) and np.all(g["dC"] == 0)


def pin_bwd_storage_types(o):
    """bf16 and fp32 storage give the gradients of the same values held in fp64."""
    rng = np.random.default_rng(RNG_SEED + 23)
    x = _case(rng, 2, 9, 3, 4, with_d=True, with_z=True, with_h0=True)
    dy = rng.standard_normal(x["u"].shape)
    for kind in ("f32", "bf16"):
        xs, x64 = dict(x), dict(x)
        for k in ("u", "delta", "B", "C", "z"):
            v32 = x[k].astype(np.float32)
            if kind == "f32":
                xs[k], x64[k] = v32, v32.astype(np.float64)
            else:
                bits = v32.view(np.uint32) >> 16
                xs[k] = bits.astype(np.uint16)
                x64[k] = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        for disc in ("euler", "zoh"):
            ga = o.selective_scan_bwd(**xs, dy=dy, disc=disc)
            gb = o.selective_scan_bwd(**x64, dy=dy, disc=disc)
            for k in ga:
                assert np.array_equal(ga[k], gb[k]), (kind, disc, k)


def pin_bwd_channel_selection(o):
    """Per-channel rows match the full backward; dB, dC of two disjoint channel sets
    add up to the full ones; the dA and dD shares add up over batch rows."""
    rng = np.random.default_rng(RNG_SEED + 24)
    x = _case(rng, 2, 8, 3, 4, with_d=True, with_z=True, with_h0=True)
    dy = rng.standard_normal(x["u"].shape)
    full = o.selective_scan_bwd(**x, dy=dy)
    s1 = [(0, 0), (1, 2), (0, 1)]
    s2 = [(0, 2), (1, 0), (1, 1)]
    g1 = o.selective_scan_bwd(**x, dy=dy, channels=s1)
    g2 = o.selective_scan_bwd(**x, dy=dy, channels=s2)
    for g, chans in ((g1, s1), (g2, s2)):
        for i, (b, d) in enumerate(chans):
            for k in ("du", "ddelta", "dz"):
                assert np.array_equal(g[k][i], full[k][b, :, d]), k
            assert np.array_equal(g["dh0"][i], full["dh0"][b, d])
    for k in ("dB", "dC"):
        assert rel_err(g1[k] + g2[k], full[k]) < 1e-14, k
    dA = np.zeros_like(full["dA"]); dD = np.zeros_like(full["dD"])
    for g, chans in ((g1, s1), (g2, s2)):
        for i, (b, d) in enumerate(chans):
            dA[d] += g["dA_c"][i]
            dD[d] += g["dD_c"][i]
    assert rel_err(dA, full["dA"]) < 1e-14 and rel_err(dD, full["dD"]) < 1e-14


def pin_delta_softplus(o):
    """A per-channel bias and softplus on delta equal running on the precomputed
    step log(1 + exp(delta + bias)) (numpy.logaddexp), for the scan and the
    decode step; a bias alone is plain addition."""
    rng = np.random.default_rng(RNG_SEED + 25)
    x = _case(rng, 2, 12, 3, 4, with_d=True, with_z=True, with_h0=True)
    raw = rng.normal(-3.0, 2.0, x["delta"].shape)
    raw[0, 0, 0], raw[1, 3, 2] = 40.0, -40.0
    bias = rng.normal(0.0, 1.0, 3)
    for disc in ("euler", "zoh"):
        y1, h1 = o.selective_scan(**dict(x, delta=raw), disc=disc, delta_bias=bias, delta_softplus=True)
        y2, h2 = o.selective_scan(**dict(x, delta=np.logaddexp(0.0, raw + bias)), disc=disc)
        assert rel_err(y1, y2) < 1e-13 and rel_err(h1, h2) < 1e-13, disc
        y3, _ = o.selective_scan(**dict(x, delta=np.abs(raw)), disc=disc, delta_bias=bias)
        y4, _ = o.selective_scan(**dict(x, delta=np.abs(raw) + bias), disc=disc)
        assert rel_err(y3, y4) < 1e-13, disc
    h = x["h0"].copy()
    hb = x["h0"].copy()
    ya = o.state_update(x["u"][:, 0], raw[:, 0], x["A"], x["B"][:, 0], x["C"][:, 0], h, D=x["D"], z=x["z"][:, 0],
                        delta_bias=bias, delta_softplus=True)
    yb = o.state_update(x["u"][:, 0], np.logaddexp(0.0, raw[:, 0] + bias), x["A"], x["B"][:, 0], x["C"][:, 0],
                        hb, D=x["D"], z=x["z"][:, 0])
    assert rel_err(ya, yb) < 1e-13 and rel_err(h, hb) < 1e-13


def pin_bwd_delta_softplus(o):
    """With bias and softplus on delta, ddelta (of the raw delta) and ddelta_bias
    equal central differences of the forward oracle's loss."""
    rng = np.random.default_rng(RNG_SEED + 26)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 6, 2, 3, with_d=True, with_z=True, with_h0=True)
        raw = rng.normal(-2.0, 1.0, x["delta"].shape)
        bias = rng.normal(0.0, 0.5, 2)
        dy = rng.standard_normal(x["u"].shape)
        dhl = rng.standard_normal(x["h0"].shape)
        g = o.selective_scan_bwd(**dict(x, delta=raw), dy=dy, dh_last=dhl, disc=disc, delta_bias=bias,
                                 delta_softplus=True)

        def loss(r, bb):
            y, hl = o.selective_scan(**dict(x, delta=r), disc=disc, delta_bias=bb, delta_softplus=True)
            return float((dy * y).sum() + (dhl * hl).sum())
        eps = 1e-6
        fd = np.zeros_like(raw)
        for idx in np.ndindex(raw.shape):
            rp, rm = raw.copy(), raw.copy()
            rp[idx] += eps
            rm[idx] -= eps
            fd[idx] = (loss(rp, bias) - loss(rm, bias)) / (2 * eps)
        assert rel_err(g["ddelta"], fd) < 1e-6, (disc, rel_err(g["ddelta"], fd))
        fdb = np.zeros_like(bias)
        for i in range(2):
            bp, bm = bias.copy(), bias.copy()
            bp[i] += eps
            bm[i] -= eps
            fdb[i] = (loss(raw, bp) - loss(raw, bm)) / (2 * eps)
        assert rel_err(g["ddelta_bias"], fdb) < 1e-6, (disc, rel_err(g["ddelta_bias"], fdb))


def _np_conv_silu(x, w, cb):
    """silu(causal depthwise conv1d(x)): numpy.convolve per channel with the
    taps reversed, first L outputs (left padding W-1)."""
    b, L, dim = x.shape
    pre = np.empty_like(x)
    for i in range(b):
        for d in range(dim):
            pre[i, :, d] = np.convolve(x[i, :, d], w[d, ::-1])[:L] + (cb[d] if cb is not None else 0.0)
    return pre / (1.0 + np.exp(-pre))


def pin_conv_prologue(o):
    """The convolution prologue equals running on silu(numpy.convolve(x, w) + b)."""
    rng = np.random.default_rng(RNG_SEED + 27)
    for W in (1, 2, 4):
        x = _case(rng, 2, 11, 3, 4, with_d=True, with_z=True, with_h0=True)
        w = rng.normal(0.0, 0.5, (3, W))
        cb = rng.normal(0.0, 0.5, 3)
        for disc in ("euler", "zoh"):
            y1, h1 = o.selective_scan(**x, disc=disc, conv_weight=w, conv_bias=cb)
            y2, h2 = o.selective_scan(**dict(x, u=_np_conv_silu(x["u"], w, cb)), disc=disc)
            assert rel_err(y1, y2) < 1e-13 and rel_err(h1, h2) < 1e-13, (W, disc)
        y3, _ = o.selective_scan(**x, conv_weight=w)
        y4, _ = o.selective_scan(**dict(x, u=_np_conv_silu(x["u"], w, None)))
        assert rel_err(y3, y4) < 1e-13, W


def pin_bwd_conv(o):
    """With the convolution prologue, the gradients of x, the taps and the conv
    bias equal central differences of the forward oracle's loss."""
    rng = np.random.default_rng(RNG_SEED + 28)
    for disc in ("euler", "zoh"):
        x = _case(rng, 2, 7, 2, 3, with_d=True, with_z=True, with_h0=True)
        w = rng.normal(0.0, 0.5, (2, 4))
        cb = rng.normal(0.0, 0.5, 2)
        dy = rng.standard_normal(x["u"].shape)
        dhl = rng.standard_normal(x["h0"].shape)
        g = o.selective_scan_bwd(**x, dy=dy, dh_last=dhl, disc=disc, conv_weight=w, conv_bias=cb)

        def loss(xx, ww, bb):
            y, hl = o.selective_scan(**dict(x, u=xx), disc=disc, conv_weight=ww, conv_bias=bb)
            return float((dy * y).sum() + (dhl * hl).sum())
        eps = 1e-6
        for name, arr, key in (("x", x["u"], "du"), ("w", w, "dconv_weight"), ("b", cb, "dconv_bias")):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                ap, am = arr.copy(), arr.copy()
                ap[idx] += eps
                am[idx] -= eps
                args_p = {"x": (ap, w, cb), "w": (x["u"], ap, cb), "b": (x["u"], w, ap)}[name]
                args_m = {"x": (am, w, cb), "w": (x["u"], am, cb), "b": (x["u"], w, am)}[name]
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert rel_err(g[key], fd) < 1e-6, (disc, name, rel_err(g[key], fd))


# ---------------------------------------------------------------------------
# Mamba-2 SSD layer (oracle_ssd)

def _ssd_case(rng, batch, L, H, P, G, N, with_d=True, with_z=False, with_h0=False):
    return dict(
        x=rng.standard_normal((batch, L, H, P)),
        dt=np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (batch, L, H))),
        A=-np.exp(rng.uniform(np.log(0.2), np.log(8.0), H)),
        B=rng.standard_normal((batch, L, G, N)),
        C=rng.standard_normal((batch, L, G, N)),
        D=rng.standard_normal(H) if with_d else None,
        z=rng.standard_normal((batch, L, H, P)) if with_z else None,
        h0=rng.standard_normal((batch, H, P, N)) if with_h0 else None,
    )


def _ssd_via_scan(o, c, disc, dt_bias=None, dt_softplus=False):
    """The SSD layer as one selective scan per group: the group's heads side by
    side as channels d = h_local*P + p, A[d, n] = A[h] for every n, each
    channel stepping with its head's dt (itwiki, "Mamba-2와 상태 공간 쌍대성":
    the SSD layer is the selective SSM whose A is a scalar times the identity)."""
    x = c["x"]
    batch, L, H, P = x.shape
    G, N = c["B"].shape[2], c["B"].shape[3]
    hpg = H // G
    y = np.empty_like(x)
    hl = np.empty((batch, H, P, N))
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        rep = lambda a: np.repeat(a[:, :, hs], P, axis=2)        # (b, L, hpg) -> (b, L, hpg*P)
        u = x[:, :, hs, :].reshape(batch, L, hpg * P)
        A = np.repeat(c["A"][hs], P)[:, None] * np.ones((1, N))
        kw = dict(D=None if c["D"] is None else np.repeat(c["D"][hs], P),
                  z=None if c["z"] is None else c["z"][:, :, hs, :].reshape(batch, L, hpg * P),
                  h0=None if c["h0"] is None else c["h0"][:, hs].reshape(batch, hpg * P, N),
                  delta_bias=None if dt_bias is None else np.repeat(dt_bias[hs], P),
                  delta_softplus=dt_softplus)
        yy, hh = o.selective_scan(u, rep(c["dt"]), A, c["B"][:, :, g, :].copy(), c["C"][:, :, g, :].copy(),
                                  disc=disc, **kw)
        y[:, :, hs, :] = yy.reshape(batch, L, hpg, P)
        hl[:, hs] = hh.reshape(batch, hpg, P, N)
    return y, hl


def pin_ssd_is_scalar_a_scan(o):
    rng = np.random.default_rng(RNG_SEED + 40)
    for disc in ("euler", "zoh"):
        for G in (1, 2):
            c = _ssd_case(rng, 2, 9, 4, 3, G, 5, with_z=True, with_h0=True)
            y, hl = o.ssd(**c, disc=disc)
            ry, rh = _ssd_via_scan(o, c, disc)
            assert rel_err(y, ry) < 1e-12 and rel_err(hl, rh) < 1e-12, (disc, G)
    c = _ssd_case(rng, 2, 6, 4, 2, 2, 3, with_h0=True)
    c["dt"] = 0.5 * rng.standard_normal(c["dt"].shape)
    bias = rng.uniform(-2.0, 0.5, 4)
    y, hl = o.ssd(**c, dt_bias=bias, dt_softplus=True)
    ry, rh = _ssd_via_scan(o, c, "euler", dt_bias=bias, dt_softplus=True)
    assert rel_err(y, ry) < 1e-12 and rel_err(hl, rh) < 1e-12


def pin_ssd_chunked_form(o):
    from oracle.ssd_chunked import ssd_chunked
    rng = np.random.default_rng(RNG_SEED + 41)
    for disc in ("euler", "zoh"):
        c = _ssd_case(rng, 2, 23, 4, 3, 2, 5, with_z=True, with_h0=True)
        y, hl = o.ssd(**c, disc=disc)
        for chunk in (1, 4, 7, 23, 64):
            cy, ch = ssd_chunked(**c, disc=disc, chunk=chunk)
            assert rel_err(cy, y) < 1e-10 and rel_err(ch, hl) < 1e-10, (disc, chunk)


def pin_ssd_a_zero_masked_matmul(o):
    """A = 0: no decay, so y is a causally masked product
    y_t = sum_{s<=t} (C_t . B_s) dt_s x_s + C_t . h0 + D x_t (both discretisations:
    the hold coefficient's A -> 0 limit is dt)."""
    rng = np.random.default_rng(RNG_SEED + 42)
    c = _ssd_case(rng, 2, 11, 3, 4, 1, 6, with_h0=True)
    c["A"] = np.zeros(3)
    scores = np.einsum("btn,bsn->bts", c["C"][:, :, 0], c["B"][:, :, 0])
    mask = np.tril(np.ones((11, 11)))
    ref = np.einsum("bts,bsh,bshp->bthp", scores * mask, c["dt"], c["x"])
    ref += np.einsum("btn,bhpn->bthp", c["C"][:, :, 0], c["h0"]) + c["D"][None, None, :, None] * c["x"]
    for disc in ("euler", "zoh"):
        y, _ = o.ssd(**c, disc=disc)
        assert rel_err(y, ref) < 1e-12, disc


def pin_ssd_fast_forgetting(o):
    """A very negative A with a positive step forgets everything before the
    current token: y_t = (C_t . B_t) wbar_t x_t + D x_t, wbar = dt (simplified)
    or expm1(dt A)/A -> -1/A (hold)."""
    rng = np.random.default_rng(RNG_SEED + 43)
    c = _ssd_case(rng, 1, 8, 2, 3, 1, 4, with_h0=True)
    c["dt"] = rng.uniform(0.5, 1.0, c["dt"].shape)
    c["A"] = np.array([-2e3, -5e3])
    cb = np.einsum("btn,btn->bt", c["C"][:, :, 0], c["B"][:, :, 0])
    for disc in ("euler", "zoh"):
        w = c["dt"] if disc == "euler" else np.broadcast_to(-1.0 / c["A"], c["dt"].shape)
        ref = cb[:, :, None, None] * w[..., None] * c["x"] + c["D"][None, None, :, None] * c["x"]
        y, hl = o.ssd(**c, disc=disc)
        assert rel_err(y, ref) < 1e-12, disc
        last = w[:, -1, :, None, None] * c["x"][:, -1, :, :, None] * c["B"][:, -1, 0][:, None, None, :]
        assert rel_err(hl, last) < 1e-12, disc


def pin_ssd_head_selection_and_types(o):
    rng = np.random.default_rng(RNG_SEED + 44)
    c = _ssd_case(rng, 2, 10, 4, 3, 2, 4, with_z=True, with_h0=True)
    y, hl = o.ssd(**c)
    heads = [(1, 3), (0, 0), (1, 1)]
    ys, hs = o.ssd(**c, heads=heads)
    for k, (b, h) in enumerate(heads):
        assert np.array_equal(ys[k], y[b, :, h]) and np.array_equal(hs[k], hl[b, h])
    # f32 and bf16 storage: the oracle widens exactly
    for name, cast in (("f32", lambda a: a.astype(np.float32)), ("bf16", _to_bf16)):
        cc = dict(c, **{k: cast(c[k]) for k in ("x", "dt", "B", "C", "z")})
        yt, ht = o.ssd(**cc)
        wide = dict(c, **{k: brute._widen(cc[k]) for k in ("x", "dt", "B", "C", "z")})
        yw, hw = o.ssd(**wide)
        assert rel_err(yt, yw) < 1e-13 and rel_err(ht, hw) < 1e-13, name


def _to_bf16(a):
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


ALL_PINS = [
    pin_brute_force,
    pin_brute_force_storage_types,
    pin_lti_direct,
    pin_lti_fft,
    pin_delta_zero,
    pin_large_delta,
    pin_zoh_exact_hold,
    pin_prefix_sum,
    pin_affine_composition,
    pin_resume,
    pin_decode_is_scan,
    pin_linear_causal,
    pin_gate_and_skip,
    pin_bwd_finite_differences,
    pin_bwd_zoh_at_a_zero,
    pin_bwd_state_only,
    pin_bwd_storage_types,
    pin_bwd_channel_selection,
    pin_delta_softplus,
    pin_bwd_delta_softplus,
    pin_conv_prologue,
    pin_bwd_conv,
    pin_channel_selection,
    pin_ssd_is_scalar_a_scan,
    pin_ssd_chunked_form,
    pin_ssd_a_zero_masked_matmul,
    pin_ssd_fast_forgetting,
    pin_ssd_head_selection_and_types,
]
