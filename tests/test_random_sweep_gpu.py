"""Seeded random parity sweep of every entry point against the fp64 oracle.

The systematic GPU tests vary one thing at a time around a few base shapes.
This sweep draws whole combinations instead, each from its own seed, so that
pairings they leave out (an odd channel count with a ragged chunk, the
convolution prologue with a forced launch shape and the state continued in
place, 5 states with the hold rule and the softplus step, ...) are run too:

* forward scan: batch, length (biased towards chunk edges), channels (biased
  towards tile edges), states, element type, discretisation, each optional
  input, the three step modes (plain, bias, bias + softplus), the
  convolution prologue (width 0..4, with or without its bias), a forced
  launch shape or the planner's, h_last in place of h0, without h_last, and
  the entry point without allocation;
* backward: the same draws at smaller sizes, through ssm_scan_bwd or the
  ssm_scan_fwd_save / ssm_scan_bwd_saved pair, every gradient;
* decode: several consecutive in-place steps of a random shape and options;
* Mamba-2 SSD layer: random heads, head size, states, groups, length and
  options.

Each case prints its draw before it runs; the bars are those of the
systematic tests (2e-2 for bf16 inputs, 1e-4 for fp32, max relative error
floored at the rms).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import ssm_inputs as si
from gpu_util import TOL_BF16, TOL_F32, rel_err, say, to_dev, to_np, torch_cuda
from test_bwd_gpu import CONV_GRADS, compare_all, make_case, widen

pytestmark = pytest.mark.gpu

N_FWD, N_BWD, N_DEC, N_SSD = 48, 16, 10, 10
TILE = 64                                            # channels per lane tile
GROUPS = {4: (1, 2, 4), 8: (1, 2, 4, 8), 16: (1, 2, 4, 8, 16), 32: (2, 4, 8, 16), 64: (4, 8, 16)}


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import selective_state_space_78_amd as ssm
    ssm.lib()
    return torch, ssm


def padded(N):
    return next(p for p in (4, 8, 16, 32, 64) if N <= p)


def draw_len(rng, hi):
    k = rng.integers(3)
    if k == 0:
        return int(rng.integers(1, 41))
    if k == 1:
        return int(min(hi, max(1, 16 * rng.integers(1, hi // 16 + 1) + rng.integers(-1, 2))))
    return int(rng.integers(1, hi + 1))


def draw_dim(rng, hi):
    if rng.integers(2):
        return int(min(hi, max(1, TILE * rng.integers(1, hi // TILE + 1) + rng.integers(-1, 2))))
    return int(rng.integers(1, hi + 1))


def draw_options(rng, hi_b, hi_L, hi_d):
    o = dict(batch=int(rng.integers(1, hi_b + 1)), L=draw_len(rng, hi_L), dim=draw_dim(rng, hi_d),
             N=int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 16, 16, 20, 32, 40, 64])),
             dtype=str(rng.choice(["bf16", "f32"])), disc=str(rng.choice(["euler", "zoh"])),
             skip=bool(rng.integers(2)), gate=bool(rng.integers(2)), h0=bool(rng.integers(2)),
             step=str(rng.choice(["plain", "bias", "softplus"])), conv=int(rng.choice([0, 0, 2, 3, 4])),
             conv_bias=bool(rng.integers(2)))
    return o


def build_inputs(o, seed):
    """Oracle-side inputs of one draw plus the extra arguments both sides take."""
    x, g = make_case("mamba130m", o["dtype"], seed=seed, batch=o["batch"], seqlen=o["L"], dim=o["dim"],
                     dstate=o["N"])
    if not o["skip"]:
        x["D"] = None
    if not o["gate"]:
        x["z"] = None
    if not o["h0"]:
        x["h0"] = None
    kw = {}
    if o["step"] == "softplus":
        cfg = dataclasses.replace(si.CONFIGS["mamba130m"], dtype=o["dtype"])
        r = si.raw_delta_inputs(cfg, seed=seed, batch=o["batch"], seqlen=o["L"], dim=o["dim"])
        x["delta"] = r["delta"]
        kw.update(delta_bias=r["delta_bias"], delta_softplus=True)
    elif o["step"] == "bias":
        rng = np.random.default_rng(3000 + seed)
        kw.update(delta_bias=rng.uniform(0.0, 0.02, o["dim"]).astype(np.float32), delta_softplus=False)
    if o["conv"]:
        c = si.conv_inputs(o["dim"], o["conv"], seed=seed)
        kw["conv_weight"] = c["conv_weight"]
        if o["conv_bias"]:
            kw["conv_bias"] = c["conv_bias"]
    return x, g, kw


def dev_kw(kw, torch):
    return {k: to_dev(v, torch) if isinstance(v, np.ndarray) else v for k, v in kw.items()}


def tol_of_dtype(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


@pytest.mark.parametrize("k", range(N_FWD))
def test_random_forward(env, k):
    torch, ssm = env
    rng = np.random.default_rng(9000 + k)
    o = draw_options(rng, 3, 700, 260)
    npad = padded(o["N"])
    route = str(rng.choice(["plan", "tuned", "tuned", "noalloc"]))
    tuning = None
    if route == "tuned":
        tuning = (int(rng.choice(GROUPS[npad])), int(rng.choice([1, 2, 3, 5, 8])))
    h_last_mode = str(rng.choice(["new", "new", "in_place", "none"])) if o["h0"] else \
        str(rng.choice(["new", "new", "none"]))
    say("fwd #%d %s route %s tuning %s h_last %s" % (k, o, route, tuning, h_last_mode))
    x, _, kw = build_inputs(o, 9000 + k)
    yr, hr = oracle.load().selective_scan(**x, disc=o["disc"], **kw)

    dev = {kk: to_dev(v, torch) for kk, v in x.items()}
    h_last = dev["h0"] if h_last_mode == "in_place" else None
    args = (dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"])
    common = dict(h0=dev["h0"], h_last=h_last, disc=o["disc"], want_h_last=h_last_mode != "none",
                  **dev_kw(kw, torch))
    if route == "noalloc":
        y, hl = ssm.ssm_scan_fwd_noalloc(*args, **common)
    else:
        y, hl = ssm.ssm_scan_fwd(*args, tuning=tuning, **common)
    torch.cuda.synchronize()
    tol = tol_of_dtype(o["dtype"])
    ey = rel_err(to_np(y), yr)
    eh = rel_err(to_np(hl), hr) if h_last_mode != "none" else 0.0
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    if h_last_mode == "none":
        assert hl is None
    assert ey <= tol and eh <= tol, (k, ey, eh)


@pytest.mark.parametrize("k", range(N_BWD))
def test_random_backward(env, k):
    torch, ssm = env
    rng = np.random.default_rng(9500 + k)
    o = draw_options(rng, 2, 400, 200)
    saved = bool(rng.integers(2))
    dhl = bool(rng.integers(2))
    want_dh0 = bool(rng.integers(2))
    say("bwd #%d %s saved %s dh_last %s want_dh0 %s" % (k, o, saved, dhl, want_dh0))
    x, g, kw = build_inputs(o, 9500 + k)
    dev = {kk: to_dev(v, torch) for kk, v in x.items()}
    dy = to_dev(g["dy"], torch)
    dh_last = to_dev(g["dh_last"], torch) if dhl else None
    dkw = dev_kw(kw, torch)
    args = (dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"])
    if saved:
        _, _, ws = ssm.ssm_scan_fwd_save(*args, dev["D"], dev["z"], h0=dev["h0"], disc=o["disc"], **dkw)
        out = ssm.ssm_scan_bwd_saved(*args, dy, ws, D=dev["D"], z=dev["z"], h0=dev["h0"], dh_last=dh_last,
                                     disc=o["disc"], want_dh0=want_dh0, **dkw)
    else:
        out = ssm.ssm_scan_bwd(*args, dy, D=dev["D"], z=dev["z"], h0=dev["h0"], dh_last=dh_last,
                               disc=o["disc"], want_dh0=want_dh0, **dkw)
    torch.cuda.synchronize()
    got = {kk: to_np(v) for kk, v in out.items()}
    ref = oracle.load().selective_scan_bwd(**x, dy=widen(g["dy"]), dh_last=g["dh_last"] if dhl else None,
                                           disc=o["disc"], **kw)
    assert (got["dh0"] is None) == (not want_dh0)
    assert (got["dz"] is None) == (x["z"] is None) and (got["dD"] is None) == (x["D"] is None)
    keys = CONV_GRADS + (("ddelta_bias",) if "delta_bias" in kw else ())
    compare_all(x, got, ref, "bwd #%d" % k, keys=keys)


@pytest.mark.parametrize("k", range(N_DEC))
def test_random_decode(env, k):
    torch, ssm = env
    rng = np.random.default_rng(9800 + k)
    batch, dim = int(rng.integers(1, 10)), draw_dim(rng, 300)
    N = int(rng.choice([1, 3, 4, 5, 8, 16, 16, 24, 33, 64]))
    dtype, disc = str(rng.choice(["bf16", "f32"])), str(rng.choice(["euler", "zoh"]))
    gate, skip, sp = bool(rng.integers(2)), bool(rng.integers(2)), bool(rng.integers(2))
    steps = int(rng.integers(1, 6))
    say("decode #%d b%d d%d N%d %s %s gate %s skip %s softplus %s steps %d"
        % (k, batch, dim, N, dtype, disc, gate, skip, sp, steps))
    cfg = si.DecodeConfig("t", batch, dim, N, steps, dtype=dtype, gate=gate)
    st = si.decode_static(cfg, seed=9800 + k)
    st["A"] = -np.exp(rng.uniform(np.log(0.3), np.log(20.0), st["A"].shape)).astype(np.float32)
    D = st["D"] if skip else None
    kw = {}
    if sp:
        kw = dict(delta_bias=rng.uniform(-1.0, 0.5, dim).astype(np.float32), delta_softplus=True)
    h = to_dev(st["h"], torch)
    href = st["h"].astype(np.float64)
    tol = tol_of_dtype(dtype)
    for s_i in range(steps):
        s = si.decode_step(cfg, s_i, seed=9800 + k, bias=st["bias"])
        y = ssm.ssm_state_update(to_dev(s["x"], torch), to_dev(s["delta"], torch), to_dev(st["A"], torch),
                                 to_dev(s["B"], torch), to_dev(s["C"], torch), h, D=to_dev(D, torch),
                                 z=to_dev(s["z"], torch), disc=disc, **dev_kw(kw, torch))
        yr = oracle.load().state_update(s["x"], s["delta"], st["A"], s["B"], s["C"], href, D=D, z=s["z"],
                                        disc=disc, **kw)
        torch.cuda.synchronize()
        ey, eh = rel_err(to_np(y), yr), rel_err(h.cpu().numpy(), href)
        say("  step %d: y err %.3e, h err %.3e" % (s_i, ey, eh))
        assert ey <= tol and eh <= tol, (k, s_i, ey, eh)


@pytest.mark.parametrize("k", range(N_SSD))
def test_random_ssd(env, k):
    torch, ssm = env
    rng = np.random.default_rng(9900 + k)
    batch, L = int(rng.integers(1, 3)), int(rng.choice([0, 1, 2]) if rng.integers(6) == 0 else draw_len(rng, 300))
    H = int(rng.integers(1, 7))
    G = int(rng.choice([g for g in (1, 2, 3, 6) if H % g == 0]))
    P, N = int(rng.choice([64, 96, 128])), int(rng.choice([64, 128]))
    gate, skip, h0, disc = bool(rng.integers(2)), bool(rng.integers(2)), bool(rng.integers(2)), \
        str(rng.choice(["euler", "zoh"]))
    sp = bool(rng.integers(2))
    in_place = h0 and bool(rng.integers(2))
    say("ssd #%d b%d L%d H%d G%d P%d N%d gate %s skip %s h0 %s in_place %s %s softplus %s"
        % (k, batch, L, H, G, P, N, gate, skip, h0, in_place, disc, sp))
    x = si.ssd_inputs(si.SSD_CONFIGS["ssd-block"], seed=9900 + k, batch=batch, seqlen=L, nheads=H, headdim=P,
                      ngroups=G, dstate=N, gate=gate, skip=skip)
    x["h0"] = rng.standard_normal((batch, H, P, N)).astype(np.float32) if h0 else None
    kw = dict(dt_bias=rng.uniform(-1.0, 0.5, H).astype(np.float32), dt_softplus=True) if sp else {}
    yr, hr = oracle.ssd(**x, disc=disc, **kw)
    dev = {kk: to_dev(v, torch) for kk, v in x.items()}
    y, hl = ssm.ssm_ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], D=dev["D"], z=dev["z"],
                            h0=dev["h0"], h_last=dev["h0"] if in_place else None, disc=disc, **dev_kw(kw, torch))
    torch.cuda.synchronize()
    if L == 0:
        assert to_np(y).size == 0
        want = x["h0"].astype(np.float64) if h0 else np.zeros((batch, H, P, N))
        assert np.array_equal(to_np(hl), want)
        return
    ey, eh = rel_err(to_np(y), yr), rel_err(to_np(hl), hr)
    say("  y err %.3e, h_last err %.3e" % (ey, eh))
    assert ey <= TOL_BF16 and eh <= TOL_BF16, (k, ey, eh)
