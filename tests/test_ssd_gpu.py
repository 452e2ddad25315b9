"""GPU parity of the Mamba-2 SSD layer (ssm_ssd_fwd) against the fp64 oracle.

Element by element on every compiled (head size, state size) pair, both input
weights, ragged chunks, groups, the step bias and softplus, h0 and the state
continued in place; the SSDBlock-shaped layer in full; the Mamba-2 layer at
the Mamba-1.4B scan scale (batch 8, 8192 tokens, 64 heads of 64, N 128) on
sampled heads over the whole sequence, in the launch configuration the bench
times.

Tolerance: 2e-2 max relative error (rms-floored), the bf16 tolerance of the
scan. The kernel rounds four operands of its products to bf16 (the decayed
scores, wbar x, the decayed wbar x of the state update, and the state for the
readout): each is a relative change of at most 2^-9 per element, which
averages down in the sums, and y itself is rounded to bf16 (2^-9).
"""
import numpy as np
import pytest

import oracle
import ssm_inputs as si
from gpu_util import TOL_BF16, rel_err, say, to_dev, to_np, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import selective_state_space_78_amd as ssm
    ssm.lib()
    return torch, ssm


def case(seed, batch=2, L=150, H=4, P=64, G=1, N=128, gate=True, skip=True, h0=True):
    cfg = si.SSD_CONFIGS["ssd-block"]
    x = si.ssd_inputs(cfg, seed=seed, batch=batch, seqlen=L, nheads=H, headdim=P, ngroups=G, dstate=N,
                      gate=gate, skip=skip)
    if h0:
        rng = np.random.default_rng(500 + seed)
        x["h0"] = rng.standard_normal((batch, H, P, N)).astype(np.float32)
    return x


def run(ssm, torch, x, disc="euler", in_place=False, **kw):
    dev = {k: to_dev(v, torch) for k, v in x.items()}
    h_last = dev["h0"] if in_place else None
    y, hl = ssm.ssm_ssd_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], D=dev["D"], z=dev["z"],
                            h0=dev["h0"], h_last=h_last, disc=disc, **{k: to_dev(v, torch) if isinstance(v, np.ndarray)
                                                                     else v for k, v in kw.items()})
    torch.cuda.synchronize()
    return to_np(y), to_np(hl)


def check(got, ref, what):
    ey, eh = rel_err(got[0], ref[0]), rel_err(got[1], ref[1])
    say("  %s: y err %.3e, h_last err %.3e" % (what, ey, eh))
    assert ey <= TOL_BF16 and eh <= TOL_BF16, (what, ey, eh)


@pytest.mark.parametrize("disc", ["euler", "zoh"])
@pytest.mark.parametrize("P,N", [(64, 64), (64, 128), (96, 64), (96, 128), (128, 64), (128, 128)])
def test_ssd_shapes(env, P, N, disc):
    torch, ssm = env
    x = case(seed=P + N, P=P, N=N, G=2)
    say("ssd P%d N%d %s b2 L150 H4 G2 (ragged last chunk), D, gate, h0" % (P, N, disc))
    check(run(ssm, torch, x, disc), oracle.ssd(**x, disc=disc), "P%d N%d" % (P, N))


@pytest.mark.parametrize("L", [0, 1, 17, 63, 64, 65, 128, 300])
def test_ssd_lengths(env, L):
    torch, ssm = env
    x = case(seed=L, L=L, H=3, G=1)
    say("ssd L%d" % L)
    got = run(ssm, torch, x)
    ref = oracle.ssd(**x)
    if L == 0:
        assert got[0].size == 0 and np.array_equal(got[1], x["h0"].astype(np.float64))
        return
    check(got, ref, "L%d" % L)


def test_ssd_without_optionals(env):
    torch, ssm = env
    x = case(seed=9, gate=False, skip=False, h0=False)
    say("ssd without D, z, h0")
    check(run(ssm, torch, x), oracle.ssd(**x), "bare")


@pytest.mark.parametrize("G", [1, 2, 8])
def test_ssd_groups(env, G):
    torch, ssm = env
    x = case(seed=20 + G, H=8, G=G, L=100)
    say("ssd H8 G%d" % G)
    check(run(ssm, torch, x), oracle.ssd(**x), "G%d" % G)


@pytest.mark.parametrize("disc", ["euler", "zoh"])
def test_ssd_dt_bias_softplus(env, disc):
    torch, ssm = env
    x = case(seed=31, L=130)
    rng = np.random.default_rng(31)
    x["dt"] = si.to_bf16_bits((0.5 * rng.standard_normal(x["dt"].shape)).astype(np.float32))
    bias = si.delta_bias(31, 4, "uniform").astype(np.float32)
    say("ssd %s with dt bias + softplus" % disc)
    got = run(ssm, torch, x, disc, dt_bias=bias, dt_softplus=True)
    check(got, oracle.ssd(**x, disc=disc, dt_bias=bias, dt_softplus=True), "softplus")


def test_ssd_state_in_place_and_resume(env):
    torch, ssm = env
    x = case(seed=41, L=200, h0=True)
    ref = oracle.ssd(**x)
    say("ssd h_last written over h0, and two halves resumed from the first's state")
    check(run(ssm, torch, x, in_place=True), ref, "in place")
    first = {k: (v[:, :90] if k in ("x", "dt", "B", "C", "z") else v) for k, v in x.items()}
    second = {k: (v[:, 90:] if k in ("x", "dt", "B", "C", "z") else v) for k, v in x.items()}
    y1, h1 = run(ssm, torch, first)
    second["h0"] = h1.astype(np.float32)
    y2, h2 = run(ssm, torch, second)
    check((np.concatenate([y1, y2], axis=1), h2), ref, "resumed")


def test_ssd_deterministic(env):
    torch, ssm = env
    x = case(seed=50, L=257, H=4)
    a, b = run(ssm, torch, x), run(ssm, torch, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ssd_block_full(env):
    torch, ssm = env
    cfg = si.SSD_CONFIGS["ssd-block"]
    x = si.ssd_inputs(cfg, seed=0)
    say("ssd SSDBlock-shaped layer b2 L1000 H8 P96 N128, in full")
    check(run(ssm, torch, x), oracle.ssd(**x), "ssd-block")


def test_ssd_mamba2_full_size(env):
    torch, ssm = env
    cfg = si.SSD_CONFIGS["mamba2-ssd"]
    x = si.ssd_inputs(cfg, seed=0)
    say("ssd Mamba-2 layer b8 L8192 H64 P64 N128 G1, sampled heads")
    y, hl = run(ssm, torch, x)
    rng = np.random.default_rng(7)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, 8, 6), rng.integers(0, 64, 6))] + [(7, 63), (0, 0)]
    ry, rh = oracle.ssd(**x, heads=heads)
    gy = np.stack([y[b, :, h] for b, h in heads])
    gh = np.stack([hl[b, h] for b, h in heads])
    check((gy, gh), (ry, rh), "mamba2-ssd sampled")
    assert np.isfinite(y).all()


def test_ssd_zero_step_keeps_state_exactly(env):
    """dt = 0: no decay and no input, so the state passes through bit for bit
    and y is the readout of h0 (itwiki "Mamba의 선택 메커니즘": a small step keeps
    the state)."""
    torch, ssm = env
    x = case(seed=61, L=150, H=4, G=2)
    x["dt"] = np.zeros_like(x["dt"])
    say("ssd dt = 0")
    y, hl = run(ssm, torch, x)
    assert np.array_equal(hl, x["h0"].astype(np.float64))
    check((y, hl), oracle.ssd(**x), "dt0")


def test_ssd_a_zero_is_masked_product(env):
    """A = 0: the layer is the causally masked product tril(C B^T)(dt x) plus
    the readout of h0 (closed form, computed here with numpy)."""
    torch, ssm = env
    x = case(seed=62, L=130, H=2, G=1, gate=False, skip=False)
    x["A"] = np.zeros_like(x["A"])
    say("ssd A = 0 against the masked product")
    y, hl = run(ssm, torch, x)
    w = lambda a: si.bf16_bits_to_f32(a).astype(np.float64)
    B, C, dt, xx = w(x["B"])[:, :, 0], w(x["C"])[:, :, 0], w(x["dt"]), w(x["x"])
    L = xx.shape[1]
    ref = np.einsum("bts,bsh,bshp->bthp", np.einsum("btn,bsn->bts", C, B) * np.tril(np.ones((L, L))), dt, xx)
    ref += np.einsum("btn,bhpn->bthp", C, x["h0"].astype(np.float64))
    e = rel_err(y, ref)
    say("  y err %.3e" % e)
    assert e <= TOL_BF16


def _sweep_cases(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        P, N = [(64, 64), (64, 128), (96, 64), (96, 128), (128, 64), (128, 128)][rng.integers(0, 6)]
        G = int(rng.choice([1, 2, 4]))
        H = G * int(rng.choice([1, 2, 3]))
        cases.append(dict(k=k, P=P, N=N, G=G, H=H, L=int(rng.integers(1, 400)), batch=int(rng.integers(1, 4)),
                          disc=str(rng.choice(["euler", "zoh"])), gate=bool(rng.integers(0, 2)),
                          skip=bool(rng.integers(0, 2)), h0=bool(rng.integers(0, 2)),
                          softplus=bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("c", _sweep_cases(), ids=lambda c: "case%d" % c["k"])
def test_ssd_sweep(env, c):
    """Seeded mixes of head size, state size, groups, heads per group (odd
    and even: one or two heads per workgroup), length, batch, input weight
    and the optional parts."""
    torch, ssm = env
    x = case(seed=300 + c["k"], batch=c["batch"], L=c["L"], H=c["H"], P=c["P"], G=c["G"], N=c["N"],
             gate=c["gate"], skip=c["skip"], h0=c["h0"])
    kw = {}
    if c["softplus"]:
        rng = np.random.default_rng(700 + c["k"])
        x["dt"] = si.to_bf16_bits((0.5 * rng.standard_normal(x["dt"].shape)).astype(np.float32))
        kw = dict(dt_bias=si.delta_bias(c["k"], c["H"], "uniform").astype(np.float32), dt_softplus=True)
    say("ssd sweep %s" % c)
    got = run(ssm, torch, x, c["disc"], **kw)
    check(got, oracle.ssd(**x, disc=c["disc"], **kw), "case%d" % c["k"])
