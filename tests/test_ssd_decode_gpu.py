"""GPU parity of the SSD decode step (ssm_ssd_state_update) against the fp64
oracle of the SSD layer run one token at a time, through the C ABI.

A step is the layer's recurrence for one token with the state continued in
place, so the reference of step k is the oracle's layer over token k alone,
started from the reference state after step k - 1. The kernel computes it in
fp32 without matrix cores (one token is a rank-1 update), so the state is held
to 1e-5; y is rounded to bf16 and held to the bf16 bar, 2e-2 (rms-floored, as
every test here).
"""
import numpy as np
import pytest

import oracle
import ssm_inputs as si
from gpu_util import TOL_BF16, rel_err, say, to_dev, to_np, torch_cuda

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-5
TOKEN = ("x", "dt", "B", "C", "z")


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import selective_state_space_78_amd as ssm
    ssm.lib()
    return torch, ssm


def inputs(seed, batch=2, steps=3, H=4, P=64, G=2, N=128, gate=True, skip=True):
    x = si.ssd_inputs(si.SSD_CONFIGS["ssd-block"], seed=seed, batch=batch, seqlen=steps, nheads=H, headdim=P,
                      ngroups=G, dstate=N, gate=gate, skip=skip)
    x["h0"] = np.random.default_rng(700 + seed).standard_normal((batch, H, P, N)).astype(np.float32)
    return x


def token(x, k):
    """Token k as a one-token sequence (the oracle's and ssm_ssd_fwd's layout)."""
    return {n: (v[:, k:k + 1] if n in TOKEN and v is not None else v) for n, v in x.items()}


def run_steps(ssm, torch, x, steps, disc="euler", **kw):
    """Decode steps on the GPU, and the oracle's reference for each."""
    dk = {n: to_dev(v, torch) if isinstance(v, np.ndarray) else v for n, v in kw.items()}
    h = to_dev(x["h0"], torch).clone()
    href = x["h0"].astype(np.float64)
    for k in range(steps):
        t = token(x, k)
        d = {n: to_dev(np.ascontiguousarray(v[:, 0]) if n in TOKEN and v is not None else v, torch)
             for n, v in t.items() if n != "h0"}
        y = ssm.ssm_ssd_state_update(d["x"], d["dt"], d["A"], d["B"], d["C"], h, D=d.get("D"), z=d.get("z"),
                                     disc=disc, **dk)
        torch.cuda.synchronize()
        yr, href = oracle.ssd(**dict(t, h0=href), disc=disc, **kw)
        ey, eh = rel_err(to_np(y), yr[:, 0]), rel_err(to_np(h), href)
        say("  step %d: y err %.3e, h err %.3e" % (k, ey, eh))
        assert ey <= TOL_BF16 and eh <= TOL_STATE, (k, ey, eh)
    return to_np(h)


@pytest.mark.parametrize("disc", ["euler", "zoh"])
@pytest.mark.parametrize("P,N", [(64, 64), (64, 128), (96, 64), (96, 128), (128, 64), (128, 128)])
def test_ssd_decode_steps(env, P, N, disc):
    torch, ssm = env
    say("ssd decode %s P%d N%d, 3 steps" % (disc, P, N))
    run_steps(ssm, torch, inputs(seed=P + N, P=P, N=N), 3, disc)


def test_ssd_decode_options(env):
    """No gate and no skip; a step bias through softplus; one group per head
    and one group for all heads."""
    torch, ssm = env
    say("ssd decode without gate and skip, one group per head")
    run_steps(ssm, torch, inputs(seed=3, G=4, gate=False, skip=False), 2)
    bias = np.random.default_rng(4).uniform(-2.0, 0.5, 4).astype(np.float32)
    x = inputs(seed=4, G=1)
    say("ssd decode with a step bias through softplus, one group")
    run_steps(ssm, torch, x, 2, "zoh", dt_bias=bias, dt_softplus=True)


def test_ssd_decode_equals_layer_of_length_one(env):
    """The decode step against ssm_ssd_fwd over the same one token from the
    same state (its matrix-core path rounds operands to bf16, so the two
    agree to the bf16 bar, not bit for bit)."""
    torch, ssm = env
    x = token(inputs(seed=9), 0)
    d = {n: to_dev(v, torch) for n, v in x.items()}
    y1, h1 = ssm.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], h0=d["h0"])
    h = d["h0"].clone()
    y2 = ssm.ssm_ssd_state_update(d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["A"],
                                  d["B"][:, 0].contiguous(), d["C"][:, 0].contiguous(), h, D=d["D"],
                                  z=d["z"][:, 0].contiguous())
    torch.cuda.synchronize()
    ey, eh = rel_err(to_np(y2), to_np(y1)[:, 0]), rel_err(to_np(h), to_np(h1))
    say("ssd decode against the layer with one token: y %.3e, h %.3e" % (ey, eh))
    assert ey <= TOL_BF16 and eh <= TOL_BF16


def test_ssd_decode_mamba2_heads(env):
    """64 batch rows of the Mamba-2 layer's heads (64 x 64, N 128, one group):
    a 134 MB state, 3 steps, every element."""
    torch, ssm = env
    say("ssd decode b64 H64 P64 N128, 3 steps")
    run_steps(ssm, torch, inputs(seed=11, batch=64, H=64, P=64, G=1, N=128), 3)


def test_ssd_decode_empty_batch(env):
    torch, ssm = env
    x = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    y = ssm.ssm_ssd_state_update(x, torch.empty((0, 4), dtype=torch.bfloat16, device="cuda"),
                                 torch.full((4,), -1.0, device="cuda"),
                                 torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda"),
                                 torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda"),
                                 torch.empty((0, 4, 64, 128), dtype=torch.float32, device="cuda"))
    assert y.shape == (0, 4, 64)
