"""GPU parity of the training pair ssm_scan_fwd_save / ssm_scan_bwd_saved,
through the C ABI.

The saving forward must give ssm_scan_fwd's h_last bit for bit and its y up
to the order of the readout's sum over state groups (it runs in the
backward's launch shape, which for some dstate splits the states over fewer
waves than the forward's own choice): within one rounding of y's type. The
backward that reads those checkpoints must give ssm_scan_bwd's gradients bit
for bit (they are the states the backward's own checkpoint pass computes).
With the convolution prologue the saving forward leaves its fp32 u where the
backward reads it, the u the recomputing backward's own pass forms, so the
pair again equals the recomputing backward bit for bit, over one segment or
several.
"""
import numpy as np
import pytest

import ssm_inputs as si
from gpu_util import rel_err, say, to_dev, to_np
from test_bwd_gpu import GRADS, CONV_GRADS, compare_all, env, make_case, ref_bwd  # noqa: F401

pytestmark = pytest.mark.gpu


def run_pair(ssm, torch, x, g, disc, **kw):
    dev = {k: to_dev(v, torch) for k, v in x.items() if k != "h0"}
    h0 = to_dev(x["h0"], torch) if x.get("h0") is not None else None
    dy, dhl = to_dev(g["dy"], torch), to_dev(g["dh_last"], torch)
    y0, hl0 = ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"), dev.get("z"),
                               h0=h0, disc=disc, **kw)
    plain = ssm.ssm_scan_bwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dy, D=dev.get("D"),
                             z=dev.get("z"), h0=h0, dh_last=dhl, disc=disc, **kw)
    y1, hl1, saved = ssm.ssm_scan_fwd_save(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                                           dev.get("z"), h0=h0, disc=disc, **kw)
    got = ssm.ssm_scan_bwd_saved(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dy, saved, D=dev.get("D"),
                                 z=dev.get("z"), h0=h0, dh_last=dhl, disc=disc, **kw)
    torch.cuda.synchronize()
    fwd = tuple(to_np(t) for t in (y0, hl0, y1, hl1))
    return fwd, {k: to_np(v) for k, v in plain.items()}, {k: to_np(v) for k, v in got.items()}


def assert_forward_same(x, y0, hl0, y1, hl1):
    assert np.array_equal(hl0, hl1)
    # one rounding of y: 2^-8 relative for bf16 outputs; for fp32 outputs the
    # sum of up to 16 partial readouts in another order, a few ulps of the rms
    tol = 4e-3 if x["u"].dtype == np.uint16 else 1e-5
    e = rel_err(y1, y0)
    assert e <= tol, e


def assert_same(a, b, keys):
    for k in keys:
        if a.get(k) is None:
            continue
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("disc", ["euler", "zoh"])
@pytest.mark.parametrize("N", [16, 4, 32, 64])
def test_saved_equals_recomputed(env, dtype, disc, N):
    """Every backward launch shape; L 40 and dim 70 leave a ragged chunk and tile."""
    torch, ssm = env
    x, g = make_case("mamba130m", dtype, seed=70 + N, batch=2, seqlen=40, dim=70, dstate=N)
    say("fwd_save / bwd_saved %s %s b2 L40 d70 N%d" % (dtype, disc, N))
    (y0, hl0, y1, hl1), plain, got = run_pair(ssm, torch, x, g, disc)
    assert_forward_same(x, y0, hl0, y1, hl1)
    assert_same(plain, got, GRADS)


def test_saved_against_oracle(env):
    torch, ssm = env
    x, g = make_case("mamba130m", "bf16", seed=77, batch=2, seqlen=100, dim=192, dstate=16)
    say("bwd_saved bf16 euler b2 L100 d192 N16 against the oracle")
    _, _, got = run_pair(ssm, torch, x, g, "euler")
    compare_all(x, got, ref_bwd(x, g, "euler"), "saved")


def test_saved_with_segments(env):
    """A long sequence is split into segments joined by the affine carry; the
    saving forward uses the backward's plan, so its checkpoints cover every
    segment."""
    torch, ssm = env
    x, g = make_case("mamba130m", "bf16", seed=78, batch=1, seqlen=4096, dim=64, dstate=16)
    assert ssm.ssm_scan_plan(1, 4096, 64, 16)[1] > 1
    say("fwd_save / bwd_saved bf16 b1 L4096 d64 (several segments)")
    (y0, hl0, y1, hl1), plain, got = run_pair(ssm, torch, x, g, "euler")
    assert_forward_same(x, y0, hl0, y1, hl1)
    assert_same(plain, got, GRADS)


def test_saved_softplus_step(env):
    torch, ssm = env
    x, g = make_case("mamba130m", "bf16", seed=79, batch=2, seqlen=70, dim=136, dstate=16)
    r = si.raw_delta_inputs(si.CONFIGS["mamba130m"], seed=79, batch=2, seqlen=70, dim=136)
    x = dict(x, delta=r["delta"])
    say("fwd_save / bwd_saved with delta bias + softplus")
    (y0, hl0, y1, hl1), plain, got = run_pair(ssm, torch, x, g, "zoh", delta_bias=to_dev(r["delta_bias"], torch),
                                               delta_softplus=True)
    assert_forward_same(x, y0, hl0, y1, hl1)
    assert_same(plain, got, GRADS + ("ddelta_bias",))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [300, 1200])
def test_saved_conv_prologue(env, dtype, L):
    """L 300 runs as one segment, L 1200 as several."""
    torch, ssm = env
    x, g = make_case("mamba130m", dtype, seed=80, batch=2, seqlen=L, dim=136, dstate=16)
    conv = si.conv_inputs(136, 4, seed=80)
    nseg = ssm.ssm_scan_plan(2, L, 136, 16)[1]
    say("fwd_save / bwd_saved %s with the width-4 conv prologue, L %d (%d segments)" % (dtype, L, nseg))
    cw = dict(conv_weight=to_dev(conv["conv_weight"], torch), conv_bias=to_dev(conv["conv_bias"], torch))
    (y0, hl0, y1, hl1), plain, got = run_pair(ssm, torch, x, g, "euler", **cw)
    assert_forward_same(x, y0, hl0, y1, hl1)
    # both backward paths read the same fp32 u from the same pass
    assert_same(plain, got, CONV_GRADS)
    compare_all(x, got, ref_bwd(x, g, "euler", **conv), "saved conv", keys=CONV_GRADS)


def test_saved_mamba14b_full_size(env):
    """The launch configuration the benchmark times: every gradient of the
    saved backward equals the recomputing one bit for bit."""
    torch, ssm = env
    cfg = si.CONFIGS["mamba1.4b"]
    x, g = si.scan_inputs(cfg, seed=0), si.grad_inputs(cfg, seed=0)
    x["h0"] = None
    say("fwd_save / bwd_saved Mamba-1.4B-shaped layer b8 L8192 d4096 N16 bf16")
    (y0, hl0, y1, hl1), plain, got = run_pair(ssm, torch, x, g, "euler")
    assert_forward_same(x, y0, hl0, y1, hl1)
    assert_same(plain, got, GRADS)
