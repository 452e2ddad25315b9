"""Helpers of the GPU parity tests: move seeded numpy inputs to the device,
run the library through its binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from pins import rel_err  # noqa: F401  (re-exported)

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    if t is None:
        return None
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def tol_of(x):
    return TOL_F32 if x["u"].dtype == np.float32 else TOL_BF16


def run_scan(ssm, torch, x, disc="euler", tuning=None, h0=None, in_place=False, want_h_last=True):
    dev = {k: to_dev(v, torch) for k, v in x.items() if k != "h0"}
    h0d = to_dev(h0, torch) if h0 is not None else None
    h_last = h0d if in_place else None
    y, hl = ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                             dev.get("z"), h0=h0d, h_last=h_last, disc=disc, tuning=tuning,
                             want_h_last=want_h_last)
    torch.cuda.synchronize()
    return y, hl
