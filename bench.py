"""Throughput of the selective scan on one MI355X.

One step = one ssm_scan_fwd over the Mamba-1.4B-shaped layer workload
(batch 8, L 8192, d_inner 4096, d_state 16; bf16 u/delta/B/C/z/y, fp32 A/D and
state; D skip, SiLU gate, final state written), inputs resident in HBM.
Prints one JSON line: selective-scan Gtokens*ch/s, the dominant kernel's
roofline position (measured with HIP events on the stream it runs on), the
algorithmic HBM rate, the backward of the same scan and the decode step
measured alongside, and the fp64 CPU oracle timed on a bounded sample of the
same workload (whose outputs are also compared with the GPU's timed outputs).

The Mamba-2 SSD layer (ssm_ssd_fwd) on its own workload is measured alongside
in the same way (roofline position and the oracle on a sample of heads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-bwd] [--no-decode] [--no-ssd]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ssm_inputs as si  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# fp32 VALU issue rate without packed instructions: 256 CU x 4 SIMD x 16 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
WORKLOAD = "mamba1.4b"
WORKLOADS = {
    "mamba1.4b": "Mamba-1.4B-shaped layer scan: batch 8, L 8192, d_inner 4096, d_state 16, "
                 "bf16 u/delta/B/C/z/y, fp32 A/D/state, D skip + SiLU gate + final state",
    "mamba130m": "Mamba-130M-shaped layer scan: batch 4, L 2048, d_inner 1536, d_state 16, "
                 "bf16 u/delta/B/C/z/y, fp32 A/D/state, D skip + SiLU gate + final state",
    "long": "Long-context scan: batch 1, L 131072, d_inner 5120, d_state 16, delta bias log-uniform "
            "[1e-4, 1e-1], bf16 u/delta/B/C/z/y, fp32 A/D/state, D skip + SiLU gate + final state",
}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "selective_state_space_78_amd", "csrc")


def valu_ops_per_token_ch(N: int, gate: bool) -> int:
    """Minimal fp32 VALU lane-operations of the method per (b, t, d):
    per state: delta*A, exp2, (delta*u)*B, fma(a, h, Bu), fma(C, h, y);
    per token: delta*u, fma(D, u, y), and for the gate z*log2e, exp2, 1+e, rcp, z*r, y*s."""
    return 5 * N + 2 + (6 if gate else 0)


def source_digest(names=("scan_kernels.hpp", "scan_bf16_euler.hip")) -> str:
    """Digest of a kernel's device source (by default the scan kernel template
    and its bf16 instantiation unit): counter summaries older than it are stale."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


SSD_SOURCES = ("ssd_kernels.hpp", "ssd_euler.hip")


def measured_ssd_traffic():
    """HBM bytes per launch of the SSD kernel from the committed counter
    summary, if it was taken on the current kernel source."""
    try:
        with open(os.path.join(PROFILES, "traffic_ssd_mamba2.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest(SSD_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def to_dev(a, torch):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


def measured_traffic(workload: str, plan, default_options=True):
    """HBM bytes per launch of the main scan kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    in the same launch shape (and with the default step and discretisation)."""
    if not default_options:
        return None
    try:
        with open(os.path.join(PROFILES, "traffic_scan_%s.json" % workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or list(rec.get("launch", [])) != list(plan):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(x, y_dev, torch, budget_s=15.0, opts=None):
    """The fp64 oracle, as it stands, on batch row 0 of the same workload for a
    bounded number of channels over the full sequence. Its outputs are also
    compared with the GPU's timed outputs for those channels."""
    import oracle
    o = oracle.load()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    batch, L, dim = x["u"].shape
    # size the sample from a short probe run: the first k channels in (b, d)
    # order, every token, k bounded by the time budget and the workload
    probe = [(0, d) for d in range(min(dim, 4 * threads))]
    t0 = time.perf_counter()
    opts = opts or {}
    o.selective_scan(**x, channels=probe, nthreads=threads, want_y=False, **opts)
    per_ch = (time.perf_counter() - t0) / len(probe)
    k = int(min(batch * dim, max(threads, budget_s / max(per_ch, 1e-12))))
    chans = [(c // dim, c % dim) for c in range(k)]
    t0 = time.perf_counter()
    yr, hr = o.selective_scan(**x, channels=chans, nthreads=threads, **opts)
    sec = time.perf_counter() - t0
    # compare with the GPU's timed outputs for a subset of the sampled channels
    sub = list(range(0, k, max(1, k // 256)))
    idx_b = torch.tensor([chans[i][0] for i in sub], device=y_dev.device)
    idx_d = torch.tensor([chans[i][1] for i in sub], device=y_dev.device)
    yg = y_dev[idx_b, :, idx_d].float().cpu().numpy()          # (len(sub), L)
    err = rel_err(yg, yr[sub])
    return {
        "value": k * L / sec / 1e9,
        "unit": "Gtokens*ch/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d of %d channels in (batch, d) order, all %d tokens (%d token*ch), fp64, %.1f s" % (
            k, batch * dim, L, k * L, sec),
        "parity_max_rel_err_vs_gpu": err,
        "parity_channels_checked": len(sub),
    }


def bench_decode(torch, ssm, steps=200, warmup=10, nsets=16):
    cfg = si.DECODE
    st = si.decode_static(cfg, seed=0)
    sets = [{k: to_dev(v, torch) for k, v in si.decode_step(cfg, i, seed=0, bias=st["bias"]).items()}
            for i in range(nsets)]
    A, D, h = to_dev(st["A"], torch), to_dev(st["D"], torch), to_dev(st["h"], torch)
    y = torch.empty((cfg.batch, cfg.dim), dtype=torch.bfloat16, device="cuda")
    for i in range(warmup):
        s = sets[i % nsets]
        ssm.ssm_state_update(s["x"], s["delta"], A, s["B"], s["C"], h, D=D, z=s["z"], y=y)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        s = sets[i % nsets]
        ssm.ssm_state_update(s["x"], s["delta"], A, s["B"], s["C"], h, D=D, z=s["z"], y=y)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    nbytes = si.decode_bytes(cfg)
    return {
        "workload": "decode b%d d%d N%d, %d in-place steps cycling %d input sets" % (
            cfg.batch, cfg.dim, cfg.dstate, steps, nsets),
        "us_per_step": us,
        "Gtokens*ch/s": cfg.batch * cfg.dim / (us * 1e-6) / 1e9,
        "algorithmic_bytes_per_step": nbytes,
        "GB/s": nbytes / (us * 1e-6) / 1e9,
        "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "note": "the 84 MB state fits the 256 MB Infinity Cache; effective rate",
    }


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (bytes read + bytes written per second, in
    GB/s) of a 1 GiB buffer on this GPU: a measured sanity denominator beside
    the published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def bench_backward(torch, ssm, cfg, dev, steps=10, warmup=2, disc="euler", step_opts=None):
    """Time ssm_scan_bwd (checkpoint pass + reverse pass + reduction) on the workload."""
    g = si.grad_inputs(cfg, seed=0)
    dy = to_dev(g["dy"], torch)
    dhl = to_dev(g["dh_last"], torch)
    step_opts = step_opts or {}
    need = ssm.ssm_scan_bwd_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, ssm.SSM_BF16, disc,
                                           **step_opts)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = {}

    def call():
        r = ssm.ssm_scan_bwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dy, D=dev["D"], z=dev["z"],
                             dh_last=dhl, workspace=ws, out=out, disc=disc, **step_opts)
        out.update(r)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps

    # the training pair: a forward that keeps the checkpoints, then the
    # backward that reads them, against the plain forward and backward
    y = torch.empty_like(dev["u"])
    hl = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device="cuda")
    fws = torch.empty(max(ssm.ssm_scan_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, ssm.SSM_BF16,
                                                      disc, **step_opts), 1), dtype=torch.uint8, device="cuda")

    def fwd_plain():
        ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"], y=y, h_last=hl,
                         workspace=fws, disc=disc, **step_opts)

    def fwd_save():
        ssm.ssm_scan_fwd_save(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"], y=y,
                              h_last=hl, workspace=ws, disc=disc, **step_opts)

    def bwd_saved():
        r = ssm.ssm_scan_bwd_saved(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dy, ws, D=dev["D"],
                                   z=dev["z"], dh_last=dhl, out=out, disc=disc, **step_opts)
        out.update(r)

    def timed(fns):
        for _ in range(warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        for e in evs:
            e[0].record()
            for f, ev in zip(fns, e[1:]):
                f()
                ev.record()
        torch.cuda.synchronize()
        return [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(len(fns))]

    t_fp, t_bp = timed([fwd_plain, call])
    t_fs, t_bs = timed([fwd_save, bwd_saved])
    return {
        "workload": "backward of the same scan: gradients of u (of x with the conv prologue), delta, A, B, C, D, z, "
                    "h0 from dy and dh_last",
        "ms_per_call": ms,
        "Gtokens*ch/s": cfg.tokens_ch / (ms * 1e-3) / 1e9,
        "workspace_bytes": need,
        "calls": steps,
        "training_step": {
            "workload": "forward + backward of the layer: ssm_scan_fwd then ssm_scan_bwd, against "
                        "ssm_scan_fwd_save (keeps the checkpoints) then ssm_scan_bwd_saved (reads them)",
            "recompute_ms": {"fwd": t_fp, "bwd": t_bp, "total": t_fp + t_bp},
            "saved_ms": {"fwd": t_fs, "bwd": t_bs, "total": t_fs + t_bs},
        },
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_ssd_decode(torch, ssm, batch=64, steps=200, warmup=10, sets=16):
    """The SSD decode step (ssm_ssd_state_update) for 64 batch rows of the
    Mamba-2 layer's heads (64 x 64, N 128, one group): a 134 MB fp32 state
    updated in place, steps cycling over `sets` per-token input sets."""
    cfg = si.SSD_CONFIGS["mamba2-ssd"]
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    x = si.ssd_inputs(cfg, seed=0, batch=batch, seqlen=sets)
    tok = [{n: to_dev(np.ascontiguousarray(x[n][:, k]), torch) if x[n] is not None else None
            for n in ("x", "dt", "B", "C", "z")} for k in range(sets)]
    A = to_dev(x["A"], torch)
    D = to_dev(x["D"], torch) if x["D"] is not None else None
    h = torch.zeros((batch, H, P, N), dtype=torch.float32, device="cuda")
    y = torch.empty((batch, H, P), dtype=torch.bfloat16, device="cuda")

    def step(k):
        t = tok[k % sets]
        ssm.ssm_ssd_state_update(t["x"], t["dt"], A, t["B"], t["C"], h, D=D, z=t["z"], y=y)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    nbytes = (2 * batch * H * P * N * 4            # state read and written
              + (3 if x["z"] is not None else 2) * batch * H * P * 2 + batch * H * 2   # x, (z,) y; dt
              + 2 * batch * G * N * 2 + (2 if x["D"] is not None else 1) * H * 4)       # B, C; A, (D)
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": "SSD decode b%d, %d heads x %d, d_state %d, %d group%s%s: %d in-place steps cycling %d input "
                    "sets" % (batch, H, P, N, G, ", gate" if x["z"] is not None else "",
                              ", D skip" if x["D"] is not None else "", steps, sets),
        "us_per_step": us,
        "algorithmic_bytes_per_step": nbytes,
        "GB/s": gbps,
        "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
        "note": "the 134 MB state fits the 256 MB Infinity Cache; effective rate",
    }


def bench_ssd(torch, ssm, steps=20, warmup=3, cpu=True, budget_s=10.0):
    """The Mamba-2 SSD layer (ssm_ssd_fwd) on the mamba2-ssd workload, with its
    roofline position and the fp64 oracle on a bounded sample of heads."""
    cfg = si.SSD_CONFIGS["mamba2-ssd"]
    x = si.ssd_inputs(cfg, seed=0)
    d = {k: to_dev(v, torch) for k, v in x.items()}
    y = torch.empty((cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim), dtype=torch.bfloat16, device="cuda")
    hl = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device="cuda")

    def call():
        ssm.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], y=y, h_last=hl)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = si.ssd_bytes(cfg)
    flops = si.ssd_flops(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "workload": "Mamba-2 SSD layer: batch %d, L %d, %d heads x %d, d_state %d, %d group, bf16 x/dt/B/C/y, "
                    "fp32 A and state, final state written" % (cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim,
                                                               cfg.dstate, cfg.ngroups),
        "ms_per_call": ms,
        "Gtokens*ch/s": cfg.tokens_ch / (ms * 1e-3) / 1e9,
        "roofline": {
            "bound": "hbm",
            "kernel": "ssd_fwd_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": nbytes,
            "traffic": measured_ssd_traffic(),
            "mfma": {"algorithmic_flops_per_launch": flops, "achieved_TFLOPs": tflops,
                     "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "note": "bf16 dense peak; the kernel issues the readout, masked-product and update "
                             "MFMAs twice (hi + lo bf16 operands)"},
        },
    }
    if cpu:
        import oracle
        o = oracle.load()
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        threads = max(1, min(16, cores))
        probe = [(0, h) for h in range(threads)]
        t0 = time.perf_counter()
        o.ssd(**x, heads=probe, nthreads=threads, want_y=False)
        per_head = (time.perf_counter() - t0) / len(probe)
        k = int(min(cfg.batch * cfg.nheads, max(threads, budget_s / max(per_head, 1e-12))))
        heads = [(c // cfg.nheads, c % cfg.nheads) for c in range(k)]
        t0 = time.perf_counter()
        yr, _ = o.ssd(**x, heads=heads, nthreads=threads)
        sec = time.perf_counter() - t0
        yg = np.stack([y[b, :, h].float().cpu().numpy() for b, h in heads])
        out["cpu_baseline"] = {
            "value": k * cfg.seqlen * cfg.headdim / sec / 1e9,
            "unit": "Gtokens*ch/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "first %d of %d heads in (batch, head) order, all %d tokens x %d channels, fp64, %.1f s" % (
                k, cfg.batch * cfg.nheads, cfg.seqlen, cfg.headdim, sec),
            "parity_max_rel_err_vs_gpu": rel_err(yg, yr),
        }
    out["decode"] = bench_ssd_decode(torch, ssm)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--disc", choices=["euler", "zoh"], default="euler",
                    help="discretisation of B (default: the simplified delta*B)")
    ap.add_argument("--delta-softplus", action="store_true",
                    help="form the step in the kernel: softplus(delta_raw + bias)")
    ap.add_argument("--conv", action="store_true",
                    help="run the width-4 causal conv1d + SiLU prologue in the kernel (u holds x)")
    ap.add_argument("--tuning", type=str, default=None, help="state_groups,segments")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=WORKLOAD,
                    help="scan workload of the timed step (the default is the headline one)")
    ap.add_argument("--no-ssd", action="store_true", help="skip the Mamba-2 SSD layer measurement")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (to scale profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every channel is independent; see the sharding note in the design document)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_78_amd as ssm

    cfg = si.CONFIGS[args.workload]
    print("bench: generating %s inputs" % args.workload, file=sys.stderr, flush=True)
    x = si.scan_inputs(cfg, seed=0)
    dev = {k: to_dev(v, torch) for k, v in x.items() if v is not None}
    step_opts = {}
    oracle_opts = {"disc": args.disc}
    if args.delta_softplus:
        r = si.raw_delta_inputs(cfg, seed=0)
        x = dict(x, delta=r["delta"])
        dev["delta"] = to_dev(r["delta"], torch)
        step_opts = dict(delta_bias=to_dev(r["delta_bias"], torch), delta_softplus=True)
        oracle_opts.update(delta_bias=r["delta_bias"], delta_softplus=True)
    if args.conv:
        c = si.conv_inputs(cfg.dim, 4, seed=0)
        step_opts.update(conv_weight=to_dev(c["conv_weight"], torch), conv_bias=to_dev(c["conv_bias"], torch))
        oracle_opts.update(c)
    y = torch.empty((cfg.batch, cfg.seqlen, cfg.dim), dtype=torch.bfloat16, device="cuda")
    h_last = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device="cuda")
    tuning = tuple(int(v) for v in args.tuning.split(",")) if args.tuning else None
    plan = tuning or ssm.ssm_scan_plan(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate)
    need = ssm.ssm_scan_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, tuning=tuning, **step_opts)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None

    def step():
        ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                         y=y, h_last=h_last, workspace=ws, tuning=tuning, disc=args.disc, **step_opts)

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-launch events on the stream the kernels run on (torch's current stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for a, b in evs:
        a.record()
        step()
        b.record()
    t_all1.record()
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    per = sorted(a.elapsed_time(b) for a, b in evs)
    mean_launch_ms = float(np.mean(per))
    ms_per_step = total_ms / args.steps
    tok = cfg.tokens_ch
    value = tok / (ms_per_step * 1e-3) / 1e9
    nbytes = si.algorithmic_bytes(cfg)
    ops = valu_ops_per_token_ch(cfg.dstate, cfg.gate) * tok
    achieved_tops = ops / (mean_launch_ms * 1e-3) / 1e12
    gbps = nbytes / (mean_launch_ms * 1e-3) / 1e9
    print("bench: %.3f ms/step (median launch %.3f ms)" % (ms_per_step, per[len(per) // 2]),
          file=sys.stderr, flush=True)

    out = {
        "metric": "selective-scan Gtokens*ch/s (+ achieved HBM GB/s, % of MI355X peak)",
        "value": value,
        "unit": "Gtokens*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "global_batch": cfg.batch, "seq_len": cfg.seqlen, "dim": cfg.dim, "dstate": cfg.dstate,
            "io_dtype": "bf16", "parallelism": "none (1 GPU)",
            "disc": args.disc, "step": "softplus(delta + bias) in the kernel" if args.delta_softplus else "delta as given",
            "prologue": "silu(causal conv1d width 4), a pass of its own before the scan" if args.conv else "none",
            "launch": {"state_groups": plan[0], "segments": plan[1]},
        },
        "roofline": {
            "bound": "alu",
            "kernel": ("scan_kernel (main pass)" if plan[1] == 1 else "scan passes (aggregate + carry + main)")
                      + (" after conv_silu_kernel" if args.conv else ""),
            "achieved": achieved_tops,
            "peak": VALU_PEAK_TOPS,
            "unit": "Top/s",
            "frac": achieved_tops / VALU_PEAK_TOPS,
            "ops_per_token_ch": valu_ops_per_token_ch(cfg.dstate, cfg.gate),
            "mean_launch_ms": mean_launch_ms,
            "median_launch_ms": per[len(per) // 2],
            "min_launch_ms": per[0],
            "traffic": measured_traffic(args.workload, plan,
                                        args.disc == "euler" and not args.delta_softplus and not args.conv),
        },
        "hbm": {
            "algorithmic_bytes_per_launch": nbytes,
            "achieved_GBps": gbps,
            "peak_GBps": HBM_PEAK_GBPS,
            "frac": gbps / HBM_PEAK_GBPS,
            "measured_copy_GBps": copy_bandwidth(torch),
        },
    }
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30
    if not args.no_bwd:
        print("bench: backward", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(torch, ssm, cfg, dev, disc=args.disc, step_opts=step_opts)
    if not args.no_decode:
        print("bench: decode", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(torch, ssm)
    if not args.no_ssd:
        print("bench: Mamba-2 SSD layer", file=sys.stderr, flush=True)
        out["ssd"] = bench_ssd(torch, ssm, cpu=not args.no_cpu)
    if not args.no_cpu:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, y, torch, opts=oracle_opts)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
