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

The other workloads are measured in the same run, each with parity on its
timed outputs: the tiny fp32 case, the Mamba-130M-shaped layer cycling 12
buffer sets (1.2 GB, more than the Infinity Cache) and on one resident set, the
131072-token long-context layer at full size, and the decode workload as 1000
consecutive in-place steps with every step's y kept.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-bwd] [--no-decode] [--no-ssd]
                       [--no-configs]
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


def measured_valu(workload: str, plan, default_options=True):
    """VALU instructions per (token, channel) of the main scan kernel and the
    shader clock during it, from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source in the same launch shape."""
    if not default_options:
        return None
    try:
        with open(os.path.join(PROFILES, "valu_scan_%s.json" % workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or list(rec.get("launch", [])) != list(plan):
        return None
    return rec


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


def host_cores() -> int:
    """Cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(o, x, opts, threads, budget_s, want_y=True):
    """Run the oracle on the first k channels (in (batch, d) order, every
    token) with k sized from a short probe so that the run takes about
    budget_s. Returns (channels, seconds, y, h_last)."""
    batch, L, dim = x["u"].shape
    probe = [(c // dim, c % dim) for c in range(min(batch * dim, 4 * threads))]
    t0 = time.perf_counter()
    o.selective_scan(**x, channels=probe, nthreads=threads, want_y=False, **opts)
    per_ch = (time.perf_counter() - t0) / len(probe)
    k = int(min(batch * dim, max(threads, budget_s * threads / max(per_ch * threads, 1e-12))))
    chans = [(c // dim, c % dim) for c in range(k)]
    t0 = time.perf_counter()
    yr, hr = o.selective_scan(**x, channels=chans, nthreads=threads, want_y=want_y, **opts)
    return chans, time.perf_counter() - t0, yr, hr


def cpu_baseline(x, y_dev, torch, budget_s=15.0, opts=None, x_c2=None, single_budget_s=5.0):
    """The fp64 oracle, as it stands, on every core of this process's affinity
    mask, over the first channels (in (batch, d) order, all tokens) of the same
    workload that fit about budget_s of work (the whole workload when it fits).
    Its outputs are compared with the GPU's timed outputs on a subset of those
    channels. With x_c2, also the per-core rate: one thread on the
    Mamba-130M-shaped workload."""
    import oracle
    o = oracle.load()
    cores = host_cores()
    opts = opts or {}
    batch, L, dim = x["u"].shape
    chans, sec, yr, _ = _oracle_rate(o, x, opts, cores, budget_s)
    k = len(chans)
    sub = list(range(0, k, max(1, k // 256)))
    idx_b = torch.tensor([chans[i][0] for i in sub], device=y_dev.device)
    idx_d = torch.tensor([chans[i][1] for i in sub], device=y_dev.device)
    yg = y_dev[idx_b, :, idx_d].float().cpu().numpy()          # (len(sub), L)
    out = {
        "value": k * L / sec / 1e9,
        "unit": "Gtokens*ch/s",
        "cores": cores,
        "threads": cores,
        "cores_available": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "first %d of %d channels in (batch, d) order, all %d tokens (%d token*ch), fp64, %.1f s on %d "
                  "threads" % (k, batch * dim, L, k * L, sec, cores),
        "parity_max_rel_err_vs_gpu": rel_err(yg, yr[sub]),
        "parity_channels_checked": len(sub),
    }
    if x_c2 is not None:
        c2, sec1, _, _ = _oracle_rate(o, x_c2, {}, 1, single_budget_s, want_y=False)
        L2 = x_c2["u"].shape[1]
        out["per_core"] = {
            "value": len(c2) * L2 / sec1 / 1e9,
            "unit": "Gtokens*ch/s",
            "threads": 1,
            "sample": "Mamba-130M-shaped layer (b4 L2048 d1536 N16): first %d channels, all %d tokens, fp64, "
                      "%.1f s on one thread" % (len(c2), L2, sec1),
        }
    return out


def sample_channels(batch, dim, k=16):
    """k (batch row, channel) pairs spread over the workload, corners included."""
    pts = {(0, 0), (batch - 1, dim - 1), (0, dim - 1), (batch - 1, 0)}
    rng = np.random.default_rng(1234)
    while len(pts) < min(k, batch * dim):
        pts.add((int(rng.integers(batch)), int(rng.integers(dim))))
    return sorted(pts)


def bench_scan_workload(torch, ssm, name, steps, warmup, sets=1):
    """ssm_scan_fwd on one more scan workload, cycling over `sets` copies of its
    buffers in device memory (inputs, outputs and workspace), so that a
    workload smaller than the 256 MB Infinity Cache is read from HBM. Parity of
    the timed outputs: every copy's y and h_last equal the first copy's (the
    copies hold the same inputs), and the first copy's equal the fp64 oracle on
    sampled channels over the whole sequence."""
    import oracle
    cfg = si.CONFIGS[name]
    print("bench: %s inputs" % name, file=sys.stderr, flush=True)
    x = si.scan_inputs(cfg, seed=0)
    fp32 = cfg.dtype == "f32"
    edt = torch.float32 if fp32 else torch.bfloat16
    plan = ssm.ssm_scan_plan(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate, ssm.SSM_F32 if fp32 else ssm.SSM_BF16)
    need = ssm.ssm_scan_workspace_size(cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate,
                                       ssm.SSM_F32 if fp32 else ssm.SSM_BF16)
    bufs = []
    for _ in range(sets):
        dev = {k: to_dev(v, torch) for k, v in x.items() if v is not None}
        y = torch.empty((cfg.batch, cfg.seqlen, cfg.dim), dtype=edt, device="cuda")
        hl = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        bufs.append((dev, y, hl, ws))

    def call(i):
        dev, y, hl, ws = bufs[i % sets]
        ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"), dev.get("z"),
                         y=y, h_last=hl, workspace=ws)

    warm = settle(torch, call, max(warmup, sets))
    torch.cuda.synchronize()
    # back-to-back calls between one pair of events (events between the calls
    # would add their own gaps to calls of ~0.1 ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = si.algorithmic_bytes(cfg)
    gbps = nbytes / (ms * 1e-3) / 1e9
    same = all(torch.equal(bufs[i][1], bufs[0][1]) and torch.equal(bufs[i][2], bufs[0][2]) for i in range(1, sets))
    chans = sample_channels(cfg.batch, cfg.dim) if cfg.batch * cfg.dim > 64 else None
    yr, hr = oracle.load().selective_scan(**x, channels=chans, nthreads=host_cores())
    y0, h0 = bufs[0][1], bufs[0][2]
    if chans is None:
        yg, hg = y0.float().cpu().numpy(), h0.cpu().numpy()
    else:
        ib = torch.tensor([c[0] for c in chans], device="cuda")
        idd = torch.tensor([c[1] for c in chans], device="cuda")
        yg, hg = y0[ib, :, idd].float().cpu().numpy(), h0[ib, idd].cpu().numpy()
    tok = cfg.tokens_ch
    out = {
        "workload": WORKLOADS[name],
        "launch": {"state_groups": plan[0], "segments": plan[1]},
        "ms_per_call": ms,
        "calls": steps,
        "warmup_calls": warm,
        "timing": "one event pair around the back-to-back calls",
        "Gtokens*ch/s": tok / (ms * 1e-3) / 1e9,
        "algorithmic_bytes_per_call": nbytes,
        "GB/s": gbps,
        "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
        "buffer_sets": sets,
        "bytes_cycled": sets * nbytes,
        "workspace_bytes": need,
        "parity": {
            "max_rel_err_y": rel_err(yg, yr),
            "max_rel_err_h_last": rel_err(hg, hr),
            "tolerance": 1e-4 if fp32 else 2e-2,
            "checked": "every channel" if chans is None else "%d sampled channels x all %d tokens" % (
                len(chans), cfg.seqlen),
            "buffer_sets_identical": same,
        },
    }
    if sets > 1:
        out["note"] = ("%d sets of %.1f MB cycled (%.2f GB), more than the 256 MB Infinity Cache, so each call "
                       "reads its inputs from HBM" % (sets, nbytes / 1e6, sets * nbytes / 1e9))
    del bufs
    return out


def bench_decode(torch, ssm, nsets=64, warmup=10, copy_gbps=None):
    """The decode workload as stated: b256 d5120 N16, the fp32 state updated
    in place over 1000 consecutive steps, each step's y written to its own row
    of a (1000, batch, dim) buffer. Steps cycle over `nsets` distinct per-token
    input sets (0.5 GB, read from HBM). Parity of the timed outputs: y of
    sampled channels at every one of the 1000 steps and their final state,
    against the fp64 oracle run over the same schedule."""
    import oracle
    cfg = si.DECODE
    steps = cfg.steps
    st = si.decode_static(cfg, seed=0)
    host_sets = [si.decode_step(cfg, i, seed=0, bias=st["bias"]) for i in range(nsets)]
    sets = [{k: to_dev(v, torch) for k, v in hs.items()} for hs in host_sets]
    A, D = to_dev(st["A"], torch), to_dev(st["D"], torch)
    h_init = to_dev(st["h"], torch)
    h = h_init.clone()
    ybuf = torch.empty((steps, cfg.batch, cfg.dim), dtype=torch.bfloat16, device="cuda")
    yv = [ybuf[k] for k in range(steps)]

    def run_steps():
        for k in range(steps):
            s = sets[k % nsets]
            ssm.ssm_state_update(s["x"], s["delta"], A, s["B"], s["C"], h, D=D, z=s["z"], y=yv[k])

    def one(i):
        s = sets[i % nsets]
        ssm.ssm_state_update(s["x"], s["delta"], A, s["B"], s["C"], h, D=D, z=s["z"], y=yv[0])

    warm = settle(torch, one, warmup)
    # eager: one binding call per step from Python (its host cost is part of this figure)
    h.copy_(h_init)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    run_steps()
    ev1.record()
    torch.cuda.synchronize()
    us_eager = ev0.elapsed_time(ev1) * 1e3 / steps
    # the 1000 steps captured once in a HIP graph and replayed, as a serving
    # loop would run them; the timed outputs checked below are this replay's
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps()
    graph.replay()                      # warm again after the capture
    h.copy_(h_init)
    ybuf.zero_()
    torch.cuda.synchronize()
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    nbytes = si.decode_bytes(cfg)
    # the oracle over the same schedule for sampled channels, each its own (batch 1, dim 1) problem
    chans = sample_channels(cfg.batch, cfg.dim, 8)
    o = oracle.load()
    yref = np.empty((steps, len(chans)))
    href = np.empty((len(chans), cfg.dstate))
    for i, (b, d) in enumerate(chans):
        hb = st["h"][b:b + 1, d:d + 1].astype(np.float64)
        for k in range(steps):
            hs = host_sets[k % nsets]
            yref[k, i] = o.state_update(hs["x"][b:b + 1, d:d + 1], hs["delta"][b:b + 1, d:d + 1],
                                        st["A"][d:d + 1], hs["B"][b:b + 1], hs["C"][b:b + 1], hb,
                                        D=st["D"][d:d + 1], z=hs["z"][b:b + 1, d:d + 1])[0, 0]
        href[i] = hb[0, 0]
    ib = torch.tensor([c[0] for c in chans], device="cuda")
    idd = torch.tensor([c[1] for c in chans], device="cuda")
    yg = ybuf[:, ib, idd].float().cpu().numpy()
    hg = h[ib, idd].cpu().numpy()
    gbps = nbytes / (us * 1e-6) / 1e9
    out = {
        "workload": "decode b%d d%d N%d: %d consecutive in-place steps, y of every step kept (%d x b x d), "
                    "cycling %d distinct input sets" % (cfg.batch, cfg.dim, cfg.dstate, steps, steps, nsets),
        "us_per_step": us,
        "ms_per_1000_steps": us * steps / 1e3,
        "timing": "the 1000 steps replayed from one HIP graph capture",
        "warmup_steps": warm,
        "eager_us_per_step": us_eager,
        "Gtokens*ch/s": cfg.batch * cfg.dim / (us * 1e-6) / 1e9,
        "algorithmic_bytes_per_step": nbytes,
        "effective_GB/s": gbps,
        "parity": {
            "max_rel_err_y_all_steps": rel_err(yg, yref),
            "max_rel_err_final_state": rel_err(hg, href),
            "tolerance": 2e-2,
            "checked": "%d sampled channels: y at each of the %d steps and the final state" % (len(chans), steps),
        },
        "note": "the 84 MB state stays in the 256 MB Infinity Cache from step to step, so this is an effective "
                "rate, not an HBM rate; it is set against the measured device copy rate, not the HBM peak",
    }
    if copy_gbps:
        out["frac_of_measured_copy"] = gbps / copy_gbps
    del graph, yv, ybuf, sets
    return out


def bench_tiny(torch, ssm, reps=20):
    """The tiny fp32 workload (b1 L64 d16 N4, no gate): latency of one call and
    its parity against the fp64 oracle over every output."""
    import oracle
    cfg = si.CONFIGS["tiny"]
    x = si.scan_inputs(cfg, seed=0)
    dev = {k: to_dev(v, torch) for k, v in x.items() if v is not None}
    y = torch.empty((cfg.batch, cfg.seqlen, cfg.dim), dtype=torch.float32, device="cuda")
    hl = torch.empty((cfg.batch, cfg.dim, cfg.dstate), dtype=torch.float32, device="cuda")

    def call():
        ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("D"), None, y=y, h_last=hl)

    settle(torch, lambda i: call(), 3, 20.0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    yr, hr = oracle.load().selective_scan(**x)
    return {
        "workload": "tiny scan: b1 L64 d16 N4, fp32, no gate (latency-bound; parity case)",
        "us_per_call_median": per[len(per) // 2] * 1e3,
        "parity": {"max_rel_err_y": rel_err(y.cpu().numpy(), yr), "max_rel_err_h_last": rel_err(hl.cpu().numpy(), hr),
                   "tolerance": 1e-4, "checked": "every output"},
    }


# The GPU's clocks ramp up over the first few tens of milliseconds of work
# after an idle spell (measured: the 1.4B-shaped scan takes 1.8 ms per call in
# its first 10 calls after a 1 s pause and settles at 1.02 ms within 30 ms).
# Every timed section therefore warms up for at least its warm-up count and at
# least this much GPU time, and reports what it ran.
SETTLE_MS = 200.0


def settle(torch, fn, min_calls, min_ms=SETTLE_MS):
    """Call fn() at least min_calls times and until min_ms of GPU time has
    elapsed; returns the number of calls."""
    n = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while True:
        fn(n)
        n += 1
        if n >= min_calls and n % 4 == 0:
            e1.record()
            e1.synchronize()
            if e0.elapsed_time(e1) >= min_ms:
                return n


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

    warm = settle(torch, lambda i: call(), warmup)
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
        settle(torch, lambda i: [f() for f in fns], warmup)
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
        "warmup_calls": warm,
        "training_step": {
            "workload": "forward + backward of the layer: ssm_scan_fwd then ssm_scan_bwd, against "
                        "ssm_scan_fwd_save (keeps the checkpoints) then ssm_scan_bwd_saved (reads them)",
            "recompute_ms": {"fwd": t_fp, "bwd": t_bp, "total": t_fp + t_bp},
            "saved_ms": {"fwd": t_fs, "bwd": t_bs, "total": t_fs + t_bs},
        },
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_ssd_decode(torch, ssm, batch=64, steps=200, warmup=10, sets=16, copy_gbps=None):
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

    settle(torch, step, warmup)
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
    out = {
        "workload": "SSD decode b%d, %d heads x %d, d_state %d, %d group%s%s: %d in-place steps cycling %d input "
                    "sets" % (batch, H, P, N, G, ", gate" if x["z"] is not None else "",
                              ", D skip" if x["D"] is not None else "", steps, sets),
        "us_per_step": us,
        "algorithmic_bytes_per_step": nbytes,
        "effective_GB/s": gbps,
        "note": "the 134 MB state stays in the 256 MB Infinity Cache from step to step, so this is an effective "
                "rate, not an HBM rate; it is set against the measured device copy rate, not the HBM peak",
    }
    if copy_gbps:
        out["frac_of_measured_copy"] = gbps / copy_gbps
    return out


def bench_ssd(torch, ssm, steps=20, warmup=3, cpu=True, budget_s=10.0, copy_gbps=None):
    """The Mamba-2 SSD layer (ssm_ssd_fwd) on the mamba2-ssd workload, with its
    roofline position and the fp64 oracle on a bounded sample of heads."""
    cfg = si.SSD_CONFIGS["mamba2-ssd"]
    x = si.ssd_inputs(cfg, seed=0)
    d = {k: to_dev(v, torch) for k, v in x.items()}
    y = torch.empty((cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim), dtype=torch.bfloat16, device="cuda")
    hl = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device="cuda")

    def call():
        ssm.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], y=y, h_last=hl)

    warm = settle(torch, lambda i: call(), warmup)
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
        "calls": steps,
        "warmup_calls": warm,
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
        threads = host_cores()
        probe = [(0, h) for h in range(min(threads, cfg.batch * cfg.nheads))]
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
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "first %d of %d heads in (batch, head) order, all %d tokens x %d channels, fp64, %.1f s" % (
                k, cfg.batch * cfg.nheads, cfg.seqlen, cfg.headdim, sec),
            "parity_max_rel_err_vs_gpu": rel_err(yg, yr),
        }
    out["decode"] = bench_ssd_decode(torch, ssm, copy_gbps=copy_gbps)
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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other scan workloads (tiny, 130M-shaped rotated and resident, long context)")
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
    inputs_bytes = sum(t.numel() * t.element_size() for t in dev.values())
    outputs_bytes = y.numel() * y.element_size() + h_last.numel() * h_last.element_size()

    def step():
        ssm.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                         y=y, h_last=h_last, workspace=ws, tuning=tuning, disc=args.disc, **step_opts)

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    warm = settle(torch, lambda i: step(), args.warmup)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
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
    peak_alloc = torch.cuda.max_memory_allocated()
    total_ms = t_all0.elapsed_time(t_all1)
    per = sorted(a.elapsed_time(b) for a, b in evs)
    mean_launch_ms = float(np.mean(per))
    ms_per_step = total_ms / args.steps
    tok = cfg.tokens_ch
    value = tok / (ms_per_step * 1e-3) / 1e9
    nbytes = si.algorithmic_bytes(cfg)
    gbps = nbytes / (mean_launch_ms * 1e-3) / 1e9
    ops = valu_ops_per_token_ch(cfg.dstate, cfg.gate)
    default_opts = args.disc == "euler" and not args.delta_softplus and not args.conv
    valu_rec = measured_valu(args.workload, plan, default_opts)
    print("bench: %.3f ms/step (median launch %.3f ms)" % (ms_per_step, per[len(per) // 2]),
          file=sys.stderr, flush=True)
    copy_gbps = copy_bandwidth(torch)

    valu = {
        "algorithmic_ops_per_token_ch": ops,
        "peak_lane_ops_per_s_at_2.4GHz": VALU_PEAK_TOPS * 1e12,
        "frac_algorithmic_ops_at_2.4GHz": ops * tok / (mean_launch_ms * 1e-3) / (VALU_PEAK_TOPS * 1e12),
    }
    if valu_rec:
        slots = valu_rec["issue_slots_per_token_ch"]
        clk = valu_rec["shader_clock_GHz"]
        valu.update({
            "issued_valu_per_token_ch": valu_rec["valu_per_token_ch"],
            "issued_transcendental_per_token_ch": valu_rec["trans_per_token_ch"],
            "issue_slots_per_token_ch": slots,
            "shader_clock_GHz_measured": clk,
            "frac_issue_slots_at_measured_clock": slots * tok / (mean_launch_ms * 1e-3) / (256 * 4 * 16 * clk * 1e9),
            "note": "issue slots count a transcendental as 2 (its measured cost); counters and clock from "
                    "rocprofv3 on the same kernel source (profiles/)",
        })
    out = {
        "metric": "selective-scan Gtokens*ch/s (+ achieved HBM GB/s, % of MI355X peak)",
        "value": value,
        "unit": "Gtokens*ch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "warmup_note": "at least --warmup steps and at least %.0f ms of GPU work, so that the timed steps run at "
                       "the clocks the GPU reaches under sustained load" % SETTLE_MS,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "global_batch": cfg.batch, "seq_len": cfg.seqlen, "dim": cfg.dim, "dstate": cfg.dstate,
            "io_dtype": "bf16", "state_dtype": "f32", "compute_dtype": "f32", "parallelism": "none (1 GPU)",
            "disc": args.disc, "step": "softplus(delta + bias) in the kernel" if args.delta_softplus else "delta as given",
            "prologue": "silu(causal conv1d width 4), a pass of its own before the scan" if args.conv else "none",
            "launch": {"state_groups": plan[0], "segments": plan[1]},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("scan_kernel (main pass)" if plan[1] == 1 else "scan passes (aggregate + carry + main)")
                      + (" after conv_silu_kernel" if args.conv else ""),
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(args.workload, plan, default_opts),
            "algorithmic_bytes_per_launch": nbytes,
            "mean_launch_ms": mean_launch_ms,
            "median_launch_ms": per[len(per) // 2],
            "min_launch_ms": per[0],
            "measured_copy_GBps": copy_gbps,
            "target_frac": 0.60,
            "limited_by": "VALU issue (the kernel is ALU-bound; see valu)",
            "valu": valu,
        },
        "memory": {
            "workspace_bytes": need,
            "inputs_bytes": inputs_bytes,
            "outputs_bytes": outputs_bytes,
            "allocated_during_steps_bytes": peak_alloc - base_alloc,
            "peak_allocated_bytes": peak_alloc,
            "memory_mb": peak_alloc / 2 ** 20,
            "note": "the library allocates nothing; the caller's inputs, outputs and workspace are all it uses",
        },
    }
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30
        del src, dst
    if not args.no_bwd:
        print("bench: backward", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(torch, ssm, cfg, dev, disc=args.disc, step_opts=step_opts)
    x_c2 = None
    if not args.no_configs:
        out["workloads"] = {}
        print("bench: tiny", file=sys.stderr, flush=True)
        out["workloads"]["tiny"] = bench_tiny(torch, ssm)
        out["workloads"]["mamba130m_rotated"] = bench_scan_workload(torch, ssm, "mamba130m", 50, 5, sets=12)
        out["workloads"]["mamba130m_resident"] = bench_scan_workload(torch, ssm, "mamba130m", 50, 5, sets=1)
        out["workloads"]["mamba130m_resident"]["note"] = (
            "one buffer set (101.7 MB) that stays in the 256 MB Infinity Cache between calls: cache-assisted, "
            "context only")
        out["workloads"]["long"] = bench_scan_workload(torch, ssm, "long", 10, 2, sets=1)
    if not args.no_decode:
        print("bench: decode", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(torch, ssm, copy_gbps=copy_gbps)
    if not args.no_ssd:
        print("bench: Mamba-2 SSD layer", file=sys.stderr, flush=True)
        out["ssd"] = bench_ssd(torch, ssm, cpu=not args.no_cpu, copy_gbps=copy_gbps)
    if not args.no_cpu:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        if not args.no_configs:
            x_c2 = si.scan_inputs(si.CONFIGS["mamba130m"], seed=0)
        out["cpu_baseline"] = cpu_baseline(x, y, torch, opts=oracle_opts, x_c2=x_c2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
