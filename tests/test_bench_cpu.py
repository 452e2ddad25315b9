"""Host-side checks of bench.py: the one-GPU guard, the per-unit figures its
roofline objects are built from, and the committed traffic records."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ssm_inputs as si  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 exits with status 2 and says why, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_scan_ops_per_token_channel():
    """16 states x 5 VALU (delta*A, exp2, (delta u)*B, state FMA, readout FMA),
    plus delta*u and the D*u FMA, plus the gate (z*log2e, exp2, 1 + e, rcp, z*r,
    y*s): 80 + 2 + 6 = 88 with the gate, 82 without."""
    assert bench.valu_ops_per_token_ch(16, True) == 88
    assert bench.valu_ops_per_token_ch(16, False) == 82


def test_scan_algorithmic_bytes():
    """u, delta, z, y in bf16 (8 B per token and channel) plus B, C, A, D, h_last."""
    cfg = si.CONFIGS["mamba1.4b"]
    tok_ch = cfg.batch * cfg.seqlen * cfg.dim
    expect = (4 * 2 * tok_ch                          # u, delta, z, y
              + 2 * 2 * cfg.batch * cfg.seqlen * cfg.dstate   # B, C
              + 4 * cfg.dim * cfg.dstate + 4 * cfg.dim         # A, D
              + 4 * cfg.batch * cfg.dim * cfg.dstate)          # h_last
    assert si.algorithmic_bytes(cfg) == expect == 2154053632


def test_ssd_algorithmic_bytes_and_flops():
    """Per (token, head): x in and y out (2 P bf16), dt, and B, C shared by the
    group's heads; per chunk of Q = 64 tokens the matrix-core flops of the
    scores, the masked product, the readout and the update."""
    cfg = si.SSD_CONFIGS["mamba2-ssd"]
    th = cfg.batch * cfg.seqlen * cfg.nheads
    P, N, Q = cfg.headdim, cfg.dstate, 64
    expect_bytes = (th * (2 * P * 2 + 2) + 2 * 2 * cfg.batch * cfg.seqlen * cfg.ngroups * N
                    + 4 * cfg.nheads + 4 * cfg.batch * cfg.nheads * P * N)
    assert si.ssd_bytes(cfg) == expect_bytes == 1132462336
    assert si.ssd_flops(cfg) == th * 2 * (Q * N // 2 + Q * P // 2 + 2 * N * P) == 188978561024


@pytest.mark.parametrize("name,workload,algorithmic", [
    ("traffic_scan_mamba1.4b.json", "mamba1.4b", lambda: si.algorithmic_bytes(si.CONFIGS["mamba1.4b"])),
    ("traffic_ssd_mamba2.json", "mamba2-ssd", lambda: si.ssd_bytes(si.SSD_CONFIGS["mamba2-ssd"])),
])
def test_committed_traffic_records(name, workload, algorithmic):
    """The counter-derived HBM bytes are recorded with the source digest they
    were taken on, and lie within a few percent above the algorithmic bytes."""
    rec = json.load(open(os.path.join(ROOT, "profiles", name)))
    assert rec["workload"] == workload
    assert isinstance(rec["source_digest"], str) and len(rec["source_digest"]) == 16
    assert rec["fetch_bytes"] + rec["write_bytes"] == pytest.approx(rec["bytes_per_launch"])
    ratio = rec["bytes_per_launch"] / algorithmic()
    assert 0.99 < ratio < 1.05, ratio


def test_sampled_channels_cover_the_corners():
    """The parity samples of the extra workloads are distinct, in range, and
    include the first and last channel of the first and last batch row."""
    for batch, dim, k in ((4, 1536, 16), (1, 5120, 16), (256, 5120, 8)):
        ch = bench.sample_channels(batch, dim, k)
        assert len(ch) == len(set(ch)) == max(k, 4)
        assert all(0 <= b < batch and 0 <= d < dim for b, d in ch)
        assert {(0, 0), (batch - 1, dim - 1)} <= set(ch)


def test_cpu_baseline_uses_every_core():
    """The oracle baseline runs on every core of the affinity mask (no cap)."""
    assert bench.host_cores() == len(os.sched_getaffinity(0))


def test_committed_valu_record():
    """The scan's instruction and clock record: counted on the current kernel
    source in the headline launch shape, issue slots = VALU + transcendentals
    (an exp costs two), and a clock near the part's 2.4 GHz."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "valu_scan_mamba1.4b.json")))
    assert rec["workload"] == "mamba1.4b" and list(rec["launch"]) == [8, 1]
    assert rec["issue_slots_per_token_ch"] == pytest.approx(rec["valu_per_token_ch"] + rec["trans_per_token_ch"], abs=0.02)
    assert bench.valu_ops_per_token_ch(16, True) <= rec["valu_per_token_ch"] <= 130
    assert 1.5 < rec["shader_clock_GHz"] <= 2.45
