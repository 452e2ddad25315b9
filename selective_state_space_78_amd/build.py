"""Compile the HIP library for gfx950 into the package directory.

The library is a plain shared object (C ABI, no torch linkage) built with
hipcc. Packed fp32 vector instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# translation units: the ABI (+ decode), one scan unit and one backward unit per
# element type and discretisation (bf16 scans also one reading u in fp32),
# compiled in parallel and linked into one shared object
UNITS = ("ssm_scan.hip", "scan_bf16_euler.hip", "scan_bf16_zoh.hip", "scan_bf16_euler_u32.hip",
         "scan_bf16_zoh_u32.hip", "scan_f32_euler.hip", "scan_f32_zoh.hip",
         "bwd_bf16_euler.hip", "bwd_bf16_zoh.hip", "bwd_f32_euler.hip", "bwd_f32_zoh.hip",
         "ssd_euler.hip", "ssd_zoh.hip")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libssm_scan.so")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# the host pass does not know the device-only feature name; drop that note
_NOISE = "is not a recognized feature for this target"


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if _NOISE not in l)


def build(output: str = LIBRARY, extra=(), quiet: bool = True, build_dir: str | None = None) -> str:
    build_dir = build_dir or os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for unit in UNITS:
        obj = os.path.join(build_dir, unit.replace(".hip", ".o"))
        cmd = ["hipcc", *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, unit)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for cmd, pr in procs:
        out, err = pr.communicate()
        err = _clean(err)
        if pr.returncode != 0:
            failed.append("%s\n%s" % (" ".join(cmd), err))
        elif err.strip() and not quiet:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), _clean(res.stderr)))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(quiet=False))
