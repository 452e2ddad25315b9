"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The fp64 oracle (oracle/ssm_oracle.c), built with gcc and both sanitizers,
  runs every entry point (scan, backward, decode step, SSD) over small inputs
  in each element type, both discretisations and every option
  (tests/sanitize/oracle_driver.c).
* The library's host code (the C ABI's validation, planning and workspace
  arithmetic in csrc/ssm_scan.hip) is built with the sanitizers on its host
  side only and linked with the other, unchanged units; a driver
  (tests/sanitize/abi_driver.cpp) makes calls that are all refused before any
  launch, so no GPU is involved.
* A control program with a planted heap overflow checks that the sanitizer
  build catches one in this toolchain at all.

Any report aborts the program being run, and the test fails with its output.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "selective_state_space_78_amd")
CSRC = os.path.join(PKG, "csrc")

# gcc (CPU-only sources): both sanitizers, every report fatal
CPU_SAN = ["-fsanitize=" + ",".join(("address", "undefined")), "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
# hipcc: the sanitizers on the host side only; device code is built as usual
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
RUN_ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, env=None, timeout=300):
    return subprocess.run([str(c) for c in cmd], capture_output=True, text=True, timeout=timeout, env=env)


def _need(tool):
    path = shutil.which(tool)
    if path is None:
        pytest.skip("%s not found" % tool)
    return path


def test_sanitizer_build_catches_a_planted_overflow(tmp_path):
    gcc = _need("gcc")
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile int *p = malloc(4 * sizeof(int));\n"
                   "  int s = p[4]; free((void *)p); return s; }\n")
    r = _run([gcc, "-O0", "-g", *CPU_SAN, "-o", tmp_path / "planted", src])
    assert r.returncode == 0, r.stderr
    r = _run([tmp_path / "planted"], env=RUN_ENV)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_under_sanitizers(tmp_path):
    gcc = _need("gcc")
    exe = tmp_path / "oracle_san"
    r = _run([gcc, "-std=c99", "-O1", "-g", "-Wall", "-Werror", *CPU_SAN, "-o", exe,
              os.path.join(ROOT, "oracle", "ssm_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm"])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env=RUN_ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "all calls clean" in r.stdout


def test_library_host_validation_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not found")
    # the other translation units as the library build left them
    others = [o for o in sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
              if os.path.basename(o) != "ssm_scan.o"]
    if len(others) < 10:
        pytest.skip("library objects not built (run __graft_entry__.build())")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    abi_o, drv_o, exe = tmp_path / "ssm_scan_san.o", tmp_path / "abi_driver.o", tmp_path / "abi_san"
    r = _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *inc, "-c", "-o", abi_o,
              os.path.join(CSRC, "ssm_scan.hip")], timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    r = _run([hipcc, "-O1", "-g", "-std=c++17", *HOST_SAN, *inc, "-c", "-o", drv_o,
              os.path.join(HERE, "abi_driver.cpp")])
    assert r.returncode == 0, r.stderr[-4000:]
    r = _run([hipcc, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, drv_o, abi_o, *others])
    assert r.returncode == 0, r.stderr[-4000:]
    # the HIP runtime's own allocations are not this library's: no leak check here
    env = dict(RUN_ENV, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0")
    r = _run([exe], env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "refused as documented" in r.stdout
