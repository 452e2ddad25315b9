"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching a device.

No compute call is made here: every call below fails validation on the host,
so the fake device addresses it passes are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import selective_state_space_78_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIAS, EWS, EHIP, EALIGN, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ssm.LIBRARY):
        pytest.skip("library not built")
    return ssm.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(ssm.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_library_links_no_torch():
    if not os.path.exists(ssm.LIBRARY):
        pytest.skip("library not built")
    data = open(ssm.LIBRARY, "rb").read()
    assert b"libtorch" not in data and b"libc10" not in data


def test_status_strings(L):
    for code in (OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIAS, EWS, EHIP, EALIGN, ESCRATCH):
        s = ssm.ssm_status_string(code)
        assert s and s != "unknown status"
    assert ssm.ssm_status_string(12345) == "unknown status"


def desc(b=2, L=100, d=64, N=16, dtype=ssm.SSM_BF16, disc=0, softplus=0, conv=0, bias=None, cw=None, cb=None):
    return ssm.ScanDesc(b, L, d, N, dtype, disc, softplus, conv, bias, cw, cb)


def fake(addr):
    return ctypes.c_void_p(addr)


GB = 1 << 30


def scan_call(L, dsc, u=1 * GB, delta=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB,
              h0=0, y=8 * GB, h_last=9 * GB, ws=11 * GB, ws_bytes=1 << 30, tuning=None):
    args = [ctypes.byref(dsc) if dsc is not None else None]
    args += [fake(a) if a else None for a in (u, delta, A, B, C, D, z, h0, y, h_last, ws)]
    args += [ws_bytes]
    if tuning is None:
        return L.ssm_scan_fwd(*args, None)
    return L.ssm_scan_fwd_tuned(*args, ctypes.byref(ssm.ScanTuning(*tuning)), None)


def test_scan_descriptor_errors(L):
    assert scan_call(L, None) == ENULL
    assert scan_call(L, desc(b=-1)) == ESHAPE
    assert scan_call(L, desc(L=-5)) == ESHAPE
    assert scan_call(L, desc(dtype=7)) == EDTYPE
    assert scan_call(L, desc(disc=3)) == EUNSUP
    assert scan_call(L, desc(N=0)) == EUNSUP
    assert scan_call(L, desc(N=65)) == EUNSUP
    assert scan_call(L, desc(b=1 << 40, L=1 << 40)) == ESHAPE
    # one segment longer than 2^31 tokens (forced by the tuning): the kernels
    # count a segment's tokens in 32 bits, so the plan is refused
    assert scan_call(L, desc(b=1, L=(1 << 31) + 16, d=64), tuning=(8, 1)) == EUNSUP
    assert scan_call(L, desc(softplus=2)) == EUNSUP
    assert scan_call(L, desc(conv=5)) == EUNSUP
    assert scan_call(L, desc(conv=-1)) == EUNSUP
    assert scan_call(L, desc(conv=4)) == ENULL                   # taps missing
    assert scan_call(L, desc(conv=4, cw=10 * GB + 2)) == EALIGN
    assert scan_call(L, desc(conv=4, cw=8 * GB + 64)) == EALIAS  # taps inside y
    assert scan_call(L, desc(bias=10 * GB + 2)) == EALIGN
    assert scan_call(L, desc(bias=8 * GB + 64)) == EALIAS        # bias inside the output y


def test_scan_dim_limit(L):
    """dim is bounded so that 16 token rows of fp32 channels span less than
    4 GiB (the kernels' 32-bit offsets within a chunk); beyond it the forward,
    the backward and the workspace queries refuse the shape on the host."""
    assert scan_call(L, desc(b=1, L=16, d=(1 << 26) + 1, N=16)) == ESHAPE
    assert L.ssm_scan_workspace_size(ctypes.byref(desc(b=1, L=16, d=(1 << 26) + 1, N=16))) == 0
    assert bwd_call(L, desc(b=1, L=16, d=(1 << 26) + 1, N=16)) == ESHAPE
    assert L.ssm_scan_workspace_size(ctypes.byref(desc(b=1, L=16, d=1 << 26, N=16))) > 0


def test_scan_empty_problem_is_ok(L):
    # nothing to compute: returns before any device work
    assert scan_call(L, desc(b=0)) == OK
    assert scan_call(L, desc(d=0)) == OK


def test_scan_null_pointers(L):
    assert scan_call(L, desc(), A=0) == ENULL
    assert scan_call(L, desc(), u=0) == ENULL
    assert scan_call(L, desc(), delta=0) == ENULL
    assert scan_call(L, desc(), B=0) == ENULL
    assert scan_call(L, desc(), C=0) == ENULL
    assert scan_call(L, desc(), y=0) == ENULL


def test_scan_alignment(L):
    assert scan_call(L, desc(), u=GB + 1) == EALIGN
    assert scan_call(L, desc(dtype=ssm.SSM_F32), delta=2 * GB + 2) == EALIGN
    assert scan_call(L, desc(), h_last=9 * GB + 2) == EALIGN
    assert scan_call(L, desc(), A=3 * GB + 2) == EALIGN


def test_scan_aliasing(L):
    # y overlapping u, h_last overlapping z, h_last == y, workspace over B
    assert scan_call(L, desc(), y=1 * GB + 64) == EALIAS
    assert scan_call(L, desc(), h_last=7 * GB + 128) == EALIAS
    assert scan_call(L, desc(), h_last=8 * GB) == EALIAS
    assert scan_call(L, desc(), h0=10 * GB, h_last=10 * GB + 4) == EALIAS
    assert scan_call(L, desc(L=4096, d=64, b=1), ws=4 * GB, ws_bytes=1 << 24, tuning=(4, 4)) == EALIAS


def test_scan_workspace(L):
    d = desc(b=1, L=4096, d=64, N=16)
    rnd = lambda v: (v + 255) // 256 * 256
    bc = rnd((1 * 4096 + 32) * 16 * 4)          # widened B (and C): rows + 32 spare, 16 states
    need = L.ssm_scan_workspace_size_tuned(ctypes.byref(d), ctypes.byref(ssm.ScanTuning(4, 4)))
    assert need == 2 * bc + 3 * rnd(1 * 4 * 64 * 16 * 4)
    assert scan_call(L, d, ws=0, ws_bytes=0, tuning=(4, 4)) == EWS
    assert scan_call(L, d, ws=11 * GB, ws_bytes=need - 4, tuning=(4, 4)) == EWS
    assert scan_call(L, d, ws=11 * GB + 128, ws_bytes=need, tuning=(4, 4)) == EALIGN
    assert L.ssm_scan_workspace_size_tuned(ctypes.byref(d), ctypes.byref(ssm.ScanTuning(4, 1))) == 2 * bc
    d5 = desc(b=1, L=4096, d=64, N=5)           # padded to 8 states
    assert L.ssm_scan_workspace_size(ctypes.byref(d5)) >= 2 * rnd((4096 + 32) * 8 * 4)
    assert L.ssm_scan_workspace_size(ctypes.byref(desc(L=0))) == 0
    assert L.ssm_scan_workspace_size(None) == 0


def noalloc_call(L, dsc, u=1 * GB, delta=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB,
                 h0=0, y=8 * GB, h_last=9 * GB):
    args = [ctypes.byref(dsc) if dsc is not None else None]
    args += [fake(a) if a else None for a in (u, delta, A, B, C, D, z, h0, y, h_last)]
    return L.ssm_scan_fwd_noalloc(*args, None)


def test_noalloc_errors_before_any_device_call(L):
    """The no-allocation forward rejects bad descriptors, and problems whose
    scratch exceeds its fixed buffer, on the host before any HIP call."""
    assert noalloc_call(L, None) == ENULL
    assert noalloc_call(L, desc(b=-1)) == ESHAPE
    assert noalloc_call(L, desc(dtype=7)) == EDTYPE
    assert noalloc_call(L, desc(N=65)) == EUNSUP
    assert noalloc_call(L, desc(b=0)) == OK                      # nothing to compute
    cap = ssm.NOALLOC_SCRATCH_BYTES
    big = desc(b=64, L=1 << 20, d=4096, N=64)
    assert L.ssm_scan_workspace_size(ctypes.byref(big)) > cap
    assert noalloc_call(L, big) == ESCRATCH
    # the 1.4B-shaped layer fits; a width-4 convolution prologue on it (its u
    # takes b*L*d bf16 elements of scratch) does not
    flag = desc(b=8, L=8192, d=4096, N=16)
    assert 0 < L.ssm_scan_workspace_size(ctypes.byref(flag)) <= cap
    conv = desc(b=8, L=8192, d=4096, N=16, conv=4, cw=12 * GB)
    assert L.ssm_scan_workspace_size(ctypes.byref(conv)) > cap
    assert noalloc_call(L, conv) == ESCRATCH
    # the scratch constant of the binding is the header's
    m = re.search(r"#define\s+SSM_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == cap


def test_scan_bad_tuning(L):
    assert scan_call(L, desc(N=16), tuning=(3, 1)) == EUNSUP      # not a power of two
    assert scan_call(L, desc(N=16), tuning=(32, 1)) == EUNSUP     # more groups than states
    assert scan_call(L, desc(N=64), tuning=(2, 1)) == EUNSUP      # 32 states per wave
    assert scan_call(L, desc(N=16), tuning=(4, 65)) == EUNSUP     # too many segments
    assert scan_call(L, desc(N=16), tuning=(-1, 1)) == EUNSUP


def test_plan_shapes(L):
    # the flagship shapes get enough waves for 256 CUs x 4 SIMDs
    assert ssm.ssm_scan_plan(8, 8192, 4096, 16) == (8, 1)
    g, s = ssm.ssm_scan_plan(1, 131072, 5120, 16)
    assert g * s * 80 >= 2048
    assert ssm.ssm_scan_plan(1, 64, 16, 4)[1] == 1
    g, s = ssm.ssm_scan_plan(4, 100, 64, 64)
    assert 64 // g <= 16


def decode_call(L, b=4, d=64, N=16, dtype=ssm.SSM_BF16, disc=0, x=1 * GB, delta=2 * GB, A=3 * GB, B=4 * GB,
                C=5 * GB, D=6 * GB, z=7 * GB, h=8 * GB, y=9 * GB, softplus=0):
    ptrs = [fake(a) if a else None for a in (x, delta, A, B, C, D, z, h, y)]
    return L.ssm_state_update(b, d, N, dtype, disc, ptrs[0], ptrs[1], None, softplus, *ptrs[2:], None)


def test_decode_errors(L):
    assert decode_call(L, b=-1) == ESHAPE
    assert decode_call(L, softplus=2) == EUNSUP
    assert decode_call(L, dtype=9) == EDTYPE
    assert decode_call(L, disc=2) == EUNSUP
    assert decode_call(L, N=0) == EUNSUP
    assert decode_call(L, N=80) == EUNSUP
    assert decode_call(L, b=0) == OK
    assert decode_call(L, h=0) == ENULL
    assert decode_call(L, y=0) == ENULL
    assert decode_call(L, x=GB + 1) == EALIGN
    assert decode_call(L, y=8 * GB + 64) == EALIAS          # y inside h
    assert decode_call(L, h=1 * GB) == EALIAS               # h over x


def bwd_call(L, dsc, u=1 * GB, delta=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB, h0=0,
             dy=8 * GB, dhl=0, du=9 * GB, dde=10 * GB, dA=11 * GB, dB=12 * GB, dC=13 * GB, dD=14 * GB,
             dz=15 * GB, dh0=0, ddb=0, dcw=0, dcb=0, ws=16 * GB, ws_bytes=1 << 30):
    ptrs = [fake(a) if a else None for a in (u, delta, A, B, C, D, z, h0, dy, dhl, du, dde, dA, dB, dC, dD, dz,
                                             dh0, ddb, dcw, dcb, ws)]
    return L.ssm_scan_bwd(ctypes.byref(dsc) if dsc is not None else None, *ptrs, ws_bytes, None)


def test_bwd_errors(L):
    assert bwd_call(L, None) == ENULL
    assert bwd_call(L, desc(b=-1)) == ESHAPE
    assert bwd_call(L, desc(dtype=5)) == EDTYPE
    assert bwd_call(L, desc(N=65)) == EUNSUP
    assert bwd_call(L, desc(b=0)) == OK
    assert bwd_call(L, desc(), dy=0) == ENULL
    assert bwd_call(L, desc(), dA=0) == ENULL
    assert bwd_call(L, desc(), dB=0) == ENULL
    assert bwd_call(L, desc(), dz=0) == ENULL           # a gate needs its gradient
    # no gate: dz is not required (the call gets past the null checks to the
    # misaligned du; every call here fails before any launch)
    assert bwd_call(L, desc(), z=0, dz=0, du=9 * GB + 1) == EALIGN
    assert bwd_call(L, desc(), dD=0) == ENULL           # a skip needs its gradient
    assert bwd_call(L, desc(), du=9 * GB + 1) == EALIGN
    assert bwd_call(L, desc(), dA=11 * GB + 2) == EALIGN
    assert bwd_call(L, desc(), ws=16 * GB + 64) == EALIGN
    assert bwd_call(L, desc(), du=1 * GB + 64) == EALIAS      # du over u
    assert bwd_call(L, desc(), dB=11 * GB + 4) == EALIAS      # dB over dA
    assert bwd_call(L, desc(), ws=12 * GB) == EALIAS          # workspace over dB
    assert bwd_call(L, desc(), dh0=8 * GB + 128) == EALIAS    # dh0 over dy
    assert bwd_call(L, desc(bias=17 * GB)) == ENULL           # a delta bias needs its gradient
    assert bwd_call(L, desc(bias=17 * GB), ddb=17 * GB + 4) == EALIAS
    # the convolution prologue's backward needs the taps' gradient
    assert bwd_call(L, desc(conv=4, cw=17 * GB)) == ENULL
    assert bwd_call(L, desc(conv=4, cw=17 * GB), dcw=18 * GB + 2) == EALIGN
    assert bwd_call(L, desc(conv=4, cw=17 * GB), dcw=17 * GB + 8) == EALIAS      # over the taps
    assert bwd_call(L, desc(conv=4, cw=17 * GB, cb=17 * GB + 4096), dcw=18 * GB,
                    dcb=18 * GB + 64) == EALIAS                                  # bias gradient over taps gradient
    assert bwd_call(L, desc(conv=4, cw=17 * GB), dcw=18 * GB, ws=0, ws_bytes=0) == EWS


def test_bwd_workspace(L):
    d = desc(b=2, L=100, d=64, N=16)
    need = L.ssm_scan_bwd_workspace_size(ctypes.byref(d))
    rnd = lambda v: (v + 255) // 256 * 256
    # at least: regrouped B, C; checkpoints every 16 tokens; per-tile dB/dC partials; dA, dD partials
    assert need >= 2 * rnd(2 * (112 + 16) * 16 * 4) + rnd(2 * 7 * 16 * 64 * 4) + rnd(2 * 1 * 100 * 16 * 8)
    assert bwd_call(L, d, ws=0, ws_bytes=0) == EWS
    assert bwd_call(L, d, ws_bytes=need - 1) == EWS
    assert L.ssm_scan_bwd_workspace_size(ctypes.byref(desc(L=0))) == 0
    assert L.ssm_scan_bwd_workspace_size(None) == 0
    # the prologue adds u and its gradient (fp32) and per-256-token-block tap and bias sums
    dc = desc(b=2, L=100, d=64, N=16, conv=3, cw=17 * GB)
    extra = L.ssm_scan_bwd_workspace_size(ctypes.byref(dc)) - need
    assert extra >= 2 * rnd(2 * 100 * 64 * 4) + rnd(2 * 1 * 64 * 3 * 4) + rnd(2 * 1 * 64 * 4)


def test_training_pair_workspace(L):
    """ssm_scan_fwd_save needs the backward's workspace (checkpoints included),
    not the forward's, and ssm_scan_bwd_saved the same; both reject less before
    any launch, and share the other calls' argument checks."""
    d = desc(b=2, L=100, d=64, N=16)
    fwd_need = L.ssm_scan_workspace_size(ctypes.byref(d))
    bwd_need = L.ssm_scan_bwd_workspace_size(ctypes.byref(d))
    assert 0 < fwd_need < bwd_need
    save = lambda **kw: _fwd_save(L, kw.pop("dsc", d), **kw)
    assert save(ws_bytes=fwd_need) == EWS
    assert save(ws_bytes=bwd_need - 1) == EWS
    assert save(ws=0, ws_bytes=0) == EWS
    assert save(dsc=None) == ENULL
    assert save(dsc=desc(N=65)) == EUNSUP
    assert save(y=1 * GB + 64) == EALIAS                  # y over u
    assert save(ws=11 * GB + 64) == EALIGN
    assert save(dsc=desc(L=0), h_last=0) == OK            # nothing to compute or keep
    ptrs = [fake(a) if a else None for a in (1 * GB, 2 * GB, 3 * GB, 4 * GB, 5 * GB, 6 * GB, 7 * GB, 0, 8 * GB, 0,
                                             9 * GB, 10 * GB, 11 * GB, 12 * GB, 13 * GB, 14 * GB, 15 * GB, 0, 0, 0,
                                             0, 16 * GB)]
    assert L.ssm_scan_bwd_saved(ctypes.byref(d), *ptrs, bwd_need - 1, None) == EWS
    assert L.ssm_scan_bwd_saved(None, *ptrs, bwd_need, None) == ENULL


def test_conv_prologue_forward_workspace(L):
    """The forward runs the convolution prologue as a pass of its own and keeps
    its u, in fp32 whatever the tensors' type, in the workspace after the
    scan's part (for any batch: the pass runs in slices of rows); a workspace
    sized without it is rejected before any launch."""
    rnd = lambda v: (v + 255) // 256 * 256
    for dtype in (ssm.SSM_BF16, ssm.SSM_F32):
        for b in (70000, 2):
            plain = L.ssm_scan_workspace_size(ctypes.byref(desc(b=b, L=100, d=64, N=16, dtype=dtype)))
            dc = desc(b=b, L=100, d=64, N=16, dtype=dtype, conv=4, cw=17 * GB)
            conv = L.ssm_scan_workspace_size(ctypes.byref(dc))
            assert conv == rnd(plain) + rnd(b * 100 * 64 * 4)
        assert scan_call(L, dc, ws_bytes=conv - 1) == EWS    # b = 2


def test_ssd_decode_errors(L):
    """ssm_ssd_state_update rejects, before any launch, what ssm_ssd_fwd would
    and a sequence length other than one."""
    def call(dsc, x=1 * GB, dt=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB, h=8 * GB, y=9 * GB):
        ptrs = [fake(a) if a else None for a in (x, dt, A, B, C, D, z, h, y)]
        return L.ssm_ssd_state_update(ctypes.byref(dsc) if dsc is not None else None, *ptrs, None)
    assert call(None) == ENULL
    assert call(ssd_desc(L=2)) == ESHAPE
    assert call(ssd_desc(L=1, H=3, G=2)) == ESHAPE
    assert call(ssd_desc(L=1, dtype=ssm.SSM_F32)) == EUNSUP
    assert call(ssd_desc(L=1, P=80)) == EUNSUP
    assert call(ssd_desc(L=1, b=0)) == OK
    assert call(ssd_desc(L=1), h=0) == ENULL
    assert call(ssd_desc(L=1), y=0) == ENULL
    assert call(ssd_desc(L=1), h=8 * GB + 8) == EALIGN
    assert call(ssd_desc(L=1), B=4 * GB + 4) == EALIGN
    assert call(ssd_desc(L=1), y=8 * GB + 64) == EALIAS       # y over h
    assert call(ssd_desc(L=1), h=1 * GB) == EALIAS            # h over x


def _fwd_save(L, dsc, u=1 * GB, delta=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB, h0=0, y=8 * GB,
              h_last=9 * GB, ws=11 * GB, ws_bytes=1 << 30):
    args = [ctypes.byref(dsc) if dsc is not None else None]
    args += [fake(a) if a else None for a in (u, delta, A, B, C, D, z, h0, y, h_last, ws)]
    return L.ssm_scan_fwd_save(*args, ws_bytes, None)


def ssd_desc(b=2, L=100, H=4, P=64, G=1, N=128, dtype=ssm.SSM_BF16, disc=0, softplus=0, bias=None):
    return ssm.SsdDesc(b, L, H, P, G, N, dtype, disc, softplus, 0, bias)


def ssd_call(L, dsc, x=1 * GB, dt=2 * GB, A=3 * GB, B=4 * GB, C=5 * GB, D=6 * GB, z=7 * GB, h0=0,
             y=8 * GB, h_last=9 * GB):
    args = [ctypes.byref(dsc) if dsc is not None else None]
    args += [fake(a) if a else None for a in (x, dt, A, B, C, D, z, h0, y, h_last)]
    return L.ssm_ssd_fwd(*args, None)


def test_ssd_descriptor_errors(L):
    assert ssd_call(L, None) == ENULL
    assert ssd_call(L, ssd_desc(b=-1)) == ESHAPE
    assert ssd_call(L, ssd_desc(L=-1)) == ESHAPE
    assert ssd_call(L, ssd_desc(H=0)) == ESHAPE
    assert ssd_call(L, ssd_desc(H=6, G=4)) == ESHAPE          # groups must divide heads
    assert ssd_call(L, ssd_desc(dtype=9)) == EDTYPE
    assert ssd_call(L, ssd_desc(dtype=ssm.SSM_F32)) == EUNSUP  # bf16 matrix-core path only
    assert ssd_call(L, ssd_desc(P=48)) == EUNSUP
    assert ssd_call(L, ssd_desc(N=16)) == EUNSUP
    assert ssd_call(L, ssd_desc(disc=2)) == EUNSUP
    assert ssd_call(L, ssd_desc(softplus=3)) == EUNSUP
    assert ssd_call(L, ssd_desc(b=1 << 40, L=1 << 30)) == ESHAPE


def test_ssd_pointer_errors(L):
    assert ssd_call(L, ssd_desc(), x=0) == ENULL
    assert ssd_call(L, ssd_desc(), dt=0) == ENULL
    assert ssd_call(L, ssd_desc(), A=0) == ENULL
    assert ssd_call(L, ssd_desc(), y=0) == ENULL
    assert ssd_call(L, ssd_desc(), x=1 * GB + 8) == EALIGN
    assert ssd_call(L, ssd_desc(), B=4 * GB + 2) == EALIGN
    assert ssd_call(L, ssd_desc(), h_last=9 * GB + 4) == EALIGN
    assert ssd_call(L, ssd_desc(), dt=2 * GB + 1) == EALIGN
    assert ssd_call(L, ssd_desc(), A=3 * GB + 2) == EALIGN


def test_ssd_alias_errors(L):
    assert ssd_call(L, ssd_desc(), y=1 * GB + 4096) == EALIAS          # y inside x
    assert ssd_call(L, ssd_desc(), h_last=5 * GB) == EALIAS             # h_last on C
    assert ssd_call(L, ssd_desc(), h_last=8 * GB + 256) == EALIAS       # h_last inside y
    assert ssd_call(L, ssd_desc(), h0=10 * GB, h_last=10 * GB + 16) == EALIAS   # shifted, not in place


def test_ssd_nothing_to_do(L):
    # no heads, or no tokens and no state wanted: success without a launch
    assert ssd_call(L, ssd_desc(b=0)) == OK
    assert ssd_call(L, ssd_desc(L=0), x=0, dt=0, B=0, C=0, y=0, h_last=0) == OK
