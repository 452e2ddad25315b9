"""Python binding of the MI355X selective-scan library (libssm_scan.so).

Argument marshalling only: every step of the scan and of the decode step runs
in the library's HIP kernels. PyTorch supplies device memory and the current
HIP stream; the library itself is a plain C ABI (include/ssm_scan.h) that
links no torch. There is no fallback: if the library is missing, every call
raises.

Names follow the C ABI: ``ssm_scan_fwd``, ``ssm_scan_fwd_noalloc``, ``ssm_scan_workspace_size``,
``ssm_scan_plan``, ``ssm_scan_bwd``, ``ssm_state_update``, ``ssm_ssd_fwd``,
``ssm_status_string``.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libssm_scan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_DISC_EULER, SSM_DISC_ZOH = 0, 1
_DISC = {"euler": SSM_DISC_EULER, "zoh": SSM_DISC_ZOH}

# Every symbol include/ssm_scan.h declares.
EXPORTS = ("ssm_scan_workspace_size", "ssm_scan_fwd", "ssm_scan_workspace_size_tuned",
           "ssm_scan_fwd_tuned", "ssm_scan_plan", "ssm_scan_bwd_workspace_size", "ssm_scan_bwd",
           "ssm_scan_fwd_save", "ssm_scan_bwd_saved", "ssm_state_update", "ssm_ssd_fwd", "ssm_ssd_state_update",
           "ssm_scan_fwd_noalloc", "ssm_status_string")

# Fixed scratch of ssm_scan_fwd_noalloc per GPU (SSM_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("dtype", ctypes.c_int32), ("disc", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("delta_bias", ctypes.c_void_p), ("conv_weight", ctypes.c_void_p), ("conv_bias", ctypes.c_void_p)]


class SsdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("ngroups", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("disc", ctypes.c_int32), ("dt_softplus", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("dt_bias", ctypes.c_void_p)]


class ScanTuning(ctypes.Structure):
    _fields_ = [("state_groups", ctypes.c_int32), ("segments", ctypes.c_int32)]


class SsmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, ssm_status_string(status), status))
        self.status = status


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise ImportError("libssm_scan.so is not built (run __graft_entry__.build() or "
                                  "python selective_state_space_78_amd/build.py); there is no fallback")
            L = ctypes.CDLL(LIBRARY)
            vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
            pdesc, ptun = ctypes.POINTER(ScanDesc), ctypes.POINTER(ScanTuning)
            L.ssm_scan_workspace_size.argtypes = [pdesc]
            L.ssm_scan_workspace_size.restype = sz
            L.ssm_scan_workspace_size_tuned.argtypes = [pdesc, ptun]
            L.ssm_scan_workspace_size_tuned.restype = sz
            L.ssm_scan_plan.argtypes = [pdesc, ptun]
            L.ssm_scan_plan.restype = ctypes.c_int
            scan_args = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz]
            L.ssm_scan_fwd.argtypes = scan_args + [vp]
            L.ssm_scan_fwd.restype = ctypes.c_int
            L.ssm_scan_fwd_noalloc.argtypes = scan_args[:-2] + [vp]
            L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
            L.ssm_scan_fwd_tuned.argtypes = scan_args + [ptun, vp]
            L.ssm_scan_fwd_tuned.restype = ctypes.c_int
            L.ssm_scan_bwd_workspace_size.argtypes = [pdesc]
            L.ssm_scan_bwd_workspace_size.restype = sz
            L.ssm_scan_bwd.argtypes = [pdesc] + [vp] * 21 + [vp, sz, vp]
            L.ssm_scan_fwd_save.restype = ctypes.c_int
            L.ssm_scan_fwd_save.argtypes = scan_args + [vp]
            L.ssm_scan_bwd_saved.restype = ctypes.c_int
            L.ssm_scan_bwd_saved.argtypes = [pdesc] + [vp] * 21 + [vp, sz, vp]
            L.ssm_scan_bwd.restype = ctypes.c_int
            L.ssm_state_update.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                           vp]
            L.ssm_state_update.restype = ctypes.c_int
            L.ssm_ssd_fwd.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 11
            L.ssm_ssd_fwd.restype = ctypes.c_int
            L.ssm_ssd_state_update.argtypes = [ctypes.POINTER(SsdDesc)] + [vp] * 10
            L.ssm_ssd_state_update.restype = ctypes.c_int
            L.ssm_status_string.argtypes = [ctypes.c_int]
            L.ssm_status_string.restype = ctypes.c_char_p
            _lib = L
        return _lib


def ssm_status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    if t.dtype == torch.float32:
        return SSM_F32
    raise TypeError("per-token tensors must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _tuning(tuning):
    if tuning is None:
        return None
    g, s = tuning
    return ctypes.byref(ScanTuning(int(g), int(s)))


def make_desc(batch, seqlen, dim, dstate, dtype, disc="euler", delta_bias=None, delta_softplus=False,
              conv_weight=None, conv_bias=None) -> ScanDesc:
    """The scan descriptor; ``delta_bias`` (dim,), ``conv_weight`` (dim, W) and
    ``conv_bias`` (dim,) are float32 device tensors or None."""
    ptr = lambda t: None if t is None else t.data_ptr()
    W = 0 if conv_weight is None else int(conv_weight.shape[1])
    return ScanDesc(int(batch), int(seqlen), int(dim), int(dstate), int(dtype), _DISC[disc],
                    int(bool(delta_softplus)), W, ptr(delta_bias), ptr(conv_weight), ptr(conv_bias))


def ssm_scan_workspace_size(batch, seqlen, dim, dstate, dtype=SSM_BF16, disc="euler", tuning=None,
                            delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None) -> int:
    """Workspace bytes of ssm_scan_fwd for this shape and these options (the
    convolution prologue adds its u)."""
    desc = make_desc(batch, seqlen, dim, dstate, dtype, disc, delta_bias, delta_softplus, conv_weight, conv_bias)
    if tuning is None:
        return int(lib().ssm_scan_workspace_size(ctypes.byref(desc)))
    return int(lib().ssm_scan_workspace_size_tuned(ctypes.byref(desc), _tuning(tuning)))


def ssm_scan_plan(batch, seqlen, dim, dstate, dtype=SSM_BF16, disc="euler"):
    """(state_groups, segments) the library picks for this shape."""
    desc = make_desc(batch, seqlen, dim, dstate, dtype, disc)
    out = ScanTuning()
    rc = lib().ssm_scan_plan(ctypes.byref(desc), ctypes.byref(out))
    if rc != 0:
        raise SsmError(rc, "ssm_scan_plan")
    return out.state_groups, out.segments


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, h0=None, y=None, h_last=None,
                 disc="euler", workspace=None, tuning=None, stream=None, want_h_last=True,
                 delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None):
    """Selective scan forward on device tensors.

    u, delta, z: (batch, L, dim); B, C: (batch, L, N) of the same dtype
    (bfloat16 or float32); A: (dim, N) float32; D: (dim,) float32; h0:
    (batch, dim, N) float32. Outputs y (batch, L, dim) and h_last
    (batch, dim, N) are allocated when not given. Returns (y, h_last).
    ``tuning`` is an optional (state_groups, segments) pair. ``delta_bias``
    (dim,) float32 and ``delta_softplus`` form the step in the kernel:
    softplus(delta + bias). With ``conv_weight`` (dim, W <= 4) float32 (and
    ``conv_bias`` (dim,)), ``u`` holds x and the scan input is
    silu(causal depthwise conv1d(x) + bias), formed in the kernel.
    """
    y, h_last, _ = _fwd(u, delta, A, B, C, D, z, h0, y, h_last, disc, workspace, tuning, stream, want_h_last,
                        delta_bias, delta_softplus, conv_weight, conv_bias, save=False)
    return y, h_last


def ssm_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, h0=None, y=None, h_last=None,
                         disc="euler", stream=None, want_h_last=True,
                         delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None):
    """ssm_scan_fwd without a workspace (the C call of the same name): the
    library's fixed per-GPU scratch serves instead, and the call allocates no
    device memory of its own. Pass ``y`` (and ``h_last``) to allocate nothing
    here either. Problems needing more than NOALLOC_SCRATCH_BYTES of scratch
    raise SsmError (SSM_ERR_SCRATCH)."""
    y, h_last, _ = _fwd(u, delta, A, B, C, D, z, h0, y, h_last, disc, None, None, stream, want_h_last,
                        delta_bias, delta_softplus, conv_weight, conv_bias, save=False, noalloc=True)
    return y, h_last


def ssm_scan_fwd_save(u, delta, A, B, C, D=None, z=None, h0=None, y=None, h_last=None,
                      disc="euler", workspace=None, stream=None, want_h_last=True,
                      delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None):
    """ssm_scan_fwd that also keeps the backward's checkpoints (the C call of
    the same name). Returns (y, h_last, saved): ``saved`` is the workspace
    (uint8, ssm_scan_bwd_workspace_size bytes; ``workspace`` if given) to pass
    unchanged to ssm_scan_bwd_saved with the same inputs."""
    return _fwd(u, delta, A, B, C, D, z, h0, y, h_last, disc, workspace, None, stream, want_h_last,
                delta_bias, delta_softplus, conv_weight, conv_bias, save=True)


def _fwd(u, delta, A, B, C, D, z, h0, y, h_last, disc, workspace, tuning, stream, want_h_last,
         delta_bias, delta_softplus, conv_weight, conv_bias, save, noalloc=False):
    import torch
    batch, L, dim = u.shape
    N = A.shape[1]
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    _check(u, "u", device=dev)
    _check(delta, "delta", (batch, L, dim), dt, dev)
    _check(z, "z", (batch, L, dim), dt, dev)
    _check(B, "B", (batch, L, N), dt, dev)
    _check(C, "C", (batch, L, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(h0, "h0", (batch, dim, N), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, L, dim), dtype=dt, device=dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _check(y, "y", (batch, L, dim), dt, dev)
    _check(h_last, "h_last", (batch, dim, N), torch.float32, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (dim, conv_weight.shape[1]), torch.float32, dev)
    _check(conv_bias, "conv_bias", (dim,), torch.float32, dev)
    desc = make_desc(batch, L, dim, N, code, disc, delta_bias, delta_softplus, conv_weight, conv_bias)
    L_ = lib()
    if noalloc:
        rc = L_.ssm_scan_fwd_noalloc(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                     _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last), _stream(stream, dev))
        if rc != 0:
            raise SsmError(rc, "ssm_scan_fwd_noalloc")
        return y, h_last, None
    if save:
        need = L_.ssm_scan_bwd_workspace_size(ctypes.byref(desc))
    elif tuning is None:
        need = L_.ssm_scan_workspace_size(ctypes.byref(desc))
    else:
        need = L_.ssm_scan_workspace_size_tuned(ctypes.byref(desc), _tuning(tuning))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(h0), _ptr(y), _ptr(h_last), _ptr(workspace), ws_bytes]
    if save:
        name = "ssm_scan_fwd_save"
        rc = L_.ssm_scan_fwd_save(*args, _stream(stream, dev))
    elif tuning is None:
        name = "ssm_scan_fwd"
        rc = L_.ssm_scan_fwd(*args, _stream(stream, dev))
    else:
        name = "ssm_scan_fwd_tuned"
        rc = L_.ssm_scan_fwd_tuned(*args, _tuning(tuning), _stream(stream, dev))
    if rc != 0:
        raise SsmError(rc, name)
    return y, h_last, workspace


def ssm_scan_bwd_workspace_size(batch, L, dim, N, dtype_code, disc="euler", delta_bias=None,
                                delta_softplus=False, conv_weight=None, conv_bias=None) -> int:
    desc = make_desc(batch, L, dim, N, dtype_code, disc, delta_bias, delta_softplus, conv_weight, conv_bias)
    return int(lib().ssm_scan_bwd_workspace_size(ctypes.byref(desc)))


def ssm_scan_bwd_saved(u, delta, A, B, C, dy, saved, D=None, z=None, h0=None, dh_last=None, disc="euler",
                       stream=None, want_dh0=True, out=None, delta_bias=None, delta_softplus=False,
                       conv_weight=None, conv_bias=None):
    """ssm_scan_bwd that reads the checkpoints an ssm_scan_fwd_save call with
    the same inputs left in ``saved`` (its returned workspace) instead of
    recomputing them (the C call of the same name). Arguments and results as
    ssm_scan_bwd."""
    if saved is None:
        raise ValueError("ssm_scan_bwd_saved needs the workspace of an ssm_scan_fwd_save call")
    return ssm_scan_bwd(u, delta, A, B, C, dy, D=D, z=z, h0=h0, dh_last=dh_last, disc=disc, workspace=saved,
                        stream=stream, want_dh0=want_dh0, out=out, delta_bias=delta_bias,
                        delta_softplus=delta_softplus, conv_weight=conv_weight, conv_bias=conv_bias,
                        _saved=True)


def ssm_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, h0=None, dh_last=None, disc="euler",
                 workspace=None, stream=None, want_dh0=True, out=None, delta_bias=None, delta_softplus=False,
                 conv_weight=None, conv_bias=None, _saved=False):
    """Backward of ssm_scan_fwd on device tensors.

    Inputs as ssm_scan_fwd, plus dy (batch, L, dim) of the input dtype and an
    optional dh_last (batch, dim, N) float32. Returns a dict with du, ddelta,
    dz (input dtype, dz only with a gate), dA (dim, N), dB, dC (batch, L, N),
    dD (dim,) (with a skip) and dh0 (batch, dim, N) (when ``want_dh0``), all
    float32 except the per-token ones, and ddelta_bias (dim,) with a
    ``delta_bias``. With ``conv_weight`` (dim, W) (and ``conv_bias``), ``u``
    holds x, du is the gradient of x, and dconv_weight (dim, W), dconv_bias
    (dim,) are added. ``out`` may hold preallocated outputs.
    """
    import torch
    batch, L, dim = u.shape
    N = A.shape[1]
    dev = u.device
    dt = u.dtype
    code = _dtype_code(u)
    _check(u, "u", device=dev)
    _check(delta, "delta", (batch, L, dim), dt, dev)
    _check(z, "z", (batch, L, dim), dt, dev)
    _check(B, "B", (batch, L, N), dt, dev)
    _check(C, "C", (batch, L, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(h0, "h0", (batch, dim, N), torch.float32, dev)
    _check(dy, "dy", (batch, L, dim), dt, dev)
    _check(dh_last, "dh_last", (batch, dim, N), torch.float32, dev)
    o = dict(out or {})
    f32 = torch.float32

    def get(name, shape, dtype, wanted=True):
        if not wanted:
            return None
        if name not in o or o[name] is None:
            o[name] = torch.empty(shape, dtype=dtype, device=dev)
        _check(o[name], name, shape, dtype, dev)
        return o[name]
    du = get("du", (batch, L, dim), dt)
    dde = get("ddelta", (batch, L, dim), dt)
    dz = get("dz", (batch, L, dim), dt, z is not None)
    dA = get("dA", (dim, N), f32)
    dB = get("dB", (batch, L, N), f32)
    dC = get("dC", (batch, L, N), f32)
    dD = get("dD", (dim,), f32, D is not None)
    dh0 = get("dh0", (batch, dim, N), f32, want_dh0)
    _check(delta_bias, "delta_bias", (dim,), f32, dev)
    ddb = get("ddelta_bias", (dim,), f32, delta_bias is not None)
    W = 0 if conv_weight is None else int(conv_weight.shape[1])
    if conv_weight is not None:
        _check(conv_weight, "conv_weight", (dim, W), f32, dev)
    _check(conv_bias, "conv_bias", (dim,), f32, dev)
    dcw = get("dconv_weight", (dim, W), f32, W > 0)
    dcb = get("dconv_bias", (dim,), f32, W > 0)
    desc = make_desc(batch, L, dim, N, code, disc, delta_bias, delta_softplus, conv_weight, conv_bias)
    L_ = lib()
    need = L_.ssm_scan_bwd_workspace_size(ctypes.byref(desc))
    if workspace is not None and workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace has %d bytes, ssm_scan_bwd needs %d" % (
            workspace.numel() * workspace.element_size(), need))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    name = "ssm_scan_bwd_saved" if _saved else "ssm_scan_bwd"
    rc = getattr(L_, name)(ctypes.byref(desc), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                           _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(du), _ptr(dde), _ptr(dA), _ptr(dB), _ptr(dC),
                           _ptr(dD), _ptr(dz), _ptr(dh0), _ptr(ddb), _ptr(dcw), _ptr(dcb), _ptr(workspace), ws_bytes,
                           _stream(stream, dev))
    if rc != 0:
        raise SsmError(rc, name)
    return dict(du=du, ddelta=dde, dz=dz, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0, ddelta_bias=ddb,
                dconv_weight=dcw, dconv_bias=dcb)


def ssm_state_update(x, delta, A, B, C, h, D=None, z=None, y=None, disc="euler", stream=None,
                     delta_bias=None, delta_softplus=False):
    """One decode step on device tensors; h (batch, dim, N) float32 is updated in place.

    x, delta, z: (batch, dim); B, C: (batch, N). Returns y (batch, dim).
    """
    import torch
    batch, dim = x.shape
    N = A.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    _check(x, "x", device=dev)
    _check(delta, "delta", (batch, dim), dt, dev)
    _check(z, "z", (batch, dim), dt, dev)
    _check(B, "B", (batch, N), dt, dev)
    _check(C, "C", (batch, N), dt, dev)
    _check(A, "A", (dim, N), torch.float32, dev)
    _check(D, "D", (dim,), torch.float32, dev)
    _check(h, "h", (batch, dim, N), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, dim), dtype=dt, device=dev)
    _check(y, "y", (batch, dim), dt, dev)
    _check(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    rc = lib().ssm_state_update(batch, dim, N, code, _DISC[disc], _ptr(x), _ptr(delta), _ptr(delta_bias),
                                int(bool(delta_softplus)), _ptr(A),
                                _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h), _ptr(y), _stream(stream, dev))
    if rc != 0:
        raise SsmError(rc, "ssm_state_update")
    return y


def make_ssd_desc(batch, seqlen, nheads, headdim, ngroups, dstate, dtype=SSM_BF16, disc="euler",
                  dt_bias=None, dt_softplus=False) -> SsdDesc:
    return SsdDesc(int(batch), int(seqlen), int(nheads), int(headdim), int(ngroups), int(dstate), int(dtype),
                   _DISC[disc], int(bool(dt_softplus)), 0, None if dt_bias is None else dt_bias.data_ptr())


def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, h0=None, y=None, h_last=None, disc="euler",
                dt_bias=None, dt_softplus=False, want_h_last=True, stream=None):
    """Mamba-2 SSD layer on device tensors.

    x, z: (batch, L, H, P) bfloat16; dt: (batch, L, H) bfloat16; B, C:
    (batch, L, G, N) bfloat16; A, D, dt_bias: (H,) float32; h0: (batch, H, P, N)
    float32. Outputs y (batch, L, H, P) and h_last (batch, H, P, N) are
    allocated when not given. Returns (y, h_last).
    """
    import torch
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    code = _dtype_code(x)
    _check(x, "x", device=dev)
    _check(dt, "dt", (batch, L, H), x.dtype, dev)
    _check(z, "z", (batch, L, H, P), x.dtype, dev)
    _check(B, "B", (batch, L, G, N), x.dtype, dev)
    _check(C, "C", (batch, L, G, N), x.dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(h0, "h0", (batch, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=x.dtype, device=dev)
    if h_last is None and want_h_last:
        h_last = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _check(y, "y", (batch, L, H, P), x.dtype, dev)
    _check(h_last, "h_last", (batch, H, P, N), torch.float32, dev)
    desc = make_ssd_desc(batch, L, H, P, G, N, code, disc, dt_bias, dt_softplus)
    rc = lib().ssm_ssd_fwd(ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                           _ptr(h0), _ptr(y), _ptr(h_last), _stream(stream, dev))
    if rc != 0:
        raise SsmError(rc, "ssm_ssd_fwd")
    return y, h_last


def ssm_ssd_state_update(x, dt, A, B, C, h, D=None, z=None, y=None, disc="euler", dt_bias=None,
                         dt_softplus=False, stream=None):
    """One SSD decode step on device tensors: x, z (batch, H, P) bfloat16, dt
    (batch, H) bfloat16, B, C (batch, G, N) bfloat16, A, D, dt_bias (H,)
    float32; h (batch, H, P, N) float32 is updated in place. Returns y
    (batch, H, P), allocated when not given."""
    import torch
    batch, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    code = _dtype_code(x)
    _check(x, "x", device=dev)
    _check(dt, "dt", (batch, H), x.dtype, dev)
    _check(z, "z", (batch, H, P), x.dtype, dev)
    _check(B, "B", (batch, G, N), x.dtype, dev)
    _check(C, "C", (batch, G, N), x.dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(h, "h", (batch, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, H, P), dtype=x.dtype, device=dev)
    _check(y, "y", (batch, H, P), x.dtype, dev)
    desc = make_ssd_desc(batch, 1, H, P, G, N, code, disc, dt_bias, dt_softplus)
    rc = lib().ssm_ssd_state_update(ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(z), _ptr(h), _ptr(y), _stream(stream, dev))
    if rc != 0:
        raise SsmError(rc, "ssm_ssd_state_update")
    return y
