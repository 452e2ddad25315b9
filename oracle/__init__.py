"""fp64 CPU oracle for the Mamba selective scan (S6), its backward, its decode
step and the Mamba-2 SSD layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
bench's CPU-baseline leg, never by the product path. It shares no code with
the HIP library: the arithmetic lives in ``ssm_oracle.c`` (plain C, fp64,
sequential recurrence; see its header for the passages each line follows) and
this module only compiles it with gcc and marshals numpy arrays into it.

Element types: ``float64``, ``float32`` and ``uint16`` arrays are accepted for
the per-token tensors (u, delta, B, C, z); a ``uint16`` array holds bf16 bit
patterns. A, D and h0 are widened to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssm_oracle.c")
LIBRARY = os.path.join(HERE, "libssm_oracle.so")

F64, F32, BF16 = 0, 1, 2
EULER, ZOH = 0, 1
_TYPE_OF = {np.dtype(np.float64): F64, np.dtype(np.float32): F32, np.dtype(np.uint16): BF16}
_DISC = {"euler": EULER, "zoh": ZOH}

_lock = threading.Lock()
_handles: dict[str, "Oracle"] = {}


def build(source: str = SOURCE, output: str = LIBRARY, strict: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into ``output``."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall"]
    cmd += ["-Werror"] if strict else ["-w"]
    cmd += ["-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _conv(weight, bias, dim):
    """fp64 copies of the convolution prologue's weights (dim, W) and bias (dim,)."""
    if weight is None:
        return None, None, 0
    w = np.ascontiguousarray(weight, dtype=np.float64)
    assert w.ndim == 2 and w.shape[0] == dim
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    return w, b, int(w.shape[1])


class Oracle:
    """ctypes handle on one compiled oracle library. ``threads`` is the OpenMP
    thread count used when a call passes ``nthreads=0`` (0: the runtime's)."""

    def __init__(self, path: str, threads: int = 0):
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_selective_scan.argtypes = [i64, i64, i64, i64, i32, i32, i32, vp, vp,
                                              vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                              i64, vp, vp, vp, i32]
        lib.oracle_selective_scan.restype = i32
        lib.oracle_state_update.argtypes = [i64, i64, i64, i32, i32,
                                            vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_state_update.restype = i32
        lib.oracle_selective_scan_bwd.argtypes = [i64, i64, i64, i64, i32, i32, i32, vp, vp,
                                                  vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_selective_scan_bwd.restype = i32
        lib.oracle_ssd.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32,
                                   vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32]
        lib.oracle_ssd.restype = i32
        self.lib = lib
        self.path = path
        self.threads = int(threads)

    @staticmethod
    def _per_token(arrays):
        types = {a.dtype for a in arrays if a is not None}
        if len(types) != 1:
            raise TypeError("u, delta, B, C and z must share one element type, got %s" % types)
        t = types.pop()
        if t not in _TYPE_OF:
            raise TypeError("unsupported element type %s" % t)
        return _TYPE_OF[t]

    def selective_scan(self, u, delta, A, B, C, D=None, z=None, h0=None,
                       disc="euler", channels=None, nthreads=0, want_y=True,
                       delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None):
        """Scan (batch, L, dim) inputs.

        Returns ``(y, h_last)``. With ``channels=None`` every channel is
        computed and ``y`` is (batch, L, dim), ``h_last`` (batch, dim, N).
        With ``channels`` a sequence of (b, d) pairs, ``y`` is (k, L) and
        ``h_last`` is (k, N), row i belonging to ``channels[i]``.
        ``delta_bias`` (dim,) is added to delta, and ``delta_softplus`` passes
        the sum through softplus, before the recurrence uses it. With
        ``conv_weight`` (dim, W) (and ``conv_bias`` (dim,)), ``u`` holds x and
        the scan input is silu(causal depthwise conv1d(x) + bias).
        """
        u = np.ascontiguousarray(u)
        batch, L, dim = u.shape
        N = A.shape[1]
        typ = self._per_token([u, delta, B, C, z])
        delta = np.ascontiguousarray(delta)
        B = np.ascontiguousarray(B)
        C = np.ascontiguousarray(C)
        assert delta.shape == u.shape and B.shape == (batch, L, N) and C.shape == (batch, L, N)
        A64 = np.ascontiguousarray(A, dtype=np.float64)
        assert A64.shape == (dim, N)
        D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
        zc = None if z is None else np.ascontiguousarray(z)
        if zc is not None:
            assert zc.shape == u.shape
        h064 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        if h064 is not None:
            assert h064.shape == (batch, dim, N)
        if channels is None:
            sel = None
            nsel = batch * dim
        else:
            sel = np.ascontiguousarray([b * dim + d for b, d in channels], dtype=np.int64)
            nsel = len(sel)
        y = np.empty((nsel, L), np.float64) if want_y else None
        hl = np.empty((nsel, N), np.float64)
        dbias = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float64)
        cw, cb, W = _conv(conv_weight, conv_bias, dim)
        rc = self.lib.oracle_selective_scan(batch, L, dim, N, typ, _DISC[disc], W, _ptr(cw), _ptr(cb),
                                            _ptr(u), _ptr(delta), _ptr(dbias), int(bool(delta_softplus)),
                                            _ptr(A64), _ptr(B), _ptr(C),
                                            _ptr(D64), _ptr(zc), _ptr(h064),
                                            nsel, _ptr(sel), _ptr(y), _ptr(hl), int(nthreads or self.threads))
        if rc != 0:
            raise ValueError("oracle_selective_scan rejected its arguments")
        if channels is None:
            if y is not None:
                y = y.reshape(batch, dim, L).transpose(0, 2, 1).copy()
            hl = hl.reshape(batch, dim, N)
        return y, hl

    def selective_scan_bwd(self, u, delta, A, B, C, dy, D=None, z=None, h0=None, dh_last=None,
                           disc="euler", channels=None, want_bc=True, want_tokens=True, nthreads=0,
                           delta_bias=None, delta_softplus=False, conv_weight=None, conv_bias=None):
        """Gradients of sum(dy * y) + sum(dh_last * h_last) with respect to every input.

        Returns a dict. With ``channels=None``: du, ddelta, dz (batch, L, dim),
        dA (dim, N), dD (dim), dh0 (batch, dim, N), dB, dC (batch, L, N). With
        ``channels`` a sequence of (b, d) pairs: du, ddelta, dz (k, L), dA_c
        (k, N) and dD_c (k) (each channel's share of dA[d] and dD[d]), dh0
        (k, N), and dB, dC summed over the selected channels only.
        ``want_tokens=False`` skips du, ddelta and dz (None in the result).
        With ``delta_bias`` / ``delta_softplus`` (as in selective_scan), ddelta is
        the gradient of the raw delta and ddelta_bias (dim) (or its per-channel
        share ddelta_bias_c) that of the bias. With the convolution prologue,
        du is the gradient of x and dconv_weight (dim, W), dconv_bias (dim)
        (or their shares dconv_weight_c, dconv_bias_c) are added.
        """
        u = np.ascontiguousarray(u)
        batch, L, dim = u.shape
        N = A.shape[1]
        typ = self._per_token([u, delta, B, C, z])
        delta = np.ascontiguousarray(delta)
        B = np.ascontiguousarray(B)
        C = np.ascontiguousarray(C)
        A64 = np.ascontiguousarray(A, dtype=np.float64)
        D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
        zc = None if z is None else np.ascontiguousarray(z)
        h064 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        dy64 = np.ascontiguousarray(dy, dtype=np.float64)
        assert dy64.shape == u.shape
        dhl = None if dh_last is None else np.ascontiguousarray(dh_last, dtype=np.float64)
        if dhl is not None:
            assert dhl.shape == (batch, dim, N)
        if channels is None:
            sel, nsel = None, batch * dim
        else:
            sel = np.ascontiguousarray([b * dim + d for b, d in channels], dtype=np.int64)
            nsel = len(sel)
        du = np.empty((nsel, L)) if want_tokens else None
        dde = np.empty((nsel, L)) if want_tokens else None
        dz = np.empty((nsel, L)) if zc is not None and want_tokens else None
        dA_c = np.empty((nsel, N)); dD_c = np.empty(nsel); dDb_c = np.empty(nsel); dh0 = np.empty((nsel, N))
        dbias = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float64)
        cw, cb, W = _conv(conv_weight, conv_bias, dim)
        dcw_c = np.empty((nsel, W)) if W else None
        dcb_c = np.empty(nsel) if W else None
        dB = np.empty((batch, L, N)) if want_bc else None
        dC = np.empty((batch, L, N)) if want_bc else None
        rc = self.lib.oracle_selective_scan_bwd(batch, L, dim, N, typ, _DISC[disc], W, _ptr(cw), _ptr(cb),
                                                _ptr(u), _ptr(delta), _ptr(dbias), int(bool(delta_softplus)),
                                                _ptr(A64), _ptr(B), _ptr(C),
                                                _ptr(D64), _ptr(zc), _ptr(h064), _ptr(dy64), _ptr(dhl),
                                                nsel, _ptr(sel), _ptr(du), _ptr(dde), _ptr(dz),
                                                _ptr(dA_c), _ptr(dD_c), _ptr(dDb_c), _ptr(dcw_c), _ptr(dcb_c),
                                                _ptr(dh0), _ptr(dB), _ptr(dC),
                                                int(nthreads or self.threads))
        if rc != 0:
            raise ValueError("oracle_selective_scan_bwd rejected its arguments")
        if channels is not None:
            return dict(du=du, ddelta=dde, dz=dz, dA_c=dA_c, dD_c=dD_c, ddelta_bias_c=dDb_c, dh0=dh0,
                        dB=dB, dC=dC, dconv_weight_c=dcw_c, dconv_bias_c=dcb_c)

        def per_token(a):
            return None if a is None else a.reshape(batch, dim, L).transpose(0, 2, 1).copy()
        return dict(du=per_token(du), ddelta=per_token(dde), dz=per_token(dz),
                    dA=dA_c.reshape(batch, dim, N).sum(axis=0), dD=dD_c.reshape(batch, dim).sum(axis=0),
                    ddelta_bias=dDb_c.reshape(batch, dim).sum(axis=0),
                    dconv_weight=None if not W else dcw_c.reshape(batch, dim, W).sum(axis=0),
                    dconv_bias=None if not W else dcb_c.reshape(batch, dim).sum(axis=0),
                    dh0=dh0.reshape(batch, dim, N), dB=dB, dC=dC)

    def state_update(self, x, delta, A, B, C, h, D=None, z=None, disc="euler", nthreads=0,
                     delta_bias=None, delta_softplus=False):
        """One decode step. ``h`` (batch, dim, N) float64 is updated in place; returns y."""
        x = np.ascontiguousarray(x)
        batch, dim = x.shape
        N = A.shape[1]
        typ = self._per_token([x, delta, B, C, z])
        assert h.dtype == np.float64 and h.flags.c_contiguous and h.shape == (batch, dim, N)
        A64 = np.ascontiguousarray(A, dtype=np.float64)
        D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
        y = np.empty((batch, dim), np.float64)
        dbias = None if delta_bias is None else np.ascontiguousarray(delta_bias, dtype=np.float64)
        rc = self.lib.oracle_state_update(batch, dim, N, typ, _DISC[disc],
                                          _ptr(x), _ptr(np.ascontiguousarray(delta)), _ptr(dbias),
                                          int(bool(delta_softplus)), _ptr(A64),
                                          _ptr(np.ascontiguousarray(B)), _ptr(np.ascontiguousarray(C)),
                                          _ptr(D64), _ptr(None if z is None else np.ascontiguousarray(z)),
                                          _ptr(h), _ptr(y), int(nthreads or self.threads))
        if rc != 0:
            raise ValueError("oracle_state_update rejected its arguments")
        return y


    def ssd(self, x, dt, A, B, C, D=None, z=None, h0=None, disc="euler", dt_bias=None,
            dt_softplus=False, heads=None, want_y=True, nthreads=0):
        """Mamba-2 SSD layer, sequential form (see ``oracle_ssd`` in ssm_oracle.c).

        x, z (batch, L, H, P); dt (batch, L, H); B, C (batch, L, G, N); A, D,
        dt_bias (H,); h0 (batch, H, P, N). Returns ``(y, h_last)``: with
        ``heads=None`` y is (batch, L, H, P) and h_last (batch, H, P, N); with
        ``heads`` a sequence of (b, h) pairs, y is (k, L, P) and h_last (k, P, N).
        """
        x = np.ascontiguousarray(x)
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        typ = self._per_token([x, dt, B, C, z])
        dt = np.ascontiguousarray(dt)
        B = np.ascontiguousarray(B)
        C = np.ascontiguousarray(C)
        assert dt.shape == (batch, L, H) and B.shape == (batch, L, G, N) and C.shape == B.shape
        A64 = np.ascontiguousarray(A, dtype=np.float64)
        assert A64.shape == (H,)
        D64 = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
        zc = None if z is None else np.ascontiguousarray(z)
        if zc is not None:
            assert zc.shape == x.shape
        h064 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        if h064 is not None:
            assert h064.shape == (batch, H, P, N)
        bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float64)
        if heads is None:
            sel, nsel = None, batch * H
        else:
            sel = np.ascontiguousarray([b * H + h for b, h in heads], dtype=np.int64)
            nsel = len(sel)
        y = np.empty((nsel, L, P)) if want_y else None
        hl = np.empty((nsel, P, N))
        rc = self.lib.oracle_ssd(batch, L, H, P, G, N, typ, _DISC[disc], _ptr(x), _ptr(dt), _ptr(bias),
                                 int(bool(dt_softplus)), _ptr(A64), _ptr(B), _ptr(C), _ptr(D64), _ptr(zc),
                                 _ptr(h064), nsel, _ptr(sel), _ptr(y), _ptr(hl), int(nthreads or self.threads))
        if rc != 0:
            raise ValueError("oracle_ssd rejected its arguments")
        if heads is None:
            if y is not None:
                y = y.reshape(batch, H, L, P).transpose(0, 2, 1, 3).copy()
            hl = hl.reshape(batch, H, P, N)
        return y, hl


def load(path: str | None = None) -> Oracle:
    """Load (building first if needed) the oracle library at ``path``."""
    path = path or LIBRARY
    with _lock:
        if path not in _handles:
            if path == LIBRARY and (not os.path.exists(path)
                                    or os.path.getmtime(path) < os.path.getmtime(SOURCE)):
                build()
            _handles[path] = Oracle(path)
        return _handles[path]


def selective_scan(*args, **kwargs):
    return load().selective_scan(*args, **kwargs)


def state_update(*args, **kwargs):
    return load().state_update(*args, **kwargs)


def selective_scan_bwd(*args, **kwargs):
    return load().selective_scan_bwd(*args, **kwargs)


def ssd(*args, **kwargs):
    return load().ssd(*args, **kwargs)
