"""fp64 CPU oracle for the selective-scan hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The GPU library never calls it and shares no
code with it.  The arithmetic lives in ``oracle.c`` (plain sequential C, fp64);
this module only builds it with gcc and marshals numpy arrays through ctypes.

Every function here takes and returns float64 numpy arrays in the layouts
documented in ``oracle.c``:
  x, dt, z, y [B, D, L];  Bm, Cm [B, L, N];  A [D, N];  dt_bias, Dskip [D];
  h0, h_last [B, D, N];  conv w [D, K];
  Mamba-2 form: x, z, y [B, L, H, P]; dt [B, L, H]; Bm, Cm [B, L, G, N];
  A, dt_bias, Dskip [H]; h0, h_last [B, H, P, N].
Parity status: every function is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")


def compile_oracle(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile an oracle C source with gcc (IEEE fp64, no fast-math)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
         "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c (always with force; else only when the library is
    missing or older than the source)."""
    stale = (not os.path.exists(LIBRARY)
             or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
    if force or stale:
        compile_oracle()
    return LIBRARY


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_zoh.restype = None
        lib.oracle_zoh.argtypes = [ctypes.c_double, ctypes.c_double, P, P]
        lib.oracle_selective_scan_fwd.restype = ctypes.c_int
        lib.oracle_selective_scan_fwd.argtypes = [P] * 11 + [I64] * 4 + [ctypes.c_int]
        lib.oracle_conv1d_silu.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [P] * 4 + [I64] * 4 + [ctypes.c_int]
        lib.oracle_selective_scan_bwd.restype = ctypes.c_int
        lib.oracle_selective_scan_bwd.argtypes = [P] * 20 + [I64] * 4
        lib.oracle_conv1d_update.restype = ctypes.c_int
        lib.oracle_conv1d_update.argtypes = [P] * 5 + [I64] * 3
        lib.oracle_ssd_scan_fwd.restype = ctypes.c_int
        lib.oracle_ssd_scan_fwd.argtypes = [P] * 11 + [I64] * 6
        lib.oracle_state_update.restype = ctypes.c_int
        lib.oracle_state_update.argtypes = [P] * 10 + [I64] * 3
        self.lib = lib
        self.path = path

    def softplus(self, v: float) -> float:
        return self.lib.oracle_softplus(float(v))

    def silu(self, v: float) -> float:
        return self.lib.oracle_silu(float(v))

    def zoh(self, delta: float, a: float):
        """Return (Abar, bcoef) with Bbar = bcoef * B for one diagonal entry."""
        ab = ctypes.c_double()
        bc = ctypes.c_double()
        self.lib.oracle_zoh(float(delta), float(a), ctypes.byref(ab), ctypes.byref(bc))
        return ab.value, bc.value

    def selective_scan(self, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                       nthreads: int = 1):
        """Selective scan forward.  Returns (y [B,D,L], h_last [B,D,N])."""
        x, dt, A, Bm, Cm = map(_f64, (x, dt, A, Bm, Cm))
        dt_bias, Dskip, z, h0 = map(_f64, (dt_bias, Dskip, z, h0))
        Bsz, D, L = x.shape
        N = A.shape[1]
        assert dt.shape == x.shape and A.shape == (D, N)
        assert Bm.shape == (Bsz, L, N) and Cm.shape == (Bsz, L, N)
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (Bsz, D, N)
        assert dt_bias is None or dt_bias.shape == (D,)
        assert Dskip is None or Dskip.shape == (D,)
        y = np.empty((Bsz, D, L), dtype=np.float64)
        h_last = np.empty((Bsz, D, N), dtype=np.float64)
        rc = self.lib.oracle_selective_scan_fwd(
            _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
            _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last), Bsz, D, L, N, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_selective_scan_fwd rejected its arguments")
        return y, h_last

    def selective_scan_bwd(self, x, dt, A, Bm, Cm, dout, dt_bias=None, Dskip=None, z=None,
                           h0=None, dh_last=None):
        """Gradients of J = sum(out * dout) (+ sum(h_last * dh_last)) of the
        forward scan.  Returns a dict: dx, ddt, dz (or None), dA, dD, ddt_bias,
        dB, dC, dh0 (or None)."""
        x, dt, A, Bm, Cm, dout = map(_f64, (x, dt, A, Bm, Cm, dout))
        dt_bias, Dskip, z, h0, dh_last = map(_f64, (dt_bias, Dskip, z, h0, dh_last))
        Bsz, D, L = x.shape
        N = A.shape[1]
        g = {"dx": np.empty_like(x), "ddt": np.empty_like(x),
             "dz": np.empty_like(x) if z is not None else None,
             "dA": np.empty((D, N)), "dD": np.empty(D), "ddt_bias": np.empty(D),
             "dB": np.empty((Bsz, L, N)), "dC": np.empty((Bsz, L, N)),
             "dh0": np.empty((Bsz, D, N)) if h0 is not None else None}
        rc = self.lib.oracle_selective_scan_bwd(
            _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
            _ptr(h0), _ptr(dout), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dz"]),
            _ptr(g["dA"]), _ptr(g["dD"]), _ptr(g["ddt_bias"]), _ptr(g["dB"]), _ptr(g["dC"]),
            _ptr(g["dh0"]), Bsz, D, L, N)
        if rc != 0:
            raise ValueError("oracle_selective_scan_bwd rejected its arguments")
        return g

    def ssd_scan(self, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None):
        """Mamba-2 form (one decay per head, B/C per group of heads).
        x, z [B,L,H,P]; dt [B,L,H]; Bm, Cm [B,L,G,N]; A, dt_bias, Dskip [H];
        h0 [B,H,P,N].  Returns (y [B,L,H,P], h_last [B,H,P,N])."""
        x, dt, A, Bm, Cm = map(_f64, (x, dt, A, Bm, Cm))
        dt_bias, Dskip, z, h0 = map(_f64, (dt_bias, Dskip, z, h0))
        Bsz, L, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        assert dt.shape == (Bsz, L, H) and A.shape == (H,)
        assert Bm.shape == (Bsz, L, G, N) and Cm.shape == Bm.shape
        assert z is None or z.shape == x.shape
        assert h0 is None or h0.shape == (Bsz, H, P, N)
        y = np.empty(x.shape, dtype=np.float64)
        h_last = np.empty((Bsz, H, P, N), dtype=np.float64)
        rc = self.lib.oracle_ssd_scan_fwd(
            _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
            _ptr(h0), _ptr(y), _ptr(h_last), Bsz, L, H, P, G, N)
        if rc != 0:
            raise ValueError("oracle_ssd_scan_fwd rejected its arguments")
        return y, h_last

    def selective_scan_reverse(self, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                               nthreads: int = 1):
        """The scan in reversed time (state from step L-1 down to step 0): by
        definition the forward scan of the time-reversed sequences, reversed
        back ("Mamba架构与SSM模型：高效序列建模技术解析" §2, both directions)."""
        flip = lambda a: None if a is None else np.ascontiguousarray(np.flip(np.asarray(a), -1))
        flip_bc = lambda a: np.ascontiguousarray(np.flip(np.asarray(a), -2))
        y, h = self.selective_scan(flip(x), flip(dt), A, flip_bc(Bm), flip_bc(Cm), dt_bias, Dskip,
                                   flip(z), h0, nthreads)
        return flip(y), h

    def conv1d_silu(self, x, w, bias=None, apply_silu: bool = True):
        """Causal depthwise conv1d (+ SiLU).  x [B,D,L], w [D,K] -> [B,D,L]."""
        x, w, bias = _f64(x), _f64(w), _f64(bias)
        Bsz, D, L = x.shape
        K = w.shape[1]
        assert w.shape[0] == D and (bias is None or bias.shape == (D,))
        out = np.empty_like(x)
        rc = self.lib.oracle_conv1d_silu(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), Bsz, D, L,
                                         K, 1 if apply_silu else 0)
        if rc != 0:
            raise ValueError("oracle_conv1d_silu rejected its arguments")
        return out

    def conv1d_update(self, state, x, w, bias=None):
        """One conv step with its state.  state [B,D,K-1] (not modified), x [B,D],
        w [D,K].  Returns (out [B,D], state_new [B,D,K-1])."""
        x, w, bias = _f64(x), _f64(w), _f64(bias)
        Bsz, D = x.shape
        K = w.shape[1]
        state = np.array(state, dtype=np.float64, copy=True, order="C").reshape(Bsz, D, K - 1)
        out = np.empty((Bsz, D), dtype=np.float64)
        rc = self.lib.oracle_conv1d_update(_ptr(state) if K > 1 else None, _ptr(x), _ptr(w),
                                           _ptr(bias), _ptr(out), Bsz, D, K)
        if rc != 0:
            raise ValueError("oracle_conv1d_update rejected its arguments")
        return out, state

    def state_update(self, h, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None):
        """One decode step.  h [B,D,N] (not modified), x/dt/z [B,D], Bm/Cm [B,N].
        Returns (y [B,D], h_new [B,D,N])."""
        h = np.array(h, dtype=np.float64, copy=True, order="C")
        x, dt, A, Bm, Cm = map(_f64, (x, dt, A, Bm, Cm))
        dt_bias, Dskip, z = map(_f64, (dt_bias, Dskip, z))
        Bsz, D, N = h.shape
        assert x.shape == (Bsz, D) and dt.shape == (Bsz, D) and A.shape == (D, N)
        assert Bm.shape == (Bsz, N) and Cm.shape == (Bsz, N)
        y = np.empty((Bsz, D), dtype=np.float64)
        rc = self.lib.oracle_state_update(_ptr(h), _ptr(x), _ptr(dt), _ptr(dt_bias),
                                          _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
                                          _ptr(y), Bsz, D, N)
        if rc != 0:
            raise ValueError("oracle_state_update rejected its arguments")
        return y, h


_default = None


def get() -> Oracle:
    """The oracle built from oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def softplus(v):
    return get().softplus(v)


def silu(v):
    return get().silu(v)


def zoh(delta, a):
    return get().zoh(delta, a)


def selective_scan(*args, **kw):
    return get().selective_scan(*args, **kw)


def conv1d_silu(*args, **kw):
    return get().conv1d_silu(*args, **kw)


def selective_scan_reverse(*args, **kw):
    return get().selective_scan_reverse(*args, **kw)


def state_update(*args, **kw):
    return get().state_update(*args, **kw)


def selective_scan_bwd(*args, **kw):
    return get().selective_scan_bwd(*args, **kw)


def conv1d_update(*args, **kw):
    return get().conv1d_update(*args, **kw)


def ssd_scan(*args, **kw):
    return get().ssd_scan(*args, **kw)
