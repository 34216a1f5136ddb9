"""MI355X (gfx950) selective state-space hot path: Python binding.

Thin ctypes marshalling over the C ABI of ``libmamba_amd.so`` (declared in
``include/mamba_amd.h``).  Every step of the computation runs in the HIP
kernels of that library; this module only checks tensor metadata, takes
device pointers and the current HIP stream, and raises on a non-OK status.
There is no CPU fallback: if the library is missing, calls raise.

Entry points (same names as the C ABI, without the ``mamba_`` prefix):
  conv1d_silu(x, w, bias=None, out=None)
  selective_scan_fwd(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                     return_last_state=False, out=None, workspace=None)
  selective_state_update(h, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, out=None)
  selective_scan_fwd_workspace_size(B, D, L, N, dtype)
  conv1d_selective_scan_fwd(x_raw, conv_w, dt, A, Bm, Cm, conv_bias=None,
                            conv_state_in=None, return_conv_state=False, ...)
  conv1d_update(state, x, w, bias=None, out=None)
  selective_scan_bwd(x, dt, A, Bm, Cm, dout, dt_bias=None, Dskip=None, z=None, h0=None,
                     dh_last=None, workspace=None)
  selective_scan_bwd_workspace_size(B, D, L, N, dtype)
  ssd_scan_fwd(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
               return_last_state=False, out=None, h_last=None)
  selective_scan_fwd_noalloc(x, dt, A, Bm, Cm, ..., out=None, h_last=None)
  selective_scan_check(workspace)        the carry's error word (after a sync)
  set_scan_spin_limit(polls)             diagnostic bound of the carry waits
Test helper: set_carry_checks(True) checks the carry after every scan call.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libmamba_amd.so")
ABI_VERSION = 9  # MAMBA_AMD_ABI_VERSION of include/mamba_amd.h that this binding follows

MAMBA_F32 = 0
MAMBA_BF16 = 1
MAMBA_SCAN_REVERSE = 1
MAMBA_SCAN_ACCUMULATE = 2

STATUS_NAMES = {0: "MAMBA_OK", 1: "MAMBA_ERR_NULL", 2: "MAMBA_ERR_SHAPE", 3: "MAMBA_ERR_DTYPE",
                4: "MAMBA_ERR_UNSUPPORTED", 5: "MAMBA_ERR_ALIGN", 6: "MAMBA_ERR_ALIAS",
                7: "MAMBA_ERR_WORKSPACE", 8: "MAMBA_ERR_LAUNCH", 9: "MAMBA_ERR_DEVICE",
                10: "MAMBA_ERR_TIMEOUT"}

# every symbol include/mamba_amd.h declares
EXPORTED = ["mamba_status_string", "mamba_abi_version", "mamba_conv1d_silu",
            "mamba_selective_scan_fwd_workspace_size", "mamba_selective_scan_fwd",
            "mamba_selective_state_update", "mamba_selective_scan_fwd_ex",
            "mamba_conv1d_selective_scan_fwd",
            "mamba_conv1d_update", "mamba_set_scan_timing_events",
            "mamba_selective_scan_bwd_workspace_size", "mamba_selective_scan_bwd",
            "mamba_ssd_scan_fwd", "mamba_conv1d_selective_state_update",
            "mamba_selective_scan_check", "mamba_set_scan_spin_limit",
            "mamba_selective_scan_fwd_noalloc"]

_lib = None


class MambaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load_library(path: str = LIBRARY):
    """Load libmamba_amd.so and declare its signatures (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m selective_state_space_80_amd.build`"
                           " (the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.mamba_status_string.restype = ctypes.c_char_p
    lib.mamba_status_string.argtypes = [I32]
    lib.mamba_abi_version.restype = I32
    lib.mamba_abi_version.argtypes = []
    if lib.mamba_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.mamba_abi_version()}, this binding "
                           f"follows {ABI_VERSION}: rebuild it (`python -m "
                           "selective_state_space_80_amd.build`)")
    lib.mamba_conv1d_silu.restype = I32
    lib.mamba_conv1d_silu.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, P]
    lib.mamba_selective_scan_fwd_workspace_size.restype = SZ
    lib.mamba_selective_scan_fwd_workspace_size.argtypes = [I64, I64, I64, I64, I32]
    lib.mamba_selective_scan_fwd.restype = I32
    lib.mamba_selective_scan_fwd.argtypes = [P] * 12 + [SZ, I64, I64, I64, I64, I32, P]
    lib.mamba_selective_state_update.restype = I32
    lib.mamba_selective_state_update.argtypes = [P] * 10 + [I64, I64, I64, I32, ctypes.c_uint, P]
    lib.mamba_selective_scan_fwd_ex.restype = I32
    lib.mamba_selective_scan_fwd_ex.argtypes = ([P] * 12 + [SZ, I64, I64, I64, I64, I32,
                                                             ctypes.c_uint, P])
    lib.mamba_conv1d_selective_scan_fwd.restype = I32
    lib.mamba_conv1d_selective_scan_fwd.argtypes = ([P, P, P, I64] + [P] * 13 +
                                                    [SZ, I64, I64, I64, I64, I32, P])
    lib.mamba_conv1d_update.restype = I32
    lib.mamba_conv1d_update.argtypes = [P] * 5 + [I64, I64, I64, I32, P]
    lib.mamba_conv1d_selective_state_update.restype = I32
    lib.mamba_conv1d_selective_state_update.argtypes = ([P] * 5 + [I64] + [P] * 8 +
                                                        [I64, I64, I64, I32, ctypes.c_uint, P])
    lib.mamba_selective_scan_bwd_workspace_size.restype = SZ
    lib.mamba_selective_scan_bwd_workspace_size.argtypes = [I64, I64, I64, I64, I32]
    lib.mamba_selective_scan_bwd.restype = I32
    lib.mamba_selective_scan_bwd.argtypes = [P] * 21 + [SZ, I64, I64, I64, I64, I32, P]
    lib.mamba_ssd_scan_fwd.restype = I32
    lib.mamba_ssd_scan_fwd.argtypes = [P] * 11 + [I64] * 6 + [I32, P]
    lib.mamba_set_scan_timing_events.restype = None
    lib.mamba_set_scan_timing_events.argtypes = [P, P]
    lib.mamba_selective_scan_fwd_noalloc.restype = I32
    lib.mamba_selective_scan_fwd_noalloc.argtypes = [P] * 11 + [I64, I64, I64, I64, I32, P]
    lib.mamba_selective_scan_check.restype = I32
    lib.mamba_selective_scan_check.argtypes = [P, SZ, P]
    lib.mamba_set_scan_spin_limit.restype = None
    lib.mamba_set_scan_spin_limit.argtypes = [I32]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().mamba_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(status), "unknown")


def _torch():
    import torch
    return torch


def _io_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MAMBA_F32
    if t.dtype == torch.bfloat16:
        return MAMBA_BF16
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype=None, device=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _raise(st, where):
    if st != 0:
        raise MambaError(st, where)


def conv1d_silu(x, w, bias=None, out=None):
    """Causal depthwise conv1d + SiLU.  x [B,D,L] (f32/bf16), w [D,K] f32,
    bias [D] f32 or None.  Returns out [B,D,L] of x's dtype."""
    torch = _torch()
    lib = load_library()
    B, D, L = x.shape
    K = w.shape[1]
    _check(x, "x", (B, D, L), device=x.device)
    _check(w, "w", (D, K), torch.float32, x.device)
    _check(bias, "bias", (D,), torch.float32, x.device, optional=True)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (B, D, L), x.dtype, x.device)
    st = lib.mamba_conv1d_silu(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), B, D, L, K,
                               _io_dtype(x), _stream(x.device))
    _raise(st, "mamba_conv1d_silu")
    return out


_carry_checks = False


def set_carry_checks(on: bool = True) -> None:
    """After every scan and backward call, wait for the stream and check the
    workspace's carry error word (raises MambaError with MAMBA_ERR_TIMEOUT).
    Each check synchronizes, so this is for tests, not for timed runs."""
    global _carry_checks
    _carry_checks = bool(on)


def selective_scan_check(workspace) -> None:
    """Wait for the workspace's stream, then raise MambaError(MAMBA_ERR_TIMEOUT)
    if a carry wait of the calls that last used it gave up (their affected
    outputs are NaN)."""
    st = load_library().mamba_selective_scan_check(_ptr(workspace), workspace.numel(),
                                                   _stream(workspace.device))
    _raise(st, "mamba_selective_scan_check")


def set_scan_spin_limit(polls: int) -> None:
    """Diagnostic: polls before a carry wait of later scans gives up (< 0: the
    default).  0 makes any wait not met at once give up, for failure-path tests."""
    load_library().mamba_set_scan_spin_limit(int(polls))


def _after_scan(workspace, need):
    # a check synchronizes, which a stream under graph capture cannot do
    if _carry_checks and need >= 256 and not _torch().cuda.is_current_stream_capturing():
        selective_scan_check(workspace)


def selective_scan_fwd_workspace_size(B, D, L, N, dtype=None) -> int:
    io = MAMBA_F32 if dtype is None else _io_dtype(_torch().empty(0, dtype=dtype))
    return int(load_library().mamba_selective_scan_fwd_workspace_size(B, D, L, N, io))


def selective_scan_fwd(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                       return_last_state=False, out=None, workspace=None, h_last=None,
                       reverse=False, accumulate=False):
    """Fused selective-scan forward.  x, dt, z [B,D,L]; Bm, Cm [B,L,N] (all of
    one dtype, f32 or bf16); A [D,N], dt_bias [D], Dskip [D], h0 [B,D,N] f32.
    Returns y [B,D,L] (x's dtype), and h_last [B,D,N] f32 if return_last_state.
    reverse: scan from step L-1 down to 0; accumulate: add into `out`."""
    torch = _torch()
    lib = load_library()
    B, D, L = x.shape
    N = A.shape[1]
    dev, io_t = x.device, x.dtype
    _check(x, "x", (B, D, L), io_t, dev)
    _check(dt, "dt", (B, D, L), io_t, dev)
    _check(z, "z", (B, D, L), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, L, N), io_t, dev)
    _check(Cm, "Cm", (B, L, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    _check(h0, "h0", (B, D, N), torch.float32, dev, optional=True)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs `out` (the tensor added to)")
        out = torch.empty_like(x)
    _check(out, "out", (B, D, L), io_t, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (B, D, N), torch.float32, dev, optional=True)
    io = _io_dtype(x)
    need = int(lib.mamba_selective_scan_fwd_workspace_size(B, D, L, N, io))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    flags = (MAMBA_SCAN_REVERSE if reverse else 0) | (MAMBA_SCAN_ACCUMULATE if accumulate else 0)
    if flags:
        st = lib.mamba_selective_scan_fwd_ex(
            _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
            _ptr(h0), _ptr(out), _ptr(h_last), _ptr(workspace), workspace.numel(), B, D, L, N, io,
            flags, _stream(dev))
        _raise(st, "mamba_selective_scan_fwd_ex")
    else:
        st = lib.mamba_selective_scan_fwd(
            _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
            _ptr(h0), _ptr(out), _ptr(h_last), _ptr(workspace), workspace.numel(), B, D, L, N,
            io, _stream(dev))
        _raise(st, "mamba_selective_scan_fwd")
    _after_scan(workspace, need)
    if return_last_state:
        return out, h_last
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MAMBA_NOALLOC_SCRATCH_BYTES of include/mamba_amd.h


def selective_scan_fwd_noalloc(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                               out=None, h_last=None):
    """mamba_selective_scan_fwd_noalloc: the scan with the library's own scratch
    in place of a workspace (the C call allocates nothing; `out` / `h_last`
    given by the caller keep this wrapper allocation-free too).  Shapes whose
    workspace exceeds NOALLOC_SCRATCH_BYTES raise MAMBA_ERR_WORKSPACE.
    Returns out, or (out, h_last) when h_last is given."""
    torch = _torch()
    lib = load_library()
    B, D, L = x.shape
    N = A.shape[1]
    dev, io_t = x.device, x.dtype
    _check(x, "x", (B, D, L), io_t, dev)
    _check(dt, "dt", (B, D, L), io_t, dev)
    _check(z, "z", (B, D, L), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, L, N), io_t, dev)
    _check(Cm, "Cm", (B, L, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    _check(h0, "h0", (B, D, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (B, D, L), io_t, dev)
    _check(h_last, "h_last", (B, D, N), torch.float32, dev, optional=True)
    st = lib.mamba_selective_scan_fwd_noalloc(
        _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
        _ptr(h0), _ptr(out), _ptr(h_last), B, D, L, N, _io_dtype(x), _stream(dev))
    _raise(st, "mamba_selective_scan_fwd_noalloc")
    return (out, h_last) if h_last is not None else out


def conv1d_selective_scan_fwd(x_raw, conv_w, dt, A, Bm, Cm, conv_bias=None, conv_state_in=None,
                              return_conv_state=False, conv_state_out=None, dt_bias=None,
                              Dskip=None, z=None, h0=None, return_last_state=False, out=None,
                              workspace=None, h_last=None):
    """conv1d (K <= 4 taps) + SiLU fused into the selective scan.  x_raw [B,D,L]
    (f32/bf16) is the raw block input; conv_w [D,K], conv_bias [D] f32;
    conv_state_in / conv_state_out [B,D,K-1] of x_raw's dtype (the raw inputs
    before t = 0 / of the last K-1 steps; out may be the same tensor as in).
    Other arguments as for selective_scan_fwd.  Returns y, then h_last if
    return_last_state, then the conv state if return_conv_state."""
    torch = _torch()
    lib = load_library()
    B, D, L = x_raw.shape
    N = A.shape[1]
    K = conv_w.shape[1]
    dev, io_t = x_raw.device, x_raw.dtype
    _check(x_raw, "x_raw", (B, D, L), io_t, dev)
    _check(conv_w, "conv_w", (D, K), torch.float32, dev)
    _check(conv_bias, "conv_bias", (D,), torch.float32, dev, optional=True)
    _check(conv_state_in, "conv_state_in", (B, D, K - 1), io_t, dev, optional=True)
    _check(dt, "dt", (B, D, L), io_t, dev)
    _check(z, "z", (B, D, L), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, L, N), io_t, dev)
    _check(Cm, "Cm", (B, L, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    _check(h0, "h0", (B, D, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty_like(x_raw)
    _check(out, "out", (B, D, L), io_t, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (B, D, N), torch.float32, dev, optional=True)
    if return_conv_state and conv_state_out is None:
        conv_state_out = torch.empty((B, D, K - 1), dtype=io_t, device=dev)
    _check(conv_state_out, "conv_state_out", (B, D, K - 1), io_t, dev, optional=True)
    io = _io_dtype(x_raw)
    need = int(lib.mamba_selective_scan_fwd_workspace_size(B, D, L, N, io))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mamba_conv1d_selective_scan_fwd(
        _ptr(x_raw), _ptr(conv_w), _ptr(conv_bias), K, _ptr(conv_state_in), _ptr(conv_state_out),
        _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0),
        _ptr(out), _ptr(h_last), _ptr(workspace), workspace.numel(), B, D, L, N, io,
        _stream(dev))
    _raise(st, "mamba_conv1d_selective_scan_fwd")
    _after_scan(workspace, need)
    res = [out]
    if return_last_state:
        res.append(h_last)
    if return_conv_state:
        res.append(conv_state_out)
    return res[0] if len(res) == 1 else tuple(res)


def conv1d_update(state, x, w, bias=None, out=None):
    """One decode step of the conv front end.  state [B,D,K-1] (x's dtype) is
    updated in place; x [B,D] f32/bf16; w [D,K], bias [D] f32.  Returns out
    [B,D] = SiLU(conv) of x's dtype."""
    torch = _torch()
    lib = load_library()
    B, D = x.shape
    K = w.shape[1]
    dev, io_t = x.device, x.dtype
    _check(x, "x", (B, D), io_t, dev)
    _check(w, "w", (D, K), torch.float32, dev)
    _check(bias, "bias", (D,), torch.float32, dev, optional=True)
    _check(state, "state", (B, D, K - 1), io_t, dev, optional=(K == 1))
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (B, D), io_t, dev)
    st = lib.mamba_conv1d_update(_ptr(state), _ptr(x), _ptr(w), _ptr(bias), _ptr(out), B, D, K,
                                 _io_dtype(x), _stream(dev))
    _raise(st, "mamba_conv1d_update")
    return out


STEP_STREAM_STATE = 1  # MAMBA_STEP_STREAM_STATE


def _step_flags(stream_state):
    return STEP_STREAM_STATE if stream_state else 0


def selective_state_update(h, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, out=None,
                           stream_state=False):
    """One decode step.  h [B,D,N] f32 is updated in place; x, dt, z [B,D] and
    Bm, Cm [B,N] share one dtype (f32/bf16).  Returns y [B,D] of that dtype.
    stream_state: h is loaded and stored with nontemporal hints (the same
    results), for a state that leaves the caches before its next step anyway."""
    torch = _torch()
    lib = load_library()
    B, D, N = h.shape
    dev, io_t = h.device, x.dtype
    _check(h, "h", (B, D, N), torch.float32, dev)
    _check(x, "x", (B, D), io_t, dev)
    _check(dt, "dt", (B, D), io_t, dev)
    _check(z, "z", (B, D), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, N), io_t, dev)
    _check(Cm, "Cm", (B, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (B, D), io_t, dev)
    st = lib.mamba_selective_state_update(
        _ptr(h), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
        _ptr(z), _ptr(out), B, D, N, _io_dtype(x), _step_flags(stream_state), _stream(dev))
    _raise(st, "mamba_selective_state_update")
    return out


def conv1d_selective_state_update(h, conv_state, x_raw, conv_w, dt, A, Bm, Cm, conv_bias=None,
                                  dt_bias=None, Dskip=None, z=None, out=None, stream_state=False):
    """The block's decode step in one kernel: the conv front end's step on the
    raw input x_raw [B,D] (conv_state [B,D,K-1] of x_raw's dtype, updated in
    place; conv_w [D,K] f32 with K <= 4, conv_bias [D] f32), feeding the state
    update of h [B,D,N] f32 (in place).  Other arguments as for
    selective_state_update.  Returns y [B,D] of x_raw's dtype."""
    torch = _torch()
    lib = load_library()
    B, D, N = h.shape
    K = conv_w.shape[1]
    dev, io_t = h.device, x_raw.dtype
    _check(h, "h", (B, D, N), torch.float32, dev)
    _check(conv_state, "conv_state", (B, D, K - 1), io_t, dev, optional=K == 1)
    _check(x_raw, "x_raw", (B, D), io_t, dev)
    _check(conv_w, "conv_w", (D, K), torch.float32, dev)
    _check(conv_bias, "conv_bias", (D,), torch.float32, dev, optional=True)
    _check(dt, "dt", (B, D), io_t, dev)
    _check(z, "z", (B, D), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, N), io_t, dev)
    _check(Cm, "Cm", (B, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty_like(x_raw)
    _check(out, "out", (B, D), io_t, dev)
    st = lib.mamba_conv1d_selective_state_update(
        _ptr(h), _ptr(conv_state), _ptr(x_raw), _ptr(conv_w), _ptr(conv_bias), K, _ptr(dt),
        _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(out), B, D, N,
        _io_dtype(x_raw), _step_flags(stream_state), _stream(dev))
    _raise(st, "mamba_conv1d_selective_state_update")
    return out


def selective_scan_bwd_workspace_size(B, D, L, N, dtype=None) -> int:
    io = MAMBA_F32 if dtype is None else _io_dtype(_torch().empty(0, dtype=dtype))
    return int(load_library().mamba_selective_scan_bwd_workspace_size(B, D, L, N, io))


def selective_scan_bwd(x, dt, A, Bm, Cm, dout, dt_bias=None, Dskip=None, z=None, h0=None,
                       dh_last=None, workspace=None):
    """Backward pass of selective_scan_fwd: gradients of sum(out * dout)
    (+ sum(h_last * dh_last)) with the forward states recomputed.  Inputs as
    for selective_scan_fwd; dout [B,D,L] of x's dtype; dh_last [B,D,N] f32 or
    None.  Returns a dict: dx, ddt, dz (None without z) of x's dtype and
    shape; dA [D,N], dB, dC [B,L,N], dD, ddt_bias [D], dh0 [B,D,N], all f32."""
    torch = _torch()
    lib = load_library()
    B, D, L = x.shape
    N = A.shape[1]
    dev, io_t = x.device, x.dtype
    _check(x, "x", (B, D, L), io_t, dev)
    _check(dt, "dt", (B, D, L), io_t, dev)
    _check(z, "z", (B, D, L), io_t, dev, optional=True)
    _check(dout, "dout", (B, D, L), io_t, dev)
    _check(Bm, "Bm", (B, L, N), io_t, dev)
    _check(Cm, "Cm", (B, L, N), io_t, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(dt_bias, "dt_bias", (D,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (D,), torch.float32, dev, optional=True)
    _check(h0, "h0", (B, D, N), torch.float32, dev, optional=True)
    _check(dh_last, "dh_last", (B, D, N), torch.float32, dev, optional=True)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty_like(x), "ddt": torch.empty_like(x),
         "dz": torch.empty_like(x) if z is not None else None,
         "dA": torch.empty((D, N), **f32), "dB": torch.empty((B, L, N), **f32),
         "dC": torch.empty((B, L, N), **f32), "dD": torch.empty((D,), **f32),
         "ddt_bias": torch.empty((D,), **f32), "dh0": torch.empty((B, D, N), **f32)}
    io = _io_dtype(x)
    need = int(lib.mamba_selective_scan_bwd_workspace_size(B, D, L, N, io))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mamba_selective_scan_bwd(
        _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
        _ptr(h0), _ptr(dout), _ptr(dh_last), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]),
        _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]),
        _ptr(g["dh0"]), _ptr(workspace), workspace.numel(), B, D, L, N, io, _stream(dev))
    _raise(st, "mamba_selective_scan_bwd")
    _after_scan(workspace, need)
    return g


def ssd_scan_fwd(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                 return_last_state=False, out=None, h_last=None):
    """Mamba-2 form of the scan (one decay per head, B/C per group of heads) on
    the matrix cores.  x, z [B,L,H,P], dt [B,L,H], Bm, Cm [B,L,G,N] bf16;
    A, dt_bias, Dskip [H] f32; h0 [B,H,P,N] f32.  Returns y [B,L,H,P] bf16,
    and h_last [B,H,P,N] f32 if return_last_state."""
    torch = _torch()
    lib = load_library()
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev, io_t = x.device, x.dtype
    _check(x, "x", (B, L, H, P), io_t, dev)
    _check(dt, "dt", (B, L, H), io_t, dev)
    _check(z, "z", (B, L, H, P), io_t, dev, optional=True)
    _check(Bm, "Bm", (B, L, G, N), io_t, dev)
    _check(Cm, "Cm", (B, L, G, N), io_t, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev, optional=True)
    _check(Dskip, "Dskip", (H,), torch.float32, dev, optional=True)
    _check(h0, "h0", (B, H, P, N), torch.float32, dev, optional=True)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (B, L, H, P), io_t, dev)
    if return_last_state and h_last is None:
        h_last = torch.empty((B, H, P, N), dtype=torch.float32, device=dev)
    _check(h_last, "h_last", (B, H, P, N), torch.float32, dev, optional=True)
    st = lib.mamba_ssd_scan_fwd(
        _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z),
        _ptr(h0), _ptr(out), _ptr(h_last), B, L, H, P, G, N, _io_dtype(x), _stream(dev))
    _raise(st, "mamba_ssd_scan_fwd")
    if return_last_state:
        return out, h_last
    return out


def set_scan_timing_events_raw(start=None, stop=None):
    """Have later scan calls from this thread record the raw hipEvent_t
    handles `start` / `stop` (ctypes.c_void_p) around their main kernel, on the
    call's stream.  None, None turns it off."""
    lib = load_library()
    if start is None or stop is None:
        lib.mamba_set_scan_timing_events(None, None)
    else:
        lib.mamba_set_scan_timing_events(start, stop)
