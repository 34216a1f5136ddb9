"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the HIP path through the binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# tolerances: |y_gpu - y_oracle| <= tau * (1 + |y_oracle|)
TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = 1e-4  # fp32 state in both I/O modes


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(io):
    import torch
    return torch.float32 if io == "f32" else torch.bfloat16


def dev(a, io=None, device="cuda"):
    """numpy float32 array -> device tensor (bf16 when io == 'bf16'; exact,
    since the generators already rounded those values)."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_within(got, want, tau, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want) / (1.0 + np.abs(want))
    bad = ~(err <= tau)  # NaN counts as bad
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(np.isnan(err), np.inf, err))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tau={tau}; worst "
                             f"at {i}: got {got[i]!r} want {want[i]!r} (rel {err[i]:.3e})")
    return float(np.nanmax(err)) if err.size else 0.0


def run_scan_gpu(p, io, h0=None, want_last=True, z=True, dskip=True, bias=True):
    import selective_state_space_80_amd as mamba
    x = dev(p["x"], io)
    r = mamba.selective_scan_fwd(
        x, dev(p["dt"], io), dev(p["A"]), dev(p["Bm"], io), dev(p["Cm"], io),
        dt_bias=dev(p["dt_bias"]) if bias else None, Dskip=dev(p["Dskip"]) if dskip else None,
        z=dev(p["z"], io) if z else None, h0=dev(h0), return_last_state=want_last)
    return r


def oracle_scan_rows(p, bs, ds, h0=None, z=True, dskip=True, bias=True):
    """Oracle on the channels bs x ds only (whole sequences)."""
    bs, ds = np.asarray(bs), np.asarray(ds)
    sub = lambda a: a[np.ix_(bs, ds)]
    y, h = oracle.selective_scan(
        sub(p["x"]), sub(p["dt"]), p["A"][ds], p["Bm"][bs], p["Cm"][bs],
        dt_bias=p["dt_bias"][ds] if bias else None, Dskip=p["Dskip"][ds] if dskip else None,
        z=sub(p["z"]) if z else None, h0=None if h0 is None else sub(h0), nthreads=8)
    return y, h


def sample_channels(B, D, k=6, seed=0):
    """Batch rows and channels to check at full size: tile edges, the last
    channel, and a few random ones."""
    rng = np.random.default_rng(seed)
    ds = {0, min(63, D - 1), min(64, D - 1), D - 1, D // 2}
    ds |= set(rng.integers(0, D, size=k).tolist())
    bs = {0, B - 1} | set(rng.integers(0, B, size=2).tolist())
    return sorted(bs), sorted(ds)
