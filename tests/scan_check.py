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


# ---- whole-tensor comparisons at full size ---------------------------------
# The oracle is sequential in time, so every output of a channel costs its
# whole prefix; at full size it runs over channel blocks (bounded host memory)
# with its POSIX threads spread over the host's cores.

def host_threads():
    import os
    return max(1, min(16, os.cpu_count() or 1))


def _block_channels(L, target=1 << 24):
    return max(1, target // max(1, L))


class MaxErr:
    """Running maximum of |got - want| / (1 + |want|) with the tolerance
    asserted on every block (NaN counts as a failure)."""

    def __init__(self, tau, what):
        self.tau, self.what, self.worst, self.n = tau, what, 0.0, 0

    def add(self, got, want, where=""):
        e = assert_within(got, want, self.tau, f"{self.what}{where}")
        self.worst = max(self.worst, e)
        self.n += np.asarray(want).size
        return e


def check_scan_full(y, hl, p, io, x=None, h0=None, reverse=False, z=True, dskip=True, bias=True,
                    label="scan"):
    """Compare every element of y [B,D,L] and h_last [B,D,N] (device tensors)
    with the fp64 oracle on the inputs p (x overrides p['x'], e.g. the
    oracle's conv output).  Returns (max rel err y, max rel err h_last)."""
    xs = p["x"] if x is None else x
    B, D, L = xs.shape
    cb = _block_channels(L)
    ey, eh = MaxErr(TOL[io], f"{label} y"), MaxErr(STATE_TOL, f"{label} h_last")
    run = oracle.selective_scan_reverse if reverse else oracle.selective_scan
    nt = host_threads()
    for b in range(B):
        for d0 in range(0, D, cb):
            d1 = min(D, d0 + cb)
            sl = (slice(b, b + 1), slice(d0, d1))
            yo, ho = run(xs[sl], p["dt"][sl], p["A"][d0:d1], p["Bm"][b:b + 1], p["Cm"][b:b + 1],
                         dt_bias=p["dt_bias"][d0:d1] if bias else None,
                         Dskip=p["Dskip"][d0:d1] if dskip else None,
                         z=p["z"][sl] if z else None,
                         h0=None if h0 is None else h0[sl], nthreads=nt)
            where = f" (batch {b}, channels {d0}..{d1 - 1})"
            ey.add(host(y[b:b + 1, d0:d1]), yo, where)
            if hl is not None:
                eh.add(host(hl[b:b + 1, d0:d1]), ho, where)
    say(f"  {label}: every element compared ({ey.n} outputs, {eh.n} states); max rel err "
        f"y {ey.worst:.3e} (tol {ey.tau}) h_last {eh.worst:.3e} (tol {eh.tau})")
    return ey.worst, eh.worst


def oracle_conv_full(x_raw, w, bias=None):
    """The oracle's conv1d+SiLU of every channel, over channel blocks."""
    B, D, L = x_raw.shape
    out = np.empty((B, D, L), dtype=np.float64)
    cb = _block_channels(L)
    for b in range(B):
        for d0 in range(0, D, cb):
            d1 = min(D, d0 + cb)
            out[b:b + 1, d0:d1] = oracle.conv1d_silu(x_raw[b:b + 1, d0:d1], w[d0:d1],
                                                     None if bias is None else bias[d0:d1])
    return out


def oracle_state_update_threaded(h, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None,
                                 nthreads=None):
    """One oracle decode step over all rows, batch rows split over host
    threads (each row's arithmetic is the oracle's own; ctypes releases the
    GIL while a call runs).  Returns (y [B,D], h_new [B,D,N])."""
    from concurrent.futures import ThreadPoolExecutor
    Bsz = h.shape[0]
    nt = nthreads or host_threads()
    cuts = [Bsz * i // nt for i in range(nt + 1)]
    y = np.empty(x.shape, dtype=np.float64)
    hn = np.empty(h.shape, dtype=np.float64)

    def one(i):
        a, b = cuts[i], cuts[i + 1]
        if a == b:
            return
        y[a:b], hn[a:b] = oracle.state_update(h[a:b], x[a:b], dt[a:b], A, Bm[a:b], Cm[a:b],
                                              dt_bias=dt_bias, Dskip=Dskip,
                                              z=None if z is None else z[a:b])

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(one, range(nt)))
    return y, hn


def oracle_bwd_threaded(x, dt, A, Bm, Cm, dout, dt_bias=None, Dskip=None, z=None, h0=None,
                        dh_last=None, nthreads=None):
    """The oracle's backward over all channels, channel blocks on host threads.
    Per-channel gradients come from the block that holds the channel (every
    batch row, so dA, dD, ddt_bias are complete); dB, dC are sums over
    channels, added up over the blocks in fp64."""
    from concurrent.futures import ThreadPoolExecutor
    Bsz, D, L = x.shape
    nt = nthreads or host_threads()
    cuts = [D * i // nt for i in range(nt + 1)]
    sl3 = lambda a, lo, hi: None if a is None else a[:, lo:hi]
    sl1 = lambda a, lo, hi: None if a is None else a[lo:hi]

    def one(i):
        lo, hi = cuts[i], cuts[i + 1]
        if lo == hi:
            return None
        return lo, hi, oracle.selective_scan_bwd(
            sl3(x, lo, hi), sl3(dt, lo, hi), A[lo:hi], Bm, Cm, sl3(dout, lo, hi),
            dt_bias=sl1(dt_bias, lo, hi), Dskip=sl1(Dskip, lo, hi), z=sl3(z, lo, hi),
            h0=sl3(h0, lo, hi), dh_last=sl3(dh_last, lo, hi))

    with ThreadPoolExecutor(nt) as ex:
        parts = [r for r in ex.map(one, range(nt)) if r is not None]
    g = {"dx": np.empty((Bsz, D, L)), "ddt": np.empty((Bsz, D, L)),
         "dz": np.empty((Bsz, D, L)) if z is not None else None,
         "dA": np.empty(A.shape), "dD": np.empty(D), "ddt_bias": np.empty(D),
         "dB": np.zeros(Bm.shape), "dC": np.zeros(Cm.shape),
         "dh0": np.empty((Bsz, D, A.shape[1])) if h0 is not None else None}
    for lo, hi, gi in parts:
        for k in ("dx", "ddt", "dz", "dh0"):
            if g[k] is not None:
                g[k][:, lo:hi] = gi[k]
        for k in ("dA", "dD", "ddt_bias"):
            g[k][lo:hi] = gi[k]
        g["dB"] += gi["dB"]
        g["dC"] += gi["dC"]
    return g


def oracle_ssd_threaded(x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                        nthreads=None):
    """The oracle's Mamba-2 form over all heads, blocks of whole B/C groups of
    heads on host threads.  Returns (y [B,L,H,P], h_last [B,H,P,N])."""
    from concurrent.futures import ThreadPoolExecutor
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    nt = nthreads or host_threads()
    # units of work: (batch row, group, head block) with head blocks inside a group
    per = max(1, (Bsz * H + nt - 1) // nt)
    units = []
    for b in range(Bsz):
        for g_ in range(G):
            for h0_ in range(g_ * hpg, (g_ + 1) * hpg, per):
                units.append((b, g_, h0_, min((g_ + 1) * hpg, h0_ + per)))
    y = np.empty((Bsz, L, H, P))
    hl = np.empty((Bsz, H, P, N))

    def one(u):
        b, g_, lo, hi = u
        sx = lambda a: None if a is None else a[b:b + 1, :, lo:hi]
        yy, hh = oracle.ssd_scan(sx(x), dt[b:b + 1, :, lo:hi], A[lo:hi],
                                 Bm[b:b + 1, :, g_:g_ + 1], Cm[b:b + 1, :, g_:g_ + 1],
                                 dt_bias=None if dt_bias is None else dt_bias[lo:hi],
                                 Dskip=None if Dskip is None else Dskip[lo:hi], z=sx(z),
                                 h0=None if h0 is None else h0[b:b + 1, lo:hi])
        y[b:b + 1, :, lo:hi] = yy
        hl[b:b + 1, lo:hi] = hh

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(one, units))
    return y, hl
