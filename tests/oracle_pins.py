"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  They check the oracle against things other than itself:
  * the Van Loan block matrix exponential (scipy.linalg.expm) for ZOH
    ("Mamba架构与SSM模型：高效序列建模技术解析", §2.1),
  * a high-accuracy ODE integration (scipy.integrate.solve_ivp) of the
    continuous system the ZOH discretises (same page, §2.1; "Mamba: Linear-Time
    Sequence Modeling with Selective SSMs", section "连续与离散SSM"),
  * the LTI convolution closed form K_k = C Abar^k Bbar and scipy.signal.lfilter
    (same page, section "S4的关键思想": a time-invariant SSM is a 1-D convolution),
  * the DC-gain fixed point h = -B x / A that only exact ZOH preserves,
  * the affine chunk composition behind the block-wise scan with prefix-state
    carry (same page, section "选择性扫描（Selective Scan）要点"),
  * special cases (B = 0, C = 0, step -> infinity, A = 0, saturated gate),
    hand expansions for L <= 3, and a hand-derived rational worked example
    (tests/golden/zoh_ln2_worked_example.txt),
  * numpy.convolve for the causal depthwise conv1d, scipy.special.expit for SiLU,
  * the Mamba-2 form against its structured-matrix (quadratic) form built in
    numpy, and against the selective scan it reduces to when every state of a
    channel shares its head's decay ("Mamba状态空间模型深度解析：挑战Transformer的
    下一代序列建模范式", §4.2).
``tests/test_oracle_mutants.py`` plants mistakes in copies of oracle.c and
checks that at least one pin fails for each of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
from scipy.integrate import solve_ivp
from scipy.linalg import expm
from scipy.signal import lfilter
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    if not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: max excess at flat index {i}: got "
                             f"{a.ravel()[i]!r} want {b.ravel()[i]!r} (err {err.ravel()[i]:.3e})")


def _delta(dt, bias):
    """softplus by the library routine numpy.logaddexp(0, v) = log(1 + e^v)."""
    return np.logaddexp(0.0, np.asarray(dt, dtype=np.float64) + bias)


def _van_loan(a, b, delta):
    """(scipy's expm is accurate to ~1e-13 relative here, so comparisons
    against it use rtol 1e-10.)  Exact ZOH of x' = a x + b u over a step delta, via expm of the
    augmented matrix [[a, b], [0, 0]] * delta.  Returns (Abar, Bbar)."""
    M = np.array([[a * delta, b * delta], [0.0, 0.0]], dtype=np.float64)
    E = expm(M)
    return E[0, 0], E[0, 1]


def pin_softplus(orc):
    for u in np.logspace(-7, 1.5, 40):
        _close(orc.softplus(np.log(np.expm1(u))), u, 1e-13, what="softplus(log(expm1(u)))")
    for v in np.linspace(-60, 60, 97):
        _close(orc.softplus(v), np.logaddexp(0.0, v), 1e-14, 1e-300, what="softplus(v)")
    _close(orc.softplus(0.0), np.log(2.0), 1e-16, what="softplus(0)")


def pin_silu(orc):
    for v in np.linspace(-40, 40, 81):
        _close(orc.silu(v), v * expit(v), 1e-14, 1e-300, what="silu")


def pin_zoh_van_loan(orc):
    rng = np.random.default_rng(11)
    cases = [(a, d) for a in (-7.0, -1.0, -0.013, 0.0, 0.4) for d in (1e-4, 0.02, 0.7, 3.0)]
    cases += [(rng.uniform(-9, 1), rng.uniform(1e-4, 2)) for _ in range(30)]
    for a, d in cases:
        b = 1.7
        Abar, Bbar = _van_loan(a, b, d)
        ab, bc = orc.zoh(d, a)
        _close(ab, Abar, 1e-10, what=f"Abar a={a} d={d}")
        _close(bc * b, Bbar, 1e-10, 1e-300, what=f"Bbar a={a} d={d}")


def pin_scan_single_step_van_loan(orc):
    """Through the scan entry point: one step from h0 with x=1 reads Bbar,
    one step with x=0 and h0=1 reads Abar."""
    rng = np.random.default_rng(12)
    N = 16
    A = np.concatenate([-rng.uniform(0.01, 9, N - 2), [0.0, 0.3]])[None, :]
    bias = np.array([rng.normal()])
    dt = np.array([[[rng.normal()]]])
    Brow = rng.normal(size=(1, 1, N))
    C = rng.normal(size=(1, 1, N))
    delta = _delta(dt[0, 0, 0], bias[0])
    want_A = np.array([_van_loan(A[0, n], Brow[0, 0, n], delta)[0] for n in range(N)])
    want_B = np.array([_van_loan(A[0, n], Brow[0, 0, n], delta)[1] for n in range(N)])
    _, h = orc.selective_scan(np.ones((1, 1, 1)), dt, A, Brow, C, dt_bias=bias)
    _close(h[0, 0], want_B, 1e-10, 1e-300, what="h_last = Bbar")
    _, h = orc.selective_scan(np.zeros((1, 1, 1)), dt, A, Brow, C, dt_bias=bias,
                              h0=np.ones((1, 1, N)))
    _close(h[0, 0], want_A, 1e-10, what="h_last = Abar")


def pin_ode(orc):
    """The discrete states equal the exact solution of h' = a h + b(t) u(t)
    with u and b held constant over each step of length delta_t."""
    rng = np.random.default_rng(13)
    N, L = 3, 12
    A = np.array([[-0.5, -2.0, -7.0]])
    x = rng.normal(size=(1, 1, L))
    dt = rng.normal(0, 0.8, size=(1, 1, L))
    bias = np.array([-0.7])
    Bm = rng.normal(size=(1, L, N))
    h0 = rng.normal(size=(1, 1, N))
    delta = _delta(dt[0, 0], bias[0])
    for n in range(N):
        C = np.zeros((1, L, N))
        C[0, :, n] = 1.0
        y, _ = orc.selective_scan(x, dt, A, Bm, C, dt_bias=bias, h0=h0)
        hn = h0[0, 0, n]
        want = []
        for t in range(L):
            a, b, u = A[0, n], Bm[0, t, n], x[0, 0, t]
            sol = solve_ivp(lambda _s, v: a * v + b * u, (0.0, delta[t]), [hn],
                            method="DOP853", rtol=1e-13, atol=1e-15)
            hn = sol.y[0, -1]
            want.append(hn)
        _close(y[0, 0], np.array(want), 1e-9, 1e-12, what=f"ODE state n={n}")


def pin_dc_gain(orc):
    """Constant x and B: h = -B x / A is a fixed point of exact ZOH for any
    (time-varying) step sequence; an Euler-type Bbar = delta*B would drift."""
    rng = np.random.default_rng(14)
    N, L = 16, 300
    A = -(np.arange(1, N + 1) * 0.37)[None, :]
    x0, Brow = 0.83, rng.normal(size=N)
    x = np.full((1, 1, L), x0)
    Bm = np.tile(Brow, (1, L, 1))
    Cm = rng.normal(size=(1, L, N))
    dt = rng.normal(0, 1.5, size=(1, 1, L))
    h0 = (-Brow * x0 / A[0])[None, None, :]
    y, h = orc.selective_scan(x, dt, A, Bm, Cm, dt_bias=np.array([0.2]),
                              Dskip=np.array([0.5]), h0=h0)
    _close(h[0, 0], h0[0, 0], 1e-12, 1e-15, what="fixed point")
    _close(y[0, 0], Cm[0] @ h0[0, 0] + 0.5 * x0, 1e-11, 1e-14, what="fixed point readout")


def pin_lti_convolution(orc):
    """Constant delta, B, C: y = K * x + D x with K_k = sum_n C_n Abar_n^k Bbar_n;
    also per-state lfilter.  Readout after the update gives K_0 = C.Bbar."""
    rng = np.random.default_rng(15)
    N, L = 16, 200
    A = -rng.uniform(0.05, 4.0, size=(1, N))
    Brow, Crow = rng.normal(size=N), rng.normal(size=N)
    x = rng.normal(size=(1, 1, L))
    bias = np.array([-1.3])
    delta = float(_delta(0.0, bias[0]))
    Ab = np.array([_van_loan(A[0, n], Brow[n], delta)[0] for n in range(N)])
    Bb = np.array([_van_loan(A[0, n], Brow[n], delta)[1] for n in range(N)])
    k = np.arange(L)
    K = (Crow[None, :] * Ab[None, :] ** k[:, None] * Bb[None, :]).sum(1)
    want = np.convolve(x[0, 0], K)[:L] + 0.7 * x[0, 0]
    y, h = orc.selective_scan(x, np.zeros((1, 1, L)), A, np.tile(Brow, (1, L, 1)),
                              np.tile(Crow, (1, L, 1)), dt_bias=bias, Dskip=np.array([0.7]))
    _close(y[0, 0], want, 1e-11, 1e-13, what="LTI convolution")
    hs = np.stack([lfilter([Bb[n]], [1.0, -Ab[n]], x[0, 0]) for n in range(N)], 1)
    _close(h[0, 0], hs[-1], 1e-11, 1e-13, what="lfilter final state")
    _close(y[0, 0], hs @ Crow + 0.7 * x[0, 0], 1e-11, 1e-13, what="lfilter readout")


def _rand_problem(rng, Bsz, D, L, N, gate=True, h0=True):
    p = dict(x=rng.normal(size=(Bsz, D, L)), dt=rng.normal(0, 0.6, size=(Bsz, D, L)),
             A=-rng.uniform(0.1, 3.0, size=(D, N)), Bm=rng.normal(size=(Bsz, L, N)),
             Cm=rng.normal(size=(Bsz, L, N)), dt_bias=rng.normal(-1, 0.5, size=D),
             Dskip=rng.normal(size=D))
    if gate:
        p["z"] = rng.normal(size=(Bsz, D, L))
    if h0:
        p["h0"] = rng.normal(size=(Bsz, D, N))
    return p


def pin_chunked_carry(orc):
    """Block-wise scan: each chunk's map h -> P h + S (P from x=0,h0=1; S from
    h0=0) composed in order reproduces the single sequential run, for every
    chunk size, and re-running each chunk from its carried prefix reproduces y."""
    rng = np.random.default_rng(16)
    L, N = 37, 5
    p = _rand_problem(rng, 1, 1, L, N)
    y_full, h_full = orc.selective_scan(**p)
    for T in range(1, L + 1):
        h = p["h0"][0, 0].copy()
        ys = []
        for s in range(0, L, T):
            e = min(s + T, L)
            sl = dict(p)
            for key in ("x", "dt", "z"):
                sl[key] = p[key][:, :, s:e]
            for key in ("Bm", "Cm"):
                sl[key] = p[key][:, s:e]
            sl["h0"] = np.zeros((1, 1, N))
            _, S = orc.selective_scan(**sl)
            sl_p = dict(sl, x=np.zeros_like(sl["x"]), h0=np.ones((1, 1, N)))
            _, P = orc.selective_scan(**sl_p)
            y_c, _ = orc.selective_scan(**dict(sl, h0=h[None, None, :]))
            ys.append(y_c[0, 0])
            h = P[0, 0] * h + S[0, 0]
        _close(h, h_full[0, 0], 1e-12, 1e-14, what=f"carried state T={T}")
        _close(np.concatenate(ys), y_full[0, 0], 1e-12, 1e-14, what=f"carried y T={T}")


def pin_special_cases(orc):
    rng = np.random.default_rng(17)
    Bsz, D, L, N = 2, 3, 19, 16
    p = _rand_problem(rng, Bsz, D, L, N, h0=False)
    gate = p["z"] * expit(p["z"])
    skip_only = p["Dskip"][None, :, None] * p["x"] * gate
    # B = 0: the state never leaves zero
    y, h = orc.selective_scan(**dict(p, Bm=np.zeros_like(p["Bm"])))
    _close(y, skip_only, 1e-14, 1e-300, what="B=0")
    _close(h, 0 * h, 0, 0, what="B=0 state")
    # C = 0: nothing is read out
    y, _ = orc.selective_scan(**dict(p, Cm=np.zeros_like(p["Cm"])))
    _close(y, skip_only, 1e-14, 1e-300, what="C=0")
    # step -> infinity: Abar -> 0, Bbar -> -B/A, so h_t = -B_t x_t / A
    q = dict(p, dt=np.full_like(p["dt"], 800.0), z=None, Dskip=None)
    y, h = orc.selective_scan(**q)
    hmem = -q["Bm"][:, None, :, :] * q["x"][..., None] / q["A"][None, :, None, :]
    _close(h, hmem[:, :, -1], 1e-12, 1e-14, what="memoryless state")
    _close(y, (hmem * q["Cm"][:, None]).sum(-1), 1e-11, 1e-13, what="memoryless readout")
    # A = 0: Abar = 1, Bbar = delta B, so h is a running sum
    q = dict(p, A=np.zeros_like(p["A"]), z=None, Dskip=None)
    y, h = orc.selective_scan(**q)
    delta = _delta(q["dt"], q["dt_bias"][None, :, None])
    inc = delta[..., None] * q["Bm"][:, None] * q["x"][..., None]
    hs = np.cumsum(inc, axis=2)
    _close(h, hs[:, :, -1], 1e-12, 1e-14, what="A=0 state")
    _close(y, (hs * q["Cm"][:, None]).sum(-1), 1e-11, 1e-13, what="A=0 readout")
    # saturated gate: z*sigmoid(z) = z for z = 60 (to 1e-26)
    y_ng, _ = orc.selective_scan(**dict(p, z=None))
    y_g, _ = orc.selective_scan(**dict(p, z=np.full_like(p["z"], 60.0)))
    _close(y_g, 60.0 * y_ng, 1e-15, 1e-300, what="saturated gate")


def pin_hand_expansions(orc):
    """L=1 with N=16 and L=3 with N=1 written out term by term."""
    rng = np.random.default_rng(18)
    N = 16
    A = -rng.uniform(0.1, 5, size=(1, N))
    x, dt, z = rng.normal(size=3)
    bias, Dv = -0.4, 0.9
    Brow, Crow = rng.normal(size=N), rng.normal(size=N)
    delta = float(_delta(dt, bias))
    Bb = np.array([_van_loan(A[0, n], Brow[n], delta)[1] for n in range(N)])
    want = (np.dot(Crow, Bb) * x + Dv * x) * z * expit(z)
    y, _ = orc.selective_scan(np.full((1, 1, 1), x), np.full((1, 1, 1), dt), A,
                              Brow[None, None, :], Crow[None, None, :],
                              dt_bias=np.array([bias]), Dskip=np.array([Dv]),
                              z=np.full((1, 1, 1), z))
    _close(y[0, 0, 0], want, 1e-10, 1e-13, what="L=1 expansion")
    # L = 3, N = 1, with an initial state
    a = -1.3
    xs, dts, zs = rng.normal(size=3), rng.normal(size=3), rng.normal(size=3)
    Bs, Cs = rng.normal(size=3), rng.normal(size=3)
    h0 = 0.45
    d = _delta(dts, bias)
    Ab = [_van_loan(a, Bs[t], d[t])[0] for t in range(3)]
    Bb = [_van_loan(a, Bs[t], d[t])[1] for t in range(3)]
    h1 = Ab[0] * h0 + Bb[0] * xs[0]
    h2 = Ab[1] * Ab[0] * h0 + Ab[1] * Bb[0] * xs[0] + Bb[1] * xs[1]
    h3 = (Ab[2] * Ab[1] * Ab[0] * h0 + Ab[2] * Ab[1] * Bb[0] * xs[0]
          + Ab[2] * Bb[1] * xs[1] + Bb[2] * xs[2])
    want = np.array([Cs[0] * h1 + Dv * xs[0], Cs[1] * h2 + Dv * xs[1],
                     Cs[2] * h3 + Dv * xs[2]]) * zs * expit(zs)
    y, h = orc.selective_scan(xs[None, None], dts[None, None], np.array([[a]]),
                              Bs[None, :, None], Cs[None, :, None], dt_bias=np.array([bias]),
                              Dskip=np.array([Dv]), z=zs[None, None],
                              h0=np.full((1, 1, 1), h0))
    _close(y[0, 0], want, 1e-10, 1e-13, what="L=3 expansion")
    _close(h[0, 0, 0], h3, 1e-10, 1e-13, what="L=3 final state")


def _parse_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            rows = [[float(Fraction(t)) for t in r.split()] for r in rest.split("|")]
            vals[key] = rows if len(rows) > 1 else rows[0]
    return vals


def pin_golden_ln2(orc):
    g = _parse_golden(os.path.join(GOLDEN, "zoh_ln2_worked_example.txt"))
    N, L = int(g["N"][0]), int(g["L"][0])
    y, h = orc.selective_scan(
        np.array(g["x"]).reshape(1, 1, L), np.array(g["dt"]).reshape(1, 1, L),
        np.array(g["A"]).reshape(1, N), np.array(g["B"]).reshape(1, L, N),
        np.array(g["C"]).reshape(1, L, N), dt_bias=np.array(g["dt_bias"]),
        Dskip=np.array(g["D"]))
    _close(y[0, 0], np.array(g["y"]), 1e-14, what="golden y")
    _close(h[0, 0], np.array(g["h_last"]), 1e-14, what="golden h_last")


def pin_conv(orc):
    rng = np.random.default_rng(19)
    for K in (1, 2, 4, 5):
        Bsz, D, L = 2, 3, 50
        x = rng.normal(size=(Bsz, D, L))
        w = rng.normal(0, 0.5, size=(D, K))
        bias = rng.normal(size=D)
        pre = np.stack([np.stack([np.convolve(x[b, d], w[d, ::-1])[:L] + bias[d]
                                  for d in range(D)]) for b in range(Bsz)])
        _close(orc.conv1d_silu(x, w, bias), pre * expit(pre), 1e-13, 1e-15,
               what=f"conv K={K}")
        _close(orc.conv1d_silu(x, w, None, apply_silu=False), pre - bias[None, :, None],
               1e-13, 1e-15, what=f"conv no-bias K={K}")
    # an impulse returns the taps reversed (causal, zero-padded on the left)
    w = np.array([[0.1, -0.2, 0.3, 0.4]])
    x = np.zeros((1, 1, 8))
    x[0, 0, 0] = 1.0
    out = orc.conv1d_silu(x, w, None, apply_silu=False)
    _close(out[0, 0], [0.4, 0.3, -0.2, 0.1, 0, 0, 0, 0], 0, 0, what="impulse")


def pin_conv_update(orc):
    """Conv steps with a carried window equal numpy.convolve over the whole
    sequence, the carried-in inputs in front (and a first window of zeros is
    the zero padding of the causal conv)."""
    rng = np.random.default_rng(23)
    for K in (1, 2, 4, 6):
        Bsz, D, T = 2, 3, 9
        pre_in = rng.normal(size=(Bsz, D, K - 1))
        xs = rng.normal(size=(Bsz, D, T))
        w = rng.normal(0, 0.5, size=(D, K))
        bias = rng.normal(size=D)
        full = np.concatenate([pre_in, xs], axis=2)
        want = np.stack([np.stack([np.convolve(full[b, d], w[d, ::-1])[K - 1:K - 1 + T] + bias[d]
                                   for d in range(D)]) for b in range(Bsz)])
        want = want * expit(want)
        state = pre_in.copy()
        for t in range(T):
            out, state = orc.conv1d_update(state, xs[:, :, t], w, bias)
            _close(out, want[:, :, t], 1e-13, 1e-15, what=f"conv update K={K} t={t}")
        _close(state, full[:, :, T:], 0, 0, what=f"conv window K={K}")
    # starting from a zero window reproduces the zero-padded conv
    K, T = 4, 6
    x = rng.normal(size=(1, 2, T))
    w = rng.normal(size=(2, K))
    state = np.zeros((1, 2, K - 1))
    got = []
    for t in range(T):
        o, state = orc.conv1d_update(state, x[:, :, t], w)
        got.append(o)
    _close(np.stack(got, axis=2), orc.conv1d_silu(x, w), 1e-14, 1e-15, what="zero window")


def pin_backward_fd(orc):
    """Every gradient of the backward against central finite differences of
    the forward (J = sum(out * dout) + sum(h_last * dh_last)), one input at a
    time along a random direction, with A holding zero, tiny (|Delta A| below
    the series switch) and ordinary entries."""
    rng = np.random.default_rng(31)
    Bsz, D, L, N = 2, 3, 7, 4
    base = {
        "x": rng.normal(size=(Bsz, D, L)), "dt": rng.normal(-0.5, 0.7, size=(Bsz, D, L)),
        "z": rng.normal(size=(Bsz, D, L)), "A": -rng.uniform(0.3, 2.5, size=(D, N)),
        "Bm": rng.normal(size=(Bsz, L, N)), "Cm": rng.normal(size=(Bsz, L, N)),
        "dt_bias": rng.normal(size=D), "Dskip": rng.normal(size=D),
        "h0": rng.normal(size=(Bsz, D, N)),
    }
    base["A"][0, 1] = 0.0
    base["A"][1, 2] = -3e-5
    base["A"][2, 0] = 0.8  # a growing state is still differentiable
    dout = rng.normal(size=(Bsz, D, L))
    dh_last = rng.normal(size=(Bsz, D, N))

    def J(p):
        y, hl = orc.selective_scan(p["x"], p["dt"], p["A"], p["Bm"], p["Cm"], p["dt_bias"],
                                   p["Dskip"], p["z"], p["h0"])
        return float(np.sum(y * dout) + np.sum(hl * dh_last))

    g = orc.selective_scan_bwd(base["x"], base["dt"], base["A"], base["Bm"], base["Cm"], dout,
                               base["dt_bias"], base["Dskip"], base["z"], base["h0"], dh_last)
    names = {"x": "dx", "dt": "ddt", "z": "dz", "A": "dA", "Bm": "dB", "Cm": "dC",
             "dt_bias": "ddt_bias", "Dskip": "dD", "h0": "dh0"}
    eps = 1e-6
    for key, gname in names.items():
        v = rng.normal(size=base[key].shape)
        hi = dict(base, **{key: base[key] + eps * v})
        lo = dict(base, **{key: base[key] - eps * v})
        fd = (J(hi) - J(lo)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        _close(an, fd, 1e-6, 1e-8, what=f"d/d{key}")
    # no gate, no initial state, no final-state gradient: the same with zeros
    g0 = orc.selective_scan_bwd(base["x"], base["dt"], base["A"], base["Bm"], base["Cm"], dout,
                                base["dt_bias"], base["Dskip"])
    assert g0["dz"] is None and g0["dh0"] is None
    v = rng.normal(size=base["x"].shape)

    def J0(xx):
        y, _ = orc.selective_scan(xx, base["dt"], base["A"], base["Bm"], base["Cm"],
                                  base["dt_bias"], base["Dskip"])
        return float(np.sum(y * dout))
    fd = (J0(base["x"] + eps * v) - J0(base["x"] - eps * v)) / (2 * eps)
    _close(float(np.sum(g0["dx"] * v)), fd, 1e-6, 1e-8, what="d/dx without gate")


def pin_reverse(orc):
    """The reversed-time scan (state runs from step L-1 down to 0) against a
    direct backward loop over the exact ZOH step, written here in numpy."""
    rng = np.random.default_rng(29)
    Bsz, D, L, N = 2, 3, 9, 4
    x, z = rng.normal(size=(Bsz, D, L)), rng.normal(size=(Bsz, D, L))
    dt = rng.normal(-1, 0.5, size=(Bsz, D, L))
    A = -rng.uniform(0.2, 3, size=(D, N))
    Bm, Cm = rng.normal(size=(Bsz, L, N)), rng.normal(size=(Bsz, L, N))
    bias, Dv = rng.normal(size=D), rng.normal(size=D)
    h0 = rng.normal(size=(Bsz, D, N))
    y, hl = orc.selective_scan_reverse(x, dt, A, Bm, Cm, bias, Dv, z, h0)
    for b in range(Bsz):
        for d in range(D):
            h = h0[b, d].copy()
            for t in range(L - 1, -1, -1):
                delta = np.log1p(np.exp(dt[b, d, t] + bias[d]))
                a = delta * A[d]
                h = np.exp(a) * h + np.expm1(a) / A[d] * Bm[b, t] * x[b, d, t]
                want = (Cm[b, t] @ h + Dv[d] * x[b, d, t]) * z[b, d, t] * expit(z[b, d, t])
                _close(y[b, d, t], want, 1e-12, 1e-14, what=f"reverse y b={b} d={d} t={t}")
            _close(hl[b, d], h, 1e-12, 1e-14, what="reverse h_last")


def pin_decode_step(orc):
    """One decode step equals the exact ZOH update and gated readout, and L
    steps equal one scan over L."""
    rng = np.random.default_rng(20)
    Bsz, D, N = 3, 4, 16
    h = rng.normal(size=(Bsz, D, N))
    A = -rng.uniform(0.1, 4, size=(D, N))
    x, dt, z = (rng.normal(size=(Bsz, D)) for _ in range(3))
    Bm, Cm = rng.normal(size=(Bsz, N)), rng.normal(size=(Bsz, N))
    bias, Dv = rng.normal(-1, 0.3, size=D), rng.normal(size=D)
    y, hn = orc.state_update(h, x, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dv, z=z)
    for b in range(Bsz):
        for d in range(D):
            delta = float(_delta(dt[b, d], bias[d]))
            Ab = np.array([_van_loan(A[d, n], Bm[b, n], delta)[0] for n in range(N)])
            Bb = np.array([_van_loan(A[d, n], Bm[b, n], delta)[1] for n in range(N)])
            hw = Ab * h[b, d] + Bb * x[b, d]
            _close(hn[b, d], hw, 1e-12, 1e-14, what="decode state")
            want = (Cm[b] @ hw + Dv[d] * x[b, d]) * z[b, d] * expit(z[b, d])
            _close(y[b, d], want, 1e-12, 1e-14, what="decode y")
    L = 9
    p = _rand_problem(rng, Bsz, D, L, N)
    y_scan, h_scan = orc.selective_scan(**p)
    hs = p["h0"]
    for t in range(L):
        yt, hs = orc.state_update(hs, p["x"][:, :, t], p["dt"][:, :, t], p["A"],
                                  p["Bm"][:, t], p["Cm"][:, t], dt_bias=p["dt_bias"],
                                  Dskip=p["Dskip"], z=p["z"][:, :, t])
        _close(yt, y_scan[:, :, t], 1e-13, 1e-15, what=f"decode==scan t={t}")
    _close(hs, h_scan, 1e-13, 1e-15, what="decode==scan state")


def pin_threads(orc):
    rng = np.random.default_rng(21)
    p = _rand_problem(rng, 3, 7, 33, 16)
    y1, h1 = orc.selective_scan(**p, nthreads=1)
    y4, h4 = orc.selective_scan(**p, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4), "thread count changed result"


def _ssd_problem(rng, Bsz, L, H, P, G, N, zero_head=True):
    x = rng.normal(size=(Bsz, L, H, P))
    z = rng.normal(size=(Bsz, L, H, P))
    dt = rng.normal(-0.5, 0.8, size=(Bsz, L, H))
    A = -rng.uniform(0.2, 3.0, size=H)
    if zero_head:
        A[1] = 0.0  # no decay: the ZOH coefficient's limit Δ
    Bm, Cm = rng.normal(size=(Bsz, L, G, N)), rng.normal(size=(Bsz, L, G, N))
    bias, Dv = rng.normal(size=H), rng.normal(size=H)
    h0 = rng.normal(size=(Bsz, H, P, N))
    return x, dt, A, Bm, Cm, bias, Dv, z, h0


def pin_ssd_matrix_form(orc):
    """Mamba-2 form against its structured-matrix (quadratic) form, built here
    in numpy: y_t = sum_{s<=t} (C_t . B_s) exp(sum_{k=s+1..t} Δ_k a) β_s x_s
    + C_t . exp(sum_{k<=t} Δ_k a) h0 + D x_t, gated; β = expm1(Δa)/a (Δ at a = 0)
    ("Mamba状态空间模型深度解析：挑战Transformer的下一代序列建模范式", §4.2:
    the SSM as a structured matrix multiplication)."""
    rng = np.random.default_rng(41)
    Bsz, L, H, P, G, N = 2, 7, 4, 3, 2, 5
    x, dt, A, Bm, Cm, bias, Dv, z, h0 = _ssd_problem(rng, Bsz, L, H, P, G, N)
    y, hl = orc.ssd_scan(x, dt, A, Bm, Cm, bias, Dv, z, h0)
    for b in range(Bsz):
        for h in range(H):
            g = h // (H // G)
            delta = np.log1p(np.exp(dt[b, :, h] + bias[h]))
            ell = delta * A[h]
            beta = delta if A[h] == 0.0 else np.expm1(ell) / A[h]
            cum = np.cumsum(ell)  # sum_{k<=t}
            M = np.zeros((L, L))
            for t in range(L):
                for s_ in range(t + 1):
                    M[t, s_] = (Cm[b, t, g] @ Bm[b, s_, g]) * np.exp(cum[t] - cum[s_]) * beta[s_]
            yy = M @ x[b, :, h, :]                                   # [L, P]
            yy += np.exp(cum)[:, None] * (Cm[b, :, g] @ h0[b, h].T)  # carried state
            yy += Dv[h] * x[b, :, h, :]
            yy *= z[b, :, h, :] * expit(z[b, :, h, :])
            _close(y[b, :, h, :], yy, 1e-12, 1e-12, f"ssd matrix form y b={b} h={h}")
            hh = np.exp(cum[-1]) * h0[b, h]
            for s_ in range(L):
                hh = hh + np.exp(cum[-1] - cum[s_]) * beta[s_] * np.outer(x[b, s_, h], Bm[b, s_, g])
            _close(hl[b, h], hh, 1e-12, 1e-12, f"ssd matrix form h_last b={b} h={h}")


def pin_ssd_reduces_to_scan(orc):
    """With one decay per head, the Mamba-2 form is the selective scan of the
    head's channels with A[d, n] = a_h for every state n and the group's B, C:
    G = 1 is one scan over all H*P channels; G = H is one scan per head."""
    rng = np.random.default_rng(43)
    Bsz, L, H, P, N = 2, 9, 4, 3, 6
    for G in (1, H):
        x, dt, A, Bm, Cm, bias, Dv, z, h0 = _ssd_problem(rng, Bsz, L, H, P, G, N)
        y, hl = orc.ssd_scan(x, dt, A, Bm, Cm, bias, Dv, z, h0)
        for h in range(H):
            g = h // (H // G)
            x1 = np.ascontiguousarray(x[:, :, h, :].transpose(0, 2, 1))      # [B, P, L]
            z1 = np.ascontiguousarray(z[:, :, h, :].transpose(0, 2, 1))
            dt1 = np.repeat(dt[:, None, :, h], P, axis=1)                   # [B, P, L]
            A1 = np.full((P, N), A[h])
            y1, h1 = orc.selective_scan(x1, dt1, A1, np.ascontiguousarray(Bm[:, :, g]),
                                        np.ascontiguousarray(Cm[:, :, g]), np.full(P, bias[h]),
                                        np.full(P, Dv[h]), z1, np.ascontiguousarray(h0[:, h]))
            _close(y[:, :, h, :], y1.transpose(0, 2, 1), 1e-12, 1e-12, f"ssd vs scan y G={G} h={h}")
            _close(hl[:, h], h1, 1e-12, 1e-12, f"ssd vs scan h_last G={G} h={h}")


ALL_PINS = [pin_ssd_matrix_form, pin_ssd_reduces_to_scan, pin_backward_fd, pin_reverse, pin_conv_update, pin_softplus, pin_silu, pin_zoh_van_loan, pin_scan_single_step_van_loan, pin_ode,
            pin_dc_gain, pin_lti_convolution, pin_chunked_carry, pin_special_cases,
            pin_hand_expansions, pin_golden_ln2, pin_conv, pin_decode_step, pin_threads]
