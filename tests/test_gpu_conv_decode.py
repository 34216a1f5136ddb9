"""GPU parity of mamba_conv1d_silu, the conv -> scan block, and
mamba_selective_state_update (decode) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from scan_check import (STATE_TOL, TOL, assert_within, check_scan_full, dev, host,
                        oracle_conv_full, oracle_state_update_threaded, say)
from selective_state_space_80_amd import workloads as W

pytestmark = pytest.mark.gpu

CONV_TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 7, 8, 100, 1024])
def test_conv_matches_oracle(K, io, L):
    import selective_state_space_80_amd as mamba
    say(f"conv K={K} io={io} L={L}")
    rng = np.random.default_rng(K * 100 + L)
    B, D = 2, 37
    x = rng.standard_normal((B, D, L)).astype(np.float32)
    if io == "bf16":
        x = W.round_bf16(x)
    w = (0.5 * rng.standard_normal((D, K))).astype(np.float32)
    bias = rng.standard_normal(D).astype(np.float32) if K % 2 else None
    out = mamba.conv1d_silu(dev(x, io), dev(w), dev(bias))
    want = oracle.conv1d_silu(x, w, bias)
    assert_within(host(out), want, CONV_TOL[io], "conv")


@pytest.mark.parametrize("case", ["many_rows", "unaligned"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_fallback_layouts(case, io):
    """Rows of whole 16-byte pieces that still take the bounds-checked kernel:
    65537 batch rows (beyond one launch dimension), or input and output that
    start one element past a 16-byte boundary."""
    import torch
    import selective_state_space_80_amd as mamba
    say(f"conv fallback {case} io={io}")
    rng = np.random.default_rng(77)
    B, D, L, K = (65537, 1, 16, 4) if case == "many_rows" else (3, 5, 64, 4)
    x = rng.standard_normal((B, D, L)).astype(np.float32)
    if io == "bf16":
        x = W.round_bf16(x)
    w = (0.5 * rng.standard_normal((D, K))).astype(np.float32)
    bias = rng.standard_normal(D).astype(np.float32)
    xd = dev(x, io)
    if case == "unaligned":
        n = x.size
        buf = torch.zeros(n + 1, dtype=xd.dtype, device="cuda")
        buf[1:].copy_(xd.reshape(-1))
        xd = buf[1:].view(B, D, L)
        obuf = torch.empty(n + 1, dtype=xd.dtype, device="cuda")
        out = obuf[1:].view(B, D, L)
        assert xd.data_ptr() % 16 != 0 and out.data_ptr() % 16 != 0
        mamba.conv1d_silu(xd, dev(w), dev(bias), out=out)
    else:
        out = mamba.conv1d_silu(xd, dev(w), dev(bias))
    want = oracle.conv1d_silu(x, w, bias)
    assert_within(host(out), want, CONV_TOL[io], "conv")


def test_block_workload_every_element():
    """The d_model=768 block (B=2 D=1536 L=8192, fp32): conv1d(k=4)+SiLU, then
    the scan, as two calls at full size; the conv output, every scan output
    and every final state against the oracle (conv, then scan, in fp64)."""
    import selective_state_space_80_amd as mamba
    wl = W.WORKLOADS[1]
    say(f"block {wl.name}: drawing inputs")
    p = W.scan_inputs(wl)
    xr = dev(p["x_raw"])
    xc = mamba.conv1d_silu(xr, dev(p["conv_w"]))
    y, hl = mamba.selective_scan_fwd(xc, dev(p["dt"]), dev(p["A"]), dev(p["Bm"]), dev(p["Cm"]),
                                     dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]),
                                     z=dev(p["z"]), return_last_state=True)
    say("  oracle conv over every channel")
    x_or = oracle_conv_full(p["x_raw"], p["conv_w"])
    e = assert_within(host(xc), x_or, CONV_TOL["f32"], "block conv")
    say(f"  conv: every element compared, max rel err {e:.3e}")
    check_scan_full(y, hl, p, "f32", x=x_or, label="block scan")


@pytest.mark.parametrize("N", [16, 5])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("A_kind", ["structured", "general"])
@pytest.mark.parametrize("stream", [False, True], ids=["plain", "stream_state"])
def test_state_update_matches_oracle(N, io, A_kind, stream):
    import selective_state_space_80_amd as mamba
    say(f"decode step N={N} io={io} A={A_kind} stream_state={stream}")
    rng = np.random.default_rng(N + len(io))
    B, D = 3, 300
    wl = W.DecodeWorkload("t", B, D, N, io, 3, 1, 77)
    init = W.decode_initial(wl)
    if A_kind == "general":
        A = -rng.uniform(0.01, 6, size=(D, N)).astype(np.float32)
        A[:, 0] = 0.0
        init["A"] = A
    h = dev(init["h0"])
    h_or = init["h0"].astype(np.float64)
    for step in range(3):
        s = W.decode_step_inputs(wl, step)
        y = mamba.selective_state_update(h, dev(s["x"], io), dev(s["dt"], io), dev(init["A"]),
                                         dev(s["Bm"], io), dev(s["Cm"], io),
                                         dt_bias=dev(init["dt_bias"]), Dskip=dev(init["Dskip"]),
                                         z=dev(s["z"], io), stream_state=stream)
        yo, h_or = oracle.state_update(h_or, s["x"], s["dt"], init["A"], s["Bm"], s["Cm"],
                                       dt_bias=init["dt_bias"], Dskip=init["Dskip"], z=s["z"])
        assert_within(host(y), yo, TOL[io], f"decode y step {step}")
        assert_within(host(h), h_or, STATE_TOL, f"decode h step {step}")


@pytest.mark.parametrize("opt", ["all_inputs", "no_optional"])
def test_state_update_many_rows(opt):
    """More batch rows than one launch's grid holds (65535: the step is launched
    again for the rest) and D = 20 (the second run of 64 quads of a row is
    partly past its end); with and without the optional inputs."""
    import selective_state_space_80_amd as mamba
    say(f"decode step B=65537 D=20 {opt}")
    B, D, N = 65537, 20, 16
    wl = W.DecodeWorkload("t", B, D, N, "bf16", 1, 1, 78)
    init = W.decode_initial(wl)
    s = W.decode_step_inputs(wl, 0)
    full = opt == "all_inputs"
    h = dev(init["h0"])
    y = mamba.selective_state_update(
        h, dev(s["x"], "bf16"), dev(s["dt"], "bf16"), dev(init["A"]), dev(s["Bm"], "bf16"),
        dev(s["Cm"], "bf16"), dt_bias=dev(init["dt_bias"]) if full else None,
        Dskip=dev(init["Dskip"]) if full else None, z=dev(s["z"], "bf16") if full else None)
    yo, ho = oracle.state_update(init["h0"], s["x"], s["dt"], init["A"], s["Bm"], s["Cm"],
                                 dt_bias=init["dt_bias"] if full else None,
                                 Dskip=init["Dskip"] if full else None,
                                 z=s["z"] if full else None)
    assert_within(host(y), yo, TOL["bf16"], "decode y, many rows")
    assert_within(host(h), ho, STATE_TOL, "decode h, many rows")


def test_decode_steps_equal_scan():
    """L decode steps from h0 give the scan's outputs and final state."""
    import torch
    import selective_state_space_80_amd as mamba
    say("decode == scan")
    B, D, L, N = 2, 70, 40, 16
    p = W.make_scan_inputs(B, D, L, N, "f32", seed=41)
    h0 = np.random.default_rng(2).standard_normal((B, D, N)).astype(np.float32)
    y_scan, h_scan = mamba.selective_scan_fwd(dev(p["x"]), dev(p["dt"]), dev(p["A"]),
                                              dev(p["Bm"]), dev(p["Cm"]), dev(p["dt_bias"]),
                                              dev(p["Dskip"]), dev(p["z"]), dev(h0),
                                              return_last_state=True)
    h = dev(h0)
    ys = []
    for t in range(L):
        ys.append(mamba.selective_state_update(
            h, dev(p["x"][:, :, t]), dev(p["dt"][:, :, t]), dev(p["A"]),
            dev(p["Bm"][:, t]), dev(p["Cm"][:, t]), dev(p["dt_bias"]), dev(p["Dskip"]),
            dev(p["z"][:, :, t])))
    y_dec = torch.stack(ys, dim=2)
    assert_within(host(y_dec), host(y_scan), 5e-5, "decode vs scan y")
    assert_within(host(h), host(h_scan), 5e-5, "decode vs scan state")


@pytest.mark.parametrize("A_kind", ["structured", "general"])
def test_decode_small_steps_1024(A_kind):
    """1024 decode steps with step sizes Δ log-uniform in [1e-5, 1e-4] from a
    given state, which then barely decays: any rounding of a small Δ (the
    softplus near 0) or of a decay within an ulp of 1 accumulates in the state.
    y is compared at every step and h at the end, fp32 I/O."""
    import selective_state_space_80_amd as mamba
    say(f"decode small steps, 1024 steps, A={A_kind}")
    B, D, L, N = 2, 128, 1024, 16
    p = W.make_scan_inputs(B, D, L, N, "f32", seed=43)
    rng = np.random.default_rng(9)
    u = np.exp(rng.uniform(np.log(1e-5), np.log(1e-4), size=D))
    p["dt_bias"] = np.log(np.expm1(u)).astype(np.float32)
    if A_kind == "general":
        p["A"] = -rng.uniform(0.05, 8.0, size=(D, N)).astype(np.float32)
    h0 = rng.standard_normal((B, D, N)).astype(np.float32)
    h = dev(h0)
    h_or = h0.astype(np.float64)
    worst = 0.0
    for t in range(L):
        y = mamba.selective_state_update(
            h, dev(p["x"][:, :, t]), dev(p["dt"][:, :, t]), dev(p["A"]),
            dev(p["Bm"][:, t]), dev(p["Cm"][:, t]), dt_bias=dev(p["dt_bias"]),
            Dskip=dev(p["Dskip"]), z=dev(p["z"][:, :, t]))
        yo, h_or = oracle.state_update(h_or, p["x"][:, :, t], p["dt"][:, :, t], p["A"],
                                       p["Bm"][:, t], p["Cm"][:, t], dt_bias=p["dt_bias"],
                                       Dskip=p["Dskip"], z=p["z"][:, :, t])
        worst = max(worst, assert_within(host(y), yo, TOL["f32"], f"decode y step {t}"))
    eh = assert_within(host(h), h_or, STATE_TOL, "decode h after 1024 steps")
    say(f"  max rel err y {worst:.2e}, h {eh:.2e}")


def test_decode_workload_1024_steps():
    """Decode workload: 1024 steps on the [256, 5120, 16] fp32 state with fresh
    bf16 tokens; every 128 steps, every output and every state element is
    compared with the oracle (which runs every step over every channel)."""
    from concurrent.futures import ThreadPoolExecutor
    import selective_state_space_80_amd as mamba
    wl = W.WORKLOADS[4]
    say(f"decode {wl.name}")
    init = W.decode_initial(wl)
    h = dev(init["h0"])
    A, bias, Dk = dev(init["A"]), dev(init["dt_bias"]), dev(init["Dskip"])
    h_or = init["h0"].astype(np.float64)
    worst_y = worst_h = 0.0
    # the seeded per-step inputs are drawn a few steps ahead on host threads
    with ThreadPoolExecutor(4) as ex:
        ahead = [ex.submit(W.decode_step_inputs, wl, s) for s in range(min(8, wl.steps))]
        for step in range(wl.steps):
            s = ahead[step].result()
            if step + 8 < wl.steps:
                ahead.append(ex.submit(W.decode_step_inputs, wl, step + 8))
            ahead[step] = None
            y = mamba.selective_state_update(h, dev(s["x"], "bf16"), dev(s["dt"], "bf16"), A,
                                             dev(s["Bm"], "bf16"), dev(s["Cm"], "bf16"), bias,
                                             Dk, dev(s["z"], "bf16"))
            yo, h_or = oracle_state_update_threaded(h_or, s["x"], s["dt"], init["A"], s["Bm"],
                                                    s["Cm"], dt_bias=init["dt_bias"],
                                                    Dskip=init["Dskip"], z=s["z"])
            if (step + 1) % wl.check_every == 0:
                e1 = assert_within(host(y), yo, TOL["bf16"], f"decode y step {step + 1}")
                e2 = assert_within(host(h), h_or, STATE_TOL, f"decode h step {step + 1}")
                worst_y, worst_h = max(worst_y, e1), max(worst_h, e2)
                say(f"  step {step + 1}: every element compared ({y.numel()} outputs, "
                    f"{h.numel()} states); max rel err y {e1:.2e} h {e2:.2e}")
    say(f"  decode: max rel err y {worst_y:.3e} (tol {TOL['bf16']}) h {worst_h:.3e} "
        f"(tol {STATE_TOL})")


@pytest.mark.parametrize("conv", [False, True], ids=["state_update", "with_conv"])
def test_stream_state_hint_gives_the_same_bits(conv):
    """MAMBA_STEP_STREAM_STATE is a cache hint: on the full decode workload
    (B=256, D=5120, N=16, bf16 tokens) two steps with it leave the same bits in
    y, h (and the conv window) as two steps without it."""
    import selective_state_space_80_amd as mamba
    wl = W.WORKLOADS[4]
    say(f"stream_state hint, {wl.name}, conv={conv}")
    init = W.decode_initial(wl)
    K = 4
    ci = W.decode_conv_initial(wl, K) if conv else None
    A, bias, Dk = dev(init["A"]), dev(init["dt_bias"]), dev(init["Dskip"])
    outs = {}
    for stream in (False, True):
        h = dev(init["h0"])
        cs = dev(ci["conv_state"], "bf16") if conv else None
        ys = []
        for t in range(2):
            s = W.decode_step_inputs(wl, t)
            x, dt, Bm, Cm, z = (dev(s[k], "bf16") for k in ("x", "dt", "Bm", "Cm", "z"))
            if conv:
                y = mamba.conv1d_selective_state_update(h, cs, x, dev(ci["conv_w"]), dt, A, Bm,
                                                        Cm, dt_bias=bias, Dskip=Dk, z=z,
                                                        stream_state=stream)
            else:
                y = mamba.selective_state_update(h, x, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dk,
                                                 z=z, stream_state=stream)
            ys.append(host(y))
        outs[stream] = (ys, host(h), host(cs) if conv else None)
    (y0, h0, c0), (y1, h1, c1) = outs[False], outs[True]
    for t in range(2):
        assert np.array_equal(y0[t], y1[t]), f"y step {t}"
    assert np.array_equal(h0, h1), "h"
    if conv:
        assert np.array_equal(c0, c1), "conv window"
    say("  y, h" + (", window" if conv else "") + " bit-identical with and without the hint")
