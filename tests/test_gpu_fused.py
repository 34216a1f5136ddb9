"""GPU parity of the fused front end (mamba_conv1d_selective_scan_fwd) and the
decode conv step (mamba_conv1d_update) against the fp64 oracle: conv1d+SiLU
over the carried-in raw inputs followed by the scan, and the windowed conv
step."""
import numpy as np
import pytest

import oracle
from scan_check import (STATE_TOL, TOL, assert_within, check_scan_full, dev, host,
                        oracle_conv_full, say)
from selective_state_space_80_amd import workloads as W

pytestmark = pytest.mark.gpu

CONV_TOL = {"f32": 1e-5, "bf16": 1e-2}


def make_inputs(B, D, L, N, K, io, seed, with_state=True, with_bias=True):
    p = W.make_scan_inputs(B, D, L, N, io, seed)
    rng = np.random.default_rng(seed + 7)
    p["x_raw"] = p["x"]
    p["conv_w"] = (0.5 * rng.standard_normal((D, K))).astype(np.float32)
    p["conv_b"] = rng.standard_normal(D).astype(np.float32) if with_bias else None
    cs = rng.standard_normal((B, D, K - 1)).astype(np.float32) if with_state else None
    if cs is not None and io == "bf16":
        cs = W.round_bf16(cs)
    p["conv_state"] = cs
    return p


def oracle_conv_front(x_raw, w, bias, state):
    """conv1d+SiLU of the sequence with the carried-in raw inputs in front."""
    B, D, L = x_raw.shape
    K = w.shape[1]
    pre = np.zeros((B, D, K - 1)) if state is None else np.asarray(state, np.float64)
    full = np.concatenate([pre, np.asarray(x_raw, np.float64)], axis=2)
    return oracle.conv1d_silu(full, w, bias)[:, :, K - 1:], full[:, :, full.shape[2] - (K - 1):]


def run_fused(p, io, h0=None, conv_state_in="from_p", **kw):
    import selective_state_space_80_amd as mamba
    cs = p["conv_state"] if conv_state_in == "from_p" else conv_state_in
    return mamba.conv1d_selective_scan_fwd(
        dev(p["x_raw"], io), dev(p["conv_w"]), dev(p["dt"], io), dev(p["A"]), dev(p["Bm"], io),
        dev(p["Cm"], io), conv_bias=dev(p["conv_b"]), conv_state_in=dev(cs, io),
        dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]), z=dev(p["z"], io), h0=dev(h0),
        return_last_state=True, return_conv_state=True, **kw)


SHAPES = [(1, 64, 256, 16), (2, 100, 300, 16), (1, 37, 33, 7), (2, 64, 129, 16),
          (1, 130, 2100, 16), (1, 64, 3, 16), (1, 64, 1, 4), (2, 100, 384, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("K", [4, 3, 2, 1])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fused_matches_oracle(shape, K, io):
    B, D, L, N = shape
    with_state = (L + K) % 2 == 0
    say(f"fused shape={shape} K={K} io={io} state_in={with_state}")
    p = make_inputs(B, D, L, N, K, io, seed=L * 10 + K, with_state=with_state,
                    with_bias=K != 2)
    h0 = np.random.default_rng(L).standard_normal((B, D, N)).astype(np.float32)
    y, hl, cs = run_fused(p, io, h0=h0)
    xc, cs_want = oracle_conv_front(p["x_raw"], p["conv_w"], p["conv_b"], p["conv_state"])
    yo, ho = oracle.selective_scan(xc, p["dt"], p["A"], p["Bm"], p["Cm"], dt_bias=p["dt_bias"],
                                   Dskip=p["Dskip"], z=p["z"], h0=h0, nthreads=8)
    assert_within(host(y), yo, TOL[io], "fused y")
    assert_within(host(hl), ho, STATE_TOL, "fused h_last")
    assert np.array_equal(host(cs), cs_want), "conv state out is not the last K-1 raw inputs"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fused_split_call_then_decode(io):
    """A prefill in two fused calls (conv state and h carried over), then
    decode steps (conv update + state update), equal the oracle over the whole
    sequence."""
    import selective_state_space_80_amd as mamba
    B, D, N, K = 2, 96, 16, 4
    L1, L2, T = 200, 77, 5
    say(f"fused split + decode io={io}")
    p = make_inputs(B, D, L1 + L2 + T, N, K, io, seed=5, with_state=False)
    sl = lambda a, lo, hi: np.ascontiguousarray(a[..., lo:hi])
    part = lambda lo, hi: dict(p, x_raw=sl(p["x_raw"], lo, hi), dt=sl(p["dt"], lo, hi),
                               z=sl(p["z"], lo, hi),
                               Bm=np.ascontiguousarray(p["Bm"][:, lo:hi]),
                               Cm=np.ascontiguousarray(p["Cm"][:, lo:hi]))
    y1, h1, cs1 = run_fused(part(0, L1), io, conv_state_in=None)
    import torch
    tdt = torch.float32 if io == "f32" else torch.bfloat16
    y2, h2, cs2 = mamba.conv1d_selective_scan_fwd(
        dev(part(L1, L1 + L2)["x_raw"], io), dev(p["conv_w"]), dev(part(L1, L1 + L2)["dt"], io),
        dev(p["A"]), dev(part(L1, L1 + L2)["Bm"], io), dev(part(L1, L1 + L2)["Cm"], io),
        conv_bias=dev(p["conv_b"]), conv_state_in=cs1, dt_bias=dev(p["dt_bias"]),
        Dskip=dev(p["Dskip"]), z=dev(part(L1, L1 + L2)["z"], io), h0=h1,
        return_last_state=True, return_conv_state=True)
    assert cs2.dtype == tdt
    h, cs = h2, cs2
    ys = [host(y1), host(y2)]
    for t in range(L1 + L2, L1 + L2 + T):
        xt = dev(np.ascontiguousarray(p["x_raw"][:, :, t]), io)
        xc = mamba.conv1d_update(cs, xt, dev(p["conv_w"]), dev(p["conv_b"]))
        yt = mamba.selective_state_update(
            h, xc, dev(np.ascontiguousarray(p["dt"][:, :, t]), io), dev(p["A"]),
            dev(np.ascontiguousarray(p["Bm"][:, t]), io), dev(np.ascontiguousarray(p["Cm"][:, t]), io),
            dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]),
            z=dev(np.ascontiguousarray(p["z"][:, :, t]), io))
        ys.append(host(yt)[:, :, None])
    xc_all, _ = oracle_conv_front(p["x_raw"], p["conv_w"], p["conv_b"], None)
    if io == "bf16":
        # the decode steps take the conv output through a bf16 tensor
        xc_all[:, :, L1 + L2:] = W.round_bf16(xc_all[:, :, L1 + L2:].astype(np.float32))
    yo, ho = oracle.selective_scan(xc_all, p["dt"], p["A"], p["Bm"], p["Cm"],
                                   dt_bias=p["dt_bias"], Dskip=p["Dskip"], z=p["z"], nthreads=8)
    assert_within(np.concatenate(ys, axis=2), yo, TOL[io], "prefill + decode y")
    # bf16: the decode steps' conv outputs pass through bf16, where the kernel's
    # and the oracle's values can round to neighbouring bf16 numbers
    assert_within(host(h), ho, STATE_TOL if io == "f32" else 2e-3, "prefill + decode h")


def test_fused_empty_sequence_passes_states_through():
    import torch
    import selective_state_space_80_amd as mamba
    B, D, N, K = 2, 70, 16, 4
    rng = np.random.default_rng(3)
    A = dev(-np.tile(np.arange(1, N + 1, dtype=np.float32), (D, 1)))
    e = lambda *s: torch.empty(s, device="cuda")
    cs_in = dev(rng.standard_normal((B, D, K - 1)).astype(np.float32))
    h0 = dev(rng.standard_normal((B, D, N)).astype(np.float32))
    y, hl, cs = mamba.conv1d_selective_scan_fwd(
        e(B, D, 0), dev(rng.standard_normal((D, K)).astype(np.float32)), e(B, D, 0), A,
        e(B, 0, N), e(B, 0, N), conv_state_in=cs_in, h0=h0, return_last_state=True,
        return_conv_state=True)
    torch.cuda.synchronize()
    assert torch.equal(hl, h0) and torch.equal(cs, cs_in)
    # in place: conv state in and out the same tensor
    st = cs_in.clone()
    mamba.conv1d_selective_scan_fwd(e(B, D, 0), dev(np.ones((D, K), np.float32)), e(B, D, 0),
                                    A, e(B, 0, N), e(B, 0, N), conv_state_in=st,
                                    conv_state_out=st)
    torch.cuda.synchronize()
    assert torch.equal(st, cs_in)


@pytest.mark.parametrize("L", [1, 2, 5, 40])
def test_fused_conv_state_in_place(L):
    """conv_state_out may be the conv_state_in tensor itself."""
    import torch
    B, D, N, K = 1, 64, 16, 4
    say(f"fused in-place conv state L={L}")
    p = make_inputs(B, D, L, N, K, "f32", seed=11 + L)
    st = dev(p["conv_state"])
    _, _, cs_sep = run_fused(p, "f32")
    import selective_state_space_80_amd as mamba
    mamba.conv1d_selective_scan_fwd(
        dev(p["x_raw"]), dev(p["conv_w"]), dev(p["dt"]), dev(p["A"]), dev(p["Bm"]),
        dev(p["Cm"]), conv_bias=dev(p["conv_b"]), conv_state_in=st, conv_state_out=st,
        dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]), z=dev(p["z"]))
    torch.cuda.synchronize()
    _, want = oracle_conv_front(p["x_raw"], p["conv_w"], p["conv_b"], p["conv_state"])
    assert np.array_equal(host(st), want) and np.array_equal(host(cs_sep), want)


# D = 320 takes the 16-byte piece kernel, D = 333 the per-channel one
@pytest.mark.parametrize("D", [320, 333])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_update_matches_oracle(K, io, D):
    import selective_state_space_80_amd as mamba
    say(f"conv update K={K} io={io} D={D}")
    rng = np.random.default_rng(40 + K)
    B, T = 3, 6
    w = (0.5 * rng.standard_normal((D, K))).astype(np.float32)
    bias = rng.standard_normal(D).astype(np.float32) if K != 2 else None
    st0 = rng.standard_normal((B, D, K - 1)).astype(np.float32)
    xs = rng.standard_normal((B, D, T)).astype(np.float32)
    if io == "bf16":
        st0, xs = W.round_bf16(st0), W.round_bf16(xs)
    st = dev(st0, io) if K > 1 else None
    st_or = st0.astype(np.float64)
    for t in range(T):
        out = mamba.conv1d_update(st, dev(np.ascontiguousarray(xs[:, :, t]), io), dev(w),
                                  dev(bias))
        want, st_or = oracle.conv1d_update(st_or, xs[:, :, t], w, bias)
        assert_within(host(out), want, CONV_TOL[io], f"conv update t={t}")
        if K > 1:
            assert np.array_equal(host(st), st_or), "conv window"


@pytest.mark.parametrize("D", [8, 3])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_update_many_rows(io, D):
    """65537 batch rows: more than one launch covers (the rows go in slices of
    65535), two steps, every output and window checked; D = 8 takes the
    16-byte piece kernel, D = 3 the per-channel one."""
    import selective_state_space_80_amd as mamba
    say(f"conv update many rows io={io} D={D}")
    rng = np.random.default_rng(48)
    B, K = 65537, 4
    w = (0.5 * rng.standard_normal((D, K))).astype(np.float32)
    bias = rng.standard_normal(D).astype(np.float32)
    st0 = rng.standard_normal((B, D, K - 1)).astype(np.float32)
    xs = rng.standard_normal((B, D, 2)).astype(np.float32)
    if io == "bf16":
        st0, xs = W.round_bf16(st0), W.round_bf16(xs)
    st = dev(st0, io)
    st_or = st0.astype(np.float64)
    for t in range(2):
        out = mamba.conv1d_update(st, dev(np.ascontiguousarray(xs[:, :, t]), io), dev(w),
                                  dev(bias))
        want, st_or = oracle.conv1d_update(st_or, xs[:, :, t], w, bias)
        assert_within(host(out), want, CONV_TOL[io], f"conv update t={t}")
        assert np.array_equal(host(st), st_or), "conv window"


def test_block_workload_fused_every_element():
    """The d_model=768 block (B=2 D=1536 L=8192, fp32, conv k=4) through the
    fused entry point at full size, in the launch configuration the benchmark
    times: every output and final state against the oracle's conv1d+SiLU
    followed by its scan."""
    import selective_state_space_80_amd as mamba
    wl = W.WORKLOADS[1]
    say(f"fused block {wl.name}: drawing inputs")
    p = W.scan_inputs(wl)
    y, hl = mamba.conv1d_selective_scan_fwd(
        dev(p["x_raw"]), dev(p["conv_w"]), dev(p["dt"]), dev(p["A"]), dev(p["Bm"]),
        dev(p["Cm"]), dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]), z=dev(p["z"]),
        return_last_state=True)
    say("  oracle conv over every channel")
    x_or = oracle_conv_full(p["x_raw"], p["conv_w"])
    check_scan_full(y, hl, p, "f32", x=x_or, label="fused block")


@pytest.mark.parametrize("N", [16, 5])  # 16: four lanes per channel; 5: one lane per channel
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fused_decode_step_matches_oracle(N, K, io):
    _fused_decode_vs_oracle(N, K, io, stream=False)


@pytest.mark.parametrize("N", [16, 5])
@pytest.mark.parametrize("K", [1, 4])
def test_fused_decode_step_stream_state_matches_oracle(N, K):
    """The same with the streaming hint on the state (bf16)."""
    _fused_decode_vs_oracle(N, K, "bf16", stream=True)


def _fused_decode_vs_oracle(N, K, io, stream):
    """mamba_conv1d_selective_state_update over several tokens against the
    oracle's conv step followed by its state update (conv output in fp64, not
    rounded), with the window checked bit for bit after every token."""
    import selective_state_space_80_amd as mamba
    say(f"fused decode step N={N} K={K} io={io} stream_state={stream}")
    B, D, T = 3, 300, 4
    wl = W.DecodeWorkload("t", B, D, N, io, T, 1, 90 + K)
    init = W.decode_initial(wl)
    ci = W.decode_conv_initial(wl, K)
    rng = np.random.default_rng(K)
    cb = rng.standard_normal(D).astype(np.float32) if K != 2 else None
    with_opt = K != 3  # K = 3: no dt_bias, Dskip, z
    h = dev(init["h0"])
    cs = dev(ci["conv_state"], io) if K > 1 else None
    h_or, cs_or = init["h0"].astype(np.float64), ci["conv_state"].astype(np.float64)
    for t in range(T):
        s = W.decode_step_inputs(wl, t)
        y = mamba.conv1d_selective_state_update(
            h, cs, dev(s["x"], io), dev(ci["conv_w"]), dev(s["dt"], io), dev(init["A"]),
            dev(s["Bm"], io), dev(s["Cm"], io), conv_bias=dev(cb),
            dt_bias=dev(init["dt_bias"]) if with_opt else None,
            Dskip=dev(init["Dskip"]) if with_opt else None,
            z=dev(s["z"], io) if with_opt else None, stream_state=stream)
        xc, cs_or = oracle.conv1d_update(cs_or, s["x"], ci["conv_w"], cb)
        yo, h_or = oracle.state_update(h_or, xc, s["dt"], init["A"], s["Bm"], s["Cm"],
                                       dt_bias=init["dt_bias"] if with_opt else None,
                                       Dskip=init["Dskip"] if with_opt else None,
                                       z=s["z"] if with_opt else None)
        assert_within(host(y), yo, TOL[io], f"fused decode y t={t}")
        assert_within(host(h), h_or, STATE_TOL, f"fused decode h t={t}")
        if K > 1:
            assert np.array_equal(host(cs), cs_or), f"conv window t={t}"


def test_fused_decode_step_equals_separate_calls():
    """fp32: the fused step gives what conv1d_update then selective_state_update
    give (the conv output is exact in fp32 either way)."""
    import selective_state_space_80_amd as mamba
    B, D, N, K = 4, 640, 16, 4
    wl = W.DecodeWorkload("t", B, D, N, "f32", 3, 1, 97)
    init, ci = W.decode_initial(wl), W.decode_conv_initial(wl, K)
    h1, h2 = dev(init["h0"]), dev(init["h0"])
    c1, c2 = dev(ci["conv_state"]), dev(ci["conv_state"])
    w, A, bias, Dk = dev(ci["conv_w"]), dev(init["A"]), dev(init["dt_bias"]), dev(init["Dskip"])
    for t in range(3):
        s = W.decode_step_inputs(wl, t)
        x, dt, Bm, Cm, z = (dev(s[k]) for k in ("x", "dt", "Bm", "Cm", "z"))
        y1 = mamba.conv1d_selective_state_update(h1, c1, x, w, dt, A, Bm, Cm, dt_bias=bias,
                                                 Dskip=Dk, z=z)
        xc = mamba.conv1d_update(c2, x, w)
        y2 = mamba.selective_state_update(h2, xc, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dk, z=z)
        assert_within(host(y1), host(y2), 1e-6, f"fused vs separate y t={t}")
        assert_within(host(h1), host(h2), 1e-6, f"fused vs separate h t={t}")
        assert np.array_equal(host(c1), host(c2)), f"fused vs separate window t={t}"


def test_fused_decode_step_many_rows():
    """65537 batch rows (two launches) through the fused step, bf16."""
    import selective_state_space_80_amd as mamba
    B, D, N, K = 65537, 4, 16, 4
    wl = W.DecodeWorkload("t", B, D, N, "bf16", 1, 1, 98)
    init, ci = W.decode_initial(wl), W.decode_conv_initial(wl, K)
    s = W.decode_step_inputs(wl, 0)
    h, cs = dev(init["h0"]), dev(ci["conv_state"], "bf16")
    y = mamba.conv1d_selective_state_update(
        h, cs, dev(s["x"], "bf16"), dev(ci["conv_w"]), dev(s["dt"], "bf16"), dev(init["A"]),
        dev(s["Bm"], "bf16"), dev(s["Cm"], "bf16"), dt_bias=dev(init["dt_bias"]),
        Dskip=dev(init["Dskip"]), z=dev(s["z"], "bf16"))
    xc, cs_or = oracle.conv1d_update(ci["conv_state"].astype(np.float64), s["x"], ci["conv_w"])
    yo, ho = oracle.state_update(init["h0"].astype(np.float64), xc, s["dt"], init["A"], s["Bm"],
                                 s["Cm"], dt_bias=init["dt_bias"], Dskip=init["Dskip"], z=s["z"])
    assert_within(host(y), yo, TOL["bf16"], "fused decode y")
    assert_within(host(h), ho, STATE_TOL, "fused decode h")
    assert np.array_equal(host(cs), cs_or), "conv window"


@pytest.mark.parametrize("shape", [(8, 3072, 300, 16), (1, 6080, 8320, 16)],
                         ids=["chain", "superblocks"])
def test_fused_f32_carry_modes_every_element(shape):
    """fp32 fused front end with 384 groups (the chain carry) and with 95
    groups x 65 segments (superblocks, a ragged last tile): every element
    against the oracle."""
    B, D, L, N = shape
    K = 4
    say(f"fused fp32 shape={shape}: drawing inputs")
    p = make_inputs(B, D, L, N, K, "f32", seed=L + D, with_state=True, with_bias=True)
    y, hl, cs = run_fused(p, "f32")
    say("  oracle conv and scan over every channel")
    xc, cs_want = oracle_conv_front(p["x_raw"], p["conv_w"], p["conv_b"], p["conv_state"])
    check_scan_full(y, hl, p, "f32", x=xc, label="fused fp32")
    assert np.array_equal(host(cs), cs_want), "conv state out is not the last K-1 raw inputs"
