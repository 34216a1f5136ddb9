"""The library's calls inside HIP graphs (torch.cuda.CUDAGraph): they launch
kernels only (no allocation, memset or synchronisation on the path), so a
captured call replays correctly.  Each graph is replayed several times, with
new input values, eager work and synchronisations between the replays, and
every replay is compared with the same call made eagerly (bit for bit: the
kernels are deterministic)."""
import numpy as np
import pytest

from scan_check import dev, say
from selective_state_space_80_amd import workloads as W

pytestmark = pytest.mark.gpu


def _replays(capture, eager, refill, n=3):
    """capture() records the call into a graph and returns its output tensors;
    eager() makes the same call eagerly; refill(k) writes replay k's inputs in
    place.  Both must give identical tensors after every replay."""
    import torch
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up off the capture
        capture()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = capture()
    for k in range(n):
        refill(k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref), f"replay {k} differs from the eager call"
        say(f"  replay {k} identical")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_graph_scan(io):
    import torch
    import selective_state_space_80_amd as mamba
    B, D, L, N = 2, 130, 700, 16
    say(f"graph scan io={io}")
    p = W.make_scan_inputs(B, D, L, N, io, seed=21)
    x, dt, z = dev(p["x"], io), dev(p["dt"], io), dev(p["z"], io)
    Bm, Cm = dev(p["Bm"], io), dev(p["Cm"], io)
    A, bias, Dk = dev(p["A"]), dev(p["dt_bias"]), dev(p["Dskip"])
    h0 = torch.randn((B, D, N), device="cuda")
    ws = torch.empty(mamba.selective_scan_fwd_workspace_size(B, D, L, N, x.dtype),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    hl = torch.empty((B, D, N), device="cuda")
    rng = np.random.default_rng(22)

    def call(out, h_last, workspace):
        return mamba.selective_scan_fwd(x, dt, A, Bm, Cm, bias, Dk, z, h0, return_last_state=True,
                                        out=out, workspace=workspace, h_last=h_last)

    def refill(k):
        x.copy_(dev(rng.standard_normal((B, D, L)).astype(np.float32), io))
        h0.copy_(torch.randn((B, D, N), device="cuda"))

    _replays(lambda: call(y, hl, ws), lambda: call(None, None, None), refill)


def test_graph_decode():
    """One decode step captured and replayed: the state advances in place, so
    k replays equal k eager steps from the same start."""
    import torch
    import selective_state_space_80_amd as mamba
    B, D, N = 4, 320, 16
    say("graph decode")
    rng = np.random.default_rng(23)
    io = "bf16"
    x = dev(rng.standard_normal((B, D)).astype(np.float32), io)
    dt = dev((0.25 * rng.standard_normal((B, D))).astype(np.float32), io)
    z = dev(rng.standard_normal((B, D)).astype(np.float32), io)
    Bm = dev(rng.standard_normal((B, N)).astype(np.float32), io)
    Cm = dev(rng.standard_normal((B, N)).astype(np.float32), io)
    p = W.make_scan_inputs(1, D, 1, N, "f32", seed=24)
    A, bias, Dk = dev(p["A"]), dev(p["dt_bias"]), dev(p["Dskip"])
    h_g = torch.randn((B, D, N), device="cuda")
    h_e = h_g.clone()
    y = torch.empty_like(x)
    # the warm-up call of _replays advances h_g once: advance h_e to match
    mamba.selective_state_update(h_e, x, dt, A, Bm, Cm, bias, Dk, z)

    def refill(k):
        x.copy_(dev(rng.standard_normal((B, D)).astype(np.float32), io))

    def eager():
        out = mamba.selective_state_update(h_e, x, dt, A, Bm, Cm, bias, Dk, z)
        return out, h_e

    _replays(lambda: (mamba.selective_state_update(h_g, x, dt, A, Bm, Cm, bias, Dk, z, out=y),
                      h_g), eager, refill, n=4)


def test_graph_ssd():
    import torch
    import selective_state_space_80_amd as mamba
    B, L, H, G, N = 1, 300, 4, 2, 64
    say("graph ssd")
    p = W.make_ssd_inputs(B, L, H, 64, G, N, seed=25)
    x, z, dt = dev(p["x"], "bf16"), dev(p["z"], "bf16"), dev(p["dt"], "bf16")
    Bm, Cm = dev(p["Bm"], "bf16"), dev(p["Cm"], "bf16")
    A, bias, Dk = dev(p["A"]), dev(p["dt_bias"]), dev(p["Dskip"])
    y = torch.empty_like(x)
    hl = torch.empty((B, H, 64, N), device="cuda")
    rng = np.random.default_rng(26)

    def call(out, h_last):
        return mamba.ssd_scan_fwd(x, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dk, z=z,
                                  return_last_state=True, out=out, h_last=h_last)

    def refill(k):
        x.copy_(dev(rng.standard_normal((B, L, H, 64)).astype(np.float32), "bf16"))

    _replays(lambda: call(y, hl), lambda: call(None, None), refill)


def test_graph_fused_decode():
    """The fused decode step (conv window and state advance in place) captured
    and replayed: k replays equal k eager steps from the same start."""
    import torch
    import selective_state_space_80_amd as mamba
    wl = W.DecodeWorkload("t", 4, 320, 16, "bf16", 1, 1, 27)
    say("graph fused decode")
    init, ci = W.decode_initial(wl), W.decode_conv_initial(wl, 4)
    s = W.decode_step_inputs(wl, 0)
    x, dt, z = dev(s["x"], "bf16"), dev(s["dt"], "bf16"), dev(s["z"], "bf16")
    Bm, Cm = dev(s["Bm"], "bf16"), dev(s["Cm"], "bf16")
    A, bias, Dk, w = dev(init["A"]), dev(init["dt_bias"]), dev(init["Dskip"]), dev(ci["conv_w"])
    h_g, c_g = dev(init["h0"]), dev(ci["conv_state"], "bf16")
    h_e, c_e = h_g.clone(), c_g.clone()
    y = torch.empty_like(x)
    rng = np.random.default_rng(28)

    def call(h, c, out=None):
        return mamba.conv1d_selective_state_update(h, c, x, w, dt, A, Bm, Cm, dt_bias=bias,
                                                   Dskip=Dk, z=z, out=out)

    # the warm-up call of _replays advances h_g and c_g once: advance h_e, c_e to match
    call(h_e, c_e)

    def refill(k):
        x.copy_(dev(rng.standard_normal((wl.B, wl.D)).astype(np.float32), "bf16"))

    def eager():
        return call(h_e, c_e), h_e, c_e

    _replays(lambda: (call(h_g, c_g, out=y), h_g, c_g), eager, refill, n=4)
