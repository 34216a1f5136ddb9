"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

import selective_state_space_80_amd as mamba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_amd.h")

F32, BF16 = mamba.MAMBA_F32, mamba.MAMBA_BF16
OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EALIGN, EALIAS, EWS, ELAUNCH, EDEV, ETIMEOUT = range(11)


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


@pytest.fixture(scope="module")
def lib():
    return mamba.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba_[a-z0-9_]+)\s*\(", text)))


def test_binding_follows_the_header_abi_version():
    m = re.search(r"#define MAMBA_AMD_ABI_VERSION (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == mamba.ABI_VERSION


def test_header_lists_what_binding_expects():
    assert declared_functions() == sorted(mamba.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported by libmamba_amd.so"


def test_status_strings(lib):
    assert lib.mamba_abi_version() == mamba.ABI_VERSION == 9
    for st in range(11):
        s = lib.mamba_status_string(st).decode()
        assert s.startswith(mamba.STATUS_NAMES[st])
    assert "unknown" in lib.mamba_status_string(99).decode()


def test_workspace_size(lib):
    assert lib.mamba_selective_scan_fwd_workspace_size(0, 64, 256, 16, F32) == 0
    assert lib.mamba_selective_scan_fwd_workspace_size(1, 64, 256, 17, F32) == 0
    small = lib.mamba_selective_scan_fwd_workspace_size(1, 64, 256, 16, F32)
    big = lib.mamba_selective_scan_fwd_workspace_size(2, 1536, 8192, 16, F32)
    assert 0 < small < big and big % 256 == 0


# fake, well-aligned, non-overlapping device addresses: validation never
# dereferences them, and every case below must fail before any HIP call
def P(k):
    return ctypes.c_void_p(0x10000000000 + k * 0x100000000)


def scan(lib, **kw):
    a = dict(x=P(1), dt=P(2), dt_bias=P(3), A=P(4), Bm=P(5), Cm=P(6), Dskip=P(7), z=P(8),
             h0=P(9), y=P(10), h_last=P(11), ws=P(12), ws_bytes=1 << 40, B=2, D=64, L=256,
             N=16, io=F32)
    a.update(kw)
    return lib.mamba_selective_scan_fwd(a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"],
                                        a["Cm"], a["Dskip"], a["z"], a["h0"], a["y"],
                                        a["h_last"], a["ws"], a["ws_bytes"], a["B"], a["D"],
                                        a["L"], a["N"], a["io"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(io=7), EDTYPE),
    (dict(N=0), EUNSUP), (dict(N=17), EUNSUP),
    (dict(B=-1), ESHAPE), (dict(L=-5), ESHAPE), (dict(D=1 << 30, L=1 << 30), ESHAPE),
    (dict(x=None), ENULL), (dict(Bm=None), ENULL), (dict(y=None), ENULL),
    (dict(x=ctypes.c_void_p(0x10000000002)), EALIGN),
    (dict(io=BF16, dt=ctypes.c_void_p(0x20000000001)), EALIGN),
    (dict(A=ctypes.c_void_p(0x40000000002)), EALIGN),
    (dict(y=P(1)), EALIAS), (dict(h_last=P(9)), EALIAS), (dict(y=P(12)), EALIAS),
    (dict(ws=None), EWS), (dict(ws_bytes=1024), EWS),
    (dict(ws=ctypes.c_void_p(0xC0000000010)), EWS),
])
def test_scan_rejects(lib, kw, want):
    assert scan(lib, **kw) == want


def scan_ex(lib, flags, **kw):
    a = dict(x=P(1), dt=P(2), dt_bias=P(3), A=P(4), Bm=P(5), Cm=P(6), Dskip=P(7), z=P(8),
             h0=P(9), y=P(10), h_last=P(11), ws=P(12), ws_bytes=1 << 40, B=2, D=64, L=256,
             N=16, io=F32)
    a.update(kw)
    return lib.mamba_selective_scan_fwd_ex(a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"],
                                           a["Cm"], a["Dskip"], a["z"], a["h0"], a["y"],
                                           a["h_last"], a["ws"], a["ws_bytes"], a["B"], a["D"],
                                           a["L"], a["N"], a["io"], flags, None)


def test_scan_ex_flags(lib):
    assert scan_ex(lib, 4) == EUNSUP
    assert scan_ex(lib, 1 << 31) == EUNSUP
    assert scan_ex(lib, 3, y=P(1)) == EALIAS
    assert scan_ex(lib, 1, B=0) == OK
    if not _gpu_visible():
        for f in (0, 1, 2, 3):
            assert scan_ex(lib, f) == EDEV


def test_scan_empty_is_ok(lib):
    assert scan(lib, B=0) == OK
    assert scan(lib, D=0, x=None) == OK


def test_conv_rejects(lib):
    f = lib.mamba_conv1d_silu
    assert f(P(1), P(2), None, P(3), 2, 8, 32, 9, F32, None) == EUNSUP
    assert f(P(1), P(2), None, P(3), 2, 8, 32, 0, F32, None) == EUNSUP
    assert f(P(1), P(2), None, P(3), 2, 8, 32, 4, 3, None) == EDTYPE
    assert f(None, P(2), None, P(3), 2, 8, 32, 4, F32, None) == ENULL
    assert f(P(1), P(2), None, P(1), 2, 8, 32, 4, F32, None) == EALIAS
    assert f(P(1), P(2), None, ctypes.c_void_p(0x30000000001), 2, 8, 32, 4, BF16, None) == EALIGN
    assert f(P(1), P(2), None, P(3), -2, 8, 32, 4, F32, None) == ESHAPE
    assert f(P(1), P(2), None, P(3), 0, 8, 32, 4, F32, None) == OK


def test_state_update_rejects(lib):
    f = lib.mamba_selective_state_update
    args = [P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), P(10)]
    assert f(*args, 4, 64, 17, F32, 0, None) == EUNSUP
    assert f(*args, 4, 64, 16, 5, 0, None) == EDTYPE
    assert f(*args, 4, 64, 16, F32, 2, None) == EUNSUP  # unknown flag
    assert f(*args, 4, 64, 16, F32, 1 | 4, None) == EUNSUP
    bad = list(args)
    bad[9] = P(1)  # y on top of h
    assert f(*bad, 4, 64, 16, F32, 0, None) == EALIAS
    bad = list(args)
    bad[0] = None
    assert f(*bad, 4, 64, 16, F32, 1, None) == ENULL
    assert f(*args, 0, 64, 16, F32, 0, None) == OK
    assert f(*args, 0, 64, 16, F32, mamba.STEP_STREAM_STATE, None) == OK


def fused(lib, **kw):
    a = dict(x=P(1), w=P(13), cb=P(14), K=4, csin=P(15), csout=P(16), dt=P(2), dt_bias=P(3),
             A=P(4), Bm=P(5), Cm=P(6), Dskip=P(7), z=P(8), h0=P(9), y=P(10), h_last=P(11),
             ws=P(12), ws_bytes=1 << 40, B=2, D=64, L=256, N=16, io=F32)
    a.update(kw)
    return lib.mamba_conv1d_selective_scan_fwd(
        a["x"], a["w"], a["cb"], a["K"], a["csin"], a["csout"], a["dt"], a["dt_bias"], a["A"],
        a["Bm"], a["Cm"], a["Dskip"], a["z"], a["h0"], a["y"], a["h_last"], a["ws"],
        a["ws_bytes"], a["B"], a["D"], a["L"], a["N"], a["io"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(io=7), EDTYPE), (dict(K=0), EUNSUP), (dict(K=5), EUNSUP), (dict(K=-1), ESHAPE),
    (dict(N=17), EUNSUP), (dict(w=None), ENULL), (dict(x=None), ENULL),
    (dict(w=ctypes.c_void_p(0xD0000000002)), EALIGN),
    (dict(io=BF16, csout=ctypes.c_void_p(0xF0000000001)), EALIGN),
    (dict(y=P(13)), EALIAS), (dict(y=P(15)), EALIAS), (dict(h_last=P(14)), EALIAS),
    (dict(csout=P(1)), EALIAS), (dict(csout=P(10)), EALIAS), (dict(csout=P(12)), EALIAS),
    (dict(csout=ctypes.c_void_p(0x10000000000 + 15 * 0x100000000 + 4)), EALIAS),
    (dict(ws=None), EWS),
])
def test_fused_scan_rejects(lib, kw, want):
    assert fused(lib, **kw) == want


def test_fused_scan_empty_is_ok(lib):
    assert fused(lib, B=0) == OK
    assert fused(lib, D=0, x=None, w=None) == OK


def fused_step(lib, **kw):
    a = dict(h=P(1), cs=P(11), x=P(2), w=P(12), cb=P(13), K=4, dt=P(3), dt_bias=P(4), A=P(5),
             Bm=P(6), Cm=P(7), Dskip=P(8), z=P(9), y=P(10), B=4, D=64, N=16, io=F32, flags=0)
    a.update(kw)
    return lib.mamba_conv1d_selective_state_update(
        a["h"], a["cs"], a["x"], a["w"], a["cb"], a["K"], a["dt"], a["dt_bias"], a["A"], a["Bm"],
        a["Cm"], a["Dskip"], a["z"], a["y"], a["B"], a["D"], a["N"], a["io"], a["flags"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(io=7), EDTYPE), (dict(K=0), EUNSUP), (dict(K=5), EUNSUP), (dict(K=-1), ESHAPE),
    (dict(N=17), EUNSUP), (dict(B=-1), ESHAPE), (dict(w=None), ENULL), (dict(cs=None), ENULL),
    (dict(h=None), ENULL), (dict(x=None), ENULL),
    (dict(w=ctypes.c_void_p(0xC0000000002)), EALIGN),
    (dict(io=BF16, cs=ctypes.c_void_p(0xB0000000001)), EALIGN),
    (dict(cs=P(2)), EALIAS), (dict(cs=P(1)), EALIAS), (dict(cs=P(10)), EALIAS),
    (dict(cs=P(12)), EALIAS), (dict(y=P(13)), EALIAS), (dict(h=P(12)), EALIAS),
    (dict(flags=2), EUNSUP), (dict(flags=0x80000001), EUNSUP),
])
def test_fused_step_rejects(lib, kw, want):
    assert fused_step(lib, **kw) == want


def test_fused_step_empty_is_ok(lib):
    assert fused_step(lib, B=0) == OK
    assert fused_step(lib, D=0, h=None, cs=None) == OK


def test_conv_update_rejects(lib):
    f = lib.mamba_conv1d_update
    assert f(P(1), P(2), P(3), None, P(4), 2, 8, 9, F32, None) == EUNSUP
    assert f(P(1), P(2), P(3), None, P(4), 2, 8, 0, F32, None) == EUNSUP
    assert f(P(1), P(2), P(3), None, P(4), 2, 8, 4, 3, None) == EDTYPE
    assert f(None, P(2), P(3), None, P(4), 2, 8, 4, F32, None) == ENULL
    assert f(P(1), None, P(3), None, P(4), 2, 8, 4, F32, None) == ENULL
    assert f(P(1), P(2), P(3), None, P(1), 2, 8, 4, F32, None) == EALIAS
    assert f(P(1), P(2), P(3), None, P(2), 2, 8, 4, F32, None) == EALIAS
    assert f(P(2), P(2), P(3), None, P(4), 2, 8, 4, F32, None) == EALIAS
    assert f(P(1), P(2), P(3), None, ctypes.c_void_p(0x40000000001), 2, 8, 4, BF16,
             None) == EALIGN
    assert f(P(1), P(2), P(3), None, P(4), -2, 8, 4, F32, None) == ESHAPE
    assert f(P(1), P(2), P(3), None, P(4), 0, 8, 4, F32, None) == OK


def bwd(lib, **kw):
    a = dict(x=P(1), dt=P(2), dt_bias=P(3), A=P(4), Bm=P(5), Cm=P(6), Dskip=P(7), z=P(8),
             h0=P(9), dout=P(10), dh_last=P(11), dx=P(12), ddt=P(13), dA=P(14), dB=P(15),
             dC=P(16), dD=P(17), dz=P(18), ddt_bias=P(19), dh0=P(20), ws=P(21),
             ws_bytes=1 << 40, B=2, D=64, L=256, N=16, io=F32)
    a.update(kw)
    return lib.mamba_selective_scan_bwd(
        a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"], a["Cm"], a["Dskip"], a["z"], a["h0"],
        a["dout"], a["dh_last"], a["dx"], a["ddt"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
        a["ddt_bias"], a["dh0"], a["ws"], a["ws_bytes"], a["B"], a["D"], a["L"], a["N"],
        a["io"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(io=5), EDTYPE), (dict(N=0), EUNSUP), (dict(N=17), EUNSUP),
    (dict(L=-1), ESHAPE), (dict(D=1 << 30, L=1 << 30), ESHAPE),
    (dict(B=1 << 20, L=1 << 12), ESHAPE),        # B*L*16 too large for the B/C grid
    (dict(x=None), ENULL), (dict(dout=None), ENULL), (dict(dA=None), ENULL),
    (dict(dB=None), ENULL), (dict(dz=None), ENULL),  # z given, dz missing
    (dict(ws=None), EWS), (dict(ws_bytes=1000), EWS),
    (dict(ws=ctypes.c_void_p(0x10000000000 + 21 * 0x100000000 + 64)), EWS),
    (dict(dx=ctypes.c_void_p(0x10000000000 + 12 * 0x100000000 + 2)), EALIGN),
    (dict(io=BF16, dout=ctypes.c_void_p(0x10000000000 + 10 * 0x100000000 + 1)), EALIGN),
    (dict(dh0=ctypes.c_void_p(0x10000000000 + 20 * 0x100000000 + 2)), EALIGN),
    (dict(dx=P(1)), EALIAS), (dict(dB=P(5)), EALIAS), (dict(dh0=P(11)), EALIAS),
    (dict(dC=P(15)), EALIAS), (dict(dA=P(21)), EALIAS),
    (dict(ddt=ctypes.c_void_p(0x10000000000 + 12 * 0x100000000 + 4096)), EALIAS),
])
def test_bwd_rejects(lib, kw, want):
    assert bwd(lib, **kw) == want


def test_bwd_optional_and_empty(lib):
    # D = 0: nothing at all to do
    assert bwd(lib, D=0, x=None, dA=None, ws=None) == OK
    # no gate: dz is not required (and never written)
    if not _gpu_visible():
        assert bwd(lib, z=None, dz=None) == EDEV
        assert bwd(lib, z=None, dz=P(18), dt_bias=None, Dskip=None, h0=None, dh_last=None,
                   dD=None, ddt_bias=None, dh0=None) == EDEV
        # L = 0: only dA (and the optional outputs) are written, no workspace
        assert bwd(lib, L=0, x=None, dt=None, Bm=None, Cm=None, dout=None, dx=None, ddt=None,
                   dB=None, dC=None, ws=None, ws_bytes=0) == EDEV
    assert bwd(lib, L=0, dA=None) == ENULL


def test_bwd_workspace_size(lib):
    f = lib.mamba_selective_scan_bwd_workspace_size
    assert f(0, 64, 256, 16, F32) == 0 and f(1, 64, 256, 0, F32) == 0
    small, big = f(1, 64, 256, 16, F32), f(2, 1536, 2048, 16, BF16)
    assert 0 < small < big and big % 256 == 0
    assert small > lib.mamba_selective_scan_fwd_workspace_size(1, 64, 256, 16, F32)


def ssd(lib, **kw):
    a = dict(x=P(1), dt=P(2), dt_bias=P(3), A=P(4), Bm=P(5), Cm=P(6), Dskip=P(7), z=P(8),
             h0=P(9), y=P(10), h_last=P(11), B=2, L=256, H=8, Pd=64, G=2, N=64, io=BF16)
    a.update(kw)
    return lib.mamba_ssd_scan_fwd(a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"], a["Cm"],
                                  a["Dskip"], a["z"], a["h0"], a["y"], a["h_last"], a["B"],
                                  a["L"], a["H"], a["Pd"], a["G"], a["N"], a["io"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(io=9), EDTYPE), (dict(io=F32), EUNSUP), (dict(Pd=32), EUNSUP), (dict(N=48), EUNSUP),
    (dict(N=256), EUNSUP), (dict(G=3), ESHAPE), (dict(G=0), ESHAPE), (dict(L=-1), ESHAPE),
    (dict(x=None), ENULL), (dict(A=None), ENULL), (dict(Cm=None), ENULL), (dict(y=None), ENULL),
    (dict(x=ctypes.c_void_p(0x10000000000 + 1 * 0x100000000 + 8)), EALIGN),
    (dict(h_last=ctypes.c_void_p(0x10000000000 + 11 * 0x100000000 + 4)), EALIGN),
    (dict(dt=ctypes.c_void_p(0x10000000000 + 2 * 0x100000000 + 1)), EALIGN),
    (dict(y=P(1)), EALIAS), (dict(h_last=P(9)), EALIAS), (dict(h_last=P(10)), EALIAS),
])
def test_ssd_rejects(lib, kw, want):
    assert ssd(lib, **kw) == want


def test_ssd_empty_is_ok(lib):
    assert ssd(lib, B=0) == OK and ssd(lib, H=0, G=1) == OK
    assert ssd(lib, L=0, h_last=None, x=None, y=None) == OK


def test_launch_grid_limits(lib):
    """Sizes whose launch grids would reach 2^32 work-items in one dimension are
    shape errors, reported before any pointer is looked at."""
    big = dict(B=1 << 16, D=1 << 15)  # 2^31 channels
    assert lib.mamba_conv1d_silu(P(1), P(2), None, P(3), 1, 1 << 20, 1 << 13, 4, F32,
                                 None) == ESHAPE
    assert lib.mamba_selective_state_update(*[P(k) for k in range(1, 11)], big["B"], big["D"],
                                            16, F32, 0, None) == ESHAPE
    assert fused_step(lib, **big) == ESHAPE
    assert lib.mamba_conv1d_update(P(1), P(2), P(3), None, P(4), big["B"], big["D"], 4, F32,
                                   None) == ESHAPE
    # an empty sequence still copies h0 into h_last over B*D*N values
    assert scan(lib, B=1 << 12, D=1 << 15, L=0) == ESHAPE
    assert scan(lib, B=1 << 12, D=1 << 15, L=0, h_last=None) == OK  # nothing to launch
    # an empty dimension leaves the others bounded
    assert scan(lib, B=1 << 30, D=1 << 30, L=0, h_last=None) == ESHAPE
    assert bwd(lib, B=1, D=64, L=1 << 25) == ESHAPE  # column sums over B*L*16 columns
    assert bwd(lib, B=1, D=1 << 16, L=1 << 18) == ESHAPE  # 2^21 segments
    assert bwd(lib, B=1 << 12, D=1 << 15, L=0) == ESHAPE  # empty problem over B*D*N
    assert ssd(lib, B=1 << 12, H=1 << 12, G=1) == ESHAPE


@pytest.mark.skipif(_gpu_visible(), reason="valid fake pointers must never reach a GPU")
def test_valid_arguments_without_gpu_report_device(lib):
    assert fused(lib) == EDEV
    assert fused(lib, csout=P(15)) == EDEV  # conv state updated in place
    assert lib.mamba_conv1d_update(P(1), P(2), P(3), None, P(4), 2, 8, 4, F32, None) == EDEV
    assert lib.mamba_conv1d_update(None, P(2), P(3), None, P(4), 2, 8, 1, F32, None) == EDEV
    assert scan(lib) == EDEV
    assert lib.mamba_conv1d_silu(P(1), P(2), None, P(3), 2, 8, 32, 4, F32, None) == EDEV
    assert lib.mamba_selective_state_update(P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8),
                                            P(9), P(10), 4, 64, 16, F32, 0, None) == EDEV
    assert lib.mamba_selective_state_update(P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8),
                                            P(9), P(10), 4, 64, 16, F32, 1, None) == EDEV
    assert bwd(lib) == EDEV
    assert fused_step(lib) == EDEV
    assert fused_step(lib, K=1, cs=None) == EDEV  # one tap: no window to carry
    assert fused_step(lib, flags=1) == EDEV
    assert ssd(lib) == EDEV
    assert ssd(lib, L=0, x=None, y=None, dt=None, Bm=None, Cm=None) == EDEV  # h_last = h0


def test_binding_fails_loudly_without_library(tmp_path):
    saved = mamba._lib
    try:
        mamba._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            mamba.load_library(str(tmp_path / "missing.so"))
    finally:
        mamba._lib = saved


def test_scan_check_rejects_bad_workspace_before_any_hip_call(lib):
    """mamba_selective_scan_check validates its workspace first (no stream is
    touched for a NULL, misaligned or too small one)."""
    buf = ctypes.create_string_buffer(1024)
    base = ctypes.addressof(buf)
    aligned = (base + 255) // 256 * 256
    assert lib.mamba_selective_scan_check(None, 4096, None) == EWS
    assert lib.mamba_selective_scan_check(ctypes.c_void_p(aligned), 255, None) == EWS
    assert lib.mamba_selective_scan_check(ctypes.c_void_p(aligned + 16), 512, None) == EWS


def test_spin_limit_hook_accepts_values(lib):
    lib.mamba_set_scan_spin_limit(0)
    lib.mamba_set_scan_spin_limit(-1)  # back to the default


def test_noalloc_scan_rejects_shapes_beyond_its_scratch(lib):
    """The entry point that allocates nothing refuses, before any HIP call, a
    shape whose workspace is larger than its 64 MiB scratch."""
    f = lib.mamba_selective_scan_fwd_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_void_p]
    fake = ctypes.c_void_p(4096)
    need = lib.mamba_selective_scan_fwd_workspace_size(1, 1536, 131072, 16, BF16)
    assert need > mamba.NOALLOC_SCRATCH_BYTES
    args = [fake, fake, None, fake, fake, fake, None, None, None, ctypes.c_void_p(1 << 40),
            None, 1, 1536, 131072, 16, BF16, None]
    assert f(*args) == EWS
    fits = lib.mamba_selective_scan_fwd_workspace_size(8, 5120, 2048, 16, BF16)
    assert fits <= mamba.NOALLOC_SCRATCH_BYTES
