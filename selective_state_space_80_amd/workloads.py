"""Seeded synthetic workloads for the selective-scan hot path.

This module only draws random inputs; it contains none of the method's
arithmetic and is shared by the GPU tests, the oracle checks and the
benchmark so that both sides consume bit-identical tensors.

Recipe (every distribution is drawn with ``numpy.random.default_rng``):
  x, z           ~ N(0, 1)                       [B, D, L]
  dt             ~ N(0, 0.25)  (0.25 = std)      [B, D, L]
  u_d            log-uniform in [1e-3, 1e-1]     per channel d
  dt_bias_d      = log(expm1(u_d))  (so a zero dt gives step u_d)
  A[d, n]        = -(n + 1)
  Bm, Cm         ~ N(0, 1)                       [B, L, N]  (shared over d)
  Dskip          = 1
  block config:  x is replaced by x_raw ~ N(0, 1) that feeds the causal
                 depthwise conv, whose weights are conv_w ~ N(0, 0.5) [D, 4]
  decode config: h0 ~ N(0, 1) [B, D, N] fp32; every step draws fresh
                 x, z, dt [B, D] and Bm, Cm [B, N] from its own stream.
  Mamba-2 form:  x, z ~ N(0, 1) [B, L, H, P]; dt ~ N(0, 0.25) [B, L, H];
                 u_h log-uniform in [1e-3, 1e-1] and dt_bias_h = log(expm1(u_h))
                 per head; A_h ~ -U(1, 16) per head; Bm, Cm ~ N(0, 1)
                 [B, L, G, N]; Dskip_h = 1 (draw order: x, z, dt, u, A, Bm, Cm).
Draw order: x (or x_raw), z, dt, u, Bm, Cm, conv_w.  bf16 tensors are drawn in
fp32 and rounded to bf16 (round-to-nearest-even); the arrays returned here
hold those rounded values in float32, so they convert to bf16 exactly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ScanWorkload:
    name: str
    B: int
    D: int
    L: int
    N: int
    io: str            # "f32" or "bf16"
    conv: bool = False  # causal conv1d(k=4)+SiLU front end feeds the scan
    seed: int = 0

    @property
    def elems(self) -> int:
        return self.B * self.D * self.L


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    D: int
    N: int
    io: str
    steps: int
    check_every: int
    seed: int = 0


@dataclass(frozen=True)
class SsdWorkload:
    name: str
    B: int
    L: int
    H: int
    P: int
    G: int
    N: int
    seed: int = 0

    @property
    def elems(self) -> int:
        return self.B * self.L * self.H * self.P


# The Mamba-2 form at the 2.8B-layer scale of the bf16 scan workload:
# d_inner 5120 = 80 heads of 64 channels, one B/C group, state size 64.
SSD_WORKLOAD = SsdWorkload("ssd_b8_l2048_h80_p64_g1_n64_bf16", 8, 2048, 80, 64, 1, 64, 1005)


WORKLOADS = {
    0: ScanWorkload("scan_b1_d64_l256_n16_f32", 1, 64, 256, 16, "f32", False, 1000),
    1: ScanWorkload("block_dmodel768_b2_d1536_l8192_n16_f32_conv4", 2, 1536, 8192, 16,
                    "f32", True, 1001),
    2: ScanWorkload("scan_b8_d5120_l2048_n16_bf16", 8, 5120, 2048, 16, "bf16", False, 1002),
    3: ScanWorkload("scan_b1_d1536_l131072_n16_bf16", 1, 1536, 131072, 16, "bf16", False,
                    1003),
    4: DecodeWorkload("decode_b256_d5120_n16_bf16_x1024", 256, 5120, 16, "bf16", 1024, 128,
                      1004),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even) with torch's
    conversion; return them as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normal(rng, shape, std=1.0):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _channel_params(rng, D: int, N: int, u_range=(1e-3, 1e-1)):
    lo, hi = np.log(u_range[0]), np.log(u_range[1])
    u = np.exp(rng.uniform(lo, hi, size=D))
    dt_bias = np.log(np.expm1(u)).astype(np.float32)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (D, 1))
    Dskip = np.ones(D, dtype=np.float32)
    return dt_bias, A, Dskip


def make_scan_inputs(B: int, D: int, L: int, N: int, io: str = "f32", seed: int = 0,
                     conv: bool = False, dt_std: float = 0.25, u_range=(1e-3, 1e-1)):
    """Draw one scan problem.  Returns a dict of float32 numpy arrays:
    x (or x_raw + conv_w when conv), z, dt, dt_bias, A, Bm, Cm, Dskip."""
    rng = np.random.default_rng(seed)
    out = {}
    first = _normal(rng, (B, D, L))
    out["z"] = _normal(rng, (B, D, L))
    out["dt"] = _normal(rng, (B, D, L), dt_std)
    out["dt_bias"], out["A"], out["Dskip"] = _channel_params(rng, D, N, u_range)
    out["Bm"] = _normal(rng, (B, L, N))
    out["Cm"] = _normal(rng, (B, L, N))
    if conv:
        out["x_raw"] = first
        out["conv_w"] = _normal(rng, (D, 4), 0.5)
    else:
        out["x"] = first
    if io == "bf16":
        for k in ("x", "x_raw", "z", "dt", "Bm", "Cm"):
            if k in out:
                out[k] = round_bf16(out[k])
    elif io != "f32":
        raise ValueError("io must be 'f32' or 'bf16'")
    return out


def scan_inputs(wl: ScanWorkload, seed: int | None = None):
    return make_scan_inputs(wl.B, wl.D, wl.L, wl.N, wl.io,
                            wl.seed if seed is None else seed, wl.conv)


def decode_initial(wl: DecodeWorkload, seed: int | None = None):
    """h0 [B,D,N] fp32 and the per-channel parameters of a decode run."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    h0 = _normal(rng, (wl.B, wl.D, wl.N))
    dt_bias, A, Dskip = _channel_params(rng, wl.D, wl.N)
    return {"h0": h0, "dt_bias": dt_bias, "A": A, "Dskip": Dskip}


def decode_step_inputs(wl: DecodeWorkload, step: int, seed: int | None = None):
    """Fresh token inputs of decode step `step`: x, z, dt [B,D]; Bm, Cm [B,N]."""
    rng = np.random.default_rng([wl.seed if seed is None else seed, 1 + step])
    out = {
        "x": _normal(rng, (wl.B, wl.D)),
        "z": _normal(rng, (wl.B, wl.D)),
        "dt": _normal(rng, (wl.B, wl.D), 0.25),
        "Bm": _normal(rng, (wl.B, wl.N)),
        "Cm": _normal(rng, (wl.B, wl.N)),
    }
    if wl.io == "bf16":
        out = {k: round_bf16(v) for k, v in out.items()}
    return out


def decode_conv_initial(wl: DecodeWorkload, K: int = 4, seed: int | None = None):
    """The conv front end of a decode run: weights [D,K] ~ N(0, 0.5) (as in the
    block workload) and the carried window of K-1 raw inputs [B,D,K-1] ~ N(0,1)
    (bf16-exact for bf16 I/O).  Each step's raw input is that step's x."""
    rng = np.random.default_rng([wl.seed if seed is None else seed, 0, K])
    w = _normal(rng, (wl.D, K), 0.5)
    state = _normal(rng, (wl.B, wl.D, K - 1))
    if wl.io == "bf16":
        state = round_bf16(state)
    return {"conv_w": w, "conv_state": state}


def make_ssd_inputs(B: int, L: int, H: int, P: int, G: int, N: int, seed: int = 0):
    """Draw one Mamba-2-form problem (bf16 I/O).  Returns float32 numpy arrays
    holding bf16-exact values: x, z [B,L,H,P]; dt [B,L,H]; Bm, Cm [B,L,G,N];
    and fp32 per-head dt_bias, A, Dskip [H]."""
    rng = np.random.default_rng(seed)
    out = {"x": round_bf16(_normal(rng, (B, L, H, P))),
           "z": round_bf16(_normal(rng, (B, L, H, P))),
           "dt": round_bf16(_normal(rng, (B, L, H), 0.25))}
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    out["dt_bias"] = np.log(np.expm1(u)).astype(np.float32)
    out["A"] = (-rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    out["Bm"] = round_bf16(_normal(rng, (B, L, G, N)))
    out["Cm"] = round_bf16(_normal(rng, (B, L, G, N)))
    out["Dskip"] = np.ones(H, dtype=np.float32)
    return out


def ssd_inputs(wl: SsdWorkload, seed: int | None = None):
    return make_ssd_inputs(wl.B, wl.L, wl.H, wl.P, wl.G, wl.N,
                           wl.seed if seed is None else seed)
