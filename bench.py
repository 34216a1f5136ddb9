#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
held in HBM: causal depthwise conv1d(k=4) + SiLU, then the fused selective
scan (softplus step, ZOH, recurrence, readout, D skip, SiLU(z) gate), on the
Mamba block at d_model=768 (B=2, D_inner=1536, L=8192, N=16, fp32 I/O).  By
default the conv runs inside the scan kernel (mamba_conv1d_selective_scan_fwd);
--unfused times the two separate calls.

Prints ONE JSON line with the metric (scanned Gelem/s = B*L*D_inner / step
time), the roofline of the dominant kernel (the main scan kernel, timed with
HIP events on its own stream through the library's timing hook) and the fp64
oracle timed on a bounded sample of the same workload on the host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from selective_state_space_80_amd import profiling  # noqa: E402  (stdlib only)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak (packed fp32)
# Without packed fp32 (the v_pk_*_f32 forms are switched off in every build here)
# a CU issues one wave64 fp32 VALU instruction per clock: 4 SIMDs x 16 lanes, a
# wave64 instruction occupying a SIMD for 4 clocks.  256 CUs at 2.4 GHz:
VALU_ISSUE_PEAK = 256 * 2.4e9    # wave64 VALU instructions per second
FP32_NOPACK_PEAK_TFLOPS = VALU_ISSUE_PEAK * 64 * 2 / 1e12  # 78.6: fma = 2 flops
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


class HipEvents:
    """Raw hipEvent_t pairs through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def scan_bytes(B, D, L, N, esz, gate=True, last_state=False):
    """Algorithmic HBM bytes of one scan: x, dt (and z) read once, y written
    once, B and C read once per (b, t), A/D/dt_bias once, h_last if returned."""
    per_elem = (3 if gate else 2) * esz + esz
    return (B * D * L * per_elem + 2 * B * L * N * esz + D * N * 4 + 2 * D * 4
            + (B * D * N * 4 if last_state else 0))


def conv_bytes(B, D, L, K, esz):
    return 2 * B * D * L * esz + D * K * 4


def traffic_record(key):
    """HBM traffic (and VALU instruction count) of a workload's dominant kernel
    measured by rocprofv3 counters, if they were taken on the current source of
    that kernel (else None: counters of an older kernel say nothing)."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(key)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or "source" not in rec:
        return None
    path = os.path.join(ROOT, rec["source"])
    if not os.path.isfile(path):
        return None
    return rec if rec.get("source_digest") == profiling.source_digest(path) else None


def traffic_bytes(tr):
    """FETCH_SIZE + WRITE_SIZE per launch, each scaled by a copy kernel of known size."""
    return None if tr is None else int(round(tr["fetch_bytes"] + tr["write_bytes"]))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, B, D, L, target_s=20.0, y_gpu=None, tol=1e-4):
    """The fp64 oracle (conv then scan) on a bounded sample of the workload:
    whole sequences of the first channels, batch row by batch row, sized for at
    most ~target_s seconds (the whole workload when it fits).  Also the rate of
    one thread on a few whole sequences, and (given the benchmarked output
    y_gpu) the largest error of that output on those few sequences,
    |y_gpu - y_oracle| / (1 + |y_oracle|), against the tolerance."""
    import oracle
    threads = min(16, os.cpu_count() or 1)

    def run(b, ch, nthreads):
        xs = oracle.conv1d_silu(p["x_raw"][b:b + 1, :ch], p["conv_w"][:ch])
        return oracle.selective_scan(xs, p["dt"][b:b + 1, :ch], p["A"][:ch], p["Bm"][b:b + 1],
                                     p["Cm"][b:b + 1], p["dt_bias"][:ch], p["Dskip"][:ch],
                                     p["z"][b:b + 1, :ch], nthreads=nthreads)[0]

    t0 = time.perf_counter()
    y_small = run(0, 4, 1)
    single = 4 * L / (time.perf_counter() - t0) / 1e9
    check = None
    if y_gpu is not None:
        err = np.abs(y_gpu - y_small) / (1.0 + np.abs(y_small))
        check = {"max_rel_err": float(err.max()), "tolerance": tol,
                 "sample": f"batch row 0, channels 0..3, all {L} steps of the benchmarked output",
                 "within": bool(err.max() <= tol)}
    t0 = time.perf_counter()
    run(0, threads, threads)
    per_ch = (time.perf_counter() - t0) / threads
    budget = int(target_s / max(per_ch, 1e-9) * threads)
    if budget >= B * D:
        rows, ch = B, D
    else:
        rows, ch = 1, max(threads, min(D, budget) // threads * threads)
    t0 = time.perf_counter()
    for b in range(rows):
        run(b, ch, threads)
    dt = time.perf_counter() - t0
    elems = rows * ch * L
    what = ("the whole workload" if rows * ch == B * D else
            f"batch row 0, channels 0..{ch - 1} of {D}")
    return {"value": round(elems / dt / 1e9, 6), "unit": "Gelem/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{what}, all {L} steps: conv1d+SiLU then scan in fp64 on {threads} "
                      f"host threads ({elems} elements)",
            "single_thread_value": round(single, 6),
            "single_thread_sample": f"batch row 0, channels 0..3, all {L} steps, 1 thread",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            **({"check": check} if check is not None else {})}


def _pool_time(jobs, threads):
    """Run oracle calls (ctypes, so they release the GIL) on a thread pool;
    return the wall-clock seconds."""
    import concurrent.futures as cf
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(j) for j in jobs]:
            f.result()
    return time.perf_counter() - t0


def cpu_baseline_bwd(p, dout, B, D, L, target_s=15.0):
    """The fp64 oracle's backward on a bounded sample: batch row 0, whole
    sequences of the first channels, one oracle call per channel on a pool of
    host threads, sized for about target_s seconds."""
    import oracle
    threads = min(16, os.cpu_count() or 1)

    def job(d):
        sl = slice(d, d + 1)
        return lambda: oracle.selective_scan_bwd(
            p["x"][0:1, sl], p["dt"][0:1, sl], p["A"][sl], p["Bm"][0:1], p["Cm"][0:1],
            dout[0:1, sl], dt_bias=p["dt_bias"][sl], Dskip=p["Dskip"][sl], z=p["z"][0:1, sl])

    t1 = _pool_time([job(0)], 1)
    ch = int(min(D, max(threads, target_s / max(t1, 1e-6) * threads)) // threads * threads)
    dt = _pool_time([job(d) for d in range(ch)], threads)
    elems = ch * L
    return {"value": round(elems / dt / 1e9, 6), "unit": "Gelem/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"batch row 0, channels 0..{ch - 1} of {D}, all {L} steps: the fp64 "
                      f"backward, one channel per call on {threads} host threads",
            "single_thread_value": round(L / t1 / 1e9, 6), "cpu_model": cpu_model()}


def cpu_baseline_ssd(p, wl, target_s=15.0):
    """The fp64 oracle's Mamba-2-form recurrence on a bounded sample: whole
    sequences of (batch row, head) pairs, one call per pair on a pool of host
    threads, sized for about target_s seconds."""
    import oracle
    threads = min(16, os.cpu_count() or 1)

    def job(b, h):
        def run():
            oracle.ssd_scan(p["x"][b:b + 1, :, h:h + 1], p["dt"][b:b + 1, :, h:h + 1],
                            p["A"][h:h + 1], p["Bm"][b:b + 1], p["Cm"][b:b + 1],
                            p["dt_bias"][h:h + 1], p["Dskip"][h:h + 1],
                            p["z"][b:b + 1, :, h:h + 1])
        return run

    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    t1 = _pool_time([job(0, 0)], 1)
    n = int(min(len(pairs), max(threads, target_s / max(t1, 1e-6) * threads)) // threads * threads)
    dt = _pool_time([job(b, h) for b, h in pairs[:n]], threads)
    elems = n * wl.L * wl.P
    return {"value": round(elems / dt / 1e9, 6), "unit": "Gelem/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the first {n} of {len(pairs)} (batch row, head) pairs, all {wl.L} steps, "
                      f"fp64 recurrence, one pair per call on {threads} host threads",
            "single_thread_value": round(wl.L * wl.P / t1 / 1e9, 6), "cpu_model": cpu_model()}


def cpu_baseline_decode(wl, init, steps, nbytes, conv=None, target_s=10.0):
    """The fp64 oracle's decode step (with `conv`: its conv step first) over the
    whole B x D problem, batch rows split across a pool of host threads, for
    about target_s seconds of steps; reported in GB/s of the same algorithmic
    bytes per step as the GPU line."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    parts = [r for r in np.array_split(np.arange(wl.B), threads) if len(r)]

    def job(r, s):
        b0, b1 = int(r[0]), int(r[-1]) + 1

        def run():
            x = s["x"][b0:b1]
            if conv is not None:
                x, _ = oracle.conv1d_update(conv["conv_state"][b0:b1], x, conv["conv_w"])
            oracle.state_update(init["h0"][b0:b1], x, s["dt"][b0:b1], init["A"], s["Bm"][b0:b1],
                                s["Cm"][b0:b1], init["dt_bias"], init["Dskip"], s["z"][b0:b1])
        return run

    t_one = _pool_time([job(r, steps[0]) for r in parts], threads)
    n = int(max(1, min(256, target_s / max(t_one, 1e-6))))
    dt = _pool_time([job(r, steps[i % len(steps)]) for i in range(n) for r in parts], threads)
    what = "conv step, then state update" if conv is not None else "state update"
    return {"value": round(nbytes * n / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{n} whole decode steps ({wl.B} x {wl.D} channels, {what}) in fp64, "
                      f"batch rows split over {threads} host threads",
            "cpu_model": cpu_model()}


def quantiles(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def valu_record(tr, elems, kernel_ms):
    """Measured VALU issue of a kernel: wave64 VALU instructions per launch
    (rocprofv3 SQ_INSTS_VALU, taken on the same kernel source) over the time of
    one launch, against one wave64 instruction per clock per CU; and the VALU
    busy cycles (SQ_ACTIVE_INST_VALU: a transcendental counts two, and they
    partly overlap other VALU work, so this may exceed 1 on exp-heavy kernels)."""
    if tr is None or "valu_insts" not in tr:
        return None
    per_s = tr["valu_insts"] / (kernel_ms * 1e-3)
    rec = {"wave_instr_per_launch": int(tr["valu_insts"]),
           "wave_instr_per_elem": round(tr["valu_insts"] * 64 / elems, 1),
           "issue_peak_per_s": VALU_ISSUE_PEAK, "frac": round(per_s / VALU_ISSUE_PEAK, 4)}
    if "valu_active" in tr:
        rec["busy_frac"] = round(tr["valu_active"] / (kernel_ms * 1e-3) / VALU_ISSUE_PEAK, 4)
    return rec


def scan_valu_per_elem(io, conv=False):
    """Algorithmic VALU instructions per scanned element of the forward scan
    (structured A, N = 16, with dt_bias, D and the gate): the arithmetic the
    chunked two-level scan performs, without loads, stores, addressing,
    register moves or waits.  A transcendental counts one instruction.
      chunk scan per step: Δ = softplus (fma, exp2, add, log2; the series
        near 0: fma, fma, mul; two compares, two selects: 11), the step decay
        (mul, exp2: 2), e and e - 1 (the subtraction; the series near 0: fma,
        fma, mul, compare, add, two selects: 8), 16 states x 3 minus the first
        power (47), readout (16), cumulative decay (add to the exponent sum,
        exp2: 2), skip and scale (2)                                     88
      fix-up: 16 products C_n/(n+1) * carried state, 15 Horner fmas, 2  33
      gate: SiLU(z) (mul, exp2, add, rcp, mul) and the product          6
      carry: chunk and segment maps, start states: about 4.25 map
        applications per 32 steps, each 16 x (exponent, exp2, fma)      6.375
      bf16 I/O: unpack x, dt, z; pack y                                 3.5
      fused conv1d, 4 taps: 4 fma + SiLU                                9"""
    n = 88 + 33 + 6 + 6.375
    if io == "bf16":
        n += 3.5
    if conv:
        n += 9
    return n


def scan_roofline(kernel, io, conv, elems, kernel_ms, alg_bytes, tr):
    """Roofline of a forward scan kernel.  Its binding roof is VALU issue: the
    counted instructions need more time at one wave64 instruction per clock per
    CU than its bytes need at 8 TB/s.  `achieved` is the algorithmic VALU
    instruction rate (scan_valu_per_elem x elements / kernel time); `hbm` is the
    metric's own figure, algorithmic bytes over kernel time against 8 TB/s."""
    per_elem = scan_valu_per_elem(io, conv)
    alg_instr = per_elem * elems / 64
    achieved = alg_instr / (kernel_ms * 1e-3)
    gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
    return {"bound": "alu", "achieved": round(achieved / 1e9, 1),
            "peak": round(VALU_ISSUE_PEAK / 1e9, 1), "unit": "G VALU instr/s (wave64)",
            "frac": round(achieved / VALU_ISSUE_PEAK, 4), "traffic": traffic_bytes(tr),
            "kernel": kernel, "kernel_ms": round(kernel_ms, 4),
            "algorithmic_instr_per_elem": per_elem, "algorithmic_instr": int(alg_instr),
            "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg_bytes}}



def settle_clocks(step, torch, seconds):
    """Run the step back to back for `seconds` of wall time before the warm-up
    steps: the GPU only reaches its steady clocks after tens of milliseconds of
    sustained work, which a few warm-up steps of a sub-millisecond kernel do
    not give.  Untimed; reported beside the result."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "steps": n}


def time_with_scan_events(step, torch, mamba, steps):
    """Time `steps` calls of step(): wall clock per step, and the main scan
    kernel's duration per launch from HIP events recorded around it on its own
    stream (the library's timing hook)."""
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        mamba.set_scan_timing_events_raw(pairs[i][0], pairs[i][1])
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mamba.set_scan_timing_events_raw(None, None)
    k_all = [ev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    return elapsed / steps * 1e3, k_all


def cpu_baseline_scan(p, wl, target_s, y_gpu_rows=None, tol=2e-2):
    """The fp64 oracle's scan on a bounded sample of a workload: whole
    sequences of the first channels of batch row 0 on the host threads, sized
    for about target_s seconds; with the benchmarked output of those channels
    (y_gpu_rows, [1, ch, L]) also its largest error against the oracle."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    L = wl.L

    def run(ch, nthreads):
        return oracle.selective_scan(p["x"][0:1, :ch], p["dt"][0:1, :ch], p["A"][:ch],
                                     p["Bm"][0:1], p["Cm"][0:1], p["dt_bias"][:ch],
                                     p["Dskip"][:ch], p["z"][0:1, :ch], nthreads=nthreads)[0]

    t0 = time.perf_counter()
    run(threads, threads)
    per_ch = (time.perf_counter() - t0) / threads
    ch = int(min(wl.D, max(threads, target_s / max(per_ch, 1e-9))) // threads * threads)
    t0 = time.perf_counter()
    y_or = run(ch, threads)
    dt = time.perf_counter() - t0
    out = {"value": round(ch * L / dt / 1e9, 6), "unit": "Gelem/s", "cores": threads,
           "kind": "oracle", "seconds": round(dt, 3),
           "sample": f"batch row 0, channels 0..{ch - 1} of {wl.D}, all {L} steps, fp64 on "
                     f"{threads} host threads ({ch * L} elements)",
           "cpu_model": cpu_model()}
    if y_gpu_rows is not None:
        k = min(ch, y_gpu_rows.shape[1])
        err = np.abs(y_gpu_rows[:, :k] - y_or[:, :k]) / (1.0 + np.abs(y_or[:, :k]))
        out["check"] = {"max_rel_err": float(err.max()), "tolerance": tol,
                        "sample": f"batch row 0, channels 0..{k - 1}, all {L} steps of "
                                  "the benchmarked output",
                        "within": bool(err.max() <= tol)}
    return out


def measure_scan(torch, mamba, W, idx, steps, warmup, settle_s, cpu_s, no_cpu=False):
    """One scan workload in the benchmark's launch: kernel and step time, the
    HBM roofline of the main kernel, its counter traffic and VALU issue when
    profiled on the current source, and the oracle on a bounded sample."""
    wl = W.WORKLOADS[idx]
    B, D, L, N = wl.B, wl.D, wl.L, wl.N
    p = W.scan_inputs(wl)
    dev = torch.device("cuda:0")
    bf = wl.io == "bf16"
    io_t = torch.bfloat16 if bf else torch.float32
    T = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    x, dt, z = T(p["x"], io_t), T(p["dt"], io_t), T(p["z"], io_t)
    Bm, Cm = T(p["Bm"], io_t), T(p["Cm"], io_t)
    A, bias, Dk = T(p["A"]), T(p["dt_bias"]), T(p["Dskip"])
    y = torch.empty_like(x)
    ws = torch.empty(max(1, mamba.selective_scan_fwd_workspace_size(B, D, L, N)),
                     dtype=torch.uint8, device=dev)

    def step():
        mamba.selective_scan_fwd(x, dt, A, Bm, Cm, bias, Dk, z, out=y, workspace=ws)

    settle = settle_clocks(step, torch, settle_s)
    for _ in range(warmup):
        step()
    ms_step, k_all = time_with_scan_events(step, torch, mamba, steps)
    k_ms = float(np.mean(k_all))
    elems = B * D * L
    sb = scan_bytes(B, D, L, N, 2 if bf else 4)
    achieved = sb / (k_ms * 1e-3) / 1e9
    tr = traffic_record(wl.name)
    out = {"config": {"batch": B, "d_inner": D, "seq_len": L, "d_state": N, "io": wl.io,
                      "state": "f32"},
           "step_gelem_s": round(elems / (ms_step * 1e-3) / 1e9, 3),
           "ms_per_step": round(ms_step, 4), "steps": steps, "warmup": warmup,
           "clock_settle": settle,
           "roofline": scan_roofline(f"main scan kernel ({wl.io})", wl.io, False, elems, k_ms,
                                     sb, tr),
           "valu": valu_record(tr, elems, k_ms),
           "kernels": {"scan_ms": quantiles(k_all),
                       "scan_gelem_s": round(elems / (k_ms * 1e-3) / 1e9, 2)}}
    if idx == 0:
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": None, "kernel": f"main scan kernel ({wl.io})",
                           "kernel_ms": round(k_ms, 4), "algorithmic_bytes": sb,
                           "note": "0.3 MB problem: cache-resident and launch-latency bound, "
                                   "reported for completeness"}
    if not no_cpu:
        ch = min(D, 64)
        y_rows = y[0:1, :ch].float().cpu().numpy().astype(np.float64)
        out["cpu_baseline"] = cpu_baseline_scan(p, wl, cpu_s, y_rows,
                                                tol=2e-2 if bf else 1e-4)
    del x, dt, z, Bm, Cm, y, ws
    torch.cuda.empty_cache()
    return out


def measure_decode(torch, mamba, W, steps, warmup, settle_s, n_sets, with_conv=False,
                   unfused=False):
    """Decode steps of the [256, 5120, 16] workload, warm and cold, each with the
    state loaded and stored plainly and with the streaming hint
    (MAMBA_STEP_STREAM_STATE).  Warm: one state buffer (84 MB, resident in the
    256 MB MALL between steps).  Cold: n_sets state buffers (and conv windows)
    used in turn, more bytes than the MALL holds, so every step reads its state
    from HBM, as a model whose layers each step their own state does."""
    wl = W.WORKLOADS[4]
    dev = torch.device("cuda:0")
    init = W.decode_initial(wl)
    T = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    hs = [T(init["h0"]) for _ in range(n_sets)]
    A, bias, Dk = T(init["A"]), T(init["dt_bias"]), T(init["Dskip"])
    toks, toks_np = [], []
    for s_ in range(8):
        st = W.decode_step_inputs(wl, s_)
        toks_np.append(st)
        toks.append({k: T(v, torch.bfloat16) for k, v in st.items()})
    y = torch.empty((wl.B, wl.D), dtype=torch.bfloat16, device=dev)
    K = 4
    if with_conv:
        ci = W.decode_conv_initial(wl, K)
        cw = T(ci["conv_w"])
        cstates = [T(ci["conv_state"], torch.bfloat16) for _ in range(n_sets)]
        xc = torch.empty((wl.B, wl.D), dtype=torch.bfloat16, device=dev)

    def step(i, k, stream=False):
        t = toks[i % len(toks)]
        x, h = t["x"], hs[k]
        if with_conv and not unfused:  # conv front end and state update in one kernel
            mamba.conv1d_selective_state_update(h, cstates[k], x, cw, t["dt"], A, t["Bm"],
                                                t["Cm"], dt_bias=bias, Dskip=Dk, z=t["z"],
                                                out=y, stream_state=stream)
            return
        if with_conv:
            mamba.conv1d_update(cstates[k], x, cw, None, out=xc)
            x = xc
        mamba.selective_state_update(h, x, t["dt"], A, t["Bm"], t["Cm"], bias, Dk, t["z"], out=y,
                                     stream_state=stream)

    nbytes = wl.B * wl.D * (2 * wl.N * 4 + 4 * 2) + wl.B * 2 * wl.N * 2 + wl.D * (wl.N + 2) * 4
    if with_conv:  # window read and written (the state update above counts the raw input's
        # read; the conv output never reaches memory when fused)
        nbytes += wl.B * wl.D * 2 * (K - 1) * 2 + wl.D * K * 4
    settle = settle_clocks(lambda: step(0, 0), torch, settle_s)
    res = {}
    for mode, sets, stream in (("warm", 1, False), ("cold", n_sets, False),
                               ("warm_stream", 1, True), ("cold_stream", n_sets, True)):
        for i in range(warmup):
            step(i, i % sets, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i, i % sets, stream)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[mode] = {"ms_per_step": round(ms, 5), "GBps": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "state_sets": sets, "state_set_bytes": hs[0].numel() * 4,
                     "stream_state": stream}
    # the practical roof of the cold step: a plain streaming kernel (torch's
    # elementwise add, in place) over the same state sets in the same turn,
    # reading and writing each 84 MB state once.  Not a multiply: the counter
    # passes scale bytes by torch's multiply kernel of known size, and its name
    # must belong to that one calibration launch.
    for i in range(warmup):
        hs[i % n_sets].add_(0.0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        hs[i % n_sets].add_(0.0)
    e1.record()
    torch.cuda.synchronize()
    cms = e0.elapsed_time(e1) / steps
    cgbs = 2 * hs[0].numel() * 4 / (cms * 1e-3) / 1e9
    res["copy_cold"] = {"ms_per_call": round(cms, 5), "GBps": round(cgbs, 1),
                        "frac": round(cgbs / HBM_PEAK_GBS, 4), "state_sets": n_sets,
                        "what": "torch elementwise add in place over the same state "
                                "sets in turn (reads and writes each state once)"}
    res["cold_stream"]["frac_of_copy"] = round(res["cold_stream"]["GBps"] / cgbs, 4)
    res["clock_settle"] = settle
    res["algorithmic_bytes_per_step"] = nbytes
    res["toks_np"], res["init"] = toks_np, init
    del hs, toks, y
    torch.cuda.empty_cache()
    return res


def run_block(args, torch, mamba, W):
    wl = W.WORKLOADS[1]
    B, D, L, N = wl.B, wl.D, wl.L, wl.N
    K = 4
    p = W.scan_inputs(wl)
    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x_raw, cw = T(p["x_raw"]), T(p["conv_w"])
    dt, A, Bm, Cm = T(p["dt"]), T(p["A"]), T(p["Bm"]), T(p["Cm"])
    bias, Dk, z = T(p["dt_bias"]), T(p["Dskip"]), T(p["z"])
    y = torch.empty_like(x_raw)
    xc = torch.empty_like(x_raw) if args.unfused else None
    ws = torch.empty(mamba.selective_scan_fwd_workspace_size(B, D, L, N), dtype=torch.uint8,
                     device=dev)

    def conv():
        mamba.conv1d_silu(x_raw, cw, None, out=xc)

    def scan():
        if args.unfused:
            mamba.selective_scan_fwd(xc, dt, A, Bm, Cm, bias, Dk, z, out=y, workspace=ws)
        else:
            mamba.conv1d_selective_scan_fwd(x_raw, cw, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dk,
                                            z=z, out=y, workspace=ws)

    def block_step():
        if args.unfused:
            conv()
        scan()

    settle = settle_clocks(block_step, torch, args.settle_seconds)
    for _ in range(args.warmup):
        block_step()
    torch.cuda.synchronize()

    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    conv_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        mamba.set_scan_timing_events_raw(pairs[i][0], pairs[i][1])
        if args.unfused:
            conv_ev[i][0].record()
            conv()
            conv_ev[i][1].record()
        scan()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mamba.set_scan_timing_events_raw(None, None)
    scan_all = [ev.elapsed_ms(a, b) for a, b in pairs]
    scan_ms = float(np.mean(scan_all))
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    ms_step = elapsed / args.steps * 1e3
    elems = B * D * L
    # the fused kernel reads the raw input where the plain scan reads the conv
    # output: the same bytes, plus the conv weights
    sb = scan_bytes(B, D, L, N, 4) + (0 if args.unfused else D * K * 4)
    cb = conv_bytes(B, D, L, K, 4)
    achieved = sb / (scan_ms * 1e-3) / 1e9
    tr = traffic_record("block_unfused" if args.unfused else "block_fused")
    # HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a
    # copy kernel of known size; null once the kernel source has changed
    traffic = traffic_bytes(tr)
    kname = "scan_main_kernel<fp32>" if args.unfused else "scan_main_kernel<fp32, conv>"
    kernels = {"scan_ms": quantiles(scan_all),
               "scan_gelem_s": round(elems / (scan_ms * 1e-3) / 1e9, 2)}
    if args.unfused:
        conv_all = [a.elapsed_time(b) for a, b in conv_ev]
        kernels["conv_ms"] = quantiles(conv_all)
        kernels["conv_GBps"] = round(cb / (float(np.mean(conv_all)) * 1e-3) / 1e9, 1)
    out = {
        "metric": "selective-scan Gelem/s (B*L*D_inner) and HBM GB/s as % of MI355X peak",
        "value": round(elems / (ms_step * 1e-3) / 1e9, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "d_model": 768, "d_inner": D, "seq_len": L,
                   "d_state": N, "d_conv": K, "io": "f32", "state": "f32",
                   "step": ("conv1d_silu, then selective_scan_fwd" if args.unfused else
                            "conv1d_selective_scan_fwd (conv1d+SiLU fused into the scan)")},
        "roofline": scan_roofline(kname, "f32", not args.unfused, elems, scan_ms, sb, tr),
        "valu": valu_record(tr, elems, scan_ms),
        "kernels": kernels,
        "clock_settle": settle,
    }
    if not args.no_cpu:
        y0 = y[0:1, :4].double().cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(p, B, D, L, y_gpu=y0)
    if not args.headline_only:
        del x_raw, cw, dt, A, Bm, Cm, bias, Dk, z, y, xc, ws
        torch.cuda.empty_cache()
        out["other_workloads"] = other_workloads(args, torch, mamba, W)
    return out


def other_workloads(args, torch, mamba, W):
    """The other configurations of the hot path, measured in the same run
    beside the headline: the 2.8B-scale layer and the long sequence (bf16 scans
    whose inputs far exceed the MALL), the small fp32 case, and the decode
    workload warm and cold, each with its roofline and an oracle baseline."""
    res = {}
    for idx in (2, 3, 0):
        wl = W.WORKLOADS[idx]
        res[wl.name] = measure_scan(torch, mamba, W, idx, steps=20, warmup=10,
                                    settle_s=min(args.settle_seconds, 0.5), cpu_s=4.0,
                                    no_cpu=args.no_cpu)
    wl = W.WORKLOADS[4]
    d = measure_decode(torch, mamba, W, steps=200, warmup=20,
                       settle_s=min(args.settle_seconds, 0.5), n_sets=args.decode_sets)
    toks_np, init = d.pop("toks_np"), d.pop("init")
    d["roofline"] = {"bound": "hbm", "achieved": d["cold_stream"]["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": d["cold_stream"]["frac"],
                     "traffic": traffic_bytes(traffic_record(wl.name)),
                     "kernel": "state update (cold: state read from HBM every step; "
                               "streaming hint)"}
    if not args.no_cpu:
        d["cpu_baseline"] = cpu_baseline_decode(wl, init, toks_np,
                                                d["algorithmic_bytes_per_step"], target_s=4.0)
    res[wl.name] = d
    return res


def run_scan(args, torch, mamba, W, idx, bidir=False, general=False):
    """One workload's scan as the JSON line.  bidir: the forward scan, then the
    reverse scan of a second parameter set added into the same y (a
    bidirectional layer); general: A[d, n] ~ -U(0.05, 5) with no structure
    across n (as after training), which takes the general path."""
    wl = W.WORKLOADS[idx]
    B, D, L, N = wl.B, wl.D, wl.L, wl.N
    line = {"metric": "selective-scan Gelem/s (B*L*D_inner) and HBM GB/s as % of MI355X peak",
            "unit": "Gelem/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16-io/f32" if wl.io == "bf16" else "f32", "data": "synthetic"}
    if not bidir and not general:
        m = measure_scan(torch, mamba, W, idx, args.steps, args.warmup, args.settle_seconds,
                         cpu_s=15.0, no_cpu=args.no_cpu)
        line.update(value=m.pop("step_gelem_s"), ms_per_step=m.pop("ms_per_step"))
        m.pop("steps"), m.pop("warmup")
        cfg = m.pop("config")
        line["config"] = {"workload": wl.name, **cfg, "step": "forward scan"}
        line.update(m)
        return line
    p = W.scan_inputs(wl)
    if general:
        p["A"] = (-np.random.default_rng(wl.seed + 77).uniform(0.05, 5.0, size=(D, N))).astype(
            np.float32)
    dev = torch.device("cuda:0")
    bf = wl.io == "bf16"
    io_t = torch.bfloat16 if bf else torch.float32
    T = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    x, dt, z = T(p["x"], io_t), T(p["dt"], io_t), T(p["z"], io_t)
    Bm, Cm = T(p["Bm"], io_t), T(p["Cm"], io_t)
    A, bias, Dk = T(p["A"]), T(p["dt_bias"]), T(p["Dskip"])
    y = torch.empty_like(x)
    ws = torch.empty(mamba.selective_scan_fwd_workspace_size(B, D, L, N), dtype=torch.uint8,
                     device=dev)
    if bidir:
        q = W.make_scan_inputs(B, D, L, N, wl.io, wl.seed + 500)
        dt2, Bm2, Cm2 = T(q["dt"], io_t), T(q["Bm"], io_t), T(q["Cm"], io_t)
        A2, bias2, Dk2 = T(q["A"]), T(q["dt_bias"]), T(q["Dskip"])

    def step():
        mamba.selective_scan_fwd(x, dt, A, Bm, Cm, bias, Dk, z, out=y, workspace=ws)
        if bidir:
            mamba.set_scan_timing_events_raw(None, None)
            mamba.selective_scan_fwd(x, dt2, A2, Bm2, Cm2, bias2, Dk2, z, out=y, workspace=ws,
                                     reverse=True, accumulate=True)

    settle = settle_clocks(step, torch, args.settle_seconds)
    for _ in range(args.warmup):
        step()
    ms_step, scan_all = time_with_scan_events(step, torch, mamba, args.steps)
    scan_ms = float(np.mean(scan_all))
    elems = B * D * L
    sb = scan_bytes(B, D, L, N, 2 if bf else 4)
    achieved = sb / (scan_ms * 1e-3) / 1e9
    key = wl.name + ("_bidirectional" if bidir else "") + ("_general_A" if general else "")
    tr = traffic_record(key)
    line.update({
        "value": round(elems * (2 if bidir else 1) / (ms_step * 1e-3) / 1e9, 3),
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": key, "batch": B, "d_inner": D, "seq_len": L, "d_state": N,
                   "io": wl.io,
                   "step": ("forward scan, then reverse scan added into y" if bidir else
                            "forward scan"),
                   "elements_per_step": elems * (2 if bidir else 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes(tr), "kernel_ms": round(scan_ms, 4),
                     "algorithmic_bytes": sb,
                     "kernel": "main scan kernel of the forward call"},
        "valu": valu_record(tr, elems, scan_ms),
        "kernels": {"scan_ms": quantiles(scan_all),
                    "scan_gelem_s": round(elems / (scan_ms * 1e-3) / 1e9, 2)},
        "clock_settle": settle})
    if general and not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_scan(
            p, wl, 15.0, y[0:1, :64].float().cpu().numpy().astype(np.float64),
            tol=2e-2 if bf else 1e-4)
    return line


def run_bwd(args, torch, mamba, W):
    """The scan's backward pass (gradients of every input, states recomputed)
    at the block's scan shape: B=2, D_inner=1536, L=8192, N=16, fp32 I/O."""
    wl = W.WORKLOADS[1]
    B, D, L, N = wl.B, wl.D, wl.L, wl.N
    p = W.make_scan_inputs(B, D, L, N, "f32", wl.seed)
    rng = np.random.default_rng(wl.seed + 7)
    dout_np = rng.standard_normal((B, D, L)).astype(np.float32)
    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, dt, z, dout = T(p["x"]), T(p["dt"]), T(p["z"]), T(dout_np)
    Bm, Cm, A, bias, Dk = T(p["Bm"]), T(p["Cm"]), T(p["A"]), T(p["dt_bias"]), T(p["Dskip"])
    ws = torch.empty(mamba.selective_scan_bwd_workspace_size(B, D, L, N), dtype=torch.uint8,
                     device=dev)

    def step(pair=None):
        if pair is not None:
            mamba.set_scan_timing_events_raw(pair[0], pair[1])
        mamba.selective_scan_bwd(x, dt, A, Bm, Cm, dout, bias, Dk, z, workspace=ws)

    settle = settle_clocks(step, torch, args.settle_seconds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mamba.set_scan_timing_events_raw(None, None)
    k_all = [ev.elapsed_ms(a, b) for a, b in pairs]
    k_ms = float(np.mean(k_all))
    ms_step = elapsed / args.steps * 1e3
    elems = B * D * L
    return {"metric": "selective-scan backward Gelem/s (B*L*D_inner)",
            "value": round(elems / (ms_step * 1e-3) / 1e9, 3), "unit": "Gelem/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "clock_settle": settle, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": f"scan_bwd_b{B}_d{D}_l{L}_n{N}_f32", "batch": B,
                       "d_inner": D, "seq_len": L, "d_state": N, "io": "f32",
                       "step": "forward recompute, adjoint scan, chunk gradients, reductions"},
            # the chunk-gradient kernel is bound by fp32 arithmetic: 30 flops of the
            # formulas per (element, state) (recompute 7, gradients 23; an fma counts
            # 2, exp and reciprocal 1), against the fp32 vector peak without packed
            # math (one wave64 fma per clock per CU: 78.6 TFLOP/s)
            "roofline": {"bound": "alu", "achieved": round(30 * elems * N / (k_ms * 1e-3) / 1e12, 2),
                         "peak": round(FP32_NOPACK_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                         "frac": round(30 * elems * N / (k_ms * 1e-3) / 1e12 / FP32_NOPACK_PEAK_TFLOPS, 4),
                         "traffic": traffic_bytes(traffic_record(f"scan_bwd_b{B}_d{D}_l{L}_n{N}_f32")),
                         "kernel": "scan_bwd_chunk_kernel<fp32>",
                         "kernel_ms": round(k_ms, 4), "algorithmic_flops": 30 * elems * N},
            "kernels": {"chunk_grad_ms": quantiles(k_all),
                        "chunk_grad_gelem_s": round(elems / (k_ms * 1e-3) / 1e9, 2)},
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline_bwd(p, dout_np, B, D, L)})}


def run_ssd(args, torch, mamba, W):
    """The Mamba-2 form of the scan (one decay per head, B/C per group) on the
    matrix cores: B=8, L=2048, 80 heads of 64 channels (d_inner 5120), G=1,
    N=64, bf16 I/O."""
    wl = W.SSD_WORKLOAD
    p = W.ssd_inputs(wl)
    dev = torch.device("cuda:0")
    T = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)
    bf = torch.bfloat16
    x, z, dt = T(p["x"], bf), T(p["z"], bf), T(p["dt"], bf)
    Bm, Cm = T(p["Bm"], bf), T(p["Cm"], bf)
    A, bias, Dk = T(p["A"]), T(p["dt_bias"]), T(p["Dskip"])
    y = torch.empty_like(x)

    def step(pair=None):
        if pair is not None:
            mamba.set_scan_timing_events_raw(pair[0], pair[1])
        mamba.ssd_scan_fwd(x, dt, A, Bm, Cm, bias, Dk, z, out=y)

    settle = settle_clocks(step, torch, args.settle_seconds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mamba.set_scan_timing_events_raw(None, None)
    k_all = [ev.elapsed_ms(a, b) for a, b in pairs]
    k_ms = float(np.mean(k_all))
    ms_step = elapsed / args.steps * 1e3
    elems = wl.elems
    # algorithmic bytes: x, z read and y written (bf16), dt per (b, t, h), B and C
    # per (b, t, g), A / dt_bias / D per head
    nbytes = (3 * elems * 2 + wl.B * wl.L * wl.H * 2 + 2 * wl.B * wl.L * wl.G * wl.N * 2
              + 3 * wl.H * 4)
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    # matrix work of the chunked form per Q-step chunk and head (the kernel's
    # chunk: 32 steps for N >= 32): the causal C B^T and M x (Q(Q+1)/2 entries
    # each), the chunk state and C H
    Q = 64 if wl.N == 16 else 32
    chunks = wl.B * wl.H * ((wl.L + Q - 1) // Q)
    flops = chunks * (2 * (Q * (Q + 1) // 2) * (wl.N + wl.P) + 2 * 2 * Q * wl.N * wl.P)
    return {"metric": "Mamba-2 form scan Gelem/s (B*L*H*P) and HBM GB/s as % of MI355X peak",
            "value": round(elems / (ms_step * 1e-3) / 1e9, 3), "unit": "Gelem/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "clock_settle": settle, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16-io/f32", "data": "synthetic",
            "config": {"workload": wl.name, "batch": wl.B, "seq_len": wl.L, "heads": wl.H,
                       "head_dim": wl.P, "groups": wl.G, "d_state": wl.N,
                       "step": "ssd_scan_fwd (chunked Mamba-2 form, bf16 MFMA)"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_bytes(traffic_record(wl.name)),
                         "kernel": f"ssd_fwd_kernel<N={wl.N}, Q={Q}>", "kernel_ms": round(k_ms, 4),
                         "algorithmic_bytes": nbytes},
            "mfma": {"achieved_tflops": round(flops / (k_ms * 1e-3) / 1e12, 2),
                     "peak_tflops": 2500.0, "frac": round(flops / (k_ms * 1e-3) / 2.5e15, 4),
                     "algorithmic_flops": flops},
            "kernels": {"ssd_ms": quantiles(k_all),
                        "ssd_gelem_s": round(elems / (k_ms * 1e-3) / 1e9, 2)},
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline_ssd(p, wl)})}


def run_decode(args, torch, mamba, W):
    wl = W.WORKLOADS[4]
    K = 4
    d = measure_decode(torch, mamba, W, args.steps, args.warmup, args.settle_seconds,
                       args.decode_sets, with_conv=args.with_conv, unfused=args.unfused)
    toks_np, init = d.pop("toks_np"), d.pop("init")
    nbytes = d["algorithmic_bytes_per_step"]
    # the serving setting: every step's state comes from HBM (a model's layers
    # each step their own state), stepped with the streaming hint
    cold = d["cold_stream"]
    metric = ("decode step (conv update + state update) GB/s" if args.with_conv else
              "decode state update GB/s")
    key = wl.name + ("_conv" if args.with_conv else "")
    return {"metric": metric, "value": cold["GBps"], "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": cold["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16-io/f32", "data": "synthetic",
            "config": {"workload": wl.name, "batch": wl.B, "d_inner": wl.D, "d_state": wl.N,
                       "state_sets": args.decode_sets, "state_hint": "stream",
                       **({"d_conv": K,
                           "step": ("conv1d_update, then selective_state_update" if args.unfused
                                    else "conv1d_selective_state_update (one kernel)")}
                          if args.with_conv else {})},
            "roofline": {"bound": "hbm", "achieved": cold["GBps"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": cold["frac"],
                         "traffic": traffic_bytes(traffic_record(key)),
                         "note": (f"cold: {args.decode_sets} state sets of "
                                  f"{cold['state_set_bytes'] / 1e6:.0f} MB used in turn, more "
                                  "than the 256 MB MALL holds; h loaded and stored with "
                                  "MAMBA_STEP_STREAM_STATE")},
            "warm": d["warm"], "cold": d["cold"], "warm_stream": d["warm_stream"],
            "cold_stream": cold, "copy_cold": d["copy_cold"], "clock_settle": d["clock_settle"],
            "algorithmic_bytes_per_step": nbytes,
            **({} if args.no_cpu else {"cpu_baseline": cpu_baseline_decode(
                wl, init, toks_np, nbytes, W.decode_conv_initial(wl, K) if args.with_conv
                else None)})}


PROBE_LIBRARY = os.path.join(ROOT, "selective_state_space_80_amd", "libmamba_probe.so")
PROBE_MODES = ((0, "8 independent fma chains", 8),
               (1, "8 chains of exp2 then mul", 16),
               (2, "1 exp2 chain and 7 fma chains", 8))


def run_probe_valu(torch):
    """The VALU issue-rate probe behind the roofline's peak: independent chains
    per lane (libmamba_probe.so, built without packed fp32 like the kernels) at
    2, 3, 4 and 8 waves per SIMD, timed with events on the launch stream.
    Reports wave64 VALU instructions per clock per CU at the 2.4 GHz peak clock,
    and the clocks one round of 8 chain steps takes per CU."""
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.mamba_probe_valu_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for mode, what, instr_per_round in PROBE_MODES:
        for wgs in (2, 3, 4, 8):
            grid = n_cu * wgs * 8  # eight workgroups per resident slot
            out = torch.empty(grid * 256, dtype=torch.float32, device="cuda:0")
            if lib.mamba_probe_valu_launch(out.data_ptr(), mode, grid, wgs, 200, stream) != 0:
                raise RuntimeError("probe launch failed")
            times = []
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                if lib.mamba_probe_valu_launch(out.data_ptr(), mode, grid, wgs, iters,
                                               stream) != 0:
                    raise RuntimeError("probe launch failed")
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = min(times)
            rounds = grid * 4 * iters * 16  # wave-level rounds of 8 chain steps
            clocks = ms * 1e-3 * 2.4e9 * n_cu
            rows.append({"mode": what, "waves_per_simd": wgs, "ms": round(ms, 3),
                         "instr_per_clock_per_cu": round(rounds * instr_per_round / clocks, 3),
                         "clocks_per_round_per_cu": round(clocks / rounds, 2)})
            del out
    return {"metric": "VALU issue probe", "unit": "wave64 VALU instructions per clock per CU "
            "at 2.4 GHz", "n_cu": n_cu, "packed_fp32": False, "results": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU takes tens of milliseconds of work to reach its steady clocks:
    # fewer warm-up steps time a partly clocked-down GPU
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="block",
                    choices=["block", "scan_bf16_l2048", "scan_bf16_l131072", "decode",
                             "bidir_bf16_l2048", "bwd", "ssd", "scan_bf16_l2048_general"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--unfused", action="store_true",
                    help="block workload: run conv1d_silu and selective_scan_fwd as two calls "
                         "instead of the fused entry point; decode --with-conv: conv1d_update "
                         "and selective_state_update as two calls")
    ap.add_argument("--with-conv", action="store_true",
                    help="decode workload: each step runs the conv front end's decode step "
                         "(K = 4) on the token's raw input, then the state update, fused into "
                         "one kernel (conv1d_selective_state_update)")
    ap.add_argument("--headline-only", action="store_true",
                    help="block workload: skip the other configurations")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed back-to-back steps before the warm-up, for steady clocks")
    ap.add_argument("--decode-sets", type=int, default=8,
                    help="decode: state buffers used in turn for the cold figure (8 x 84 MB)")
    ap.add_argument("--probe-valu", action="store_true",
                    help="instead of a workload, run the VALU issue-rate probe that the "
                         "roofline's peak rests on (libmamba_probe.so)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one elementwise kernel that reads and writes "
                         "this many MiB (known traffic for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the hot path "
              "shards over batch/channels with no communication between GPUs", file=sys.stderr)
        sys.exit(2)
    import torch

    import selective_state_space_80_amd as mamba
    from selective_state_space_80_amd import workloads as W

    mamba.load_library()
    if args.probe_valu:
        print(json.dumps(run_probe_valu(torch)), flush=True)
        return
    if args.copy_calibration_mib:
        # one plain streaming kernel (torch's elementwise multiply) that reads
        # and writes exactly this many bytes with ordinary loads and stores
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "block":
        out = run_block(args, torch, mamba, W)
    elif args.workload == "scan_bf16_l2048":
        out = run_scan(args, torch, mamba, W, 2)
    elif args.workload == "scan_bf16_l131072":
        out = run_scan(args, torch, mamba, W, 3)
    elif args.workload == "scan_bf16_l2048_general":
        out = run_scan(args, torch, mamba, W, 2, general=True)
    elif args.workload == "bidir_bf16_l2048":
        out = run_scan(args, torch, mamba, W, 2, bidir=True)
    elif args.workload == "bwd":
        out = run_bwd(args, torch, mamba, W)
    elif args.workload == "ssd":
        out = run_ssd(args, torch, mamba, W)
    else:
        out = run_decode(args, torch, mamba, W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
