"""Host-side logic of the benchmark and of the profile summaries: the one-GPU
guard, the scaling of rocprofv3 byte counters by the copy calibration, and the
rule that counter traffic is reported only for the kernel source it was taken
on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from selective_state_space_80_amd import profiling  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


COUNTERS = """# a comment line
calibration_MulFunctor
    FETCH_SIZE                              262,144
    WRITE_SIZE                              524,288
state_update_quad_kernel<true, 2, 0, false>
    FETCH_SIZE                               50,000
state_update_quad_kernel<true, 2, 0, true>
    FETCH_SIZE                               45,000
    WRITE_SIZE                               84,000
    SQ_INSTS_VALU                        10,240,000
    SQ_WAVES                                 40,960
traffic (scaled by the copy calibration), per dispatch of state_update_quad_kernel<true, 2, 0, true>:
    fetch    92.2 MB   write    86.0 MB
"""


def test_counter_text_is_read_back_per_kernel(tmp_path):
    f = tmp_path / "c.txt"
    f.write_text(COUNTERS)
    d = profiling.counters(str(f))
    assert d["calibration_MulFunctor"] == {"FETCH_SIZE": 262144.0, "WRITE_SIZE": 524288.0}
    assert d["state_update_quad_kernel<true, 2, 0, false>"] == {"FETCH_SIZE": 50000.0}
    k = d["state_update_quad_kernel<true, 2, 0, true>"]
    assert k["FETCH_SIZE"] == 45000.0 and k["WRITE_SIZE"] == 84000.0
    assert k["SQ_INSTS_VALU"] == 10240000.0 and k["SQ_WAVES"] == 40960.0


def test_traffic_refuses_a_calibration_kernel_launched_more_than_once(tmp_path):
    """The counters of a database keep each kernel's dispatch count; a pass in
    which the calibration kernel ran twice (another multiply beside the one of
    known size) cannot scale bytes, and the traffic step says so."""
    import sqlite3
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(str(db))
    con.execute("create table counters_collection (dispatch_id, kernel_name, counter_name, value)")
    rows = [(1, "void at::native::elementwise<MulFunctor<float>>(int)", "FETCH_SIZE", 262144.0),
            (2, "void at::native::elementwise<MulFunctor<float>>(int)", "FETCH_SIZE", 20000.0),
            (3, "mamba::foo_kernel(int)", "FETCH_SIZE", 1000.0),
            (3, "mamba::foo_kernel(int)", "FETCH_SIZE", 500.0)]  # two XCD rows: summed
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    d = profiling.counters(str(db))
    assert d["calibration_MulFunctor"]["dispatches"] == 2.0
    assert d["calibration_MulFunctor"]["FETCH_SIZE"] == pytest.approx(141072.0)
    assert d["foo_kernel"] == {"FETCH_SIZE": 1500.0, "dispatches": 1.0}
    with pytest.raises(ValueError, match="launched 2 times"):
        profiling.traffic(str(db), str(db), 512 << 20, "foo_kernel")


def test_traffic_is_scaled_by_the_copy_kernel(tmp_path):
    """A copy of 512 MiB that the counters see as 256 MiB fetched and 512 MiB
    written gives scales 2 and 1; the kernel's KiB are scaled alike, and the
    hinted kernel is not confused with the plain one of the same prefix."""
    f = tmp_path / "c.txt"
    f.write_text(COUNTERS)
    src = tmp_path / "k.hip"
    src.write_text("// kernel source\n")
    rec = profiling.traffic(str(f), str(f), 512 << 20, "state_update_quad_kernel<true, 2, 0, true>",
                            source=str(src), sq_db=str(f))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(45000 * 1024 * 2.0)
    assert rec["write_bytes"] == pytest.approx(84000 * 1024 * 1.0)
    assert rec["valu_insts"] == 10240000.0 and rec["waves"] == 40960.0
    assert rec["source_digest"] == profiling.source_digest(str(src))


def test_source_digest_follows_local_includes(tmp_path):
    """The digest changes with the source and with a local header it includes,
    directly or through another header, and not with an unrelated file."""
    (tmp_path / "k.hip").write_text('#include "a.h"\n#include <hip/hip_runtime.h>\nk\n')
    (tmp_path / "a.h").write_text('#include "b.h"\na\n')
    (tmp_path / "b.h").write_text("b\n")
    (tmp_path / "c.h").write_text("c\n")
    k = str(tmp_path / "k.hip")
    d0 = profiling.source_digest(k)
    (tmp_path / "c.h").write_text("c changed\n")
    assert profiling.source_digest(k) == d0
    (tmp_path / "b.h").write_text("b changed\n")
    d1 = profiling.source_digest(k)
    assert d1 != d0
    (tmp_path / "k.hip").write_text('#include "a.h"\n#include <hip/hip_runtime.h>\nk2\n')
    assert profiling.source_digest(k) != d1


def test_traffic_record_only_for_the_current_source(tmp_path, monkeypatch):
    src = os.path.join("selective_state_space_80_amd", "csrc", "state_update.hip")
    dig = profiling.source_digest(os.path.join(ROOT, src))
    rec = {"kernel": "k", "fetch_bytes": 100.4, "write_bytes": 50.2, "source": src}
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps({"cur": dict(rec, source_digest=dig),
                                 "old": dict(rec, source_digest="0" * 64),
                                 "nosrc": {"kernel": "k", "fetch_bytes": 1.0,
                                           "write_bytes": 1.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.traffic_bytes(bench.traffic_record("cur")) == 151
    assert bench.traffic_record("old") is None      # counters of an older kernel
    assert bench.traffic_record("nosrc") is None    # no source to check against
    assert bench.traffic_record("missing") is None
    assert bench.traffic_bytes(None) is None



def test_valu_peak_is_one_wave64_instruction_per_clock_per_cu():
    """Without packed fp32 a CU issues one wave64 VALU instruction per clock:
    256 CUs at 2.4 GHz; twice that rate in fma flops with packed math is the
    published 157.3 TFLOP/s fp32 vector peak."""
    assert bench.VALU_ISSUE_PEAK == pytest.approx(614.4e9)
    assert bench.FP32_NOPACK_PEAK_TFLOPS * 2 == pytest.approx(157.3, rel=1e-3)


def test_scan_roofline_is_the_alu_roof_with_hbm_beside_it():
    # design count per element: fp32 plain, bf16, fp32 with the fused conv
    assert bench.scan_valu_per_elem("f32") == pytest.approx(133.375)
    assert bench.scan_valu_per_elem("bf16") == pytest.approx(136.875)
    assert bench.scan_valu_per_elem("f32", conv=True) == pytest.approx(142.375)
    elems, ms, nbytes = 64 * 1000 * 1000, 0.25, 8 * 64 * 10 ** 6
    tr = {"fetch_bytes": 600.0e6, "write_bytes": 200.0e6, "valu_insts": 140.0e6,
          "valu_active": 146.0e6}
    r = bench.scan_roofline("k", "bf16", False, elems, ms, nbytes, tr)
    assert r["bound"] == "alu"
    # 136.875 instructions per element x 1e6 wave-steps in 0.25 ms
    assert r["achieved"] == pytest.approx(136.875e6 / 0.25e-3 / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(136.875e6 / 0.25e-3 / 614.4e9, abs=1e-4)
    assert r["traffic"] == 800000000
    assert r["hbm"]["frac"] == pytest.approx(nbytes / 0.25e-3 / 8e12, abs=1e-4)
    v = bench.valu_record(tr, elems, ms)
    assert v["wave_instr_per_elem"] == pytest.approx(140.0)
    assert v["frac"] == pytest.approx(140e6 / 0.25e-3 / 614.4e9, abs=1e-4)
    assert v["busy_frac"] == pytest.approx(146e6 / 0.25e-3 / 614.4e9, abs=1e-4)


def test_probe_library_exports_its_launch():
    """The issue-rate probe is built beside the library (build() links it) and
    exports its one launch function; no GPU call here."""
    import ctypes
    if not os.path.exists(bench.PROBE_LIBRARY):
        pytest.skip("libmamba_probe.so not built")
    lib = ctypes.CDLL(bench.PROBE_LIBRARY)
    assert hasattr(lib, "mamba_probe_valu_launch")
