"""Host-side logic of the benchmark and of the profile summaries: the one-GPU
guard, the scaling of rocprofv3 byte counters by the copy calibration, and the
rule that counter traffic is reported only for the kernel source it was taken
on."""
import hashlib
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
    assert rec["source_sha256"] == hashlib.sha256(src.read_bytes()).hexdigest()


def test_traffic_record_only_for_the_current_source(tmp_path, monkeypatch):
    src = os.path.join("selective_state_space_80_amd", "csrc", "state_update.hip")
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    rec = {"kernel": "k", "fetch_bytes": 100.4, "write_bytes": 50.2, "source": src}
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps({"cur": dict(rec, source_sha256=sha),
                                 "old": dict(rec, source_sha256="0" * 64),
                                 "nosrc": {"kernel": "k", "fetch_bytes": 1.0,
                                           "write_bytes": 1.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.traffic_bytes(bench.traffic_record("cur")) == 151
    assert bench.traffic_record("old") is None      # counters of an older kernel
    assert bench.traffic_record("nosrc") is None    # no source to check against
    assert bench.traffic_record("missing") is None
    assert bench.traffic_bytes(None) is None

