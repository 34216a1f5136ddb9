"""Summaries of rocprofv3 result databases (SQLite, ``*_results.db``).

    python -m selective_state_space_80_amd.profiling trace  RESULTS.db
    python -m selective_state_space_80_amd.profiling counters RESULTS.db [RESULTS.db ...]
    python -m selective_state_space_80_amd.profiling traffic --fetch F.db --write W.db \
        --copy-bytes N --kernel KERNEL --source SRC [--sq SQ.db] [--variant WORKLOAD] \
        --out profiles/traffic.json

(``traffic`` also takes the text that ``counters`` prints in place of each database.)

``trace`` prints per-kernel call counts and average durations in microseconds (from
``rocprofv3 --kernel-trace --stats``); ``counters`` prints per-kernel averages of
every counter collected with ``--pmc`` (summed over the per-XCD/SE rows of a
dispatch, averaged over dispatches); ``traffic`` turns FETCH_SIZE / WRITE_SIZE
(KiB per dispatch) into bytes, scaled so that a plain streaming kernel of the
same run (bench.py --copy-calibration-mib: torch's elementwise multiply), which
reads and writes a known number of bytes, reads and writes exactly that.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3
import sys

_LOCAL_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def source_digest(source):
    """sha256 over a kernel source and the local headers it includes
    (``#include "..."`` found beside it, recursively, each once, in the order
    first met): counters describe the compiled kernel, so a change to a shared
    device header makes them as stale as a change to the source itself."""
    h = hashlib.sha256()
    seen = set()

    def add(path):
        path = os.path.abspath(path)
        if path in seen or not os.path.isfile(path):
            return
        seen.add(path)
        text = open(path, "rb").read()
        h.update(os.path.basename(path).encode() + b"\0" + text + b"\0")
        for inc in _LOCAL_INCLUDE.findall(text.decode("utf-8", "replace")):
            add(os.path.join(os.path.dirname(path), inc))

    add(source)
    return h.hexdigest()


COPY_KERNEL = "MulFunctor"  # torch elementwise multiply: reads N bytes, writes N bytes


def short_name(kernel: str) -> str:
    if COPY_KERNEL in kernel:
        return "calibration_" + COPY_KERNEL
    k = kernel.replace("(anonymous namespace)", "anon")
    m = re.search(r"::(\w+)(<[^>]*>)?\(", k)
    if m:
        return m.group(1) + (m.group(2) or "")
    return k.split("(")[0][:60]


def kernel_trace(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels").fetchall()
    return [(short_name(n), int(c), float(t), float(a), float(p)) for n, c, t, a, p in rows]


def counters_text(path: str):
    """The same dictionary, read back from the text that ``counters`` prints
    (several passes may follow each other in one file: a kernel's counters are
    merged; lines starting with '#' are comments)."""
    out, cur = {}, None
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        if line.startswith(" "):
            parts = line.split()
            if len(parts) == 2 and cur is not None:
                try:
                    out[cur][parts[0]] = float(parts[1].replace(",", ""))
                except ValueError:
                    pass
        elif not line.startswith(("traffic", "{", "}")):
            cur = line.strip()
            out.setdefault(cur, {})
    return out


def counters(db: str):
    """{kernel: {counter: mean over dispatches of the per-dispatch total}}
    from a rocprofv3 database, or from a ``counters`` text summary (.txt)."""
    if db.endswith(".txt"):
        return counters_text(db)
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, counter_name, value "
                       "from counters_collection").fetchall()
    per_dispatch = collections.defaultdict(float)
    names = {}
    for did, kn, cn, v in rows:
        per_dispatch[(did, cn)] += float(v)
        names[did] = kn
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for (did, cn), v in per_dispatch.items():
        acc[short_name(names[did])][cn].append(v)
    out = {k: {cn: sum(v) / len(v) for cn, v in d.items()} for k, d in acc.items()}
    for k, d in acc.items():
        out[k]["dispatches"] = float(max(len(v) for v in d.values()))
    return out


def _find(d, sub):
    for k, v in d.items():
        if sub in k:
            return v
    raise KeyError(sub)


def traffic(fetch_db, write_db, copy_bytes, kernel, source=None, sq_db=None):
    f = counters(fetch_db)
    w = counters(write_db)
    for d in (f, w):
        # the scale rests on one launch of known size: an average with other
        # launches of the same kernel would scale by the wrong bytes
        if _find(d, COPY_KERNEL).get("dispatches", 1.0) != 1.0:
            raise ValueError("the calibration kernel %s was launched %d times in one pass"
                             % (COPY_KERNEL, _find(d, COPY_KERNEL)["dispatches"]))
    copy_f = _find(f, COPY_KERNEL)["FETCH_SIZE"] * 1024.0
    copy_w = _find(w, COPY_KERNEL)["WRITE_SIZE"] * 1024.0
    kf = _find(f, kernel)["FETCH_SIZE"] * 1024.0
    kw = _find(w, kernel)["WRITE_SIZE"] * 1024.0
    out = {"kernel": kernel, "copy_bytes": copy_bytes,
           "copy_fetch_raw_bytes": copy_f, "copy_write_raw_bytes": copy_w,
           "fetch_scale": copy_bytes / copy_f, "write_scale": copy_bytes / copy_w,
           "fetch_raw_bytes": kf, "write_raw_bytes": kw,
           "fetch_bytes": kf * copy_bytes / copy_f, "write_bytes": kw * copy_bytes / copy_w}
    if sq_db:
        sq = _find(counters(sq_db), kernel)
        out["valu_insts"] = sq["SQ_INSTS_VALU"]
        out["waves"] = sq["SQ_WAVES"]
        # VALU busy time in wave64 issue cycles of a CU (one fp32 operation
        # per cycle, two for a transcendental)
        if "SQ_ACTIVE_INST_VALU" in sq:
            out["valu_active"] = sq["SQ_ACTIVE_INST_VALU"]
    if source:
        out["source"] = os.path.relpath(source, os.path.dirname(os.path.dirname(
            os.path.abspath(__file__))))
        out["source_digest"] = source_digest(source)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    c = sub.add_parser("counters")
    c.add_argument("db", nargs="+")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--copy-bytes", type=int, required=True)
    tr.add_argument("--kernel", default="scan_main_kernel")
    tr.add_argument("--source", default=None, help="kernel source to fingerprint")
    tr.add_argument("--sq", default=None,
                    help="run with SQ_INSTS_VALU, SQ_WAVES (and SQ_ACTIVE_INST_VALU)")
    tr.add_argument("--variant", default="block_fused",
                    help="key of the record in --out: the workload it was taken on")
    tr.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(f"{'kernel':44s} {'calls':>6s} {'avg_us':>10s} {'total_us':>11s} {'pct':>6s}")
        for n, calls, tot, avg, pct in kernel_trace(a.db):
            print(f"{n:44s} {calls:6d} {avg:10.2f} {tot:11.1f} {pct:6.2f}")
    elif a.cmd == "counters":
        merged = collections.defaultdict(dict)
        for db in a.db:
            for k, d in counters(db).items():
                merged[k].update(d)
        for k, d in merged.items():
            print(k)
            for cn, v in sorted(d.items()):
                print(f"    {cn:28s} {v:18,.0f}")
    else:
        rec = traffic(a.fetch, a.write, a.copy_bytes, a.kernel, a.source, a.sq)
        print(json.dumps(rec, indent=1))
        if a.out:
            try:
                allrec = json.load(open(a.out))
                if "kernel" in allrec:  # a single record of an older layout
                    allrec = {}
            except (OSError, ValueError):
                allrec = {}
            allrec[a.variant] = rec
            os.makedirs(os.path.dirname(a.out) or ".", exist_ok=True)
            with open(a.out, "w") as fh:
                fh.write(json.dumps(allrec, indent=1) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
