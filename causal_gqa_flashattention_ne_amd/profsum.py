"""Summaries of rocprofv3 output.

    python -m causal_gqa_flashattention_ne_amd.profsum <results.db | kernel_stats.csv>
        one line per kernel: dispatch count, average / min / max duration in microseconds.
    python -m causal_gqa_flashattention_ne_amd.profsum traffic <FETCH_SIZE dir> <WRITE_SIZE dir> <out.json>
        per-kernel HBM bytes per dispatch from two counter runs (--pmc FETCH_SIZE, then
        --pmc WRITE_SIZE) of `bench.py --copy-calibration`, each scaled by what the same counter
        reads for the calibration copy (256 MiB read + 256 MiB written per launch), tagged with a
        hash of each kernel's sources so that the benchmark stops quoting it once that kernel changes.
    python -m causal_gqa_flashattention_ne_amd.profsum last <N> <kernel_trace.csv>
        per-kernel average duration over each kernel's last N dispatches (for bench.py, whose last
        K dispatches of each call are that call's back-to-back launches).
    python -m causal_gqa_flashattention_ne_amd.profsum counters <dir> [<dir> ...]
        per-kernel averages over dispatches of every counter or derived metric in the
        counter_collection.csv files of one or more --pmc runs (e.g. MfmaUtil, MfmaFlopsBF16,
        VALUBusy, LdsUtil, LDSBankConflict, OccupancyPercent).
"""
import collections
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNELS = {"fwd_bf16_kernel": "fwd", "bwd_pre_bf16_kernel": "bwd_pre", "bwd_bf16_kernel": "bwd_main",
           "fwd_kernel": "fwd", "bwd_pre_kernel": "bwd_pre", "bwd_main_kernel": "bwd_main",
           "rope_apply_kernel": "rope_keys", "key_rot_kernel": "key_rot", "decode_split_kernel": "decode_split",
           "decode_merge_kernel": "decode_merge", "decode16_kernel": "decode16",
           "proj_kernel": "qkv_proj"}
CAL_BYTES = 256 << 20


# the sources each kernel is built from (shared headers included); a stored traffic figure stays
# valid while these hash the same
_HEADERS = ("common.hpp", "tiles.hpp", "kernels.hpp")
KERNEL_SOURCES = {
    "fwd": ("fwd_bf16.hip", "fwd.hip"), "bwd_pre": ("bwd_bf16.hip", "bwd.hip"), "bwd_main": ("bwd_bf16.hip", "bwd.hip"),
    "rope_keys": ("rope.hip",), "key_rot": ("fwd_bf16.hip",), "decode16": ("decode.hip",), "decode_split": ("decode.hip",),
    "decode_merge": ("decode.hip",), "qkv_proj": ("proj.hip",),
}


def source_hash(kernel=None) -> str:
    """sha256 over the sources of `kernel` (a short name of KERNELS) and the shared headers, or over
    every source file when kernel is None."""
    if kernel is None:
        files = sorted(glob.glob(os.path.join(HERE, "csrc", "*")))
    else:
        files = [os.path.join(HERE, "csrc", f) for f in sorted(KERNEL_SOURCES[kernel] + _HEADERS)]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def counter_avgs(d):
    vals = collections.defaultdict(list)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)   # KiB -> bytes
    return {k: sum(v) / len(v) for k, v in vals.items()}


def traffic(fetch_dir, write_dir, out):
    fetch, write = counter_avgs(fetch_dir), counter_avgs(write_dir)
    cal = [k for k in fetch if "neg_kernel" in k]
    if not cal:
        raise SystemExit("no calibration copy kernel in %s" % fetch_dir)
    rf = CAL_BYTES / fetch[cal[0]]
    wf = CAL_BYTES / write[cal[0]]
    res = {"read_scale": rf, "write_scale": wf, "kernels": {}}
    for name in fetch:
        for key, short in KERNELS.items():
            if key + "<" in name or name.endswith(key) or ("::" + key + "(") in name:
                res["kernels"][short] = {"name": name, "read_bytes": fetch[name] * rf,
                                         "write_bytes": write.get(name, 0.0) * wf,
                                         "source_sha256": source_hash(short)}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def counters(dirs):
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in vals.values() for c in k})
    print("%-40s" % "kernel" + "".join("%17s" % c[:16] for c in names))
    for kname, cs in vals.items():
        short = next((v for key, v in KERNELS.items() if key + "<" in kname or ("::" + key + "(") in kname
                      or kname.endswith(key) or key in kname), kname[:40])
        print("%-40s" % short[:40] + "".join("%17.4g" % (sum(cs[c]) / len(cs[c])) if cs.get(c) else "%17s" % "-"
                                            for c in names))


def last_n(n, path):
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    print("%-64s %6s %10s" % ("kernel", "last_n", "avg_us"))
    for name, v in sorted(per.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        v.sort()
        tail = v[-n:]
        print("%-64s %6d %10.2f" % (name[:64], len(tail), sum(e - s for s, e in tail) / len(tail) / 1e3))


def rows_from_db(path):
    c = sqlite3.connect(path)
    q = ("select name, count(*), avg(end-start)/1000.0, min(end-start)/1000.0, max(end-start)/1000.0, "
         "sum(end-start)/1000.0 from kernels group by name order by sum(end-start) desc")
    return c.execute(q).fetchall()


def rows_from_csv(path):
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                        float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3))
    return out


def main(path):
    rows = rows_from_db(path) if path.endswith(".db") else rows_from_csv(path)
    print("%-64s %6s %10s %10s %10s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "total_us"))
    for name, n, avg, mn, mx, tot in rows:
        print("%-64s %6d %10.2f %10.2f %10.2f %12.1f" % (name[:64], n, avg, mn, mx, tot))


if __name__ == "__main__":
    if sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "last":
        last_n(int(sys.argv[2]), sys.argv[3])
    elif sys.argv[1] == "counters":
        counters(sys.argv[2:])
    else:
        main(sys.argv[1])
