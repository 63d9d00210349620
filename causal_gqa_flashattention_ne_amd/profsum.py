"""Summarise a rocprofv3 kernel trace (rocpd SQLite database or kernel_stats CSV) per kernel.

    python -m causal_gqa_flashattention_ne_amd.profsum <results.db | kernel_stats.csv>
Prints one line per kernel: dispatch count, average / min / max duration in microseconds.
"""
import csv
import sqlite3
import sys


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
    main(sys.argv[1])
