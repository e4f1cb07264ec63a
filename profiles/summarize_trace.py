"""Summarise a rocprofv3 kernel-trace database (rocpd SQLite) as a per-kernel table.

usage: python profiles/summarize_trace.py <results.db> "<command that produced it>" [skip_first_n_per_kernel]
"""
import sqlite3
import sys


def main():
    db, cmd = sys.argv[1], sys.argv[2]
    skip = int(sys.argv[3]) if len(sys.argv) > 3 else 0
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels order by start").fetchall()
    per = {}
    for name, s, e in rows:
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        per.setdefault(short, []).append((e - s) / 1e3)
    print(f"# rocprofv3 --kernel-trace --stats summary\n# command: {cmd}\n# first {skip} dispatches of each kernel skipped (warm-up)")
    print(f"{'kernel':48s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s}")
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v = v[skip:] if len(v) > skip else v
        print(f"{k[:48]:48s} {len(v):6d} {sum(v)/len(v):9.2f} {min(v):9.2f} {max(v):9.2f} {sum(v):10.1f}")


if __name__ == "__main__":
    main()
