"""Summaries of rocprofv3 output as short text tables (measurement plumbing, not part of the path).

usage:
  python -m speculative_decoding_moe_amd.profiling trace <results.db> "<command>" [skip_first_n_per_kernel]
      per-kernel durations from a `rocprofv3 --kernel-trace` database (rocpd SQLite)
  python -m speculative_decoding_moe_amd.profiling traffic <fetch_dir> <write_dir> <profiled program's log>
      "<fetch command>" "<write command>" <kernel substring> <source file>
      HBM bytes per dispatch from one `--pmc FETCH_SIZE` run and one `--pmc WRITE_SIZE` run (csv output),
      each scaled by what the same counter reads for the plain copy kernel of known size that the
      profiled program runs last (`bench.py --profile-run` prints its size as JSON).
  python -m speculative_decoding_moe_amd.profiling counters "<command>" <pmc_dir> [<pmc_dir> ...]
      per-kernel means of the SQ counters of one or more `--pmc` runs (csv output) that each
      include SQ_WAVE_CYCLES: every other wave-cycle counter as a fraction of it, and the other
      counters per dispatch
"""
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

COPY_KERNEL = "k_copy16"


def _short(name):
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def trace(db, cmd, skip=0):
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels order by start").fetchall()
    per = {}
    for name, s, e in rows:
        per.setdefault(_short(name), []).append((e - s) / 1e3)
    out = [f"# rocprofv3 --kernel-trace --stats summary\n# command: {cmd}\n"
           f"# first {skip} dispatches of each kernel skipped (warm-up)",
           f"{'kernel':48s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v = v[skip:] if len(v) > skip else v
        out.append(f"{k[:48]:48s} {len(v):6d} {sum(v)/len(v):9.2f} {min(v):9.2f} {max(v):9.2f} {sum(v):10.1f}")
    return "\n".join(out)


def _counter_rows(d):
    """(dispatch id, kernel name, counter value) from the counter_collection csv under directory d."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def _per_kernel(rows):
    """Mean counter value per dispatch for each kernel (values of one dispatch summed first)."""
    by_dispatch = {}
    for did, name, v in rows:
        key = (did, _short(name))
        by_dispatch[key] = by_dispatch.get(key, 0.0) + v
    per = {}
    for (_, name), v in by_dispatch.items():
        per.setdefault(name, []).append(v)
    return {n: (sum(v) / len(v), len(v)) for n, v in per.items()}


def traffic(fetch_dir, write_dir, run_json, cmd_fetch, cmd_write, kernel, source):
    run = None
    if os.path.exists(run_json):  # the profiled program's output: its {"profile_run": ...} line
        for line in open(run_json):
            if line.startswith('{"profile_run"'):
                run = json.loads(line)
    else:
        run = json.loads(run_json)
    if run is None:
        raise ValueError(f"no profile_run line in {run_json}")
    fetch = _per_kernel(_counter_rows(fetch_dir))
    write = _per_kernel(_counter_rows(write_dir))
    copy_bytes = float(run["copy_bytes"])
    cf = [v for n, v in fetch.items() if COPY_KERNEL in n][0][0]
    cw = [v for n, v in write.items() if COPY_KERNEL in n][0][0]
    fscale, wscale = copy_bytes / cf, copy_bytes / cw  # bytes per counter unit
    src_hash = hashlib.sha256(open(source, "rb").read()).hexdigest()
    out = ["# HBM traffic per dispatch from rocprofv3 FETCH_SIZE and WRITE_SIZE (separate runs), each",
           "# scaled by the counter's reading for a plain copy of known size in the same run",
           f"# fetch command: {cmd_fetch}", f"# write command: {cmd_write}",
           f"# copy kernel {COPY_KERNEL}: {int(copy_bytes)} B read and written; FETCH_SIZE reads {cf:.1f}, "
           f"WRITE_SIZE reads {cw:.1f} per dispatch",
           f"{'kernel':40s} {'calls':>6s} {'fetch_raw':>12s} {'write_raw':>12s} {'fetch_MB':>10s} {'write_MB':>10s}"]
    for n in sorted(fetch, key=lambda n: -fetch[n][0]):
        f, c = fetch[n]
        w = write.get(n, (float("nan"), 0))[0]
        out.append(f"{n[:40]:40s} {c:6d} {f:12.1f} {w:12.1f} {f * fscale / 1e6:10.2f} {w * wscale / 1e6:10.2f}")
    name = [n for n in fetch if n == kernel] or [n for n in fetch if kernel in n]  # an exact name first
    if len(name) != 1:
        raise ValueError(f"kernel substring {kernel!r} matches {name}")
    name = name[0]
    fb, wb = fetch[name][0] * fscale, write[name][0] * wscale
    out += ["", f"kernel: {name}", f"source: {os.path.basename(source)}", f"source_sha256: {src_hash}",
            f"fetch_scale_bytes_per_unit: {fscale:.4f}", f"write_scale_bytes_per_unit: {wscale:.4f}",
            f"fetch_bytes_per_launch: {fb:.0f}", f"write_bytes_per_launch: {wb:.0f}",
            f"traffic_bytes_per_launch: {fb + wb:.0f}"]
    # algorithmic bytes per launch that the profiled program reports for each kernel
    keys = [("k_bexp<true, false>", "bexp_gateup_bytes"), ("k_bexp<false, false>", "bexp_down_bytes"),
            ("k_bexp<true, true>", "mx_bexp_gateup_bytes"), ("k_bexp<false, true>", "mx_bexp_down_bytes"),
            ("k_layer<2, 4, true>", "mx_layer_bytes_mean"), ("k_layer<2, 4, false>", "layer_bytes_mean"),
            ("k_accept", "accept_bytes"), ("k_head", "head_bytes")]
    alg = next((float(run[key]) for sub, key in keys if sub in name and key in run), None)
    if alg:
        out += [f"algorithmic_bytes_per_launch: {alg:.0f}", f"traffic_over_algorithmic: {(fb + wb) / alg:.4f}"]
    return "\n".join(out)


def _counter_means(d):
    """{kernel: {counter: (mean per dispatch, dispatches)}} of one counter_collection csv directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    by_dispatch = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (int(r["Dispatch_Id"]), _short(r["Kernel_Name"]), r["Counter_Name"])
                by_dispatch[key] = by_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (_, name, ctr), v in by_dispatch.items():
        per.setdefault(name, {}).setdefault(ctr, []).append(v)
    return {n: {c: (sum(v) / len(v), len(v)) for c, v in cs.items()} for n, cs in per.items()}


# counters in wave-cycles (quad-cycles), shown as fractions of SQ_WAVE_CYCLES
_WAVE_CYCLE_COUNTERS = ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                        "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC")


def counters(cmd, *dirs):
    runs = [_counter_means(d) for d in dirs]
    kernels = sorted(set().union(*runs), key=lambda n: -max(r.get(n, {}).get("SQ_WAVE_CYCLES", (0, 0))[0]
                                                             for r in runs))
    out = ["# SQ counters per kernel from rocprofv3 --pmc runs (csv output), one run per counter set;",
           "# wave-cycle counters as fractions of the same run's SQ_WAVE_CYCLES, others per dispatch",
           f"# command: {cmd}", "# runs: " + " ".join(os.path.basename(d.rstrip('/')) for d in dirs)]
    for n in kernels:
        cols = []
        for r in runs:
            cs = r.get(n)
            if not cs or "SQ_WAVE_CYCLES" not in cs:
                continue
            wc = cs["SQ_WAVE_CYCLES"][0]
            for c, (v, _) in sorted(cs.items()):
                if c == "SQ_WAVE_CYCLES":
                    continue
                cols.append(f"{c[3:]}={v / wc:.3f}" if c in _WAVE_CYCLE_COUNTERS else f"{c[3:]}={v:.4g}")
            cols.append(f"WAVE_CYCLES={wc:.4g}")
        calls = max(r.get(n, {}).get("SQ_WAVE_CYCLES", (0, 0))[1] for r in runs)
        out.append(f"{n[:28]:28s} calls {calls:3d}  " + " ".join(cols))
    return "\n".join(out)


def main(argv):
    if argv[0] == "trace":
        print(trace(argv[1], argv[2], int(argv[3]) if len(argv) > 3 else 0))
    elif argv[0] == "traffic":
        print(traffic(*argv[1:8]))
    elif argv[0] == "counters":
        print(counters(argv[1], *argv[2:]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
