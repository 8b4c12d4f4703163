"""Summaries of rocprofv3 CSV output (``-f csv``) for the files kept under ``profiles/``.

    python -m attention_backward_fmha_amd.rocprof_summary stats DIR [--match TEXT] [--top N]
        per-kernel calls / total / average duration from DIR/*kernel_stats.csv, and the
        median duration of each kernel's dispatches from DIR/*kernel_trace.csv
    python -m attention_backward_fmha_amd.rocprof_summary traffic --kernel NAME \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-mib N
        HBM bytes per launch of NAME: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by
        what the same counters read for a plain copy of N MiB (bytes moved / counter value)
"""

import argparse
import csv
import glob
import os


def _one(dir_, pattern):
    files = sorted(glob.glob(os.path.join(dir_, "**", pattern), recursive=True))
    if not files:
        raise FileNotFoundError("no %s under %s" % (pattern, dir_))
    return files[0]


def kernel_stats(dir_):
    rows = []
    with open(_one(dir_, "*kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r.get("Percentage", 0.0))))
    rows.sort(key=lambda x: -x[2])
    return rows


def median_durations(dir_):
    """Kernel name -> median dispatch duration (ns) from the kernel trace, if there is one."""
    try:
        path = _one(dir_, "*kernel_trace.csv")
    except FileNotFoundError:
        return {}
    durs = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for name, d in durs.items():
        d.sort()
        n = len(d)
        out[name] = d[n // 2] if n % 2 else 0.5 * (d[n // 2 - 1] + d[n // 2])
    return out


def counter_avg(dir_, counter, kernel):
    vals = []
    with open(_one(dir_, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError("no %s samples for %s in %s" % (counter, kernel, dir_))
    return sum(vals) / len(vals), len(vals)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--match", default="", help="only kernels whose name contains this")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--copy-kernel", default="copyBuffer")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print("| kernel | calls | total ms | average us | median us | % |")
        print("|---|---:|---:|---:|---:|---:|")
        rows = [r for r in kernel_stats(a.dir) if a.match in r[0]]
        med = median_durations(a.dir)
        for name, calls, tot, avg, pct in rows[: a.top]:
            m = "%.1f" % (med[name] / 1e3) if name in med else "-"
            print("| %s | %d | %.3f | %.1f | %s | %.1f |" % (name[:90], calls, tot / 1e6, avg / 1e3, m, pct))
    else:
        nbytes = a.copy_mib * (1 << 20)
        cf, _ = counter_avg(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
        cw, _ = counter_avg(a.copy_write, "WRITE_SIZE", a.copy_kernel)
        kf, nf = counter_avg(a.fetch, "FETCH_SIZE", a.kernel)
        kw, nw = counter_avg(a.write, "WRITE_SIZE", a.kernel)
        rf, rw = nbytes / cf, nbytes / cw
        print("copy probe: %d MiB; FETCH_SIZE %.0f KiB -> %.4f bytes per unit; WRITE_SIZE %.0f KiB -> "
              "%.4f bytes per unit" % (a.copy_mib, cf, rf, cw, rw))
        print("kernel %s: FETCH_SIZE %.0f KiB/dispatch (%d samples), WRITE_SIZE %.0f KiB/dispatch (%d)"
              % (a.kernel, kf, nf, kw, nw))
        print("read_bytes_per_launch: %.0f" % (kf * rf))
        print("write_bytes_per_launch: %.0f" % (kw * rw))


if __name__ == "__main__":
    main()
