"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

  python profile_summary.py trace DIR OUT.md --cmd "COMMAND"
      kernel-trace statistics (rocprofv3 --kernel-trace --stats, CSV output)
      per kernel and per (kernel, grid size), as markdown.

  python profile_summary.py legs TRACE_DIR FETCH_DIR WRITE_DIR OUT.json --cmd "COMMANDS"
      per-leg kernel-trace averages and HBM bytes of a `bench.py --profile` run
      (one run with --kernel-trace, one with --pmc FETCH_SIZE, one with --pmc
      WRITE_SIZE).  The legs are told apart by the marker launches that
      profile run makes (the probe-read kernel with 1000 + leg index
      workgroups); the counters are scaled by what they read for the run's
      512 MiB device copy.  The file records a hash of the kernel sources;
      bench.py reports these figures only while the kernels are unchanged.

  python profile_summary.py traffic FETCH_DIR WRITE_DIR OUT.json --cmd "COMMAND"
      mean HBM bytes per dispatch from two counter runs (--pmc FETCH_SIZE, then
      --pmc WRITE_SIZE).  The counters are scaled by what they read for the
      512 MiB device copy that `bench.py --profile` runs first (a plain copy
      of known size).  The file records a hash of the kernel sources; bench.py
      reports the traffic only while the kernels are unchanged.

  python profile_summary.py sq OUT.md DIR... --cmd "COMMAND" ... --title TITLE
      mean SQ counter values per leg and kernel of `bench.py --profile`
      counter runs.

Reads rocprofv3 CSV output only; runs nothing on the GPU.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "q4_weight_only_amd", "csrc")
COPY_BYTES = 512 << 20


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def short_name(name):
    base = name.split("(")[0]
    return base.replace("void ", "").strip()


def _one(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise SystemExit(f"no file matches {pattern}")
    return files[0]


def trace_summary(d, out, cmd):
    trace = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv")))))
    per_kernel = collections.defaultdict(list)
    per_grid = collections.defaultdict(list)
    for r in trace:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        k = short_name(r["Kernel_Name"])
        per_kernel[k].append(dur)
        per_grid[(k, int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))].append(dur)
    lines = [f"# rocprofv3 kernel trace: {os.path.basename(out)[:-3]}", "",
             "Command (from the repository root):", "", "```", cmd, "```", "",
             "Durations are the kernel-trace start/end timestamps, in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | total us |",
             "|---|---:|---:|---:|---:|---:|"]
    for k, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | "
                     f"{max(v):.2f} | {sum(v):.1f} |")
    lines += ["", "Per kernel and grid size (workgroups per dispatch):", "",
              "| kernel | workgroups | calls | avg us | median us |", "|---|---:|---:|---:|---:|"]
    for (k, g), v in sorted(per_grid.items()):
        lines.append(f"| `{k}` | {g} | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def _counter(d):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    per = collections.defaultdict(list)
    for r in rows:
        wg = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
        per[(short_name(r["Kernel_Name"]), wg)].append(float(r["Counter_Value"]))
    return per


def traffic(fetch_dir, write_dir, out, cmd):
    fetch, write = _counter(fetch_dir), _counter(write_dir)

    def copy_ref(per):
        vals = [statistics.median(v) for (k, _), v in per.items()
                if "copyBuffer" in k and statistics.median(v) > 1e5]
        if not vals:
            raise SystemExit("no 512 MiB copy dispatch in the counter run")
        return COPY_BYTES / (max(vals) * 1024)   # counters are KiB per dispatch

    fs, ws = copy_ref(fetch), copy_ref(write)
    kernels = {}
    for key in fetch:
        k, wg = key
        if "jq4k" not in k:
            continue
        kernels[f"{k}@{wg}"] = {
            "kernel": k, "workgroups": wg, "dispatches": len(fetch[key]),
            "fetch_bytes": round(statistics.mean(fetch[key]) * 1024 * fs),
            "write_bytes": round(statistics.mean(write.get(key, [0.0])) * 1024 * ws)}
    doc = {"command": cmd, "copy_reference_bytes": COPY_BYTES,
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "kernel_sources_sha256": kernel_source_hash(), "kernels": kernels}
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {out}")


MARKER_KERNEL = "probe_read_kernel"
MARKER_BASE = 1000
PROFILE_LEGS = ["copy_512MiB", "single", "decode", "lm_head", "m33", "prefill", "lm_head_m512",
                "warmup"]


def _segments(rows, key, wg_of, name_of):
    """Split dispatch rows (sorted by `key`) at the marker launches; returns
    {leg: [rows]}."""
    legs = collections.defaultdict(list)
    cur = None
    for r in sorted(rows, key=key):
        name = name_of(r)
        wg = wg_of(r)
        if MARKER_KERNEL in name and MARKER_BASE <= wg < MARKER_BASE + len(PROFILE_LEGS):
            cur = PROFILE_LEGS[wg - MARKER_BASE]
            continue
        if cur is not None:
            legs[cur].append(r)
    return legs


def legs_summary(trace_dir, fetch_dir, write_dir, out, cmd):
    trace = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    tl = _segments(trace, key=lambda r: int(r["Start_Timestamp"]),
                   wg_of=lambda r: int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                   name_of=lambda r: r["Kernel_Name"])

    def counters(d):
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        return _segments(rows, key=lambda r: int(r["Dispatch_Id"]),
                         wg_of=lambda r: int(r["Grid_Size"]) // int(r["Workgroup_Size"]),
                         name_of=lambda r: r["Kernel_Name"])
    fl, wl = counters(fetch_dir), counters(write_dir)

    def scale(seg):
        # the 512 MiB copies (other copies in the segment are the next leg's
        # weight rotation, a few MB each)
        vals = [float(r["Counter_Value"]) for r in seg.get("copy_512MiB", [])
                if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 1e5]
        if not vals:
            raise SystemExit("no 512 MiB copy in the counter run")
        return COPY_BYTES / (statistics.median(vals) * 1024)   # counters: KiB per dispatch
    fs, ws = scale(fl), scale(wl)
    legs = {}
    for leg in PROFILE_LEGS[1:]:
        per = collections.defaultdict(list)
        for r in tl.get(leg, []):
            per[short_name(r["Kernel_Name"])].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        fetch = collections.defaultdict(list)
        for r in fl.get(leg, []):
            fetch[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]) * 1024 * fs)
        write = collections.defaultdict(list)
        for r in wl.get(leg, []):
            write[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]) * 1024 * ws)
        legs[leg] = {}
        for k, v in per.items():
            if "jq4k" not in k:
                continue
            legs[leg][k] = {"calls": len(v), "avg_us": round(statistics.mean(v), 3),
                            "median_us": round(statistics.median(v), 3),
                            "fetch_bytes": round(statistics.mean(fetch[k])) if fetch.get(k) else None,
                            "write_bytes": round(statistics.mean(write[k])) if write.get(k) else None}
    doc = {"command": cmd, "copy_reference_bytes": COPY_BYTES,
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "kernel_sources_sha256": kernel_source_hash(), "legs": legs}
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {out}")


def sq_summary(dirs, out, cmds, title):
    """Mean value per dispatch of every counter in the counter runs `dirs`
    (each a `bench.py --profile` run), per leg and jq4k kernel, as
    markdown."""
    table = collections.defaultdict(dict)   # (leg, kernel) -> counter -> mean
    names = []
    for d in dirs:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        segs = _segments(rows, key=lambda r: int(r["Dispatch_Id"]),
                         wg_of=lambda r: int(r["Grid_Size"]) // int(r["Workgroup_Size"]),
                         name_of=lambda r: r["Kernel_Name"])
        for leg, seg in segs.items():
            per = collections.defaultdict(list)
            for r in seg:
                k = short_name(r["Kernel_Name"])
                if "jq4k" in k:
                    per[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
            for (k, c), v in per.items():
                table[(leg, k)][c] = statistics.mean(v)
                if c not in names:
                    names.append(c)
    cols = [key for key in sorted(table, key=lambda kv: PROFILE_LEGS.index(kv[0]))]
    lines = [f"# rocprofv3 counters: {title}", "", "Commands (from the repository root):", "",
             "```", *cmds, "```", "",
             "Mean counter value per dispatch, in millions, per leg of `bench.py --profile` "
             "(weights rotated over >= 1 GiB of copies, as the benchmark runs them).", "",
             "| counter | " + " | ".join(f"{leg}: `{k.replace('jq4k::', '')}`" for leg, k in cols)
             + " |", "|---|" + "---:|" * len(cols)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(
            f"{table[key].get(c, float('nan')) / 1e6:.2f}" for key in cols) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    g = sub.add_parser("legs")
    g.add_argument("trace_dir")
    g.add_argument("fetch_dir")
    g.add_argument("write_dir")
    g.add_argument("out")
    g.add_argument("--cmd", required=True)
    q = sub.add_parser("sq")
    q.add_argument("out")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--cmd", action="append", required=True)
    q.add_argument("--title", required=True)
    a = ap.parse_args()
    if a.what == "sq":
        sq_summary(a.dirs, a.out, a.cmd, a.title)
        return
    if a.what == "trace":
        trace_summary(a.dir, a.out, a.cmd)
    elif a.what == "legs":
        legs_summary(a.trace_dir, a.fetch_dir, a.write_dir, a.out, a.cmd)
    else:
        traffic(a.fetch_dir, a.write_dir, a.out, a.cmd)


if __name__ == "__main__":
    main()
