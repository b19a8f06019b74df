"""Short text summaries of rocprofv3 CSV output (kernel traces and counter
runs), in the form kept under profiles/.

    python -m paged_kv_cache_64_amd.prof_summary trace DIR --title T --command C [--note N ...]
        [--skip KERNEL=N ...]
    python -m paged_kv_cache_64_amd.prof_summary counters --kernel K --fetch DIR --write DIR
        --cal-fetch DIR --cal-write DIR --cal-bytes B --bytes B --title T --workload W
        --command-fetch C --command-write C --command-cal C [--note N ...]
    python -m paged_kv_cache_64_amd.prof_summary sq DIR --kernel K [--title T --command C ... --note N ...]
        [--code-root CHECKOUT]

Every summary records the kernel source hash of bench.py's kernel_code_hash()
at the time it was written (right after the run, from the tree that ran), so a
figure can be matched to the kernel source it was measured on; bench.py reads
the traffic figures of a counter summary only while that source is unchanged.
"""
import argparse
import csv
import glob
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csv_files(path, suffix):
    files = sorted(glob.glob(os.path.join(path, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {path}")
    return files


def kernel_stats(path):
    """Rows (name, calls, average ns, min ns, max ns, total ns), largest total first."""
    rows = []
    for f in _csv_files(path, "kernel_stats.csv"):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                             float(r["MaxNs"]), float(r["TotalDurationNs"])))
    rows.sort(key=lambda x: -x[5])
    return rows


def dispatch_stats(path, skip=None):
    """Per-kernel rows from the per-dispatch kernel trace: (name, calls, mean ns,
    median ns, min ns, max ns, total ns, skipped), largest total first.

    skip maps a kernel-name substring to a number of that kernel's first
    dispatches (in dispatch order) to leave out, e.g. a bench's warm-up
    launches.  Returns None when the directory holds no kernel_trace.csv."""
    files = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        return None
    per = defaultdict(list)
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
                per[r["Kernel_Name"]].append((key, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows = []
    for name, ds in per.items():
        ds.sort()
        n_skip = 0
        for sub, n in (skip or {}).items():
            if sub in name:
                n_skip = min(len(ds), n)
        kept = [end - start for _, start, end in ds[n_skip:]]
        if not kept:
            continue
        kept.sort()
        mid = len(kept) // 2
        median = kept[mid] if len(kept) % 2 else (kept[mid - 1] + kept[mid]) / 2
        rows.append((name, len(kept), sum(kept) / len(kept), median, kept[0], kept[-1], sum(kept), n_skip))
    rows.sort(key=lambda x: -x[6])
    return rows


def counter_means(path, counter):
    """{kernel name: (mean value per dispatch, dispatches)} for one counter."""
    acc = defaultdict(lambda: [0.0, 0])
    for f in _csv_files(path, "counter_collection.csv"):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                a = acc[r["Kernel_Name"]]
                a[0] += float(r["Counter_Value"])
                a[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items() if v[1]}


def _match(means, kernel):
    hits = {k: v for k, v in means.items() if kernel in k}
    if not hits:
        raise SystemExit(f"kernel {kernel} not in the counter output")
    if len(hits) > 1:  # several instantiations: weight by dispatches
        tot = sum(v[1] for v in hits.values())
        return sum(v[0] * v[1] for v in hits.values()) / tot, tot
    return next(iter(hits.values()))


def _code_hash(root=None):
    sys.path.insert(0, ROOT)
    import bench

    return bench.kernel_code_hash(root)


def _short(name, width=88):
    return name if len(name) <= width else name[:width - 3] + "..."


def _skips(items):
    skip = {}
    for it in items or []:
        sub, _, n = it.rpartition("=")
        if not sub:
            raise SystemExit(f"--skip wants KERNEL=N, got {it!r}")
        skip[sub] = int(n)
    return skip


def cmd_trace(args):
    out = [f"# {args.title}", f"# command: {args.command}", f"# kernel_code_sha256: {_code_hash()}"]
    out += [f"# {n}" for n in args.note or []]
    rows = dispatch_stats(args.dir, _skips(args.skip))
    if rows is None:
        if args.skip:
            raise SystemExit("--skip needs the per-dispatch kernel_trace.csv")
        out.append("# name | calls | average ns | min ns | max ns | total ns")
        for name, calls, avg, mn, mx, tot in kernel_stats(args.dir)[: args.top]:
            out.append(f"{_short(name)} | {calls} | {avg:.0f} | {mn:.0f} | {mx:.0f} | {tot:.0f}")
        return "\n".join(out) + "\n"
    for name, calls, *_rest, skipped in rows:
        if skipped:
            out.append(f"# {_short(name, 60)}: its first {skipped} dispatches (warm-up) are left out")
    out.append("# name | calls | average ns | median ns | min ns | max ns | total ns")
    for name, calls, avg, med, mn, mx, tot, _ in rows[: args.top]:
        out.append(f"{_short(name)} | {calls} | {avg:.0f} | {med:.0f} | {mn:.0f} | {mx:.0f} | {tot:.0f}")
    return "\n".join(out) + "\n"


def cmd_counters(args):
    cal_f = _match(counter_means(args.cal_fetch, "FETCH_SIZE"), "probe_copy_kernel")[0]
    cal_w = _match(counter_means(args.cal_write, "WRITE_SIZE"), "probe_copy_kernel")[0]
    fetch_scale = args.cal_bytes / (cal_f * 1024.0)
    write_scale = args.cal_bytes / (cal_w * 1024.0)
    f, nf = _match(counter_means(args.fetch, "FETCH_SIZE"), args.kernel)
    w, nw = _match(counter_means(args.write, "WRITE_SIZE"), args.kernel)
    fetch_bytes = f * 1024.0 * fetch_scale
    write_bytes = w * 1024.0 * write_scale
    out = [f"# {args.title}",
           f"# FETCH_SIZE run:  {args.command_fetch}",
           f"# WRITE_SIZE run:  {args.command_write}",
           f"# calibration:     {args.command_cal}",
           f"#   a plain copy of {args.cal_bytes} B read FETCH_SIZE = {cal_f:.1f} KiB and WRITE_SIZE = "
           f"{cal_w:.1f} KiB per launch,",
           f"#   so FETCH_SIZE is scaled by {fetch_scale:.4f} and WRITE_SIZE by {write_scale:.4f} to give bytes",
           f"# {args.kernel}: FETCH_SIZE {f:.1f} KiB/launch over {nf} launches, WRITE_SIZE {w:.1f} KiB/launch "
           f"over {nw} launches",
           f"# algorithmic bytes per launch: {args.bytes}",
           f"# traffic / algorithmic = {(fetch_bytes + write_bytes) / args.bytes:.4f}"]
    out += [f"# {n}" for n in args.note or []]
    out += [f"kernel: {args.kernel}",
            f"workload: {args.workload}",
            f"kernel_code_sha256: {_code_hash()}",
            f"fetch_scale: {fetch_scale:.6f}",
            f"write_scale: {write_scale:.6f}",
            f"fetch_bytes_per_launch: {fetch_bytes:.0f}",
            f"write_bytes_per_launch: {write_bytes:.0f}"]
    return "\n".join(out) + "\n"


def cmd_sq(args):
    """Mean per-dispatch value of every counter in the run, for one kernel."""
    names = set()
    for f in _csv_files(args.dir, "counter_collection.csv"):
        with open(f, newline="") as fh:
            names.update(r["Counter_Name"] for r in csv.DictReader(fh))
    out = []
    if args.title:
        out.append(f"# {args.title}")
    for cmd in args.command or []:
        out.append(f"# command: {cmd}")
    out.append(f"# kernel_code_sha256: {_code_hash(args.code_root)}"
               + (f" (kernel sources of {args.code_root})" if args.code_root else ""))
    out += [f"# {n}" for n in args.note or []]
    for c in sorted(names):
        v, n = _match(counter_means(args.dir, c), args.kernel)
        out.append(f"{args.kernel} {c}: {v:.6g} per launch over {n} launches")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--note", action="append")
    t.add_argument("--top", type=int, default=12)
    t.add_argument("--skip", action="append", metavar="KERNEL=N",
                   help="leave out the first N dispatches of kernels whose name contains KERNEL")
    c = sub.add_parser("counters")
    for k in ("kernel", "fetch", "write", "cal_fetch", "cal_write", "title", "workload", "command_fetch",
              "command_write", "command_cal"):
        c.add_argument("--" + k.replace("_", "-"), required=True)
    c.add_argument("--cal-bytes", type=int, required=True)
    c.add_argument("--bytes", type=int, required=True)
    c.add_argument("--note", action="append")
    q = sub.add_parser("sq")
    q.add_argument("dir")
    q.add_argument("--kernel", required=True)
    q.add_argument("--title")
    q.add_argument("--command", action="append", help="one per counter pass whose output lies under DIR")
    q.add_argument("--note", action="append")
    q.add_argument("--code-root", help="the checkout whose kernels ran (default: this one)")
    ap.add_argument("-o", "--out")
    args = ap.parse_args(argv)
    text = {"trace": cmd_trace, "counters": cmd_counters, "sq": cmd_sq}[args.cmd](args)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
