"""Summaries of rocprofv3 CSV output for this library's kernels (text for profiles/).

  python -m gemm_gate_softmax_amd.profile_summary stats KERNEL_STATS.csv --command "..."
        [--trace KERNEL_TRACE.csv --kernel PREFIX --last N]
      Markdown table of a ``rocprofv3 --kernel-trace --stats --output-format csv`` run; with
      --trace, also the mean duration of the last N dispatches of the kernel named PREFIX
      (e.g. the calls a benchmark times last, when earlier calls of the same kernel ran
      with other arguments).

  python -m gemm_gate_softmax_amd.profile_summary traffic --kernel PREFIX --workload NAME \\
      --fetch BENCH_FETCH.csv --write BENCH_WRITE.csv \\
      --copy-fetch COPY_FETCH.csv --copy-write COPY_WRITE.csv --copy-bytes B --command "..."
      HBM bytes per launch of one kernel from ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
      runs (KiB per dispatch), each scaled by what the same counter reads for a plain
      device copy of B bytes (the copy kernel is the largest dispatch of its run).

  python -m gemm_gate_softmax_amd.profile_summary steps KERNEL_TRACE.csv --command "..."
        [--first dense_gemm_kernel --last combine_kernel --exclude dispatch_kernel]
      Per-dispatch durations and the gaps between consecutive dispatches of the layer steps
      in a kernel trace (medians over the last steps).

  python -m gemm_gate_softmax_amd.profile_summary counters PASS1.csv [PASS2.csv ...] \\
      --kernel PREFIX --last N --command "..." [--command "..."]
      Mean per dispatch of every counter of ``rocprofv3 --pmc`` passes over the last N
      dispatches of one kernel.

Only the standard library is used; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("gemm_gate_softmax_amd/csrc/gemm.hip", "gemm_gate_softmax_amd/csrc/device.h")


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name, width=96):
    name = name.replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    cut = name.find(">(")
    if cut > 0:
        name = name[:cut + 1]
    return name if len(name) <= width else name[:width - 3] + "..."


def _code_only(text):
    """Source text without comments and with whitespace runs collapsed (string literals
    in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_digest():
    """sha256 over the expert kernel's code (comments and layout ignored): the traffic
    counters recorded in profiles/ are tied to it."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def last_dispatches(trace, prefix, n):
    """Durations (us) of the last n dispatches of kernels whose name contains prefix."""
    rows = [r for r in _rows(trace) if prefix in _short(r["Kernel_Name"], 10**6)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[-n:]]


def stats_markdown(path, command, title, trace=None, prefix=None, last=0):
    rows = sorted(_rows(path), key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Command (repository root, one MI355X):", "", f"    {command}", "",
           "`Calls` counts dispatches over the whole run (warm-up, timed steps, per-stage",
           "timing, input generation); durations are per dispatch.", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f} |")
    if trace and prefix and last > 0:
        d = last_dispatches(trace, prefix, last)
        out += ["", f"Last {len(d)} dispatches of `{prefix}` (the calls the benchmark times "
                "last, from the kernel trace of the same run): mean "
                f"{statistics.mean(d):.1f} us, min {min(d):.1f}, max {max(d):.1f}."]
    return "\n".join(out) + "\n"


def _per_dispatch(path, prefix):
    """Counter value (summed over its instances) for each dispatch of kernels whose name
    contains prefix."""
    per = {}
    for r in _rows(path):
        if prefix in _short(r["Kernel_Name"], 10**6):
            d = r["Dispatch_Id"]
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    return list(per.values())


def _copy_reading(path):
    """Counter reading (KiB) of the plain copy: the largest dispatch of the run."""
    per = {}
    for r in _rows(path):
        d = r["Dispatch_Id"]
        per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    vals = sorted(per.values())
    return vals[-1]


def traffic_markdown(a):
    fetch = _per_dispatch(a.fetch, a.kernel)
    write = _per_dispatch(a.write, a.kernel)
    if not fetch or not write:
        raise SystemExit(f"no dispatch of {a.kernel!r} in the counter files")
    cf, cw = _copy_reading(a.copy_fetch), _copy_reading(a.copy_write)
    f_scale = a.copy_bytes / (cf * 1024.0)
    w_scale = a.copy_bytes / (cw * 1024.0)
    fetch_b = statistics.mean(fetch) * 1024.0 * f_scale
    write_b = statistics.mean(write) * 1024.0 * w_scale
    total = int(round(fetch_b + write_b))
    out = [f"# L2<->fabric bytes per launch: {a.kernel} ({a.workload})", "",
           "Commands (repository root, one MI355X), one counter per run:", ""]
    out += [f"    {c}" for c in a.command]
    out += ["",
            "FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  A plain device copy of "
            f"{a.copy_bytes} bytes reads {cf:.1f} KiB of FETCH_SIZE and {cw:.1f} KiB of WRITE_SIZE, "
            f"so kernel readings are scaled by {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
            "| | dispatches | mean reading (KiB) | scaled bytes per launch |",
            "|---|---|---|---|",
            f"| fetch | {len(fetch)} | {statistics.mean(fetch):.1f} | {fetch_b:.4g} |",
            f"| write | {len(write)} | {statistics.mean(write):.1f} | {write_b:.4g} |", "",
            "Fields read by bench.py (traffic is reported only while the kernel sources hash",
            "to source_sha256):", "",
            f"- workload: `{a.workload}`",
            f"- kernel: `{a.kernel}`",
            f"- source_sha256: `{kernel_digest()}`",
            f"- fetch_scale: `{f_scale:.6f}`",
            f"- write_scale: `{w_scale:.6f}`",
            f"- fabric_bytes_per_launch: `{total}`", "",
            "FETCH_SIZE and WRITE_SIZE count what the L2 exchanged with the memory fabric; the",
            "fabric's own cache (MALL) may serve part of it, so these are fabric bytes, an upper",
            "bound on HBM bytes.", ""]
    return "\n".join(out)


def layer_steps(trace, first, last, exclude=(), max_kernels=16):
    """The layer steps of a kernel trace: runs of consecutive dispatches that start with a
    kernel whose name contains `first`, end with one containing `last`, and hold none
    containing a name in `exclude`.  Each step is a list of (short name, start, end) in ns."""
    rows = sorted(_rows(trace), key=lambda r: int(r["Start_Timestamp"]))
    k = [(_short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
         for r in rows]
    steps, i = [], 0
    while i < len(k):
        if first in k[i][0]:
            j = i
            while j < len(k) and j - i < max_kernels and not (j > i and first in k[j][0]):
                if last in k[j][0]:
                    break
                j += 1
            if j < len(k) and last in k[j][0] and not any(x in n for n, _, _ in k[i:j + 1]
                                                          for x in exclude):
                steps.append(k[i:j + 1])
                i = j + 1
                continue
        i += 1
    return steps


def steps_markdown(a):
    steps = layer_steps(a.trace, a.first, a.last, a.exclude or ())
    steps = steps[-a.last_steps:] if a.last_steps > 0 else steps
    if not steps:
        raise SystemExit("no layer step found in the trace")
    shape = [n for n, _, _ in steps[-1]]
    steps = [st for st in steps if [n for n, _, _ in st] == shape]
    med = statistics.median
    out = [f"# {a.title}", "", "Command (repository root, one MI355X):", "", f"    {a.command}", "",
           f"The last {len(steps)} layer steps of the run (dispatches from `{a.first}` through "
           f"`{a.last}`), medians over the steps; a gap is the time from the end of the previous "
           "dispatch to the start of this one (0 when they overlap).", "",
           "| # | kernel | duration (us) | gap before (us) |", "|---|---|---|---|"]
    for p, name in enumerate(shape):
        d = med([(st[p][2] - st[p][1]) / 1e3 for st in steps])
        g = max(med([(st[p][1] - st[p - 1][2]) / 1e3 for st in steps]), 0.0) if p else 0.0
        out.append(f"| {p} | `{name}` | {d:.1f} | {g:.1f} |")
    span = med([(st[-1][2] - st[0][1]) / 1e3 for st in steps])
    busy = med([sum(e - b for _, b, e in st) / 1e3 for st in steps])
    gaps = max(span - busy, 0.0)            # (rounding of the medians can dip below 0)
    out += ["", f"Step span {span:.1f} us: kernels {busy:.1f} us, gaps {gaps:.1f} us "
            f"({len(shape)} dispatches)."]
    return "\n".join(out) + "\n"


def counter_means(path, prefix, last):
    """Mean per dispatch (each counter summed over its instances) over the last `last`
    dispatches of kernels whose name contains prefix: {counter: mean}."""
    per = {}
    for r in _rows(path):
        if prefix in _short(r["Kernel_Name"], 10**6):
            d = int(r["Dispatch_Id"])
            per.setdefault(d, {})
            per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)[-last:]
    names = sorted({n for d in ids for n in per[d]})
    return {n: statistics.mean(per[d].get(n, 0.0) for d in ids) for n in names}, len(ids)


def counters_markdown(a):
    out = [f"# {a.title}", "", "Commands (repository root, one MI355X), one pass each:", ""]
    out += [f"    {c}" for c in a.command]
    out += ["", f"Each counter summed over its instances, mean over the last {a.last} dispatches "
            f"of `{a.kernel}`.", "", "| counter | per dispatch |", "|---|---|"]
    for path in a.csv:
        means, n = counter_means(path, a.kernel, a.last)
        for name, v in means.items():
            out.append(f"| {name} | {v:.4g} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel summary")
    s.add_argument("--trace")
    s.add_argument("--kernel")
    s.add_argument("--last", type=int, default=0)
    t = sub.add_parser("traffic")
    for k in ("kernel", "workload", "fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", action="append", required=True)
    g = sub.add_parser("steps")
    g.add_argument("trace")
    g.add_argument("--command", required=True)
    g.add_argument("--title", default="Layer steps: kernel durations and launch gaps")
    g.add_argument("--first", default="dense_gemm_kernel")
    g.add_argument("--last", default="combine_kernel")
    g.add_argument("--exclude", action="append")
    g.add_argument("--last-steps", type=int, default=20)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--last", type=int, default=5)
    c.add_argument("--title", default="Hardware counters")
    c.add_argument("--command", action="append", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        sys.stdout.write(counters_markdown(a))
        return 0
    if a.cmd == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.command, a.title, a.trace, a.kernel, a.last))
    elif a.cmd == "traffic":
        sys.stdout.write(traffic_markdown(a))
    else:
        sys.stdout.write(steps_markdown(a))
    return 0


if __name__ == "__main__":
    sys.exit(main())
