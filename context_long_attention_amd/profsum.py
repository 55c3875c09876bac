"""Short text summaries of rocprofv3 CSV output, and the traffic lookup bench.py uses.

Four summaries are produced (all markdown with the exact commands that made
them):

* ``stats``: the per-kernel table of a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (calls, total, average, min, max duration).
* ``traffic``: HBM traffic of one kernel from two ``--pmc`` runs (``FETCH_SIZE``
  and ``WRITE_SIZE``, KiB per dispatch).  The raw counters are scaled by what
  the same counters read for a plain device-to-device copy of known size made
  at the start of the same program (``bench.py --calibrate-copy-mib``), so the
  result is in bytes of memory traffic per launch.  The summary records a
  SHA-256 of the kernel's source code (comments and layout ignored);
  ``read_traffic`` returns the figure only while that code is unchanged.
* ``counters``: MFMA utilisation and instruction mix per kernel from one
  ``--pmc`` pass over the SQ counters listed in ``SQ_COUNTERS``.
* ``dispatches``: the individual dispatches of chosen kernels from a
  ``--kernel-trace`` run, in order, with their workgroup counts and durations.

Usage::

    python -m context_long_attention_amd.profsum stats --csv K_kernel_stats.csv \
        --command "<rocprofv3 command>" --out profiles/NAME.md
    python -m context_long_attention_amd.profsum traffic --fetch F.csv --write W.csv \
        --kernel "fwd_step_kernel<128, 4, true>" --workload llama3_8b_fwd --copy-mib 1024 \
        --command "<fetch command>" --command "<write command>" --out profiles/NAME.md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# source files that define each kernel whose traffic may be reported
KERNEL_SOURCES = {
    "fwd_step_kernel": ["context_long_attention_amd/csrc/attn_fwd.hip", "context_long_attention_amd/csrc/tiles.h",
                        "context_long_attention_amd/csrc/internal.h"],
    "bwd_dkdv_kernel": ["context_long_attention_amd/csrc/attn_bwd.hip", "context_long_attention_amd/csrc/tiles.h",
                        "context_long_attention_amd/csrc/internal.h"],
    "bwd_dq_kernel": ["context_long_attention_amd/csrc/attn_bwd.hip", "context_long_attention_amd/csrc/tiles.h",
                      "context_long_attention_amd/csrc/internal.h"],
    "merge_kernel": ["context_long_attention_amd/csrc/merge.hip"],
}
COPY_KERNEL = "copyBuffer"


def _family(kernel: str) -> str:
    for fam in KERNEL_SOURCES:
        if fam in kernel:
            return fam
    raise KeyError(f"no source list for kernel {kernel!r}")


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed: what the
    compiler sees, so that editing a comment does not mark measurements stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel: str) -> str:
    """SHA-256 over the code (comments and layout ignored) of a kernel's sources."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[_family(kernel)]:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def short_name(name: str) -> str:
    """``void ns::(anonymous namespace)::fwd_step_kernel<128, 4>(Params)`` -> ``fwd_step_kernel<128, 4>``."""
    n = re.sub(r"^void\s+", "", name).replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            n = n[:i]
            break
    head, sep, tail = n.partition("<")
    return head.split("::")[-1] + sep + tail


def kernel_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "total_ms": float(r["TotalDurationNs"]) / 1e6, "avg_ms": float(r["AverageNs"]) / 1e6,
                         "min_ms": float(r["MinNs"]) / 1e6, "max_ms": float(r["MaxNs"]) / 1e6,
                         "pct": float(r["Percentage"])})
    rows.sort(key=lambda r: -r["total_ms"])
    return rows


def stats_markdown(path: str, commands, top: int = 12, title: str | None = None, trace: str | None = None,
                   timed=()) -> str:
    """``timed``: (kernel, skip_first, skip_last) triples; with the run's
    ``--kernel-trace`` CSV (``trace``), each adds the kernel's average over its
    launches without the first and last ones given (the untimed passes)."""
    rows = kernel_stats(path)
    out = [f"# {title or 'Kernel trace summary'}", "", "Made by:", ""]
    out += ["```", *commands, "```", ""]
    out += ["| kernel | calls | total ms | avg ms | min ms | max ms | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        out.append(f"| `{r['name']}` | {r['calls']} | {r['total_ms']:.3f} | {r['avg_ms']:.4f} | {r['min_ms']:.4f} | "
                   f"{r['max_ms']:.4f} | {r['pct']:.2f} |")
    for kernel, first, last in timed:
        ms = [d[3] for d in dispatch_rows(trace, [kernel]) if d[1] == kernel]
        sel = ms[first:len(ms) - last]
        if not sel:
            raise SystemExit(f"no launches of {kernel!r} left after skipping {first} + {last}")
        out += ["", f"`{kernel}` over the launches of the timed passes only (launches {first + 1}–{len(ms) - last} "
                    f"of {len(ms)}): average {sum(sel) / len(sel):.4f} ms."]
    return "\n".join(out) + "\n"


def dispatch_rows(path: str, match, last: int | None = None):
    """Dispatches of a ``--kernel-trace`` CSV whose kernel short name contains one of
    the ``match`` strings, in dispatch order: (id, name, workgroups, ms); the last
    ``last`` of them if given."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Kernel_Name"])
            if not any(m in name for m in match):
                continue
            wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            ms = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
            rows.append((int(r["Dispatch_Id"]), name, wgs, ms))
    rows.sort()
    return rows[-last:] if last else rows


def dispatches_markdown(path: str, commands, match, last, title: str) -> str:
    out = [f"# {title}", "", "Made by:", "", "```", *commands, "```", "",
           "| dispatch | kernel | workgroups | ms |", "|---:|---|---:|---:|"]
    for d, name, wgs, ms in dispatch_rows(path, match, last):
        out.append(f"| {d} | `{name}` | {wgs} | {ms:.4f} |")
    return "\n".join(out) + "\n"


def counters_by_dispatch(path: str, counter: str):
    """kernel short name -> list of (dispatch id, value summed over the counter's
    instances, grid size in work-items)."""
    acc = defaultdict(float)
    names, grids = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            acc[d] += float(r["Counter_Value"])
            names[d] = short_name(r["Kernel_Name"])
            grids[d] = int(r["Grid_Size"])
    out = defaultdict(list)
    for d in sorted(acc):
        out[names[d]].append((d, acc[d], grids[d]))
    return out


def _copy_calibration(by_kernel, copy_count: int):
    """Counter total of the calibration copies: the leading run of copy dispatches
    before the first dispatch of any other kernel (the program makes them first and
    then launches a one-element fill).  A copy split over several dispatches is
    summed whole."""
    order = sorted((d, name, v) for name, vals in by_kernel.items() for d, v, _ in vals)
    lead = []
    for d, name, v in order:
        if COPY_KERNEL not in name:
            break
        lead.append(v)
    if len(lead) < copy_count or len(lead) % copy_count:
        raise SystemExit(f"found {len(lead)} leading {COPY_KERNEL} dispatches, expected a multiple of {copy_count}")
    per = len(lead) // copy_count
    copies = [sum(lead[i * per:(i + 1) * per]) for i in range(copy_count)]
    spread = (max(copies) - min(copies)) / max(copies)
    if spread > 0.02:
        raise SystemExit(f"calibration copies disagree by {100 * spread:.1f}%: {copies}")
    return sum(copies) / copy_count


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int, copy_count: int = 3,
            grid: int | None = None):
    """grid: only the kernel's dispatches of this grid size (work-items), when one
    program launches it at several shapes."""
    fetch = counters_by_dispatch(fetch_csv, "FETCH_SIZE")
    write = counters_by_dispatch(write_csv, "WRITE_SIZE")
    copy_fetch = _copy_calibration(fetch, copy_count)
    copy_write = _copy_calibration(write, copy_count)
    keep = lambda g: grid is None or g == grid
    kf = [v for name, vals in fetch.items() if name == kernel for _, v, g in vals if keep(g)]
    kw = [v for name, vals in write.items() if name == kernel for _, v, g in vals if keep(g)]
    if not kf or not kw:
        raise SystemExit(f"kernel {kernel!r} not in the counter files (have {sorted(fetch)})")
    copy_kib = copy_bytes / 1024.0
    fs, ws = copy_kib / copy_fetch, copy_kib / copy_write
    f_kib, w_kib = sum(kf) / len(kf), sum(kw) / len(kw)
    return {"kernel": kernel, "dispatches": len(kf),
            "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
            "copy_bytes": copy_bytes, "copy_fetch_kib": round(copy_fetch, 1), "copy_write_kib": round(copy_write, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "fetch_bytes_per_launch": round(f_kib * fs * 1024),
            "write_bytes_per_launch": round(w_kib * ws * 1024),
            "traffic_bytes_per_launch": round((f_kib * fs + w_kib * ws) * 1024),
            "source_sha256": source_digest(kernel)}


def traffic_markdown(t: dict, workload: str, commands, algorithmic_bytes: int | None = None) -> str:
    t = dict(t, workload=workload)
    if algorithmic_bytes:
        t["algorithmic_bytes_per_launch"] = algorithmic_bytes
        t["traffic_over_algorithmic"] = round(t["traffic_bytes_per_launch"] / algorithmic_bytes, 3)
    out = [f"# HBM traffic of `{t['kernel']}` on {workload}", "", "Made by (one counter per run):", ""]
    out += ["```", *commands, "```", ""]
    out += [f"- raw counters per dispatch (average of {t['dispatches']}): FETCH_SIZE {t['fetch_kib_per_dispatch']} KiB,"
            f" WRITE_SIZE {t['write_kib_per_dispatch']} KiB",
            f"- calibration: a {t['copy_bytes'] / 2**20:.0f} MiB device-to-device copy reads as FETCH_SIZE "
            f"{t['copy_fetch_kib']} KiB and WRITE_SIZE {t['copy_write_kib']} KiB, so the scale factors are "
            f"{t['fetch_scale']} and {t['write_scale']}",
            f"- traffic per launch: {t['fetch_bytes_per_launch'] / 2**20:.1f} MiB read + "
            f"{t['write_bytes_per_launch'] / 2**20:.1f} MiB written = {t['traffic_bytes_per_launch'] / 2**20:.1f} MiB"]
    if algorithmic_bytes:
        out.append(f"- algorithmic bytes per launch: {algorithmic_bytes / 2**20:.1f} MiB "
                   f"(ratio {t['traffic_over_algorithmic']})")
    out += ["", "```json", json.dumps(t, indent=1), "```", ""]
    return "\n".join(out)


def read_traffic(path: str, kernel: str, workload: str):
    """Measured traffic (bytes per launch) from a traffic summary, or None when the
    summary is missing, is for another kernel or workload, or the kernel's sources
    changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    if not m:
        return None
    t = json.loads(m.group(1))
    if t.get("kernel") != kernel or t.get("workload") != workload:
        return None
    if t.get("source_sha256") != source_digest(kernel):
        return None
    return t


# Counters of the MFMA-utilisation summary (one rocprofv3 --pmc pass: 8 SQ and 1 GRBM counters).
SQ_COUNTERS = ["SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"]
N_XCD, N_SIMD = 8, 1024  # MI355X: GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs


def counters(path: str, grids=None):
    """Per kernel: launches and the per-launch average of every counter in
    SQ_COUNTERS (only dispatches whose size in work-items is one of `grids`, if
    given)."""
    per = defaultdict(lambda: defaultdict(float))
    names = {}
    keep = None if not grids else set(grids)
    with open(path) as f:
        for r in csv.DictReader(f):
            if keep is not None and int(r["Grid_Size"]) not in keep:
                continue
            d = int(r["Dispatch_Id"])
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
            names[d] = short_name(r["Kernel_Name"])
    out = defaultdict(lambda: defaultdict(list))
    for d, cs in per.items():
        for c, v in cs.items():
            out[names[d]][c].append(v)
    return {k: {"launches": len(next(iter(cs.values()))), **{c: sum(v) / len(v) for c, v in cs.items()}}
            for k, cs in out.items()}


def counters_markdown(path: str, commands, kernels, title: str, grids=None) -> str:
    cs = counters(path, grids)
    out = [f"# {title}", "", "Made by:", "", "```", *commands, "```", "",
           "Per launch (average over launches). cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs);",
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); VALU/MFMA counts the non-MFMA vector",
           "instructions per MFMA; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (waves stalled on a dependency counter).", "",
           "| kernel | launches | cycles | MFMA busy | MFMAs | VALU/MFMA | LDS/MFMA | LDS bank conflicts | waiting |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k in kernels:
        if k not in cs:
            raise SystemExit(f"kernel {k!r} not in {path} (have {sorted(cs)})")
        c = cs[k]
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
        mf = c["SQ_INSTS_MFMA"]
        out.append(f"| `{k}` | {c['launches']} | {cyc:.4g} | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMD * cyc):.3f} | "
                   f"{mf:.4g} | {(c['SQ_INSTS_VALU'] - mf) / mf:.2f} | {c['SQ_INSTS_LDS'] / mf:.2f} | "
                   f"{c['SQ_LDS_BANK_CONFLICT']:.0f} | {c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.2f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", action="append", default=[])
    s.add_argument("--title")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--trace", help="the run's *_kernel_trace.csv (for --timed)")
    s.add_argument("--timed", action="append", default=[],
                   help="KERNEL:SKIP_FIRST:SKIP_LAST: also average KERNEL over its launches without the first and last ones")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--copy-count", type=int, default=3)
    t.add_argument("--algorithmic-bytes", type=int)
    t.add_argument("--grid", type=int, help="only dispatches of this grid size (work-items)")
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--out", required=True)
    d = sub.add_parser("dispatches")
    d.add_argument("--csv", required=True, help="the *_kernel_trace.csv of a --kernel-trace run")
    d.add_argument("--match", action="append", required=True, help="substring of the kernel names to list")
    d.add_argument("--last", type=int, help="only the last N matching dispatches")
    d.add_argument("--command", action="append", default=[])
    d.add_argument("--title", default="Kernel dispatches")
    d.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--title", default="MFMA utilisation from SQ counters")
    c.add_argument("--grid", type=int, action="append",
                   help="only dispatches of this grid size (work-items); may be repeated")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        timed = []
        for spec in a.timed:
            kernel, first, last = spec.rsplit(":", 2)
            timed.append((kernel, int(first), int(last)))
        if timed and not a.trace:
            raise SystemExit("--timed needs --trace")
        text = stats_markdown(a.csv, a.command, a.top, a.title, a.trace, timed)
    elif a.cmd == "dispatches":
        text = dispatches_markdown(a.csv, a.command, a.match, a.last, a.title)
    elif a.cmd == "counters":
        text = counters_markdown(a.csv, a.command, a.kernel, a.title, a.grid)
    else:
        tr = traffic(a.fetch, a.write, a.kernel, a.copy_mib << 20, a.copy_count, a.grid)
        if a.grid is not None:
            tr["grid_size"] = a.grid
        text = traffic_markdown(tr, a.workload, a.command, a.algorithmic_bytes)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
