"""Summaries of rocprofv3 output for the profile notes kept with the repository.

* ``stats``: per-kernel calls, average and total duration from a ``--kernel-trace --stats`` run
  (the ``*_kernel_stats.csv`` file).
* ``traffic``: HBM bytes per dispatch of the kernels matching a name pattern, from two
  ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs, each scaled by what the same counter reads for
  a plain device copy of known size (``bench.py --copy-calibration``). The result also goes to a
  JSON file that ``bench.py`` reads for ``roofline.traffic`` as long as the hash of the kernel
  sources it records still matches.

    python -m selective_recompute_cf_amd.profiles stats <kernel_stats.csv> <out.md> --command "..."
* ``counters``: per kernel group, the average of each counter per dispatch over ``--pmc`` passes,
  with the matrix-core busy share, the waiting share, the LDS bank-conflict share and vector-ALU
  instructions per MFMA instruction.
* ``overlap``: from a ``--kernel-trace --memory-copy-trace`` run, how much of the host-to-device
  copy time (and of the kernels matching a side pattern, e.g. the copy stream's re-position)
  falls inside the execution intervals of the other kernels, counted from the first dispatch of
  a start kernel on.

    python -m selective_recompute_cf_amd.profiles traffic --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --pattern gemm_bf16 \
        --out-md OUT.md --out-json OUT.json --command "..."
    python -m selective_recompute_cf_amd.profiles overlap <kernel_trace.csv> <memory_copy_trace.csv> <out.md> \
        --start embed_kernel --side reposition --command "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import shutil
import subprocess
from collections import OrderedDict

PKG = os.path.dirname(os.path.abspath(__file__))
# sources whose compiled code the GEMM traffic figures describe: the GEMM file, the common header
# and the GEMM section of the shared declarations header (from its section marker to the next)
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h", "csrc/kernels.h#GEMM (gemm.hip)")


def _source_text(rel: str) -> bytes:
    path, _, section = rel.partition("#")
    with open(os.path.join(PKG, path), "rb") as f:
        text = f.read()
    if not section:
        return text
    lines = text.decode().splitlines(keepends=True)
    start = next(i for i, l in enumerate(lines) if l.startswith("// ---") and l.rstrip().endswith(section))
    end = next((i for i in range(start + 1, len(lines)) if lines[i].startswith("// ---")), len(lines))
    return "".join(lines[start:end]).encode()


def sources_sha256(rel_paths=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in rel_paths:
        h.update(rel.encode() + b"\0" + _source_text(rel) + b"\0")
    return h.hexdigest()


def _demangle(name: str) -> str:
    if not name.startswith("_Z"):
        return name
    if shutil.which("c++filt"):
        out = subprocess.run(["c++filt", name], capture_output=True, text=True).stdout.strip()
        if out and not out.startswith("_Z"):
            return out
    # names this c++filt cannot read (the bf16 type): namespace::name<element type>
    m = re.match(r"_ZN(\d+)(\w+)", name)
    if not m:
        return name
    n1 = int(m.group(1))
    ns, rest = m.group(2)[:n1], m.group(2)[n1:]
    m2 = re.match(r"(\d+)", rest)
    if not m2:
        return name
    n2 = int(m2.group(1))
    base = rest[len(m2.group(1)):len(m2.group(1)) + n2]
    tail = rest[len(m2.group(1)) + n2:]
    targ = "<__bf16>" if tail.startswith("IDF16b") else "<float>" if tail.startswith("IfE") else ""
    return f"{ns}::{base}{targ}"


def short_name(name: str) -> str:
    """Kernel name without the argument list (template arguments kept)."""
    name = _demangle(name.strip().strip('"'))
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def kernel_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "avg_us": float(r["AverageNs"]) / 1e3, "pct": float(r["Percentage"])})
    rows.sort(key=lambda x: -x["total_ms"])
    return rows


def counter_per_dispatch(path: str, counter: str, pattern: str):
    """[(kernel name, summed counter value)] per dispatch whose name matches `pattern`."""
    per = OrderedDict()
    rx = re.compile(pattern)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not rx.search(r["Kernel_Name"]):
                continue
            key = (int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(k[1], v) for k, v in per.items()]


def copy_factor(path: str, counter: str, copy_bytes: int, pattern: str = "copyBuffer") -> float:
    """Bytes per counter KiB: the copy moves copy_bytes in (FETCH) and out (WRITE) per dispatch."""
    vals = [v for _, v in counter_per_dispatch(path, counter, pattern)]
    if not vals:
        raise SystemExit(f"no '{pattern}' dispatch with {counter} in {path}")
    kib = sum(vals) / len(vals)
    return copy_bytes / (kib * 1024.0)


def cmd_stats(a):
    rows = kernel_stats(a.csv)
    tot = sum(r["total_ms"] for r in rows)
    lines = [f"# {a.title}", "", "Command:", "", "```", a.command, "```", "",
             f"rocprofv3 kernel-trace statistics, {sum(r['calls'] for r in rows)} dispatches, "
             f"{tot:.2f} ms of kernel time in total.", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows[: a.top]:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['total_ms']:.3f} | {r['pct']:.2f} |")
    if a.group:
        rx = re.compile(a.group)
        g = [r for r in rows if rx.search(r["name"])]
        calls = sum(r["calls"] for r in g)
        ms = sum(r["total_ms"] for r in g)
        lines += ["", f"Kernels matching `{a.group}` together: {calls} calls, {ms:.3f} ms, "
                      f"average {ms / max(calls, 1) * 1e3:.2f} us per launch."]
        if a.tail_trace:
            # the last dispatches of the group are the event-timed steps when nothing runs after them
            with open(a.tail_trace) as f:
                tr = [r for r in csv.DictReader(f) if rx.search(short_name(r["Kernel_Name"]))]
            tr.sort(key=lambda r: int(r["Start_Timestamp"]))
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr[-a.tail:]]
            lines += [f"The last {len(d)} of them in the kernel trace (the event-timed steps, which run last): "
                      f"average {sum(d) / max(len(d), 1):.2f} us per launch."]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def cmd_traffic(a):
    ff = copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    wf = copy_factor(a.copy_write, "WRITE_SIZE", a.copy_bytes)
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.pattern)
    write = counter_per_dispatch(a.write, "WRITE_SIZE", a.pattern)
    if not fetch or not write:
        raise SystemExit("no matching dispatches")
    by_name = OrderedDict()
    for (n, v) in fetch:
        by_name.setdefault(n, {"fetch": [], "write": []})["fetch"].append(v * 1024 * ff)
    for (n, v) in write:
        by_name.setdefault(n, {"fetch": [], "write": []})["write"].append(v * 1024 * wf)
    allf = [x for d in by_name.values() for x in d["fetch"]]
    allw = [x for d in by_name.values() for x in d["write"]]
    res = {
        "kernel_pattern": a.pattern,
        "source_sha256": sources_sha256(),
        "copy_bytes": a.copy_bytes,
        "fetch_factor": ff,
        "write_factor": wf,
        "dispatches": len(allf),
        "fetch_bytes_per_launch": sum(allf) / len(allf),
        "write_bytes_per_launch": sum(allw) / len(allw),
        "command": a.command,
        "per_kernel": {n: {"dispatches": len(d["fetch"]),
                           "fetch_bytes_per_launch": sum(d["fetch"]) / max(len(d["fetch"]), 1),
                           "write_bytes_per_launch": sum(d["write"]) / max(len(d["write"]), 1)}
                       for n, d in by_name.items()},
    }
    res["traffic_bytes_per_launch"] = res["fetch_bytes_per_launch"] + res["write_bytes_per_launch"]
    if a.out_json:
        with open(a.out_json, "w") as f:
            json.dump(res, f, indent=1)
    # average durations from a kernel-trace run without counters, for the bytes' rate
    avg_us = {r["name"]: r["avg_us"] for r in kernel_stats(a.durations)} if a.durations else {}
    lines = [f"# {a.title}", "", "Commands:", "", "```", a.command, "```", "",
             f"Copy calibration: a {a.copy_bytes / 2**30:.2f} GiB device copy reads FETCH_SIZE "
             f"{a.copy_bytes / ff / 1024:.0f} KiB and WRITE_SIZE {a.copy_bytes / wf / 1024:.0f} KiB per dispatch, "
             f"so FETCH_SIZE x {ff:.3f} and WRITE_SIZE x {wf:.3f} give bytes.", "",
             f"Dispatches matching `{a.pattern}`: {len(allf)}; per launch on average "
             f"{res['fetch_bytes_per_launch'] / 1e6:.2f} MB fetched + {res['write_bytes_per_launch'] / 1e6:.2f} MB "
             f"written = {res['traffic_bytes_per_launch'] / 1e6:.2f} MB.", "",
             "| kernel | dispatches | fetch MB / launch | write MB / launch |"
             + (" avg us | GB/s | of 8 TB/s |" if avg_us else ""),
             "|---|---:|---:|---:|" + ("---:|---:|---:|" if avg_us else "")]
    for n, d in res["per_kernel"].items():
        row = (f"| `{n}` | {d['dispatches']} | {d['fetch_bytes_per_launch'] / 1e6:.2f} | "
               f"{d['write_bytes_per_launch'] / 1e6:.2f} |")
        if avg_us:
            us = avg_us.get(n)
            if us:
                gbs = (d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]) / (us * 1e3)
                row += f" {us:.2f} | {gbs:.0f} | {100 * gbs / 8000:.0f}% |"
            else:
                row += " n/a | n/a | n/a |"
        lines.append(row)
    if avg_us:
        lines += ["", "Rates divide the counted bytes by the average duration of the same kernel in the kernel-trace "
                      "run (no counters): bytes served by the MALL count as traffic, so a rate can exceed what HBM "
                      "alone delivers."]
    if a.out_json:
        lines += ["", f"Kernel sources hash (sha256 of {', '.join(GEMM_SOURCES)}): `{res['source_sha256']}`"]
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _union(intervals):
    out = []
    for s, e in sorted(intervals):
        if out and s <= out[-1][1]:
            out[-1][1] = max(out[-1][1], e)
        else:
            out.append([s, e])
    return out


def _covered(union, s, e):
    """Length of [s, e) inside the (sorted, disjoint) union."""
    import bisect
    i = max(0, bisect.bisect_right([u[0] for u in union], s) - 1)
    c = 0
    while i < len(union) and union[i][0] < e:
        c += max(0, min(e, union[i][1]) - max(s, union[i][0]))
        i += 1
    return c


def cmd_overlap(a):
    kt = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
          for r in csv.DictReader(open(a.kernel_trace))]
    cp = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
          for r in csv.DictReader(open(a.copy_trace)) if r["Direction"] == "MEMORY_COPY_HOST_TO_DEVICE"]
    starts = [s for s, _, n in kt if a.start in n]
    if not starts:
        raise SystemExit(f"no '{a.start}' dispatch in {a.kernel_trace}")
    t0 = min(starts)
    side = [(s, e) for s, e, n in kt if s >= t0 and a.side in n]
    main_u = _union([(s, e) for s, e, n in kt if s >= t0 and a.side not in n])
    copies = [(s, e) for s, e in cp if s >= t0]
    if not copies:
        raise SystemExit("no host-to-device copy after the start kernel")
    c_tot = sum(e - s for s, e in copies)
    c_cov = sum(_covered(main_u, s, e) for s, e in copies)
    s_tot = sum(e - s for s, e in side)
    s_cov = sum(_covered(main_u, s, e) for s, e in side)
    m_tot = sum(e - s for s, e in main_u)
    lines = [f"# {a.title}", "", "Commands:", "", "```", a.command, "```", "",
             f"Counted from the first `{a.start}` dispatch on; the other kernels are every dispatch whose name does "
             f"not contain `{a.side}`.", "",
             f"- Host-to-device copies: {len(copies)}, {c_tot / 1e6:.2f} ms in total, "
             f"{c_tot / len(copies) / 1e3:.1f} us on average; {c_cov / 1e6:.2f} ms "
             f"({100 * c_cov / c_tot:.1f}%) of it while other kernels ran.",
             f"- `{a.side}` dispatches: {len(side)}, {s_tot / 1e6:.2f} ms in total"
             + (f", {s_tot / len(side) / 1e3:.1f} us on average; {s_cov / 1e6:.2f} ms ({100 * s_cov / s_tot:.1f}%) "
                f"of it while other kernels ran." if side else "."),
             f"- The other kernels were busy (union of their intervals) for {m_tot / 1e6:.2f} ms."]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


CLOCK_GHZ = 2.4  # MI355X peak engine clock
SIMDS = 256 * 4  # compute units x SIMDs per unit


def cmd_counters(a):
    """Per kernel group: each counter's average per dispatch over one or more --pmc passes, and the
    derived shares: matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / (dispatch time x clock x SIMDs);
    waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS bank conflicts = SQ_LDS_BANK_CONFLICT /
    SQ_LDS_IDX_ACTIVE; vector-ALU instructions per MFMA instruction."""
    groups = [(g.split("=", 1)[0], re.compile(g.split("=", 1)[1])) for g in a.group]
    val = {g: {} for g, _ in groups}   # counter -> [sum, dispatches]
    dur = {g: {} for g, _ in groups}   # counter -> summed dispatch ns (for the MFMA share)
    for path in a.csv:
        for r in csv.DictReader(open(path)):
            for g, rx in groups:
                if rx.search(r["Kernel_Name"]):
                    c = r["Counter_Name"]
                    v = val[g].setdefault(c, [0.0, 0])
                    v[0] += float(r["Counter_Value"])
                    v[1] += 1
                    dur[g][c] = dur[g].get(c, 0) + int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    break
    lines = [f"# {a.title}", "", "Commands:", "", "```", a.command, "```", "",
             f"Derived shares: matrix cores busy = SQ_VALU_MFMA_BUSY_CYCLES / (dispatch time x {CLOCK_GHZ} GHz x "
             f"{SIMDS} SIMDs); waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS bank conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; VALU per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA.", "",
             "| group | dispatches | matrix cores busy | waiting | LDS bank conflicts | VALU per MFMA |",
             "|---|---:|---:|---:|---:|---:|"]

    def avg(g, c):
        v = val[g].get(c)
        return v[0] / v[1] if v and v[1] else None

    def pct(x):
        return "n/a" if x is None else f"{100 * x:.1f}%"

    for g, _ in groups:
        if not val[g]:
            continue
        n = max(v[1] for v in val[g].values())
        mf = val[g].get("SQ_VALU_MFMA_BUSY_CYCLES")
        busy = mf[0] / (dur[g]["SQ_VALU_MFMA_BUSY_CYCLES"] * CLOCK_GHZ * SIMDS) if mf else None
        wc, wi = avg(g, "SQ_WAVE_CYCLES"), avg(g, "SQ_WAIT_INST_ANY")
        li, lb = avg(g, "SQ_LDS_IDX_ACTIVE"), avg(g, "SQ_LDS_BANK_CONFLICT")
        iv, im = avg(g, "SQ_INSTS_VALU"), avg(g, "SQ_INSTS_MFMA")
        lines.append(f"| {g} | {n} | {pct(busy)} | {pct(wi / wc if wi is not None and wc else None)} | "
                     f"{pct(lb / li if lb is not None and li else None)} | "
                     f"{'n/a' if not (iv and im) else f'{iv / im:.2f}'} |")
    lines += ["", "Average per dispatch:", "", "| group | counter | value |", "|---|---|---:|"]
    for g, _ in groups:
        for c in sorted(val[g]):
            lines.append(f"| {g} | {c} | {avg(g, c):.0f} |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--title", default="Kernel statistics")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=25)
    s.add_argument("--group", default=None, help="also total the kernels whose names match this pattern")
    s.add_argument("--tail-trace", default=None, help="kernel_trace.csv: also average the group's last --tail dispatches")
    s.add_argument("--tail", type=int, default=0)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--pattern", required=True)
    t.add_argument("--out-md", required=True)
    t.add_argument("--out-json", default=None, help="also write the JSON that bench.py reads (GEMM traffic)")
    t.add_argument("--durations", default=None, help="kernel_stats.csv of a run without counters: adds GB/s")
    t.add_argument("--title", default="HBM traffic per dispatch")
    t.add_argument("--command", required=True)
    o = sub.add_parser("overlap")
    o.add_argument("kernel_trace")
    o.add_argument("copy_trace")
    o.add_argument("out")
    o.add_argument("--start", required=True, help="count from the first dispatch whose name contains this")
    o.add_argument("--side", required=True, help="kernels on the copy stream, reported like the copies")
    o.add_argument("--title", default="Copy and compute overlap")
    o.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+", help="counter_collection.csv files of one or more --pmc passes")
    c.add_argument("--out", required=True)
    c.add_argument("--group", action="append", required=True, help="NAME=REGEX over kernel names")
    c.add_argument("--title", default="Counters per kernel group")
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "overlap": cmd_overlap, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
