"""Summaries of rocprofv3 CSV output for the draft-step kernels (host only).

    python -m tree_causal_draft_parent_amd.profsum stats DIR [--by-grid] [--cold-after SUBSTR]
        per-kernel calls / average / total duration from *_kernel_stats.csv
        (--by-grid: per kernel and grid size, from *_kernel_trace.csv;
        --cold-after: split each row into flushed and warm launches, a
        launch being flushed when a kernel whose name holds SUBSTR -- the
        cache-evicting write -- ran after the previous launch of the same
        kernel)
    python -m tree_causal_draft_parent_amd.profsum traffic --fetch DIR --write DIR \
            --copy-fetch DIR --copy-write DIR --copy-bytes N --out JSON
        per-launch FETCH_SIZE / WRITE_SIZE of every libjf kernel, scaled by the
        factor that makes the same counters read N bytes for a plain copy
        kernel of N bytes read and N bytes written; written as JSON together
        with hashes of the kernel sources, whole and per file (a reader treats
        a call's figures as stale once its kernel's source file changes).

FETCH_SIZE and WRITE_SIZE are rocprofv3 derived counters in KiB per dispatch
(bytes the L2 requested from / wrote to the memory fabric; on MI355X the
fabric side holds the 256 MiB last-level cache in front of HBM).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def short_name(name: str) -> str:
    """'void jf::(anonymous namespace)::k_fuse_gemm_bf16<256>(jf::...)' -> 'k_fuse_gemm_bf16<256>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, c in enumerate(n):          # first '(' outside template brackets ends the name
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0 and not n[:i].endswith("anonymous namespace") and \
                not n[i:].startswith("(anonymous namespace)"):
            cut = i
            break
    n = n[:cut]
    n = n.replace("jf::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return n


def file_hashes() -> dict:
    """sha256 of each kernel source file (basename -> hex digest)."""
    out = {}
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))):
        with open(p, "rb") as f:
            out[os.path.basename(p)] = hashlib.sha256(f.read()).hexdigest()
    return out


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _one(dirname: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirname}")
    return hits[-1]


def read_stats(dirname: str):
    rows = []
    with open(_one(dirname, "_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append(dict(name=short_name(r["Name"]), calls=int(r["Calls"]),
                             avg_us=float(r["AverageNs"]) / 1e3, total_us=float(r["TotalDurationNs"]) / 1e3,
                             min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3,
                             pct=float(r["Percentage"])))
    return rows


def read_counter(dirname: str, counter: str):
    """kernel short name -> list of per-dispatch values (KiB for *_SIZE)."""
    per = defaultdict(dict)
    with open(_one(dirname, "_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            # one derived value per dispatch; sum if the tool split it
            d = per[short_name(r["Kernel_Name"])]
            did = r["Dispatch_Id"]
            d[did] = d.get(did, 0.0) + float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def read_trace_by_grid(dirname: str):
    """(kernel short name, grid size) -> per-dispatch durations in us, from
    *_kernel_trace.csv: one kernel launched at two shapes shows as two rows."""
    per = defaultdict(list)
    with open(_one(dirname, "_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]))
            per[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return per


def read_trace_split(dirname: str, flush_substr: str):
    """(kernel short name, grid size) -> (flushed durations, warm durations)
    in us.  In dispatch (start-time) order, a launch is flushed when a kernel
    whose full name contains flush_substr started after the previous launch
    of the same kernel (or before the first one)."""
    rows = []
    with open(_one(dirname, "_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                         int(r["Grid_Size_X"])))
    rows.sort(key=lambda t: t[0])
    last_flush = -1
    last_seen = {}
    per = defaultdict(lambda: ([], []))
    for i, (t0, t1, name, grid) in enumerate(rows):
        if flush_substr in name:
            last_flush = i
            continue
        key = (short_name(name), grid)
        cold = last_flush > last_seen.get(key, -1)
        last_seen[key] = i
        per[key][0 if cold else 1].append((t1 - t0) / 1e3)
    return per


def cmd_stats(a):
    if a.cold_after:
        per = read_trace_split(a.dir, a.cold_after)
        print("| kernel | grid (threads) | flushed calls | flushed avg us | warm calls | warm avg us |")
        print("|---|---:|---:|---:|---:|---:|")
        for (name, grid), (c, w) in sorted(per.items(), key=lambda kv: -sum(kv[1][0]) - sum(kv[1][1])):
            if not name.startswith("k_"):
                continue
            fmt = lambda v: f"{_mean(v):.2f}" if v else "-"
            print(f"| `{name}` | {grid} | {len(c)} | {fmt(c)} | {len(w)} | {fmt(w)} |")
        return
    if a.by_grid:
        per = read_trace_by_grid(a.dir)
        print(f"{'kernel':44s} {'grid':>8s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}")
        for (name, grid), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            print(f"{name[:44]:44s} {grid:8d} {len(v):6d} {_mean(v):9.2f} {min(v):9.2f} {max(v):9.2f}")
        return
    rows = read_stats(a.dir)
    print(f"{'kernel':44s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'total %':>8s}")
    for r in rows:
        print(f"{r['name'][:44]:44s} {r['calls']:6d} {r['avg_us']:9.2f} {r['min_us']:9.2f} "
              f"{r['max_us']:9.2f} {r['pct']:8.2f}")


def _mean(v):
    return sum(v) / len(v) if v else 0.0


def read_counters_by_grid(dirname: str):
    """(kernel short name, grid size) -> {counter: [per-dispatch values]} from
    *_counter_collection.csv (values of one dispatch summed when the tool
    splits them)."""
    per = defaultdict(lambda: defaultdict(dict))
    with open(_one(dirname, "_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            d = per[key][r["Counter_Name"]]
            did = r["Dispatch_Id"]
            d[did] = d.get(did, 0.0) + float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def cmd_counters(a):
    """Per (kernel, grid) average of every counter over the given runs."""
    merged = defaultdict(dict)
    for d in a.dirs:
        for key, cs in read_counters_by_grid(d).items():
            for c, v in cs.items():
                merged[key][c] = _mean(v)
    for (name, grid), cs in sorted(merged.items()):
        if not name.startswith("k_"):
            continue
        print(f"{name} grid={grid}")
        for c, v in sorted(cs.items()):
            print(f"    {c:32s} {v:16.1f}")


def cmd_traffic(a):
    fetch = read_counter(a.fetch, "FETCH_SIZE")
    write = read_counter(a.write, "WRITE_SIZE")
    cf = read_counter(a.copy_fetch, "FETCH_SIZE")
    cw = read_counter(a.copy_write, "WRITE_SIZE")
    # the copy kernel is the one with the largest per-dispatch read volume
    ck = max(cf, key=lambda k: _mean(cf[k]))
    f_kib, w_kib = _mean(cf[ck]), _mean(cw.get(ck, [0.0]))
    factor_f = a.copy_bytes / (f_kib * 1024.0) if f_kib > 0 else None
    factor_w = a.copy_bytes / (w_kib * 1024.0) if w_kib > 0 else None
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        if not k.startswith("k_"):
            continue
        fk, wk = _mean(fetch.get(k, [])), _mean(write.get(k, []))
        kernels[k] = {"launches": len(fetch.get(k, [])),
                      "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                      "fetch_bytes": round(fk * 1024.0 * factor_f) if factor_f else None,
                      "write_bytes": round(wk * 1024.0 * factor_w) if factor_w else None}
    out = {"sources_sha256": sources_hash(),
           "file_sha256": file_hashes(),
           "workload": a.workload,
           "copy_calibration": {"kernel": ck, "bytes_each_way": a.copy_bytes,
                                "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1),
                                "factor_fetch": factor_f, "factor_write": factor_w},
           "kernels": kernels,
           "commands": a.commands}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--by-grid", action="store_true",
                   help="per (kernel, grid size) from the kernel trace instead of the stats file")
    s.add_argument("--cold-after", default="",
                   help="split launches into flushed / warm by the last kernel whose name holds this")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", default="")
    t.add_argument("--commands", nargs="*", default=[])
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
