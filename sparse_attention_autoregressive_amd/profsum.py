"""Summaries of rocprofv3 result databases (SQLite) for the files under profiles/.

    python -m sparse_attention_autoregressive_amd.profsum trace DB --title T --cmd C
        per-kernel calls and mean / median / min duration (us) of a --kernel-trace run.

    python -m sparse_attention_autoregressive_amd.profsum traffic --fetch DB --write DB \
        --kernel REGEX --copy-mib N --workload W --cmd C
        HBM bytes per dispatch of the kernels matching REGEX from a FETCH_SIZE run and a
        WRITE_SIZE run, each scaled by what the same counter reads for the plain device
        copy of N MiB that bench.py --calib-copy-mib N runs first (the largest copy
        kernel in the run), so that a counter that over- or under-counts is corrected by
        a transfer of known size. Also records the SHA-256 of the kernel source, so a
        reader (bench.py) can tell whether the figures still describe the current kernel.

    python -m sparse_attention_autoregressive_amd.profsum counters CSV [CSV ...] \
        --title T --cmd C [--sets S ...]
        mean per-dispatch value of every counter in the --pmc runs' counter_collection
        CSV files (one run per counter set), for each library kernel, the wave-cycle
        split of the attention kernel and each kernel's L2 hit rate (when TCC_HIT_sum and
        TCC_MISS_sum were collected); C is the command with <set> for the counter list.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sqlite3
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(PKG, "csrc", "attn.hip")


def source_sha(path: str = ATTN_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _short(name: str) -> str:
    n = re.sub(r"\(.*", "", name.replace("(anonymous namespace)", "anon"))
    return n if len(n) < 90 else n[:87] + "..."


def trace(db: str, title: str, cmd: str) -> str:
    """Per-kernel table; a kernel launched with several grid sizes (e.g. pooling a whole
    key prefix and pooling one chunk's frames) gets one row per grid size."""
    c = sqlite3.connect(db)
    try:
        rows = c.execute("select name, duration, grid_x / workgroup_x from kernels").fetchall()
        with_grid = True
    except sqlite3.OperationalError:                    # a database without launch shapes
        rows = [(n, d, None) for n, d in c.execute("select name, duration from kernels").fetchall()]
        with_grid = False
    by = {}
    for n, d, wgs in rows:
        by.setdefault((n, wgs), []).append(d / 1000.0)
    out = [f"# {title}", "", f"Command: `{cmd}`", ""]
    if with_grid:
        out += ["| kernel | workgroups | calls | mean us | median us | min us |", "|---|---|---|---|---|---|"]
    else:
        out += ["| kernel | calls | mean us | median us | min us |", "|---|---|---|---|---|"]
    for (n, wgs), ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        if "lf::" not in n and "_ZN2lf" not in n:
            continue
        grid = f" {wgs} |" if with_grid else ""
        out.append(f"| `{_short(n)}` |{grid} {len(ds)} | {statistics.mean(ds):.2f} | "
                   f"{statistics.median(ds):.2f} | {min(ds):.2f} |")
    return "\n".join(out)


def _per_kernel(db: str, counter: str):
    c = sqlite3.connect(db)
    q = "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?"
    by = {}
    for name, disp, v in c.execute(q, (counter,)):
        by.setdefault(name, {}).setdefault(disp, 0.0)
        by[name][disp] += v
    return by


def traffic(fetch_db: str, write_db: str, kernel: str, copy_mib: int, workload: str, cmd: str) -> str:
    pat = re.compile(kernel)
    ref_kib = copy_mib * 1024.0
    res = {}
    for label, db, counter in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        by = _per_kernel(db, counter)
        # the calibration copy: the copy kernel with the largest counter value
        copies = [max(d.values()) for n, d in by.items() if "copy" in n.lower()]
        if not copies:
            raise SystemExit(f"no copy kernel found in {db}")
        copy_kib = max(copies)
        hits = [v for n, d in by.items() if pat.search(n) for v in d.values()]
        if not hits:
            raise SystemExit(f"no dispatch of {kernel} in {db}")
        res[label] = dict(kib=statistics.median(hits), copy_kib=copy_kib, factor=ref_kib / copy_kib, n=len(hits))
    f, w = res["fetch"], res["write"]
    total = (f["kib"] * f["factor"] + w["kib"] * w["factor"]) * 1024.0
    lines = [
        f"# HBM traffic per dispatch: {kernel} on {workload}",
        "",
        f"Commands (two runs, one counter each): `{cmd}`",
        "",
        f"kernel_regex: {kernel}",
        f"workload: {workload}",
        f"source_sha256: {source_sha()}",
        f"fetch_kib_per_dispatch: {f['kib']:.1f}",
        f"write_kib_per_dispatch: {w['kib']:.1f}",
        f"dispatches: {f['n']} / {w['n']}",
        f"calibration_copy_mib: {copy_mib}",
        f"copy_fetch_kib: {f['copy_kib']:.1f}",
        f"copy_write_kib: {w['copy_kib']:.1f}",
        f"fetch_factor: {f['factor']:.4f}",
        f"write_factor: {w['factor']:.4f}",
        f"traffic_bytes_per_dispatch: {total:.0f}",
    ]
    return "\n".join(lines)


_KERNELS = (("attn_bf16_kernel", "attention"), ("select_kernel", "selection"),
            ("select_1d_kernel", "single-level selection"), ("block_mean_kernel", "block means"),
            ("frame_mean_kernel", "frame means"), ("prologue_kernel", "prologue"))


def counters(csvs, title: str, cmd: str, asked=None) -> str:
    vals, sets, durs = {}, [], {}
    for path in csvs:
        names = []
        for r in csv.DictReader(open(path)):
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            for key, label in _KERNELS:
                if key in r["Kernel_Name"]:
                    vals.setdefault(label, {}).setdefault(c, []).append(float(r["Counter_Value"]))
                    if key == "attn_bf16_kernel":
                        durs[(path, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        sets.append(" ".join(names))
    cols = [c for s_ in sets for c in s_.split()]
    out = [f"# {title}", "", "Commands (one run per counter set, from /tmp):", ""]
    for i, found in enumerate(sets):
        given = asked[i] if asked and i < len(asked) and asked[i] else found
        out.append(f"- `{cmd.replace('<set>', given)}`")
    out += ["", f"attn.hip sha256: {source_sha()}"]
    if durs:
        out.append(f"attention dispatch duration under counters: median {statistics.median(durs.values()):.1f} us")
    out += ["", "Mean per dispatch (derived counters in rocprofv3's definitions; SQ counters summed over the device):",
            "", "| kernel | dispatches | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
    for _, label in _KERNELS:
        if label not in vals:
            continue
        m = vals[label]
        n = max(len(v) for v in m.values())
        out.append(f"| {label} | {n} | " + " | ".join(
            f"{statistics.mean(m[c]):.4g}" if c in m else "-" for c in cols) + " |")
    a = vals.get("attention", {})
    if "SQ_WAVE_CYCLES" in a:
        w = statistics.mean(a["SQ_WAVE_CYCLES"])
        out += ["", "Attention wave cycles (same units):", ""]
        for c, what in (("SQ_WAIT_ANY", "waiting on s_waitcnt"), ("SQ_WAIT_INST_ANY", "ready, not issued"),
                        ("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_ACTIVE_INST_LDS", "issuing LDS"),
                        ("SQ_ACTIVE_INST_VMEM", "issuing vector memory"), ("SQ_WAIT_INST_LDS", "waiting on LDS issue")):
            if c in a:
                out.append(f"- {what} ({c}): {statistics.mean(a[c]) / w * 100:.1f}%")
    hits = [(label, vals[label]) for _, label in _KERNELS
            if label in vals and "TCC_HIT_sum" in vals[label] and "TCC_MISS_sum" in vals[label]]
    if hits:
        out += ["", "L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)):", ""]
        for label, m in hits:
            h, s = statistics.mean(m["TCC_HIT_sum"]), statistics.mean(m["TCC_MISS_sum"])
            out.append(f"- {label}: {h / (h + s) * 100:.1f}% of {h + s:.4g} requests")
    return "\n".join(out)


def read_traffic(path: str):
    """(bytes per dispatch, workload) from a traffic summary if its source hash matches the
    current kernel source, else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "Commands")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha():
        return None
    return float(kv["traffic_bytes_per_dispatch"]), kv.get("workload")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--copy-mib", type=int, required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--cmd", required=True)
    k = sub.add_parser("counters")
    k.add_argument("csv", nargs="+")
    k.add_argument("--title", required=True)
    k.add_argument("--cmd", required=True)
    k.add_argument("--sets", nargs="*", help="the --pmc lists as given, one per CSV (default: names found)")
    a = ap.parse_args(argv)
    if a.cmd_ == "trace":
        print(trace(a.db, a.title, a.cmd))
    elif a.cmd_ == "counters":
        print(counters(a.csv, a.title, a.cmd, a.sets))
    else:
        print(traffic(a.fetch, a.write, a.kernel, a.copy_mib, a.workload, a.cmd))


if __name__ == "__main__":
    sys.exit(main())
