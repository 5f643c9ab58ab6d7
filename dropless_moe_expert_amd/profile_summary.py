"""Text summaries of rocprofv3 counter runs, for the committed profiles.

Measurement only: reads the CSV files that `rocprofv3 --pmc ... -f csv`
writes (one row per dispatch and counter, values summed over the chip) and
prints a markdown table per kernel:

* MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE / 8 XCCs x
  1024 SIMDs), i.e. the fraction of the kernel's cycles in which an average
  SIMD's matrix core was busy, and the clock the kernel ran at
  (GRBM_GUI_ACTIVE / 8 over its duration);
* HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
  what the same counter reads for a plain 1 GiB device copy in the same run
  (`bench.py --calibrate-copy` adds one), and the rate over the kernel's
  average duration.

    python -m dropless_moe_expert_amd.profile_summary --title T --command C \\
        [--trace kernel_stats.csv] [--mfma mfma.csv] [--fetch fetch.csv --write write.csv] \\
        [--json OUT --json-kernel NAME --source FILE]

--json writes {source hash, the kernel's HBM bytes per launch, its MFMA
busy fraction} for bench.py to quote while the source is unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import sys

XCC = 8            # GRBM_GUI_ACTIVE is summed over the XCCs
SIMDS = 1024       # 256 CUs x 4 SIMDs
COPY_KIB = 1 << 20  # the calibration copy moves 1 GiB each way


def _dispatches(path):
    """-> {dispatch id: {"name", "dur_ns", "grid", counter: value}}"""
    out = collections.defaultdict(dict)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            d = out[r["Dispatch_Id"]]
            d["name"] = r["Kernel_Name"]
            d["grid"] = int(r["Grid_Size"])
            d["dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _by_kernel(disp):
    k = collections.defaultdict(list)
    for d in disp.values():
        k[d["name"]].append(d)
    return k


def _mean(xs):
    xs = list(xs)
    return sum(xs) / len(xs) if xs else float("nan")


def _copy_scale(disp, counter):
    """COPY_KIB over what the counter reads for the run's 1 GiB copies: the
    largest device copies of the run (within 5 % of the largest reading),
    so that smaller copies in the same run do not enter the mean."""
    vals = [d[counter] for d in disp.values() if "copyBuffer" in d["name"] and d.get(counter)]
    if not vals:
        return None
    top = max(vals)
    return COPY_KIB / _mean(v for v in vals if v >= 0.95 * top)


def short(name: str) -> str:
    name = name.replace("|", "/")
    return name if len(name) <= 90 else name[:87] + "..."


def calibration(args) -> str:
    """Per-dispatch table of the counter passes of counter_calibration.py:
    each kernel's reading against the bytes it reads and writes."""
    lines = [f"# {args.title}", "", "Commands (from the repository root), one counter pass each:", ""]
    lines += ["    " + c for c in args.command] + [""]
    rows = collections.OrderedDict()
    for path in (args.fetch, args.write, args.mfma):
        if not path:
            continue
        for i, d in enumerate(_dispatches(path).values()):
            r = rows.setdefault(i, {"name": d["name"]})
            r.update({k: v for k, v in d.items() if k.isupper()})
    sizes = [int(x) for x in args.sizes.split(",")]
    lines.append("| dispatch | kernel | MiB read and written | FETCH_SIZE MiB | read / FETCH_SIZE | WRITE_SIZE MiB | "
                 "written / WRITE_SIZE |")
    lines.append("|---|---|---|---|---|---|---|")
    si = -1
    for i, r in rows.items():
        if "Fill" in r["name"]:   # each size starts with the fill of its source
            si += 1
            continue
        if si < 0 or ("copyBuffer" not in r["name"] and "elementwise" not in r["name"]):
            continue
        mib = sizes[min(si, len(sizes) - 1)]
        f, w = r.get("FETCH_SIZE", 0) / 1024, r.get("WRITE_SIZE", 0) / 1024
        lines.append(f"| {i} | `{short(r['name'])}` | {mib} | {f:.1f} | {mib / f if f else float('nan'):.3f} | "
                     f"{w:.1f} | {mib / w if w else float('nan'):.3f} |")
    return "\n".join(lines) + "\n"


def counters_table(args) -> str:
    """Per-kernel averages of every counter in one --pmc CSV (--counters),
    with the LDS figures derived from them when present: utilisation
    (SQ_LDS_IDX_ACTIVE over GRBM_GUI_ACTIVE / 8 XCCs x 256 CUs, the tool's
    own LDS-utilisation formula), bank-conflict cycles per active cycle, and
    the share of wave cycles spent waiting to issue an LDS instruction
    (SQ_WAIT_INST_LDS counts units of 4 cycles)."""
    lines = [f"# {args.title}", ""]
    for src in args.source or []:
        lines.append(f"{src.split('/')[-1]} sha256[:16] = {hashlib.sha256(open(src, 'rb').read()).hexdigest()[:16]}  ")
    lines += ["", "Command (from the repository root):", ""] + ["    " + c for c in args.command] + [""]
    kern = _by_kernel(_dispatches(args.counters))
    names = sorted({c for ds in kern.values() for c in ds[0] if c.isupper()})
    lines.append("| kernel | calls | avg us | LDS util | bank conflict / active | LDS issue wait / wave cycles | "
                 + " | ".join(names) + " |")
    lines.append("|---" * (6 + len(names)) + "|")
    for name, ds in kern.items():
        if args.kernel_filter and not any(f in name for f in args.kernel_filter):
            continue
        m = {c: _mean(d.get(c, 0.0) for d in ds) for c in names}
        cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / XCC
        util = 100 * m["SQ_LDS_IDX_ACTIVE"] / (cyc * 256) if cyc and "SQ_LDS_IDX_ACTIVE" in m else None
        conf = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"] if m.get("SQ_LDS_IDX_ACTIVE") else None
        wait = 4 * m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"] if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_LDS" in m else None
        f = lambda v, fmt: "" if v is None else fmt.format(v)   # noqa: E731
        lines.append(f"| `{short(name)}` | {len(ds)} | {_mean(d['dur_ns'] for d in ds) / 1e3:.1f} | "
                     f"{f(util, '{:.1f} %')} | {f(conf, '{:.3f}')} | {f(wait, '{:.2f}')} | "
                     + " | ".join(f"{m[c]:.4g}" for c in names) + " |")
    return "\n".join(lines) + "\n"


def summarise(args) -> str:
    lines = [f"# {args.title}", ""]
    for s in args.source or []:
        lines.append(f"{s.split('/')[-1]} sha256[:16] = {hashlib.sha256(open(s, 'rb').read()).hexdigest()[:16]}  ")
    lines += ["", "Commands (from the repository root), one counter pass each:", ""]
    lines += ["    " + c for c in args.command]
    lines.append("")
    rows = collections.OrderedDict()
    if args.mfma:
        for name, ds in _by_kernel(_dispatches(args.mfma)).items():
            if "SQ_VALU_MFMA_BUSY_CYCLES" not in ds[0]:
                continue
            dur = _mean(d["dur_ns"] for d in ds)
            cyc = _mean(d["GRBM_GUI_ACTIVE"] / XCC for d in ds)
            busy = _mean(d["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS for d in ds)
            r = rows.setdefault(name, {})
            r.update(calls=len(ds), dur_us=dur / 1e3, ghz=cyc / dur, mfma=busy / cyc if cyc else float("nan"))
    scales = {}
    for counter, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        if not path:
            continue
        disp = _dispatches(path)
        scales[counter] = _copy_scale(disp, counter)
        for name, ds in _by_kernel(disp).items():
            if counter not in ds[0] or "copyBuffer" in name:
                continue
            r = rows.setdefault(name, {})
            r.setdefault("calls", len(ds))
            r.setdefault("dur_us", _mean(d["dur_ns"] for d in ds) / 1e3)
            r[counter] = _mean(d[counter] for d in ds) * (scales[counter] or float("nan")) * 1024
    if scales:
        lines.append("Copy calibration (a plain 1 GiB device copy in the same run): " + ", ".join(
            f"{c} x {v:.3f}" if v else f"{c}: no copy found" for c, v in scales.items()))
        lines.append("")
    if args.trace:
        lines += ["Kernel trace (every dispatch of the run):", "",
                  "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
        with open(args.trace) as fh:
            for r in csv.DictReader(fh):
                lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                             f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                             f"{float(r['Percentage']):.2f} % |")
        lines.append("")
    if not rows:
        return "\n".join(lines) + "\n"
    lines.append("| kernel | calls | avg us | clock GHz | MFMA busy | HBM read GB | HBM write GB | HBM GB/s |")
    lines.append("|---|---|---|---|---|---|---|---|")
    for name, r in rows.items():
        rd, wr = r.get("FETCH_SIZE"), r.get("WRITE_SIZE")
        rate = (rd + wr) / (r["dur_us"] * 1e-6) / 1e9 if rd is not None and wr is not None else None
        f = lambda v, fmt: "" if v is None else fmt.format(v)   # noqa: E731
        lines.append(f"| `{short(name)}` | {r.get('calls', '')} | {r['dur_us']:.1f} | {f(r.get('ghz'), '{:.2f}')} "
                     f"| {f(r.get('mfma'), '{:.1%}')} | {f(rd and rd / 1e9, '{:.3f}')} | "
                     f"{f(wr and wr / 1e9, '{:.3f}')} | {f(rate, '{:.0f}')} |")
    if args.json:
        r = rows.get(args.json_kernel)
        if r is None:
            raise SystemExit(f"{args.json_kernel!r} not among the profiled kernels")
        src = args.source[0]
        json.dump({"source_sha256_16": hashlib.sha256(open(src, "rb").read()).hexdigest()[:16],
                   "kernel": args.json_kernel,
                   "hbm_bytes_per_launch": int(r["FETCH_SIZE"] + r["WRITE_SIZE"]) if "FETCH_SIZE" in r else None,
                   "mfma_busy": round(r["mfma"], 4) if "mfma" in r else None,
                   "clock_ghz": round(r["ghz"], 3) if "ghz" in r else None}, open(args.json, "w"), indent=1)
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", default=[], help="a command that made one of the CSV files")
    ap.add_argument("--source", action="append", help="source files whose hashes head the summary")
    ap.add_argument("--trace", help="kernel_stats CSV of a --kernel-trace --stats run")
    ap.add_argument("--mfma", help="CSV of SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    ap.add_argument("--fetch", help="CSV of FETCH_SIZE")
    ap.add_argument("--write", help="CSV of WRITE_SIZE")
    ap.add_argument("--json", help="write the named kernel's figures here")
    ap.add_argument("--json-kernel")
    ap.add_argument("--calibration", action="store_true",
                    help="per-dispatch table of counter_calibration.py's copies (--sizes: MiB per side, in order)")
    ap.add_argument("--sizes", default="256,1024,2048")
    ap.add_argument("--counters", help="one --pmc CSV: a per-kernel table of all its counters")
    ap.add_argument("--kernel-filter", action="append", help="with --counters: kernels whose name holds this")
    args = ap.parse_args(argv)
    if args.counters:
        sys.stdout.write(counters_table(args))
    else:
        sys.stdout.write(calibration(args) if args.calibration else summarise(args))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
