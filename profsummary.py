"""Summaries of rocprofv3 output for the committed profiles.

    python profsummary.py trace <kernel_stats.csv> <out.md> "<command>"
    python profsummary.py traffic <fetch_counter.csv> <write_counter.csv> \\
        <traffic.json> <workload> <path> <steps>

`trace` condenses a --kernel-trace --stats run into a markdown table grouped by
kernel class.  `counters` condenses --pmc runs (with --kernel-trace) into a
per-class table of clock, MFMA-busy fraction, achieved MFMA rate and LDS
figures:

    python profsummary.py counters <out.md> "<title>" <counter_collection.csv> ["<command>"] ...
  `traffic` takes the FETCH_SIZE and WRITE_SIZE passes (KiB per
dispatch), scales them by what the same counters read for the plain 1 GiB
copy that bench.py --copy-calibration runs, and records HBM bytes per launch
for every kernel class in traffic.json under (workload, path), tagged with the
hash of the kernel sources (other entries of the file are kept).
"""
from __future__ import annotations

import collections
import csv
import json
import sys

CLASSES = (("fwd_lse", "fwd_lse"), ("bwd_grad", "bwd_grad"), ("gemm_store", "gemm_dhdw"),
           ("gpass", "g_pass"), ("transpose", "transpose"), ("teacher_prep", "teacher_prep"),
           ("fwd_finalize", "fwd_finalize"), ("loss_reduce", "fwd_finalize"))


def kernel_class(name: str) -> str:
    for key, cls in CLASSES:
        if key in name:
            return cls
    if "ckl" in name:
        return "other"
    if "copyBuffer" in name:  # the runtime's device-to-device copy (bench.py --copy-calibration)
        return "copy"
    return "foreign"


def trace(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    agg = collections.OrderedDict()
    for r in rows:
        cls = kernel_class(r["Name"])
        a = agg.setdefault(cls, [0, 0.0])
        a[0] += int(r["Calls"])
        a[1] += float(r["TotalDurationNs"])
    tot = sum(v[1] for k, v in agg.items() if k != "foreign")
    with open(out_md, "w") as f:
        f.write(f"# rocprofv3 kernel trace: {command}\n\n")
        f.write("| kernel class | launches | total ms | avg ms / launch | share |\n|---|---|---|---|---|\n")
        for cls, (n, ns) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            if cls == "foreign":
                continue
            f.write(f"| {cls} | {n} | {ns / 1e6:.3f} | {ns / n / 1e6:.4f} | {100 * ns / tot:.1f}% |\n")
        f.write("\nPer kernel symbol:\n\n| kernel | calls | avg ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                    f"{float(r['MaxNs']):.0f} |\n")


def _per_dispatch(csv_path: str, counter: str):
    out = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            out.append((kernel_class(r["Kernel_Name"]), float(r["Counter_Value"]) * 1024.0))
    return out


def traffic(fetch_csv: str, write_csv: str, out_json: str, workload: str, path: str, steps: int) -> None:
    from bench import kernel_source_hash
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_f = [b for c, b in fetch if c == "copy"]
    copy_w = [b for c, b in write if c == "copy"]
    if not copy_f or not copy_w:
        raise SystemExit("no copy-calibration dispatch found (run bench.py --copy-calibration)")
    gib = float(1 << 30)
    fscale = gib / max(copy_f)  # counter bytes per true byte, from the 1 GiB copy
    wscale = gib / max(copy_w)
    res = {}
    for name, data, scale in (("read", fetch, fscale), ("write", write, wscale)):
        by = collections.defaultdict(list)
        for c, b in data:
            if c not in ("copy", "foreign"):
                by[c].append(b * scale)
        for c, v in by.items():
            d = res.setdefault(c, {})
            d[f"hbm_{name}_bytes_per_launch"] = sum(v) / len(v)
            d["launches"] = len(v)
    for c, d in res.items():
        d["hbm_bytes_per_launch"] = d.get("hbm_read_bytes_per_launch", 0.0) + d.get("hbm_write_bytes_per_launch", 0.0)
    try:
        doc = json.load(open(out_json))
    except (OSError, ValueError):
        doc = {}
    entries = [e for e in doc.get("entries", []) if (e.get("workload"), e.get("path")) != (workload, path)]
    entries.append({"workload": workload, "path": path, "source_hash": kernel_source_hash(), "steps_profiled": steps,
                    "copy_scale": {"FETCH_SIZE": 1.0 / fscale, "WRITE_SIZE": 1.0 / wscale}, "kernels": res})
    json.dump({"entries": entries}, open(out_json, "w"), indent=1)


def _per_class(csv_path: str):
    """{class: {counter: sum over dispatches, 'dur': seconds, 'n': dispatches}}."""
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(csv_path)):
        d = per[int(r["Dispatch_Id"])]
        d["cls"] = kernel_class(r["Kernel_Name"])
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = collections.OrderedDict()
    for d in per.values():
        if d["cls"] in ("foreign", "copy"):
            continue
        a = agg.setdefault(d["cls"], collections.defaultdict(float))
        a["n"] += 1
        for k, v in d.items():
            if k != "cls":
                a[k] += v
    return agg


# gfx950 reports GRBM_GUI_ACTIVE summed over its 8 XCDs; 256 CUs, 1024 SIMDs
_XCD, _CU, _SIMD = 8, 256, 1024


def counters(out_md: str, title: str, pairs) -> None:
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("Clock = GRBM_GUI_ACTIVE per XCD / kernel duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                "(cycles x 1024 SIMDs); MFMA rate = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flop / duration; "
                "LDS read = SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 B / (cycles x 256 CUs); waits as a fraction of "
                "SQ_WAVE_CYCLES.  Averages over the profiled launches.\n\n")
        for csv_path, command in pairs:
            agg = _per_class(csv_path)
            f.write(f"## `{command}`\n\n")
            f.write("| kernel class | launches | avg ms | clock GHz | MFMA busy | MFMA TFLOP/s | LDS read B/clk/CU | "
                    "wait any | wait LDS |\n|---|---|---|---|---|---|---|---|---|\n")
            for cls, a in agg.items():
                g = a.get("GRBM_GUI_ACTIVE", 0.0) / _XCD
                dur = a["dur"]
                def pct(key, denom):
                    return f"{100.0 * a[key] / denom:.1f}%" if key in a and denom > 0 else "-"
                clk = f"{g / dur / 1e9:.2f}" if g else "-"
                mfma = pct("SQ_VALU_MFMA_BUSY_CYCLES", g * _SIMD)
                rate = (f"{a['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / dur / 1e12:.0f}"
                        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in a else "-")
                lds = (f"{a['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / (g * _CU):.1f}"
                       if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in a and g else "-")
                wa = pct("SQ_WAIT_ANY", a.get("SQ_WAVE_CYCLES", 0.0))
                wl = pct("SQ_WAIT_INST_LDS", a.get("SQ_WAVE_CYCLES", 0.0))
                f.write(f"| {cls} | {int(a['n'])} | {dur * 1e3 / a['n']:.3f} | {clk} | {mfma} | {rate} | {lds} | "
                        f"{wa} | {wl} |\n")
            f.write("\n")


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "counters":
        rest = sys.argv[4:]
        counters(sys.argv[2], sys.argv[3], [(rest[i], rest[i + 1]) for i in range(0, len(rest), 2)])
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], int(sys.argv[7]))
    else:
        raise SystemExit(__doc__)
