"""Turn rocprofv3 CSV output into the short text summaries kept with the
library (kernel durations, HBM traffic per launch).

    python -m lora_fine_tuning_mlp_amd.profiling stats  <kernel_stats.csv> <out.md> --cmd "<command>"
    python -m lora_fine_tuning_mlp_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> <copy bytes> <out.json> <out.md> --cmd "<fetch cmd>" --cmd "<write cmd>"
    python -m lora_fine_tuning_mlp_amd.profiling counters <counter_collection.csv> <out.md> --cmd "<command>" \
        [--bench-flops]

Traffic: FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Both are
calibrated against the largest device copy kernel of the same run (a plain
copy of a known byte count), so bytes = counter * 1024 * (known / measured).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_fine_tuning_mlp_amd", "csrc")


def source_hash() -> str:
    """Hash of the HIP sources, so stored counter figures can be recognised as
    stale once a kernel has changed."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip")):
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _unmangle_nested(n: str) -> str:
    """Outer qualified name of an Itanium-mangled function (_ZN4lora12k_fooI...)."""
    i, parts = 3, []
    while i < len(n) and n[i].isdigit():
        j = i
        while n[j].isdigit():
            j += 1
        ln = int(n[i:j])
        parts.append(n[j:j + ln])
        i = j + ln
    return "::".join(parts) if parts else n


def short_name(name: str) -> str:
    n = name.strip('"')
    if n.startswith("_ZN"):
        n = _unmangle_nested(n)
    n = n.split("(")[0]
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("lora::", "")
    return n


def base_name(name: str) -> str:
    return short_name(name).split("<")[0]


def stats_summary(path: str, out: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(path)))
    lines = ["# rocprofv3 kernel-trace summary", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{base_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    lines.append("")
    lines.append(f"HIP sources hash: `{source_hash()}`")
    open(out, "w").write("\n".join(lines) + "\n")


def _per_kernel(path: str, counter: str):
    vals = collections.defaultdict(list)
    copies = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        name = r["Kernel_Name"]
        if "copyBuffer" in name or "copy_kernel" in name:
            copies.append(v)
        vals[base_name(name)].append(v)
    return vals, copies


def traffic_summary(fetch_csv: str, write_csv: str, copy_bytes: int, out_json: str, out_md: str, cmds) -> None:
    fv, fcopy = _per_kernel(fetch_csv, "FETCH_SIZE")
    wv, wcopy = _per_kernel(write_csv, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("no copy kernel in the counter runs: cannot calibrate")
    f_scale = copy_bytes / (max(fcopy) * 1024.0)
    w_scale = copy_bytes / (max(wcopy) * 1024.0)
    sh = source_hash()
    res = {"_calibration": {"copy_bytes": copy_bytes, "fetch_kib": max(fcopy), "write_kib": max(wcopy),
                            "fetch_scale": f_scale, "write_scale": w_scale, "source_hash": sh}}
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "", "Commands:", ""]
    for c in cmds:
        lines += ["```", c, "```", ""]
    lines += [f"Calibration: a device copy of {copy_bytes} bytes reads FETCH_SIZE {max(fcopy):.0f} KiB and "
              f"WRITE_SIZE {max(wcopy):.0f} KiB; scale factors {f_scale:.4f} (fetch), {w_scale:.4f} (write).", "",
              "| kernel | dispatches | fetch MB | write MB | total MB |", "|---|---:|---:|---:|---:|"]
    for k in sorted(fv):
        if not k.startswith("k_"):
            continue
        fb = sum(fv[k]) / len(fv[k]) * 1024.0 * f_scale
        wb = (sum(wv[k]) / len(wv[k]) * 1024.0 * w_scale) if wv.get(k) else 0.0
        res[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb, "dispatches": len(fv[k]),
                  "source_hash": sh}
        lines.append(f"| `{k}` | {len(fv[k])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |")
    lines += ["", f"HIP sources hash: `{sh}`"]
    json.dump(res, open(out_json, "w"), indent=1)
    open(out_md, "w").write("\n".join(lines) + "\n")


def counters_summary(path: str, out: str, cmd: str, kflops=None) -> None:
    """Per-kernel averages of rocprofv3 derived metrics (MfmaUtil, LdsUtil,
    LDSBankConflict, MfmaFlopsBF16, ...) from one counter-collection run.
    With `kflops` (kernel -> algorithmic FLOPs per launch) the table also
    gives executed MFMA FLOPs over algorithmic FLOPs."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = base_name(r["Kernel_Name"])
        if not k.startswith("k_"):
            continue
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in vals for c in vals[k]})
    lines = ["# rocprofv3 derived counters per kernel (average over dispatches)", "", "Command:", "", "```", cmd, "```",
             "", "| kernel | dispatches | " + " | ".join(names) + (" | MFMA FLOPs / algorithmic |" if kflops else " |"),
             "|---|---:|" + "---:|" * len(names) + ("---:|" if kflops else "")]
    for k in sorted(vals):
        n = max(len(v) for v in vals[k].values())
        row = [f"{sum(vals[k][c]) / len(vals[k][c]):.4g}" if vals[k].get(c) else "" for c in names]
        extra = ""
        if kflops:
            mf = vals[k].get("MfmaFlopsBF16")
            extra = f" {sum(mf) / len(mf) / kflops[k]:.3f} |" if (mf and k in kflops) else " |"
        lines.append(f"| `{k}` | {n} | " + " | ".join(row) + " |" + extra)
    lines += ["", f"HIP sources hash: `{source_hash()}`"]
    open(out, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("copy_bytes", type=int)
    t.add_argument("out_json")
    t.add_argument("out_md")
    t.add_argument("--cmd", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--bench-flops", action="store_true",
                   help="divide MfmaFlopsBF16 by the headline step's algorithmic FLOPs per launch")
    a = ap.parse_args()
    if a.what == "stats":
        stats_summary(a.csv, a.out, a.cmd)
    elif a.what == "counters":
        kf = None
        if a.bench_flops:
            import sys
            sys.path.insert(0, ROOT)
            import bench
            from lora_fine_tuning_mlp_amd import synthetic as S
            kf = bench.kernel_flops(S.C1, S.C2)
        counters_summary(a.csv, a.out, a.cmd, kf)
    else:
        traffic_summary(a.fetch_csv, a.write_csv, a.copy_bytes, a.out_json, a.out_md, a.cmd)


if __name__ == "__main__":
    main()
