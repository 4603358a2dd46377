"""Turn rocprofv3 CSV output into the short text summaries kept with the
library (kernel durations, HBM traffic per launch, wave states).

    python -m lora_fine_tuning_mlp_amd.profiling stats  <kernel_stats.csv> <out.md> --cmd "<command>"
    python -m lora_fine_tuning_mlp_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> <copy bytes> <out.json> <out.md> --cmd "<fetch cmd>" --cmd "<write cmd>"
    python -m lora_fine_tuning_mlp_amd.profiling counters <counter_collection.csv> <out.md> --cmd "<command>" \
        [--bench-flops]
    python -m lora_fine_tuning_mlp_amd.profiling stalls <out.md> <SQ counter_collection.csv>... --cmd "<command>"...

Traffic: FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Both are
calibrated against the largest device copy kernel of the same run (a plain
copy of a known byte count), so bytes = counter * 1024 * (known / measured).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import re
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_fine_tuning_mlp_amd", "csrc")


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed (the
    sources hold no string literal with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the HIP sources' code (comments and layout ignored), so stored
    counter figures can be recognised as stale once a kernel has changed."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip")):
            h.update(_code_only(open(os.path.join(CSRC, f)).read()).encode())
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


# The library's per-launch recorder names a launch by the step it performs;
# where a step has more than one kernel variant, the variant's own name (as
# rocprofv3 reports it) maps to that step's name.
RECORDER_NAME = {"k_gateup_run": "k_gateup_fwd", "k_bwd_prologue8": "k_bwd_prologue", "k_mlp_dx_pp": "k_mlp_dx_bwd", "k_linear_run": "k_linear_fwd", "k_qkv_run": "k_qkv_fwd"}


def base_name(name: str) -> str:
    b = short_name(name).split("<")[0]
    return RECORDER_NAME.get(b, b)


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


def _trace_avg_us(stats_csv: str):
    """Average duration (us) per kernel from a kernel_stats.csv (with the
    recorder names of base_name)."""
    out = {}
    for r in csv.DictReader(open(stats_csv)):
        k = base_name(r["Name"])
        n, tot = int(r["Calls"]), float(r["TotalDurationNs"])
        pn, pt = out.get(k, (0, 0.0))
        out[k] = (pn + n, pt + tot)
    return {k: t / n / 1e3 for k, (n, t) in out.items() if n}


def traffic_summary(fetch_csv: str, write_csv: str, copy_bytes: int, out_json: str, out_md: str, cmds,
                    stats_csv=None, note=None) -> None:
    """Bytes per launch from FETCH_SIZE / WRITE_SIZE runs (out_json "-": no
    JSON); with stats_csv (a kernel trace of the same program) also the
    achieved rate of those bytes over the traced average duration."""
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
              f"WRITE_SIZE {max(wcopy):.0f} KiB; scale factors {f_scale:.4f} (fetch), {w_scale:.4f} (write).", ""]
    if note:
        lines += [note, ""]
    avg = _trace_avg_us(stats_csv) if stats_csv else {}
    if avg:
        lines += ["| kernel | dispatches | fetch MB | write MB | total MB | avg us (trace) | GB/s | of 8 TB/s |",
                  "|---|---:|---:|---:|---:|---:|---:|---:|"]
    else:
        lines += ["| kernel | dispatches | fetch MB | write MB | total MB |", "|---|---:|---:|---:|---:|"]
    for k in sorted(fv):
        if not k.startswith("k_"):
            continue
        fb = sum(fv[k]) / len(fv[k]) * 1024.0 * f_scale
        wb = (sum(wv[k]) / len(wv[k]) * 1024.0 * w_scale) if wv.get(k) else 0.0
        res[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb, "dispatches": len(fv[k]),
                  "source_hash": sh}
        row = f"| `{k}` | {len(fv[k])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |"
        if avg:
            us = avg.get(k)
            row += (f" {us:.1f} | {(fb + wb) / (us * 1e-6) / 1e9:.0f} | {(fb + wb) / (us * 1e-6) / 8e12:.2f} |"
                    if us else " | | |")
        lines.append(row)
    lines += ["", f"HIP sources hash: `{sh}`"]
    if out_json != "-":
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


# Wave-state counters (SQ block), read as fractions of the wave-resident
# time SQ_WAVE_CYCLES (all in quad-cycles, summed over the chip).
STALL_RATIOS = [
    ("issue", "SQ_ACTIVE_INST_ANY"),       # issuing an instruction
    ("wait_issue", "SQ_WAIT_INST_ANY"),    # next instruction ready, waiting for its issue slot
    ("wait_any", "SQ_WAIT_ANY"),           # waiting on anything else: s_waitcnt, barrier
    ("wait_lds", "SQ_WAIT_INST_LDS"),      # waiting to issue an LDS instruction
    ("valu", "SQ_ACTIVE_INST_VALU"),       # issue split by instruction type (VALU includes MFMA)
    ("vmem", "SQ_ACTIVE_INST_VMEM"),
    ("flat", "SQ_ACTIVE_INST_FLAT"),
    ("lds", "SQ_ACTIVE_INST_LDS"),
    ("salu", "SQ_ACTIVE_INST_SCA"),
    ("misc", "SQ_ACTIVE_INST_MISC"),
]


def stalls_summary(paths, out: str, cmds) -> None:
    """Per-kernel wave-state breakdown from raw SQ counters collected over one
    or more rocprofv3 --pmc runs of the same program (each run's counters
    averaged over its dispatches)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    clk = collections.defaultdict(list)
    for p in paths:
        for r in csv.DictReader(open(p)):
            k = base_name(r["Kernel_Name"])
            if k.startswith("k_"):
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                    if ns > 0:
                        clk[k].append(float(r["Counter_Value"]) / 8 / ns)

    def avg(k, c):
        v = vals[k].get(c)
        return sum(v) / len(v) if v else None

    cols = [n for n, _ in STALL_RATIOS]
    lines = ["# Wave-state breakdown per kernel (rocprofv3 SQ counters)", "", "Commands:", ""]
    for c in cmds:
        lines += ["```", c, "```", ""]
    lines += ["Each state column is a counter divided by SQ_WAVE_CYCLES (the time waves are resident), "
              "so it reads as the share of a wave's lifetime in that state: `issue` (SQ_ACTIVE_INST_ANY), "
              "`wait_issue` (SQ_WAIT_INST_ANY: next instruction ready, waiting for an issue slot, e.g. the "
              "MFMA pipe the SIMD's other wave holds), `wait_any` (SQ_WAIT_ANY: s_waitcnt, barrier); the three "
              "add up to about 1. `wait_lds` is SQ_WAIT_INST_LDS; `valu` ... `misc` split `issue` by "
              "instruction type. GRBM_GUI_ACTIVE is summed over the 8 XCDs (it reads 8 x the kernel's "
              "cycles), so `mfma_busy` = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), "
              "the MFMA pipes' busy share at the clock the kernel ran (`clock`, from the duration of the "
              "same dispatches), and `waves/CU` = 4 SQ_WAVE_CYCLES / (256 CUs x GRBM_GUI_ACTIVE / 8). "
              "`lds_conflict` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. The clock is only meaningful "
              "for kernels that run for hundreds of microseconds (GRBM_GUI_ACTIVE also counts the dispatch "
              "around a short kernel). Empty cells: counter not collected.", "",
              "| kernel | dispatches | clock GHz | waves/CU | " + " | ".join(cols) + " | mfma_busy | lds_conflict |",
              "|---|---:|---:|---:|" + "---:|" * len(cols) + "---:|---:|"]
    for k in sorted(vals):
        wc = avg(k, "SQ_WAVE_CYCLES")
        if not wc:
            continue
        n = min(len(v) for v in vals[k].values())
        row = []
        for _, c in STALL_RATIOS:
            v = avg(k, c)
            row.append(f"{v / wc:.3f}" if v is not None else "")
        gui = avg(k, "GRBM_GUI_ACTIVE")
        mb = avg(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        busy = f"{mb / (1024 * gui / 8):.3f}" if (gui and mb is not None) else ""
        occ = f"{4 * wc / (256 * gui / 8):.2f}" if gui else ""
        la, lc = avg(k, "SQ_LDS_IDX_ACTIVE"), avg(k, "SQ_LDS_BANK_CONFLICT")
        conf = f"{lc / la:.3f}" if (la and lc is not None) else ""
        ghz = f"{sum(clk[k]) / len(clk[k]):.2f}" if clk[k] else ""
        lines.append(f"| `{k}` | {n} | {ghz} | {occ} | " + " | ".join(row) + f" | {busy} | {conf} |")
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
    t.add_argument("--stats", default=None, help="kernel_stats.csv of a trace of the same program (adds GB/s)")
    t.add_argument("--note", default=None)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--bench-flops", action="store_true",
                   help="divide MfmaFlopsBF16 by the headline step's algorithmic FLOPs per launch")
    w = sub.add_parser("stalls")
    w.add_argument("out")
    w.add_argument("csv", nargs="+")
    w.add_argument("--cmd", action="append", default=[])
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
    elif a.what == "stalls":
        stalls_summary(a.csv, a.out, a.cmd)
    else:
        traffic_summary(a.fetch_csv, a.write_csv, a.copy_bytes, a.out_json, a.out_md, a.cmd, a.stats, a.note)


if __name__ == "__main__":
    main()
