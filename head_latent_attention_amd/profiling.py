"""Summaries of rocprofv3 CSV output: per-kernel time statistics and HBM traffic per
launch of an entry point (FETCH_SIZE / WRITE_SIZE counters scaled by a plain copy of
known size).

Usage:
  python -m head_latent_attention_amd.profiling stats RUN_kernel_stats.csv
  python -m head_latent_attention_amd.profiling summary RUN_kernel_stats.csv "TITLE" "COMMAND" > OUT.md
  python -m head_latent_attention_amd.profiling traffic FETCH_DIR WRITE_DIR CALIB_FETCH_DIR CALIB_WRITE_DIR OUT.json
  python -m head_latent_attention_amd.profiling counters "TITLE" "COMMANDS" DIR [DIR ...] > OUT.md
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

# kernels launched once by each mla_decode_attn_absorbed call (MFMA path; the fold launch also plans)
DECODE_ATTN_KERNELS = ("fold_kernel", "decode_attn_kernel", "combine_kernel")
COPY_BYTES = 1 << 30


def kernel_stats(path: str):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    return out


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def per_kernel_counter(d: str, counter: str):
    """{kernel short name: mean counter value per dispatch}"""
    acc = {}
    for r in _counter_rows(d):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _largest(d: str, counter: str) -> float:
    vals = per_kernel_counter(d, counter)
    return max(vals.values())


# files holding the device code of the decode-attention kernels the counters measure
DECODE_ATTN_SOURCES = ("mla_decode_fast.hip", "mla_device.h")


def source_hash(csrc: str, files=DECODE_ATTN_SOURCES) -> str:
    """Short sha256 of the given kernel source files: a stored traffic figure is valid only
    while it matches the sources."""
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic(fetch_dir, write_dir, calib_fetch_dir, calib_write_dir, out_json, kernels=DECODE_ATTN_KERNELS):
    # the copy reads and writes COPY_BYTES once; its counters give KiB -> bytes factors
    f_copy = _largest(calib_fetch_dir, "FETCH_SIZE") * 1024.0
    w_copy = _largest(calib_write_dir, "WRITE_SIZE") * 1024.0
    f_factor, w_factor = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    fetch = per_kernel_counter(fetch_dir, "FETCH_SIZE")
    write = per_kernel_counter(write_dir, "WRITE_SIZE")
    parts = {}
    total = 0.0
    for short in kernels:
        fk = [v for k, v in fetch.items() if short in k]
        wk = [v for k, v in write.items() if short in k]
        if not fk or not wk:
            raise KeyError(f"kernel {short} missing from the counter runs")
        b = fk[0] * 1024.0 * f_factor + wk[0] * 1024.0 * w_factor
        parts[short] = {"fetch_bytes": fk[0] * 1024.0 * f_factor, "write_bytes": wk[0] * 1024.0 * w_factor}
        total += b
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    rec = {"kernel_src_sha": source_hash(csrc), "bytes_per_launch": total, "kernels": parts,
           "copy_calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": f_factor, "write_factor": w_factor}}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def summary_md(stats_csv: str, title: str, command: str) -> str:
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```",
             "cd /tmp && export TMPDIR=/tmp", command, "```", "",
             "| kernel | calls | average (us) | share of GPU time |", "|---|---:|---:|---:|"]
    for name, calls, avg_us, pct in kernel_stats(stats_csv):
        short = name.replace("(anonymous namespace)::", "").split("(")[0]
        short = short[5:] if short.startswith("void ") else short
        short = short if len(short) <= 80 else short[:77] + "..."
        lines.append(f"| `{short}` | {calls} | {avg_us:.1f} | {pct:.2f}% |")
    trace = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace("kernel_stats", "kernel_trace"))
    if os.path.exists(trace):
        lines += ["", "Library kernels by launch grid (one row per distinct launch shape, from the kernel trace):", "",
                  "| kernel | grid (x, y, z) | launches | average (us) |", "|---|---|---:|---:|"]
        for (name, grid), durs in by_grid(trace):
            lines.append(f"| `{name}` | {grid} | {len(durs)} | {sum(durs) / len(durs):.1f} |")
    lines.append("")
    return "\n".join(lines)


def by_grid(trace_csv: str):
    """Durations (us) of the library's kernels grouped by (name, launch grid), in launch order."""
    groups = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "mla::" not in name:
                continue
            short = name.replace("(anonymous namespace)::", "").split("(")[0]
            short = short[5:] if short.startswith("void ") else short
            grid = f"{r['Grid_Size_X']}, {r['Grid_Size_Y']}, {r['Grid_Size_Z']}"
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            groups.setdefault((short, grid), []).append(dur)
    return list(groups.items())


MOPS_FLOP = 512   # flop per unit of the SQ_INSTS_VALU_MFMA_MOPS_* counters (checked against the probe loop)


def _short(name: str) -> str:
    short = name.replace("(anonymous namespace)::", "").split("(")[0]
    return short[5:] if short.startswith("void ") else short


def counter_table(dirs):
    """{(kernel, grid threads): {"n": dispatches, "us": mean duration, counter: mean per dispatch}}
    over the counter_collection CSVs of several rocprofv3 --pmc runs."""
    acc = {}
    for d in dirs:
        for r in _counter_rows(d):
            if "mla::" not in r["Kernel_Name"] and "peak_" not in r["Kernel_Name"]:
                continue   # torch's own kernels (input set-up, fills)
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            e = acc.setdefault(key, {})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            e.setdefault("_dur", {})[(d, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for key, e in acc.items():
        durs = list(e.pop("_dur").values())
        row = {"n": len(durs), "us": sum(durs) / len(durs)}
        for c, v in e.items():
            row[c] = sum(v) / len(v)
        out[key] = row
    return out


def counters_md(dirs, title: str, commands: str) -> str:
    tab = counter_table(dirs)
    names = sorted({c for r in tab.values() for c in r if c not in ("n", "us")})
    lines = [f"# {title}", "", "Commands (run from the repository root on one MI355X, one counter pass each):", "",
             "```", "cd /tmp && export TMPDIR=/tmp", commands, "```", "",
             "Mean per dispatch; `us` is the dispatch duration under counter collection.", ""]
    probe = [r for (k, g), r in tab.items() if "peak_mfma" in k and "SQ_VALU_MFMA_BUSY_CYCLES" in r]
    probe_rate = None
    if probe and "SQ_INSTS_VALU_MFMA_MOPS_BF16" in probe[0]:
        p = max(probe, key=lambda r: r["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / r["us"])
        probe_rate = (p["SQ_VALU_MFMA_BUSY_CYCLES"] / p["us"], MOPS_FLOP * p["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / p["us"] / 1e6)
        lines += [f"Matrix-op loop probe (no memory traffic): {probe_rate[1]:.0f} TFLOP/s bf16 from "
                  f"{MOPS_FLOP} flop per MOPS unit; its `SQ_VALU_MFMA_BUSY_CYCLES` per us is the 'busy' reference "
                  "below (busy = a kernel's busy cycles per us over the probe's).", ""]
    derived = []
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in names or "SQ_INSTS_VALU_MFMA_MOPS_F8" in names:
        derived.append("MFMA TFLOP/s (hw)")
    if probe_rate and "SQ_VALU_MFMA_BUSY_CYCLES" in names:
        derived.append("MFMA busy vs probe")
    head = ["kernel", "grid threads", "dispatches", "us"] + derived + names
    lines += ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for (k, g), r in sorted(tab.items(), key=lambda kv: -kv[1]["us"] * kv[1]["n"]):
        cells = [f"`{k if len(k) <= 60 else k[:57] + '...'}`", str(g), str(r["n"]), f"{r['us']:.1f}"]
        if "MFMA TFLOP/s (hw)" in derived:
            mops = r.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + r.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
            cells.append(f"{MOPS_FLOP * mops / r['us'] / 1e6:.0f}" if mops else "")
        if "MFMA busy vs probe" in derived:
            b = r.get("SQ_VALU_MFMA_BUSY_CYCLES")
            cells.append(f"{b / r['us'] / probe_rate[0]:.2f}" if b is not None else "")
        for c in names:
            v = r.get(c)
            cells.append("" if v is None else (f"{v:.0f}" if abs(v) >= 100 else f"{v:.3g}"))
        lines.append("| " + " | ".join(cells) + " |")
    lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "summary":
        print(summary_md(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "stats":
        for name, calls, avg_us, pct in kernel_stats(sys.argv[2]):
            print(f"{avg_us:10.1f} us  {calls:6d}  {pct:6.2f}%  {name[:110]}")
    elif sys.argv[1] == "counters":
        print(counters_md(sys.argv[4:], sys.argv[2], sys.argv[3]))
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:7]), indent=1))
