"""Summaries of rocprofv3 CSV output for the benchmark (measurement tooling).

Usage (after the rocprofv3 runs whose commands are recorded in the output):
  python -m online_softmax_fa2_amd.rocprof_summary trace  <kernel_stats.csv> <out.txt> "<command>"
  python -m online_softmax_fa2_amd.rocprof_summary traffic <fetch_counters.csv> <write_counters.csv>
         <copy_fetch_counters.csv> <copy_write_counters.csv> <out.txt> <traffic.json> "<commands>"
  python -m online_softmax_fa2_amd.rocprof_summary sq <sq_counters.csv> <out.txt> "<command>"

The traffic summary scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by the
ratio between the bytes a plain 1 GiB device copy moves and what the same
counter reports for it, and records, per kernel, the resulting HBM bytes per
launch together with a SHA-256 of the kernel sources, so that the benchmark
reports the figure only while the kernel is unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30  # the calibration copy moves 1 GiB each way

# Kernel-name pattern -> the sources that define it (for the staleness hash).
KERNEL_SOURCES = {
    "fwd_bf16_d128_kernel": ["csrc/attn_fwd.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h",
                             "csrc/tile_layout.h"],
    "fwd_bf16_kernel": ["csrc/attn_fwd.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h"],
    "fwd_f32_kernel": ["csrc/attn_fwd.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h"],
    "fwd_f32_split_kernel": ["csrc/attn_fwd.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h"],
    "fwd_f32_split16_kernel": ["csrc/attn_fwd.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h"],
    "fwd_fp8_d128_kernel": ["csrc/attn_fwd_fp8.hip", "csrc/fwd_common.h", "csrc/masks.h", "csrc/device_common.h",
                            "csrc/tile_layout.h"],
    "decode_partial_kernel": ["csrc/decode.hip", "csrc/device_common.h"],
    "decode_merge_kernel": ["csrc/decode.hip", "csrc/device_common.h"],
    "softmax_rows_reg_kernel": ["csrc/softmax.hip", "csrc/device_common.h"],
    "softmax_rows_wave_kernel": ["csrc/softmax.hip", "csrc/device_common.h"],
    "softmax_rows_stream_kernel": ["csrc/softmax.hip", "csrc/device_common.h"],
    "softmax_topk_kernel": ["csrc/softmax.hip", "csrc/device_common.h"],
    "bwd_dq_kernel": ["csrc/attn_bwd.hip", "csrc/masks.h", "csrc/device_common.h", "csrc/tile_layout.h"],
    "bwd_dkdv_kernel": ["csrc/attn_bwd.hip", "csrc/masks.h", "csrc/device_common.h", "csrc/tile_layout.h"],
    "bwd_prep_kernel": ["csrc/attn_bwd.hip", "csrc/masks.h", "csrc/device_common.h", "csrc/tile_layout.h"],
    "bwd_dqs_kernel": ["csrc/attn_bwd.hip", "csrc/masks.h", "csrc/device_common.h", "csrc/tile_layout.h",
                       "csrc/launch.h"],
}


def short_name(name: str) -> str:
    m = re.search(r"decode_partial_kernelI(DF16b|f)Li(\d+)E", name)
    if m:
        return f"decode_partial_kernel<{'bf16' if m.group(1) == 'DF16b' else 'f32'}, {m.group(2)}>"
    m = re.search(r"(fwd_bf16_d128_kernel<[^>]*>|fwd_bf16_kernel<\d+>|fwd_f32_kernel<\d+>|fwd_f32_split_kernel<[^>]*>|fwd_f32_split16_kernel<[^>]*>|"
                  r"decode_partial_kernel\w*|decode_merge_kernel<\d+>|softmax_topk_kernel<\d, (?:true|false)>|"
                  r"softmax_rows_\w+<[\d, ]+>|bwd_dkdv_kernel(?:<\w+>)?|bwd_dq_kernel|bwd_dqs_kernel|bwd_prep_kernel|fwd_fp8_d128_kernel|"
                  r"__amd_rocclr_copyBuffer|copyBuffer)", name)
    if m:
        return m.group(1)
    return name.split("(")[0][-60:]


def family(short: str) -> str | None:
    for k in KERNEL_SOURCES:
        if short.startswith(k):
            return k
    return None


def source_sha(fam: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[fam]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def dispatch_keys(rows, name_col: str, grid_col: str) -> list[str]:
    """One key per row: the kernel's short name, followed by " [grid G]" (G = work-items of the launch) for a
    kernel launched with more than one grid size, so that launches on different workloads stay apart."""
    shorts = [short_name(r[name_col]) for r in rows]
    grids = defaultdict(set)
    for sname, r in zip(shorts, rows):
        grids[sname].add(r[grid_col])
    return [f"{sname} [grid {r[grid_col]}]" if len(grids[sname]) > 1 else sname for sname, r in zip(shorts, rows)]


def per_kernel_counter(path: str) -> dict[str, dict[str, float]]:
    rows = list(csv.DictReader(open(path)))
    acc: dict[str, dict[str, list[float]]] = defaultdict(lambda: defaultdict(list))
    for key, r in zip(dispatch_keys(rows, "Kernel_Name", "Grid_Size"), rows):
        acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def per_kernel_duration_ns(path: str) -> dict[str, float]:
    """Mean dispatch duration (ns) per kernel from the counter CSV's timestamps."""
    rows = list(csv.DictReader(open(path)))
    acc: dict[str, dict[str, float]] = defaultdict(dict)
    for key, r in zip(dispatch_keys(rows, "Kernel_Name", "Grid_Size"), rows):
        acc[key][r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items() if v}


def copy_factor(path: str, counter: str) -> float:
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no copy-kernel {counter} values in {path}")
    kib = max(vals)  # the three 1 GiB copies; small host<->device copies read less
    return COPY_BYTES / (kib * 1024.0)


def trace(trace_csv: str, out_txt: str, command: str) -> None:
    """Per-kernel dispatch statistics from the per-dispatch kernel trace (…_kernel_trace.csv)."""
    rows = list(csv.DictReader(open(trace_csv)))
    durs: dict[str, list[float]] = defaultdict(list)
    for key, r in zip(dispatch_keys(rows, "Kernel_Name", "Grid_Size_X"), rows):
        durs[key].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    total = sum(sum(v) for v in durs.values()) or 1.0
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {command}",
             "# (a kernel launched with more than one grid size has one row per grid: G = work-items)", "",
             f"{'kernel':56s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for key, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{key:56s} {len(v):6d} {sum(v) / len(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} {max(v) / 1e3:10.2f} "
                     f"{100 * sum(v) / total:6.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_txt, out_json, commands) -> None:
    fk = per_kernel_counter(fetch_csv)
    wk = per_kernel_counter(write_csv)
    ff = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    wf = copy_factor(copy_write_csv, "WRITE_SIZE")
    lines = ["# HBM traffic per launch from rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE in KiB per dispatch)",
             f"# commands: {commands}",
             f"# calibration: a 1 GiB device copy reads FETCH_SIZE x {ff:.4f} and writes WRITE_SIZE x {wf:.4f} bytes",
             "", f"{'kernel':56s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'read_MB':>10s} {'write_MB':>10s} {'total_MB':>10s}"]
    table = {}
    for k in sorted(set(fk) | set(wk)):
        fam = family(k)
        if fam is None:
            continue
        f_kib = fk.get(k, {}).get("FETCH_SIZE", float("nan"))
        w_kib = wk.get(k, {}).get("WRITE_SIZE", float("nan"))
        rb, wb = f_kib * 1024 * ff, w_kib * 1024 * wf
        lines.append(f"{k:56s} {f_kib:12.1f} {w_kib:12.1f} {rb / 1e6:10.1f} {wb / 1e6:10.1f} {(rb + wb) / 1e6:10.1f}")
        table[k] = {"fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": ff, "write_scale": wf,
                    "read_bytes": rb, "write_bytes": wb, "bytes": rb + wb, "source_sha256": source_sha(fam)}
    open(out_txt, "w").write("\n".join(lines) + "\n")
    json.dump(table, open(out_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def sq(counters_csv: str, out_txt: str, command: str, out_json: str | None = None, n_xcd: int = 8,
       n_simd: int = 1024) -> None:
    """MFMA and stall evidence per kernel from SQ counters.

    SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512-FLOP units of bf16 MFMA work;
    SQ_VALU_MFMA_BUSY_CYCLES sums, over all SIMDs, the cycles the matrix
    pipe was busy; GRBM_GUI_ACTIVE sums the active GPU cycles over the XCDs.
    SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_LDS and SQ_ACTIVE_INST_VALU are
    wave-cycle totals (same unit), so their ratios are fractions of wave time.
    clock_GHz is the active cycles of one XCD over the dispatch duration: the
    shader clock the kernel actually ran at (mfma_busy% is relative to it).
    """
    k = per_kernel_counter(counters_csv)
    dur = per_kernel_duration_ns(counters_csv)
    lines = ["# rocprofv3 SQ counters per kernel (averages per dispatch)", f"# command: {command}",
             "# clock_GHz = GRBM_GUI_ACTIVE / 8 XCDs / dispatch time; dispatches shorter than ~50 us overstate it",
             "# (the counters' window is longer than the dispatch)", "",
             f"{'kernel':56s} {'mfma_TFLOP':>10s} {'mfma_busy%':>10s} {'wait_any%':>9s} {'wait_lds%':>9s} "
             f"{'valu%':>6s} {'lds_bank_conf':>14s} {'clock_GHz':>9s}"]
    table = {}
    for name, c in sorted(k.items()):
        if family(name) is None:
            continue
        flop = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        active = c.get("GRBM_GUI_ACTIVE", 0.0) / n_xcd
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (active * n_simd) if active else 0.0
        wc = c.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        lines.append(f"{name[:56]:56s} {flop / 1e12:10.4f} {100 * busy:10.1f} {100 * c.get('SQ_WAIT_ANY', 0) / wc:9.1f} "
                     f"{100 * c.get('SQ_WAIT_INST_LDS', 0) / wc:9.1f} {100 * c.get('SQ_ACTIVE_INST_VALU', 0) / wc:6.1f} "
                     f"{c.get('SQ_LDS_BANK_CONFLICT', 0):14.0f} {active / dur.get(name, float('inf')):9.2f}")
        table[name] = {"clock_ghz": active / dur.get(name, float("inf")), "mfma_busy": busy,
                       "dispatch_ns": dur.get(name), "source_sha256": source_sha(family(name))}
    open(out_txt, "w").write("\n".join(lines) + "\n")
    if out_json:
        json.dump(table, open(out_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def lookup(kernel: str, path: str, field: str = "bytes", grid: int | None = None) -> float | None:
    """A recorded per-launch figure of the kernel (HBM bytes by default), or None if absent or measured on
    different sources.  `grid` (work-items) selects the launch of a kernel recorded with several grid sizes."""
    try:
        table = json.load(open(path))
    except (OSError, ValueError):
        return None
    for k, v in table.items():
        if k == kernel or (grid is not None and k == f"{kernel} [grid {grid}]"):
            fam = family(k)
            if fam and v.get("source_sha256") == source_sha(fam) and v.get(field) is not None:
                return float(v[field])
    return None


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:9])
    elif sys.argv[1] == "sq":
        sq(*sys.argv[2:6])
    else:
        raise SystemExit(__doc__)
