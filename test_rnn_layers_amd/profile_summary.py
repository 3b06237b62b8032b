"""Turn rocprofv3 CSV output into the short text summaries kept with the
sources, and the per-launch HBM traffic record that bench.py reports.

    # kernel-trace statistics (rocprofv3 --kernel-trace --stats --output-format csv -d DIR ...)
    python -m test_rnn_layers_amd.profile_summary stats DIR --kernel linear_dual_kernel \
        --cmd "<the rocprofv3 command>" --out profiles/linear_dual_kernel_linear_1b.md

    # HBM bytes: one --pmc FETCH_SIZE run and one --pmc WRITE_SIZE run of a
    # bench command that ends with a plain copy of known size (--copy-probe-mb)
    python -m test_rnn_layers_amd.profile_summary traffic --fetch DIR1 --write DIR2 \
        --kernel linear_dual_kernel --workload linear_1b_B4_H32_L8192_bf16 --copy-mb 1024 \
        --cmd "<the two rocprofv3 commands>" --out profiles/linear_dual_kernel_linear_1b_traffic.md

    # matrix-core use: one --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE
    # and the SQ_INSTS_VALU_MFMA_MOPS_* counters
    python -m test_rnn_layers_amd.profile_summary mfma DIR --kernel linear_dual_kernel \
        --workload linear_1b_B4_H32_L8192_bf16 --workgroups 128 --flops 30064771072 \
        --cmd "<the rocprofv3 command>" --out profiles/linear_dual_kernel_linear_1b_mfma.md

The byte counters read KiB per dispatch; each is scaled by the ratio of the
copy's known byte count to what the same counter read for the copy.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCES = {"linear_dual_kernel": "linear_dual.hip", "mlp_dual_kernel": "mlp_dual.hip",
                  "linear_token_kernel": "linear_token.hip", "mlp_token_kernel": "mlp_token.hip",
                  "post_proj_kernel": "post_proj.hip"}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_JSON = os.path.join(ROOT, "profiles", "mfma.json")
SIMDS_PER_CU = 4
CUS = 256
XCCS = 8  # GRBM_GUI_ACTIVE is reported once per XCC; the dispatch's cycles are their maximum


def source_digest(kernel: str) -> str:
    """sha256 over the kernel's source file and the headers it includes."""
    h = hashlib.sha256()
    extra = ("post_proj.hpp",) if kernel == "post_proj_kernel" else ()
    for f in (KERNEL_SOURCES[kernel], "device_common.hpp", "launch.hpp", "gelu.hpp") + extra:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _find(d: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _short(name: str, width: int = 90) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def stats_summary(d: str, kernel: str, cmd: str) -> str:
    files = _find(d, "kernel_stats.csv")
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# rocprofv3 kernel statistics: {kernel}", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        mark = "**" if kernel in r["Name"] else ""
        lines.append(f"| {mark}{_short(r['Name'])}{mark} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    tr = _find(d, "kernel_trace.csv")
    if tr:
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
               for r in csv.DictReader(open(tr[0])) if kernel in r["Kernel_Name"]]
        if dur:
            lines += ["", f"{kernel}: {len(dur)} dispatches, median {statistics.median(dur):.1f} us, "
                          f"mean {statistics.mean(dur):.1f} us"]
    return "\n".join(lines) + "\n"


def _counter(d: str, name: str) -> list[tuple[str, int, float]]:
    """(kernel name, grid size, value) per dispatch of one counter."""
    out = []
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == name:
                out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _copy_value(rows, copy_bytes: int) -> float:
    """The counter for the copy probe: the two copy dispatches the run ends
    with (bench.py --copy-probe-mb issues them after everything else)."""
    vals = [v for (k, g, v) in rows if "copy" in k.lower()]
    if len(vals) < 2:
        raise SystemExit("copy probe dispatches not found")
    return statistics.median(vals[-2:])


def traffic_summary(fetch_dir, write_dir, kernel, workload, copy_mb, cmd):
    copy_bytes = copy_mb << 20
    fr, wr = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")
    kf = [v for (k, g, v) in fr if kernel in k]
    kw = [v for (k, g, v) in wr if kernel in k]
    if not kf or not kw:
        raise SystemExit(f"no {kernel} dispatches with FETCH_SIZE / WRITE_SIZE")
    cf, cw = _copy_value(fr, copy_bytes), _copy_value(wr, copy_bytes)
    sf, sw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fb, wb = statistics.median(kf) * 1024 * sf, statistics.median(kw) * 1024 * sw
    rec = {"source_sha256": source_digest(kernel), "fetch_bytes": fb, "write_bytes": wb,
           "hbm_bytes_per_launch": fb + wb, "fetch_kib_raw": statistics.median(kf),
           "write_kib_raw": statistics.median(kw), "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": sf, "write_scale": sw, "dispatches": [len(kf), len(kw)]}
    _record(TRAFFIC_JSON, f"{kernel}@{workload}", rec)
    lines = [f"# HBM traffic of {kernel} ({workload})", "", "Commands:", "", "```", cmd, "```", "",
             f"- copy probe: {copy_bytes} bytes read and written; FETCH_SIZE read {cf:.0f} KiB, WRITE_SIZE "
             f"{cw:.0f} KiB -> scale {sf:.4f} (fetch), {sw:.4f} (write)",
             f"- {kernel}: FETCH_SIZE {statistics.median(kf):.0f} KiB, WRITE_SIZE {statistics.median(kw):.0f} KiB "
             f"per dispatch (median of {len(kf)} / {len(kw)})",
             f"- scaled: {fb / 1e6:.1f} MB read + {wb / 1e6:.1f} MB written = {(fb + wb) / 1e6:.1f} MB per launch",
             f"- kernel source sha256 {rec['source_sha256'][:16]}..."]
    return "\n".join(lines) + "\n"


def _record(path, key, rec):
    db = json.load(open(path)) if os.path.exists(path) else {}
    db[key] = rec
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
        fh.write("\n")


def mfma_summary(d, kernel, workload, workgroups, flops, cmd):
    """Matrix-core use of one kernel from SQ_VALU_MFMA_BUSY_CYCLES (cycles a
    SIMD's matrix core is busy, summed over SIMDs) against GRBM_GUI_ACTIVE
    (the dispatch's GPU cycles, summed over the XCCs), and the flops the MFMA
    op counters report (SQ_INSTS_VALU_MFMA_MOPS_*: units of 512 flops)."""
    names = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_F16",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_MFMA"]
    per = {}
    for nm in names:
        v = [x for (k, g, x) in _counter(d, nm) if kernel in k]
        if v:
            per[nm] = statistics.median(v)
    if "SQ_VALU_MFMA_BUSY_CYCLES" not in per or "GRBM_GUI_ACTIVE" not in per:
        raise SystemExit(f"no {kernel} dispatches with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE")
    cycles = per["GRBM_GUI_ACTIVE"] / XCCS
    busy = per["SQ_VALU_MFMA_BUSY_CYCLES"]
    chip = busy / (cycles * CUS * SIMDS_PER_CU)
    held = busy / (cycles * min(workgroups, CUS) * SIMDS_PER_CU)
    mops = sum(per.get(n, 0.0) for n in names[2:5])
    rec = {"source_sha256": source_digest(kernel), "mfma_busy_frac_chip": chip,
           "mfma_busy_frac_occupied_cus": held, "occupied_cus": min(workgroups, CUS), "dispatch_cycles": cycles,
           "mfma_busy_simd_cycles": busy, "counter_flops": mops * 512, "algorithmic_flops": flops,
           "counters": per}
    _record(MFMA_JSON, f"{kernel}@{workload}", rec)
    lines = [f"# Matrix-core use of {kernel} ({workload})", "", "Command:", "", "```", cmd, "```", "",
             "| counter | median per dispatch |", "|---|---|"]
    for k in names:
        if k in per:
            lines.append(f"| {k} | {per[k]:.6g} |")
    lines += ["",
              f"- dispatch: {cycles:.0f} GPU cycles (GRBM_GUI_ACTIVE / {XCCS} XCCs)",
              f"- MFMA busy: {busy:.4g} SIMD-cycles = **{chip:.2%} of the chip's {CUS * SIMDS_PER_CU} SIMDs** "
              f"over the dispatch; {held:.2%} of the {min(workgroups, CUS) * SIMDS_PER_CU} SIMDs of the "
              f"{min(workgroups, CUS)} CUs that hold a workgroup",
              f"- MFMA flops by op counters: {mops * 512:.4g}" + (
                  f" (algorithmic {flops:.4g}: ratio {mops * 512 / flops:.3f})" if flops else ""),
              f"- kernel source sha256 {rec['source_sha256'][:16]}..."]
    return "\n".join(lines) + "\n"


def sq_summary(dirs, kernel, cmd, blocks_per_chain, cus=0):
    """Shader-sequencer counters of one kernel (SQ_*), summed over its
    dispatches and divided by the dispatch count, with per-wave figures.
    SQ_WAVE_CYCLES, SQ_BUSY_CYCLES and the SQ_ACTIVE_* / SQ_WAIT_* counters
    count in units of four cycles."""
    vals = collections.defaultdict(list)
    for d in dirs:
        for f in _find(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if kernel in r["Kernel_Name"]:
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {kernel} dispatches with SQ counters")
    m = {k: statistics.mean(v) for k, v in vals.items()}
    lines = [f"# Shader-sequencer counters of {kernel}", "", "Commands:", "", "```", cmd, "```", "",
             "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
    for k in sorted(m):
        lines.append(f"| {k} | {m[k]:.4g} | {len(vals[k])} |")
    waves = m.get("SQ_WAVES", 0)
    if waves and "SQ_WAVE_CYCLES" in m:
        wc = m["SQ_WAVE_CYCLES"] / waves
        lines += ["", f"Per wave ({waves:.0f} waves per dispatch, {wc * 4:.0f} cycles each):"]
        if "SQ_INSTS_VALU" in m:
            per = m["SQ_INSTS_VALU"] / waves
            lines.append(f"- VALU instructions: {per:.0f}" + (
                f" ({per / blocks_per_chain:.0f} per mini-batch)" if blocks_per_chain else ""))
        for name in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS",
                     "SQ_LDS_BANK_CONFLICT"):
            if name in m:
                lines.append(f"- {name}: {m[name] / waves / wc:.1%} of the wave's cycles (counter / waves / "
                             f"SQ_WAVE_CYCLES per wave)")
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_ACTIVE_INST_LDS"):
            lines.append(f"- SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS = "
                         f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_ACTIVE_INST_LDS']:.2f} (mixed units: the first counts "
                         f"cycles the LDS is stalled, the second quad-cycles of each wave)")
    if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_LDS_IDX_ACTIVE"):
        lines.append(f"- SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = "
                     f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.3f} (both cycles of the LDS: the share of "
                     f"its busy cycles lost to bank conflicts)")
    if "SQ_LDS_BANK_CONFLICT" in m and m.get("GRBM_GUI_ACTIVE") and cus:
        cyc = m["GRBM_GUI_ACTIVE"] / XCCS
        lines.append(f"- bank-conflict stall cycles per CU that holds a workgroup: "
                     f"{m['SQ_LDS_BANK_CONFLICT'] / cus / cyc:.1%} of the dispatch ({cyc:.0f} cycles, {cus} CUs)")
    lines.append(f"- kernel source sha256 {source_digest(kernel)[:16]}...")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-mb", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    q = sub.add_parser("sq")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--kernel", required=True)
    q.add_argument("--blocks-per-chain", type=int, default=0, help="mini-batches per chain (per-mini-batch figures)")
    q.add_argument("--cus", type=int, default=0, help="CUs that hold a workgroup (per-CU figures)")
    q.add_argument("--cmd", required=True)
    q.add_argument("--out", required=True)
    f = sub.add_parser("mfma")
    f.add_argument("dir")
    f.add_argument("--kernel", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--workgroups", type=int, required=True, help="workgroups per dispatch (one per CU)")
    f.add_argument("--flops", type=float, default=0.0, help="algorithmic MFMA flops per dispatch")
    f.add_argument("--cmd", required=True)
    f.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd_name == "stats":
        text = stats_summary(a.dir, a.kernel, a.cmd)
    elif a.cmd_name == "sq":
        text = sq_summary(a.dirs, a.kernel, a.cmd, a.blocks_per_chain, a.cus)
    elif a.cmd_name == "mfma":
        text = mfma_summary(a.dir, a.kernel, a.workload, a.workgroups, a.flops, a.cmd)
    else:
        text = traffic_summary(a.fetch, a.write, a.kernel, a.workload, a.copy_mb, a.cmd)
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
