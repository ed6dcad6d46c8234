"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m rejection_sampling_verifier_spec_amd.profile_summary stats DIR OUT --command CMD
      kernel-trace --stats run -> per-kernel calls, mean / min / max duration
  python -m rejection_sampling_verifier_spec_amd.profile_summary traffic OUT --fetch DIR --write DIR
          --copy-fetch DIR --copy-write DIR --copy-bytes N --command CMD [--command CMD ...]
      --pmc FETCH_SIZE / WRITE_SIZE runs of the benchmark and of the copy
      calibration -> HBM bytes per launch of each launch of the per-row pass
      and of the per-request stage, and per call, with the source hash of the
      kernels they were taken on
  python -m rejection_sampling_verifier_spec_amd.profile_summary counters OUT --dir DIR [--dir DIR ...]
          --command CMD [--command CMD ...]
      --pmc runs of SQ counters -> per launch: duration, waves, VALU
      instructions, VALU issue utilisation, LDS instructions and bank
      conflicts, memory-wait share, mean occupancy
Launches are told apart by kernel family and grid size (the two launches of
the per-row pass, the slice pass and the finish of the per-request stage).
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verifier_spec_amd", "csrc", "specverify.hip")

FAMILIES = {"rows": "lazy_rows_kernel", "request": "request_kernel", "eager_rows": "probs_rows_kernel",
            "exact": "exact_kernel", "greedy": "greedy_rows_kernel", "copy": "copyBuffer"}
CLOCK_MHZ = 2400.0  # MI355X engine clock for the utilisation figures
SIMDS = 1024        # 256 compute units x 4 SIMDs


def short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    return re.sub(r"\(.*", "", name).replace("void ", "").strip()


def one_csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def family(name: str):
    for k, pat in FAMILIES.items():
        if pat in name:
            return k
    return None


def per_launch(d: str, counter: str) -> dict:
    """{(family, grid size): (mean counter value per dispatch, dispatches)}."""
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(one_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        f = family(r["Kernel_Name"])
        if f is not None:
            vals[(f, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return {k: (statistics.mean(v), len(v)) for k, v in vals.items()}


def cmd_stats(args) -> None:
    rows = list(csv.DictReader(open(one_csv(args.dir, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {args.command}", "",
             f"{'kernel':60s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>7s}"]
    for r in rows:
        lines.append(f"{short(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}%")
    # per launch (kernel family and grid size) from the trace, when present
    traces = glob.glob(os.path.join(args.dir, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        durs = collections.defaultdict(list)
        for r in csv.DictReader(open(traces[0])):
            f = family(r["Kernel_Name"])
            if f is not None and f != "copy":
                durs[(f, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "# per launch (family, grid threads, block threads): dispatches, median / mean us"]
        for k, v in sorted(durs.items()):
            lines.append(f"{k[0]:8s} grid {k[1]:9d} block {k[2]:5d}: {len(v):5d} {statistics.median(v):9.2f} "
                         f"{statistics.mean(v):9.2f}")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(args) -> None:
    f = per_launch(args.fetch, "FETCH_SIZE")
    w = per_launch(args.write, "WRITE_SIZE")
    cf = [v[0] for k, v in per_launch(args.copy_fetch, "FETCH_SIZE").items() if k[0] == "copy"][0]
    cw = [v[0] for k, v in per_launch(args.copy_write, "WRITE_SIZE").items() if k[0] == "copy"][0]
    # counter units -> bytes: the copy reads and writes exactly copy_bytes per dispatch
    sf = args.copy_bytes / cf
    sw = args.copy_bytes / cw
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    lines = ["# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (one counter per run),",
             "# scaled by the same counters on a plain device-to-device copy of known size.",
             *[f"# command: {c}" for c in args.command],
             f"source_sha256: {sha}",
             f"copy_bytes_per_dispatch: {args.copy_bytes}",
             f"copy_fetch_counter_per_dispatch: {cf:.1f}",
             f"copy_write_counter_per_dispatch: {cw:.1f}",
             f"fetch_scale_bytes_per_unit: {sf:.4f}",
             f"write_scale_bytes_per_unit: {sw:.4f}"]
    per_call = collections.defaultdict(float)
    for k in sorted(set(f) & set(w)):
        if k[0] == "copy":
            continue
        (fv, fn), (wv, _) = f[k], w[k]
        name = f"{k[0]}_grid{k[1]}"
        b = fv * sf + wv * sw
        per_call[k[0]] += b
        lines += [f"{name}_dispatches: {fn}",
                  f"{name}_fetch_bytes_per_launch: {fv * sf:.0f}",
                  f"{name}_write_bytes_per_launch: {wv * sw:.0f}",
                  f"{name}_hbm_bytes_per_launch: {b:.0f}"]
    for fam, b in per_call.items():
        lines.append(f"{fam}_kernel_hbm_bytes_per_call: {b:.0f}")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_counters(args) -> None:
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in args.dir:
        for r in csv.DictReader(open(one_csv(d, "counter_collection.csv"))):
            f = family(r["Kernel_Name"])
            if f not in ("rows", "request"):
                continue
            k = (f, int(r["Grid_Size"]))
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            vals[k]["dur_us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 SQ counters per launch (median over dispatches; counters summed over the device)",
             *[f"# command: {c}" for c in args.command],
             "# valu_issue_util = SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x duration x 2.4 GHz): the share of",
             "#   SIMD issue cycles spent on VALU instructions (wave64 on a 16-lane SIMD takes 4 cycles; fp32",
             "#   transcendentals and some fp64 operations take longer, so this is a lower bound)",
             "# mem_wait_share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: the waves' share of cycles waiting on a",
             "#   memory counter; occupancy = SQ_LEVEL_WAVES accumulated / busy cycles (when collected)",
             ""]
    for k in sorted(vals):
        v = {c: statistics.median(x) for c, x in vals[k].items()}
        dur = v.get("dur_us", 0.0)
        parts = [f"{k[0]}_grid{k[1]}", f"dur_us {dur:.1f}"]
        if "SQ_WAVES" in v:
            parts.append(f"waves {v['SQ_WAVES']:.0f}")
        if "SQ_INSTS_VALU" in v and dur > 0:
            parts.append(f"valu_instr {v['SQ_INSTS_VALU'] / 1e6:.2f}M")
            parts.append(f"valu_issue_util {v['SQ_INSTS_VALU'] * 4 / (SIMDS * dur * CLOCK_MHZ):.2f}")
        for c, lab in (("SQ_INSTS_VALU_TRANS_F32", "trans_f32"), ("SQ_INSTS_VALU_FMA_F64", "fma_f64"),
                       ("SQ_INSTS_LDS", "lds_instr"), ("SQ_LDS_BANK_CONFLICT", "lds_bank_conflict_cycles")):
            if c in v:
                parts.append(f"{lab} {v[c] / 1e6:.2f}M")
        if "SQ_WAIT_INST_ANY" in v and v.get("SQ_WAVE_CYCLES"):
            parts.append(f"mem_wait_share {v['SQ_WAIT_INST_ANY'] / v['SQ_WAVE_CYCLES']:.2f}")
        if "MeanOccupancyPerActiveCU" in v:
            parts.append(f"occupancy_waves_per_cu {v['MeanOccupancyPerActiveCU']:.1f}")
        lines.append("  ".join(parts))
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("out")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("--dir", action="append", required=True)
    c.add_argument("--command", action="append", required=True)
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.what](args)


if __name__ == "__main__":
    main()
