"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m rejection_sampling_verifier_spec_amd.profile_summary stats DIR OUT --command CMD
      kernel-trace --stats run -> per-kernel calls, mean / min / max duration
  python -m rejection_sampling_verifier_spec_amd.profile_summary traffic OUT --fetch DIR --write DIR
          --copy-fetch DIR --copy-write DIR --copy-bytes N --command CMD [--command CMD ...]
      --pmc FETCH_SIZE / WRITE_SIZE runs of the benchmark and of the copy
      calibration -> HBM bytes per launch of the per-row kernel and the two
      per-request kernels, with the source hash of the kernels they were taken on
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verifier_spec_amd", "csrc", "specverify.hip")

KERNELS = {"rows": "lazy_rows_kernel", "request_pass": "request_pass_kernel",
           "request_finish": "request_finish_kernel", "copy": "copyBuffer"}
# launches per call of the verifier's default mode (the per-row pass runs as two launches)
PER_CALL = {"rows": 2, "request_pass": 1, "request_finish": 1}


def short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    return re.sub(r"\(.*", "", name).replace("void ", "").strip()


def one_csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def per_dispatch(d: str, counter: str) -> dict:
    """Mean counter value per dispatch for each kernel family."""
    vals = {k: [] for k in KERNELS}
    for r in csv.DictReader(open(one_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        for k, pat in KERNELS.items():
            if pat in r["Kernel_Name"]:
                vals[k].append(float(r["Counter_Value"]))
    return {k: (statistics.mean(v) if v else None, len(v)) for k, v in vals.items()}


def cmd_stats(args) -> None:
    rows = list(csv.DictReader(open(one_csv(args.dir, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {args.command}", "",
             f"{'kernel':60s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>7s}"]
    for r in rows:
        lines.append(f"{short(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}%")
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(args) -> None:
    f = per_dispatch(args.fetch, "FETCH_SIZE")
    w = per_dispatch(args.write, "WRITE_SIZE")
    cf = per_dispatch(args.copy_fetch, "FETCH_SIZE")["copy"][0]
    cw = per_dispatch(args.copy_write, "WRITE_SIZE")["copy"][0]
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
    for k in ("rows", "request_pass", "request_finish"):
        (fv, fn), (wv, wn) = f[k], w[k]
        if fv is None or wv is None:
            continue
        lines += [f"{k}_kernel_dispatches: {fn}",
                  f"{k}_kernel_fetch_counter_per_dispatch: {fv:.1f}",
                  f"{k}_kernel_write_counter_per_dispatch: {wv:.1f}",
                  f"{k}_kernel_hbm_bytes_per_launch: {fv * sf + wv * sw:.0f}",
                  f"{k}_kernel_launches_per_call: {PER_CALL[k]}",
                  f"{k}_kernel_hbm_bytes_per_call: {(fv * sf + wv * sw) * PER_CALL[k]:.0f}"]
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
    args = ap.parse_args()
    cmd_stats(args) if args.what == "stats" else cmd_traffic(args)


if __name__ == "__main__":
    main()
