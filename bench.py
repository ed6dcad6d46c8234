"""Benchmark of the speculative-sampling verifier on one MI355X.

One step = one call of spec_verify_probs on the headline workload: B=256
requests, gamma=7 drafts each, V=128256, bf16 target logits (N(0, 4^2) with
1% of each row boosted by 8), fp32 draft probabilities, T=0.7 — the whole hot
path (temperature softmax, accept test, residual and bonus sampling, first
rejection select). Inputs are synthetic and seeded, already resident in HBM
when the timed region starts: four input sets (the batch with its request
order rotated), cycled through every timed loop so that no cache holds a
call's inputs from the call before.

Prints one JSON line. `value` is verified draft positions per second
(B * gamma per call). Bytes count every input element a call reads once
(`unique`); the deciding rows' logits, which the per-request stage reads a
second time, are reported apart (`reread`). The roofline object prices the
dominant stage (the per-row pass, two launches per call) against HBM: its
algorithmic bytes are the logit rows it reads (a row after a position already
known to be a certain rejection is not read), 16 B of token, q(x) and uniform
per draft row read, and the records and statistics it writes; its duration is
the mean of HIP events the library records on the launch stream around the
two launches over the timed region. The per-request stage is timed the same
way in a loop after the timed region and reported beside it. `traffic` is the
HBM traffic per call of the dominant stage from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters scaled by a copy-kernel calibration, read from the
committed summary under profiles/ only when that summary was taken on the
current kernel source (else null). The oracle (float64 numpy) is timed on
the host cores on the same inputs as the CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verifier_spec_amd", "csrc", "specverify.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lazy_rows_kernel_peaked_bf16_b256_g7_v128256_traffic.txt")
SPEC_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "probs_rows_kernel_speculative_peaked_bf16_b256_g7_v128256_traffic.txt")


def source_sha256() -> str:
    import hashlib

    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(path=TRAFFIC_FILE, keys=("rows_kernel_hbm_bytes_per_call",)):
    """HBM bytes per call of the given kernels (default: the per-row pass,
    both launches) from a committed rocprofv3 summary, or None when it is
    missing or was taken on another source."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_sha256():
        return None
    try:
        return sum(float(vals[k]) for k in keys)
    except (KeyError, ValueError):
        return None


METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak), B=256 γ=7 V=128k"


_CPU_W = None  # the workload the oracle workers read (inherited through fork, not pickled)


def _oracle_chunk(job):
    """Requests [lo, hi) of the workload through the oracle, `reps` times
    over (the same work each time); returns the last pass's results."""
    import oracle

    lo, hi, reps = job
    w = _CPU_W
    logits, q, x, u, T = w["logits"], w["draft_probs"], w["draft_tokens"], w["uniforms"], w["temperature"]
    for _ in range(reps):
        out = []
        for b in range(lo, hi):
            p_rows = [oracle.target_probs(logits[b, i], T) for i in range(logits.shape[1])]
            toks, nb = oracle.verify_request(p_rows, [q[b, i] for i in range(q.shape[1])], x[b], u[b])
            out.append((toks, nb))
    return out


def cpu_baseline(w, max_requests: int, reps: int):
    """Time the oracle over the first `max_requests` requests, `reps` passes
    over them, with one worker per host core (the workers inherit the inputs
    through fork; each gets a range of requests); returns (dict, oracle
    results)."""
    global _CPU_W
    import multiprocessing as mp

    import numpy as np

    _CPU_W = w
    nb = min(max_requests, w["B"])
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, nb))
    jobs = [(int(c[0]), int(c[-1]) + 1, reps) for c in np.array_split(np.arange(nb), workers) if len(c)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(jobs)) as pool:
        res = pool.map(_oracle_chunk, jobs)
    dt = time.perf_counter() - t0
    flat = [r for part in res for r in part]
    positions = nb * w["gamma"] * reps
    # one core: the first few requests in this process
    n1 = min(8, nb)
    t1 = time.perf_counter()
    _oracle_chunk((0, n1, 1))
    single = n1 * w["gamma"] / (time.perf_counter() - t1)
    return dict(value=positions / dt, unit="positions/s", cores=len(jobs), kind="oracle",
                sample=f"first {nb} of {w['B']} requests of the same inputs, {reps} passes, float64 numpy, "
                       f"{len(jobs)} worker processes (pool start included), {dt:.2f} s wall",
                single_core_value=single, single_core_sample=f"first {n1} requests in one process"), flat


def measure_loop(steps: int, dev):
    """The synthetic end-to-end loop (bigram target and draft tables, iid
    acceptance) at B=256, gamma=7, V=32000, T=0.7: tokens per target call
    against Eq. (1), and the wall time per step (drafting included)."""
    import numpy as np
    import torch

    from rejection_sampling_verifier_spec_amd import loop

    B, g, V, T = 256, 7, 32000, 0.7
    pair = loop.make_bigram_pair(V, seed=11, kind="iid", dtype="bf16", temperature=T, device=dev)
    loop.run(pair, B, g, 3, seed=10)  # warm-up
    st = loop.run(pair, B, g, steps, seed=11)
    p = np.exp((pair.base_target.astype(np.float64) - pair.base_target.max()) / T)
    p /= p.sum()
    qd = torch.softmax(torch.from_numpy(pair.base_draft).to(dev) / T, dim=-1).cpu().numpy().astype(np.float64)
    beta = float(np.minimum(p, qd).sum())
    mean, var = loop.eq1_tokens_per_step(beta, g)
    return {"workload": f"bigram loop: B={B} gamma={g} V={V} T={T} bf16 target, iid tables",
            "steps": st.steps, "tokens_per_step": st.tokens_per_step, "eq1_tokens_per_step": mean,
            "eq1_std_error": float(np.sqrt(var / st.request_steps)), "beta": beta,
            "ms_per_step": st.seconds / st.steps * 1e3, "tokens_per_s": st.tokens / st.seconds,
            "note": "drafting (7 fp32 softmax + inverse-CDF draws), gathers and bookkeeping in torch; "
                    "the verifier through the C ABI"}


def call_percentiles(call, steps, stream):
    """Per-call times (ms) of `steps` further calls, each bracketed by a pair of
    events on the launch stream: {p10, p50, p90}."""
    import numpy as np
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)), "p90": float(np.percentile(t, 90)),
            "calls": steps}


def measured_beta(lrows, qrows, xs, T, chunk=256):
    """Mean over draft rows of beta = sum_k min(p_k, q_k) (the row's accept
    probability), with p = softmax(l / T) in fp32 by torch (a reported
    statistic of the synthetic workload, not part of the verifier); one-hot
    drafts (qrows None): beta = p(x)."""
    import torch

    tot, n = 0.0, lrows.shape[0]
    for i in range(0, n, chunk):
        p = torch.softmax(lrows[i:i + chunk].float() / T, dim=-1)
        if qrows is None:
            b = p.gather(1, xs[i:i + chunk].clamp(0, p.shape[1] - 1).view(-1, 1)).view(-1)
        else:
            b = torch.minimum(p, qrows[i:i + chunk]).sum(-1)
        tot += float(b.double().sum().item())
    return tot / max(n, 1)


def draft_views(logits, q, x, cu, B, g, V):
    """(target rows of the draft positions [N, V], q rows [N, V] or None, x [N])."""
    import torch

    if cu is None:
        return logits[:, :g].reshape(-1, V), None if q is None else q.reshape(-1, V), x.reshape(-1)
    n = x.numel()
    req = torch.repeat_interleave(torch.arange(B, device=x.device), (cu[1:] - cu[:-1]).long())
    return logits[torch.arange(n, device=x.device) + req], q, x


def copy_ceiling(dev, mib=2048, reps=10):
    """Practical HBM ceilings as context: the library's read-only stream
    (spec_verify_stream_read: 16-byte loads, every byte once), torch's fp32
    `amax` (read only) and a device-to-device copy (bytes read + written)."""
    import torch

    from rejection_sampling_verifier_spec_amd import api

    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    word_sum = torch.empty(1, dtype=torch.int64, device=dev)
    out = {}
    for name, fn, nbytes in (("stream_read", lambda: api.stream_read(a, out=word_sum), 4 * n),
                             ("read_amax", lambda: a.amax(), 4 * n), ("copy", lambda: b.copy_(a), 8 * n)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name + "_GBps"] = nbytes * reps / (time.perf_counter() - t0) / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["buffer_MiB"] = mib
    return out


OTHER_CONFIGS = ("dense_f32", "ragged_bf16", "greedy_bf16", "onehot_bf16")

NSETS = 4  # input sets resident in HBM, cycled through every timed loop
PROFILE_EVERY = 4  # calls per call carrying the library's timing events


def device_tensors(w, dev):
    """(logits, q or None, x, u, cu or None) of workload w on the device."""
    import numpy as np
    import torch

    if w["dtype"] == "bf16":
        logits = torch.from_numpy(w["logits_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        logits = torch.from_numpy(w["logits"]).to(dev)
    q = None if w["draft_probs"] is None else torch.from_numpy(w["draft_probs"]).to(dev)
    x = torch.from_numpy(w["draft_tokens"]).to(dev)
    u = torch.from_numpy(w["uniforms"]).to(dev)
    cu = torch.from_numpy(w["cu"].astype(np.int32)).to(dev) if w["kind"] == "ragged" else None
    return logits, q, x, u, cu


def input_sets(t, w):
    """NSETS copies of the batch on the device, set k with the request order
    rotated by k * B / NSETS: the same values at other addresses, so that no
    cache (the 256 MB Infinity Cache included) still holds a call's inputs
    from the call before; set 0 is the batch itself."""
    import numpy as np
    import torch

    logits, q, x, u, cu = t
    B = w["B"]
    sets = [t]
    for k in range(1, NSETS):
        perm = np.roll(np.arange(B), -(k * B // NSETS))
        if cu is None:
            idx = torch.from_numpy(perm).to(logits.device)
            sets.append((logits[idx].contiguous(), None if q is None else q[idx].contiguous(), x[idx].contiguous(),
                         u[idx].contiguous(), None))
            continue
        cu_h = w["cu"].astype(np.int64)
        lens = np.diff(cu_h)
        t_idx = np.concatenate([np.arange(cu_h[b] + b, cu_h[b + 1] + b + 1) for b in perm])
        d_idx = np.concatenate([np.arange(cu_h[b], cu_h[b + 1]) for b in perm])
        ncu = np.concatenate([[0], np.cumsum(lens[perm])]).astype(np.int32)
        ti = torch.from_numpy(t_idx).to(logits.device)
        di = torch.from_numpy(d_idx).to(logits.device)
        sets.append((logits[ti].contiguous(), None if q is None else q[di].contiguous(), x[di].contiguous(),
                     u[ti].contiguous(), torch.from_numpy(ncu).to(logits.device)))
    return sets


def time_calls(call, sets, steps):
    """Wall time per call of `steps` calls cycling through the input sets
    (synchronize on both sides)."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(sets[i % len(sets)])
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def call_bytes(rec, nacc, V, esz, has_q, gamma=None, cu=None):
    """Bytes one call reads, from its row records: `unique` counts every
    input element once (the logit rows the per-row pass read, the q rows of
    the replacement draws, 16 B of token, q(x) and uniform per draft row
    read); `reread` the logits the per-request stage reads again: each
    request's deciding row, or only the 2048-element tile the draw falls in
    when the per-row pass kept the row's tile sums (SV_ROW_TILE_SUMS: one-hot
    drafts with bf16 logits). Returns a dict with the row counts."""
    import numpy as np

    flags = rec[:, 1].astype(np.int64)
    rows = len(flags)
    B = len(nacc)
    if cu is None:
        draft = (np.arange(rows) % (gamma + 1)) < gamma
    else:
        draft = np.ones(rows, dtype=bool)
        draft[cu[1:].astype(np.int64) + np.arange(B)] = False
    read = (flags & 0x1000) == 0  # not SV_ROW_UNREAD
    resid = int(np.count_nonzero(flags & 0x4))  # SV_ROW_RESIDUAL
    bonus = int(np.count_nonzero(nacc == (np.full(B, gamma) if cu is None else np.diff(cu))))
    rows_read = int(np.count_nonzero(read))
    drafts_read = int(np.count_nonzero(read & draft))
    unique = rows_read * V * esz + drafts_read * 16 + (resid * V * 4 if has_q else 0)
    nacc64 = np.asarray(nacc).astype(np.int64)
    if cu is None:
        deciding = np.arange(B) * (gamma + 1) + nacc64
    else:
        deciding = cu[:-1].astype(np.int64) + np.arange(B) + nacc64
    kept = (flags[deciding] & 0x8000) != 0  # SV_ROW_TILE_SUMS
    reread = int(np.where(kept, min(V, 2048), V).sum()) * esz
    needed = int(np.sum(nacc + 1)) * V * esz + (resid * V * 4 if has_q else 0)
    return dict(unique=unique, reread=reread, rows_read=rows_read, drafts_read=drafts_read, residual=resid,
                bonus=bonus, rows=rows, needed=needed)


def mean_bytes(items):
    keys = items[0].keys()
    return {k: sum(d[k] for d in items) / len(items) for k in keys}


def measure_config(name: str, steps: int, dev):
    """One of the other workloads (fp32 batch, ragged batch, greedy argmax,
    one-hot drafts): `steps` calls cycling through NSETS input sets after 3
    warm-up calls: wall time per call, verified positions per second, and
    the bytes a call reads (every input element once; the deciding rows read
    again reported apart) against HBM peak."""
    import numpy as np
    import torch

    from rejection_sampling_verifier_spec_amd import api
    from rejection_sampling_verifier_spec_amd.workloads import make_workload

    w = make_workload(name, 0)
    V, T, B = w["V"], w["temperature"], w["B"]
    esz = 2 if w["dtype"] == "bf16" else 4
    sets = input_sets(device_tensors(w, dev), w)
    ragged = w["kind"] == "ragged"
    rows = sets[0][0].shape[0] if ragged else B * (w["gamma"] + 1)
    positions = int(sets[0][2].numel())
    ws = torch.zeros(api.workspace_size(rows, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call(st):
        logits, q, x, u, cu = st
        if ragged:
            return api.verify_ragged(logits, q, x, cu, u, T, workspace=ws, stream=stream)[:2]
        if T == 0.0:
            return api.verify_greedy(logits, x, workspace=ws, stream=stream)[:2]
        return api.verify_probs(logits, q, x, u, T, workspace=ws, stream=stream)[:2]

    for i in range(3):
        call(sets[i % NSETS])
    dt = time_calls(call, sets, steps)
    k = [0]

    def one():
        call(sets[k[0] % NSETS])
        k[0] += 1

    pct = call_percentiles(one, steps, stream)
    per_set = []
    for st in sets:
        out, nacc = call(st)
        rec = api.row_records(ws, rows).cpu().numpy().astype(np.int64)
        cu_h = st[4].cpu().numpy().astype(np.int64) if ragged else None
        if T == 0.0:  # greedy: every logit row once, and the tokens
            per_set.append(dict(unique=rows * V * esz + positions * 8, reread=0, rows_read=rows, needed=rows * V * esz))
        else:
            per_set.append(call_bytes(rec, nacc.cpu().numpy(), V, esz, st[1] is not None, w["gamma"], cu_h))
    b = mean_bytes(per_set)
    mode = "greedy argmax" if T == 0.0 else ("one-hot drafts" if sets[0][1] is None else "lazy")
    logits, q, x, _, cu = sets[0]
    return {"workload": f"{name}: B={B} V={V} T={T} {w['dtype']} logits, {mode}", "steps": steps,
            "input_sets": NSETS, "ms_per_call": dt * 1e3, "positions_per_s": positions / dt,
            "rows_read": b["rows_read"], "target_rows": rows,
            "unique_bytes_per_call": b["unique"], "reread_bytes_per_call": b["reread"],
            "achieved_GBps": b["unique"] / dt / 1e9, "frac_of_hbm_peak": b["unique"] / dt / 1e9 / HBM_PEAK_GBS,
            "mean_accepted": float(nacc.float().mean().item()), "call_ms": pct,
            "beta_mean": (measured_beta(*draft_views(logits, q, x, cu, B, w["gamma"], V), T) if T > 0 else None)}


def measure_filtered(steps, sets, T, ws, stream, top_k=50, top_p=0.9):
    """The same batch through spec_verify_probs_filtered (top-k then top-p on
    the target), cycling through the input sets: wall time per call and the
    per-row pass's event time."""
    import torch

    from rejection_sampling_verifier_spec_amd import api

    def call(st):
        logits, q, x, u, _ = st
        return api.verify_probs_filtered(logits, q, x, u, T, top_k, top_p, workspace=ws, stream=stream)

    for i in range(3):
        call(sets[i % NSETS])
    torch.cuda.synchronize()
    api.profile_start((api.SV_PROFILE_ROWS,), capacity=steps, every=PROFILE_EVERY)
    wall = time_calls(call, sets, steps)
    rows_ms, rows_n = api.profile_stop()[api.SV_PROFILE_ROWS]
    out, nacc, _ = call(sets[0])
    B, g = sets[0][2].shape
    flags = api.row_records(ws, B * (g + 1))[:, 1].cpu().numpy()
    read = (flags & api.SV_ROW_UNREAD) == 0
    tiers = {"rows_read": int(read.sum()),
             "second_tier": int(((flags & api.SV_ROW_HEAD2) != 0).sum()),
             "row_select": int(((flags & api.SV_ROW_ROW_SELECT) != 0).sum())}
    return {"top_k": top_k, "top_p": top_p, "steps": steps, "input_sets": NSETS, "ms_per_call": wall * 1e3,
            "positions_per_s": B * g / wall, "per_row_pass_ms_mean": rows_ms / max(rows_n, 1),
            "mean_accepted": float(nacc.float().mean().item()), "threshold_tiers": tiers}


def measure_speculative(steps, sets, T, ws, stream, esz, V):
    """SV_FLAG_ALL_RESIDUALS, the design that draws every draft row's
    replacement speculatively (every logit row and every q row read once,
    then a per-request select), on the same input sets."""
    from rejection_sampling_verifier_spec_amd import api

    def call(st):
        logits, q, x, u, _ = st
        return api.verify_probs(logits, q, x, u, T, flags=api.SV_FLAG_ALL_RESIDUALS, workspace=ws, stream=stream)

    for i in range(3):
        call(sets[i % NSETS])
    wall = time_calls(call, sets, steps)
    B, g = sets[0][2].shape
    nbytes = B * (g + 1) * V * esz + B * g * (V * 4 + 16)
    # the bytes its kernels move (rocprofv3 summary of this source, or None):
    # every logit row is read twice, once for Z and once with q for the
    # residual tile sums, which need Z
    moved = measured_traffic(SPEC_TRAFFIC_FILE, ("eager_rows_kernel_hbm_bytes_per_call",
                                                 "exact_kernel_hbm_bytes_per_call"))
    return {"flags": api.SV_FLAG_ALL_RESIDUALS, "steps": steps, "input_sets": NSETS, "ms_per_call": wall * 1e3,
            "positions_per_s": B * g / wall, "unique_bytes_per_call": nbytes, "achieved_GBps": nbytes / wall / 1e9,
            "frac_of_hbm_peak": nbytes / wall / 1e9 / HBM_PEAK_GBS, "measured_hbm_bytes_per_call": moved,
            "measured_GBps_over_call": None if moved is None else moved / wall / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="peaked_bf16")
    ap.add_argument("--flags", type=int, default=0,
                    help="SV_FLAG_* bits passed to the library (0: lazy residuals, 4: eager, 2: all residuals)")
    ap.add_argument("--cpu-requests", type=int, default=256, help="requests in the oracle baseline sample (0: skip)")
    ap.add_argument("--cpu-passes", type=int, default=20,
                    help="passes of the oracle over its sample (about 10 s of CPU work on 16 cores at the default)")
    ap.add_argument("--config-steps", type=int, default=100,
                    help="calls timed for each of the other workloads after the timed region (0: skip)")
    ap.add_argument("--filtered-steps", type=int, default=30,
                    help="calls of the top-k / top-p entry point timed after the timed region (0: skip)")
    ap.add_argument("--speculative-steps", type=int, default=30,
                    help="calls of the all-residuals mode timed after the timed region (0: skip)")
    ap.add_argument("--loop-steps", type=int, default=30,
                    help="steps of the synthetic end-to-end loop measured after the timed region (0: skip)")
    ap.add_argument("--only-config", choices=OTHER_CONFIGS, default=None,
                    help="measure only this one of the other workloads (--steps calls) and print its object "
                         "(for profiling it alone)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rejection_sampling_verifier_spec_amd import api
    from rejection_sampling_verifier_spec_amd.workloads import make_workload

    api.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only_config:
        print(json.dumps(measure_config(args.only_config, args.steps, dev)))
        return
    w = make_workload(args.workload, 0)
    B, g, V, T = w["B"], w["gamma"], w["V"], w["temperature"]
    sets = input_sets(device_tensors(w, dev), w)
    rows = B * (g + 1)
    ws = torch.zeros(api.workspace_size(rows, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    esz = 2 if w["dtype"] == "bf16" else 4
    has_q = sets[0][1] is not None

    def step(st):
        logits, q, x, u, _ = st
        return api.verify_probs(logits, q, x, u, T, flags=args.flags, workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(sets[i % NSETS])
    torch.cuda.synchronize()
    # timed region: exactly --steps calls, cycling through the input sets; the
    # library records timing-only events (no system fence) on the launch
    # stream around the dominant stage (the per-row pass, both launches) on
    # one call in PROFILE_EVERY: an event recorded between two kernels delays
    # the next by a few microseconds, so recording every call would slow the
    # region it measures. The whole call is timed by the wall clock. The first
    # per-row launch alone and the per-request stage are timed the same way in
    # a loop of their own after the timed region.
    api.profile_start((api.SV_PROFILE_ROWS,), capacity=args.steps, every=PROFILE_EVERY)
    wall = time_calls(step, sets, args.steps)
    prof = api.profile_stop()
    ms_per_step = wall * 1e3
    api.profile_start((api.SV_PROFILE_REQUEST, api.SV_PROFILE_ROWS_FIRST), capacity=args.steps,
                      every=PROFILE_EVERY)
    time_calls(step, sets, args.steps)
    after = api.profile_stop()
    prof[api.SV_PROFILE_REQUEST] = after[api.SV_PROFILE_REQUEST]
    prof[api.SV_PROFILE_ROWS_FIRST] = after[api.SV_PROFILE_ROWS_FIRST]
    k = [0]

    def one():
        step(sets[k[0] % NSETS])
        k[0] += 1

    pct = call_percentiles(one, args.steps, stream)
    positions = B * g

    # bytes per call from each input set's row records (which rows the
    # per-row pass read and which were drawn from depends on the batch and,
    # for rows read speculatively, on timing)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    p1 = max(1, min(2 * cus // B, g + 1))
    per_set, rows_info = [], []
    for st in sets:
        out, nacc, _, _ = step(st)
        rec = api.row_records(ws, rows).cpu().numpy().astype(np.int64)
        na = nacc.cpu().numpy()
        cb = call_bytes(rec, na, V, esz, has_q, g)
        flags = rec[:, 1]
        handed = int(np.count_nonzero(((flags & api.SV_ROW_UNREAD) == 0) & ((flags & api.SV_ROW_ACCEPTED) == 0)))
        # per-row pass: logits of the rows read, 16 B per draft row read (token,
        # q(x), uniform), and what it writes: an 8-byte record per row and the
        # 32-byte statistics of the rows it hands to the per-request stage
        cb["rows_kernel"] = cb["rows_read"] * V * esz + cb["drafts_read"] * 16 + rows * 8 + handed * 32
        # the first per-row launch: every row at positions 0 .. p1 - 1 (p1 as the
        # library takes it: as many positions as fill the chip's 2 blocks per CU once)
        pos = np.arange(g + 1)[None, :].repeat(B, 0).reshape(-1)
        first = pos < p1
        cb["rows_first"] = int(np.count_nonzero(first)) * V * esz + int(np.count_nonzero(first & (pos < g))) * 16
        cb["rows_second"] = int(np.count_nonzero(~first & ((flags & api.SV_ROW_UNREAD) == 0))) * V * esz
        # per-request stage: the deciding rows' logits (read again) and q rows
        cb["request_stage"] = cb["reread"] + (cb["residual"] * V * 4 if has_q else 0)
        per_set.append(cb)
        fl = flags.reshape(B, g + 1)
        rows_info.append(dict(accepted=int(np.count_nonzero(fl[:, :g] & api.SV_ROW_ACCEPTED)),
                              exact=int(np.count_nonzero(fl & api.SV_ROW_EXACT)),
                              mean_accepted=float(na.mean())))
    b = mean_bytes(per_set)
    out0, nacc0, _, _ = step(sets[0])  # set 0 = the batch in its own order (the oracle's)
    torch.cuda.synchronize()
    full_bytes = rows * V * esz + (0 if not has_q else positions * (V * 4 + 16))
    rows_ms, rows_n = prof[api.SV_PROFILE_ROWS]
    req_ms, req_n = prof[api.SV_PROFILE_REQUEST]
    first_ms, first_n = prof[api.SV_PROFILE_ROWS_FIRST]
    rows_s = rows_ms / max(rows_n, 1) * 1e-3
    req_s = req_ms / max(req_n, 1) * 1e-3
    first_s = first_ms / max(first_n, 1) * 1e-3
    achieved = b["rows_kernel"] / rows_s / 1e9 if rows_n else None
    traffic = measured_traffic()
    logits0, q0, x0, _, _ = sets[0]

    result = {
        "metric": METRIC,
        "value": positions / wall,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 logits, fp32 q, fp32 arithmetic with fp64 accumulation" if esz == 2 else "fp32",
        "data": f"synthetic, seeded (numpy PCG64), same recipe as the parity tests; {NSETS} input sets resident in "
                f"HBM (request order rotated), cycled through every timed loop",
        "config": {"workload": f"{args.workload}: B={B} gamma={g} V={V} T={T} {w['dtype']} logits",
                   "global_batch": B, "gamma": g, "vocab": V, "flags": args.flags},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": None if achieved is None else achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "lazy_rows_kernel (per-row pass, two launches per call)",
                     "bytes_per_launch": b["rows_kernel"],
                     "launch_ms_mean": rows_s * 1e3, "launches_timed": rows_n,
                     "first_launch": {"positions": p1, "ms_mean": first_s * 1e3 if first_n else None,
                                      "bytes": b["rows_first"],
                                      "achieved_GBps": b["rows_first"] / first_s / 1e9 if first_n else None},
                     "second_launch": {"ms_mean": (rows_s - first_s) * 1e3 if first_n and rows_n else None,
                                       "bytes": b["rows_second"],
                                       "achieved_GBps": (b["rows_second"] / (rows_s - first_s) / 1e9
                                                         if first_n and rows_n and rows_s > first_s else None)},
                     "note": f"HIP events recorded by the library on the launch stream around the per-row "
                             f"pass (both launches) on one call in {PROFILE_EVERY} of the timed region; bytes: the "
                             f"logit rows it read, 16 B per draft row read, its records and statistics (mean over "
                             f"the input sets). first_launch: events around the first launch alone in a loop after "
                             f"the timed region; second_launch: the difference"},
        "request_stage": {"kernel": "request_kernel (per-request fp64 slice pass, then the finish; both in one "
                                    "launch when one slice per request fills the chip)",
                          "bytes_per_launch": b["request_stage"],
                          "launch_ms_mean": req_s * 1e3 if req_n else None, "launches_timed": req_n,
                          "achieved_GBps": b["request_stage"] / req_s / 1e9 if req_n else None},
        "whole_call": {"unique_bytes": b["unique"], "reread_bytes": b["reread"], "ms_mean": ms_per_step,
                       "achieved_GBps": b["unique"] / wall / 1e9,
                       "frac_of_hbm_peak": b["unique"] / wall / 1e9 / HBM_PEAK_GBS,
                       "ms_event_percentiles": pct,
                       "note": "unique_bytes: every input element the call reads, once (logit rows read, q rows "
                               "of the replacement draws, tokens, q(x), uniforms); reread_bytes: the deciding "
                               "rows' logits read again by the per-request stage (not counted in achieved); "
                               "ms_mean: wall clock over the timed steps; percentiles: further calls, one event "
                               "pair each"},
        "rows": {"draft": positions, "target_rows": rows, "read_by_per_row_pass": b["rows_read"],
                 "needed_by_the_method": int(round(sum(r["mean_accepted"] for r in rows_info) / NSETS * B + B)),
                 "accepted_own_test": sum(r["accepted"] for r in rows_info) / NSETS,
                 "residual_drawn": b["residual"], "bonus_drawn": b["bonus"],
                 "fp64_recomputed": sum(r["exact"] for r in rows_info) / NSETS,
                 "mean_accepted": sum(r["mean_accepted"] for r in rows_info) / NSETS,
                 "beta_mean": measured_beta(*draft_views(logits0, q0, x0, None, B, g, V), T) if T > 0 else None},
        "speculative_full_bytes_per_call": full_bytes,
        "method_minimum_bytes_per_call": b["needed"],
    }
    if args.speculative_steps > 0 and has_q and T > 0:
        result["speculative"] = measure_speculative(args.speculative_steps, sets, T, ws, stream, esz, V)
    if args.filtered_steps > 0 and has_q and T > 0:
        result["filtered"] = measure_filtered(args.filtered_steps, sets, T, ws, stream)
    if args.loop_steps > 0:
        result["loop"] = measure_loop(args.loop_steps, dev)
    if args.cpu_requests > 0 and has_q:
        base, ref = cpu_baseline(w, args.cpu_requests, args.cpu_passes)
        o = out0.cpu().numpy()
        na = nacc0.cpu().numpy()
        mism = sum(1 for bi, (toks, n) in enumerate(ref) if n != na[bi] or list(o[bi, :n + 1]) != toks)
        base["parity_mismatches_in_sample"] = mism
        result["cpu_baseline"] = base
    if args.config_steps > 0:
        del sets, ws, w, logits0, q0, x0, out0, nacc0
        torch.cuda.empty_cache()
        result["hbm_ceiling_context"] = copy_ceiling(dev)
        result["other_configs"] = []
        for n in OTHER_CONFIGS:
            print(f"bench: {n}", file=sys.stderr, flush=True)
            result["other_configs"].append(measure_config(n, args.config_steps, dev))
            torch.cuda.empty_cache()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
