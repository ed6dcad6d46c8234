"""Shared helpers of the GPU parity tests: move seeded workloads to the
device, run the HIP path through the C ABI binding, run the oracle, compare.

Comparison rule (fixed before any run): tokens, accept counts and argmax
results must be equal. A mismatch is classified with the tolerance the
verifier's target states - an accept flip is tolerated when |u - p(x)/q(x)|
<= 1e-6, a sampled-token flip when the uniform lies within 1e-6 of a CDF
boundary of the oracle's (normalised) sampling distribution - and such
tolerated flips must stay below 1e-4 of the rows checked; anything else is a
hard failure. With top-k / top-p (`filt` = (top_k, top_p)) the oracle's
target rows are its adjusted distributions and the same rule applies. Row
statistics: max(l/T) within 1e-6 relative, ln Z within
1e-5 absolute (Z within 1e-5 relative), p(x) within 1e-5 relative (floor
1e-30), R within 1e-5 relative plus 2e-6 absolute.
"""

from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from rejection_sampling_verifier_spec_amd import api

DEV = torch.device("cuda:0")


def logits_tensor(w, dev=DEV):
    if w["dtype"] == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w["logits_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w["logits"])).to(dev)


def dev_inputs(w, dev=DEV):
    t = dict(logits=logits_tensor(w, dev))
    t["q"] = None if w["draft_probs"] is None else torch.from_numpy(w["draft_probs"]).to(dev)
    t["x"] = torch.from_numpy(np.ascontiguousarray(w["draft_tokens"])).to(dev)
    t["u"] = torch.from_numpy(np.ascontiguousarray(w["uniforms"])).to(dev)
    t["cu"] = None if w.get("cu") is None else torch.from_numpy(w["cu"].astype(np.int32)).to(dev)
    return t


def run_gpu(w, flags=0, stats=False, t=None):
    """Run the HIP path on workload w; returns numpy (out, nacc, stats, records)."""
    t = t or dev_inputs(w)
    if w["kind"] == "ragged":
        out, nacc, st, ws = api.verify_ragged(t["logits"], t["q"], t["x"], t["cu"], t["u"], w["temperature"],
                                              flags=flags, row_stats=stats)
        rows = out.numel()
    elif w["temperature"] == 0.0 and w["draft_probs"] is None and not stats and flags == 0:
        out, nacc, ws = api.verify_greedy(t["logits"], t["x"])
        st = None
        rows = out.numel()
    else:
        out, nacc, st, ws = api.verify_probs(t["logits"], t["q"], t["x"], t["u"], w["temperature"],
                                             flags=flags, row_stats=stats)
        rows = out.numel()
    torch.cuda.synchronize()
    rec = api.row_records(ws, rows).cpu().numpy()
    return (out.cpu().numpy(), nacc.cpu().numpy(), None if st is None else st.cpu().numpy(), rec)


def run_gpu_filtered(w, top_k, top_p, t=None):
    """Run the filtered HIP path; returns numpy (out, nacc, None, records)."""
    t = t or dev_inputs(w)
    if w["kind"] == "ragged":
        out, nacc, ws = api.verify_ragged_filtered(t["logits"], t["q"], t["x"], t["cu"], t["u"], w["temperature"],
                                                   top_k, top_p)
    else:
        out, nacc, ws = api.verify_probs_filtered(t["logits"], t["q"], t["x"], t["u"], w["temperature"], top_k,
                                                  top_p)
    torch.cuda.synchronize()
    rec = api.row_records(ws, out.numel()).cpu().numpy()
    return out.cpu().numpy(), nacc.cpu().numpy(), None, rec


def target_rows(l, T, filt=None, rows=None):
    """The oracle's target distributions of the rows of l (adjusted by top-k /
    top-p when filt = (top_k, top_p))."""
    rows = range(len(l)) if rows is None else rows
    if filt is None:
        return [oracle.target_probs(l[i], T) for i in rows]
    return [oracle.adjusted_target_probs(l[i], T, filt[0], filt[1]) for i in rows]


def request_view(w, b):
    """(logits rows [g+1, V], q rows [g, V] or None, x [g], u [g+1], slice of target rows)."""
    if w["kind"] == "ragged":
        cu = w["cu"]
        d0, d1 = int(cu[b]), int(cu[b + 1])
        t0 = d0 + b
        sl = slice(t0, d1 + b + 1)
        q = None if w["draft_probs"] is None else w["draft_probs"][d0:d1]
        return w["logits"][sl], q, w["draft_tokens"][d0:d1], w["uniforms"][sl], sl
    q = None if w["draft_probs"] is None else w["draft_probs"][b]
    return w["logits"][b], q, w["draft_tokens"][b], w["uniforms"][b], b


def oracle_request(w, b, stats=False, filt=None):
    l, q, x, u, _ = request_view(w, b)
    T = w["temperature"]
    g = len(x)
    if T == 0.0:
        r_out, r_n = oracle.verify_greedy(l[None], np.asarray(x)[None])
        toks = [int(v) for v in r_out[0][: r_n[0] + 1]]
        return toks, int(r_n[0]), None
    p_rows = target_rows(l, T, filt, range(g + 1))
    toks, n = oracle.verify_request(p_rows, None if q is None else [q[i] for i in range(g)], x, u)
    st = None
    if stats:
        st = np.array([oracle.row_statistics(l[i], T, None if (q is None or i == g) else q[i],
                                             None if i == g else int(x[i])) for i in range(g + 1)])
    return toks, n, st


def _flip_tolerated(w, b, gpu_toks, gpu_n, ref_toks, ref_n, filt=None):
    """Classify one mismatching request; returns True for a tolerated flip."""
    l, q, x, u, _ = request_view(w, b)
    T = w["temperature"]
    g = len(x)
    p_rows = target_rows(l, T, filt, range(g + 1))
    if gpu_n != ref_n:
        i = min(gpu_n, ref_n)  # first position whose decision differs
        qx = 1.0 if q is None else float(q[i][int(x[i])])
        px = float(p_rows[i][int(x[i])])
        return qx > 0 and abs(float(u[i]) - px / qx) <= 1e-6
    n = ref_n
    if n < g:
        qrow = np.zeros(len(p_rows[n])) if q is None else np.asarray(q[n], dtype=np.float64)
        if q is None:
            qrow[int(x[n])] = 1.0
        wts, _, _ = oracle.residual_weights(p_rows[n], qrow)
    else:
        wts = p_rows[g]
    c = np.cumsum(wts) / np.cumsum(wts)[-1]
    gt = gpu_toks[n]
    if not 0 <= gt < len(c):
        return False
    us = float(u[g])
    lo = c[gt - 1] if gt > 0 else 0.0
    return (lo - 1e-6) < us <= c[gt] + 1e-6


def _compare_range(w, gpu, reqs, stats, label, filt):
    """(hard mismatches, tolerated flips, rows checked) over requests `reqs`."""
    out, nacc, gst, _ = gpu
    hard, flips, rows = [], 0, 0
    for b in reqs:
        l, q, x, u, sl = request_view(w, b)
        g = len(x)
        rows += g + 1
        ref_toks, ref_n, rst = oracle_request(w, b, stats, filt)
        go = out[sl] if w["kind"] == "ragged" else out[b]
        gn = int(nacc[b])
        gtoks = [int(v) for v in go[: gn + 1]]
        pad_ok = all(int(v) == -1 for v in go[gn + 1:])
        if not pad_ok:
            hard.append((b, "padding", go.tolist()))
        if gtoks != ref_toks or gn != ref_n:
            if _flip_tolerated(w, b, gtoks, gn, ref_toks, ref_n, filt):
                flips += 1
            else:
                hard.append((b, gtoks, ref_toks, gn, ref_n))
        if stats:
            gs = gst[sl] if w["kind"] == "ragged" else gst[b]
            check_stats(gs, rst, f"{label} request {b}")
    return hard, flips, rows


def compare(w, gpu, reqs=None, stats=False, label="", filt=None):
    """Compare GPU results with the oracle on requests `reqs` (all if None)."""
    reqs = range(w["B"]) if reqs is None else reqs
    hard, flips, rows = _compare_range(w, gpu, reqs, stats, label, filt)
    assert not hard, f"{label}: {len(hard)} hard mismatches, first: {hard[:3]}"
    assert flips <= 1e-4 * rows, f"{label}: {flips} tolerated flips in {rows} rows"
    return rows, flips


_JOB = None  # (w, gpu, stats, label, filt) inherited by the forked workers


def _compare_job(rng):
    w, gpu, stats, label, filt = _JOB
    return _compare_range(w, gpu, range(*rng), stats, label, filt)


def compare_all(w, gpu, stats=False, label="", filt=None, workers=16):
    """compare() on every request of the batch, the oracle run by forked worker
    processes over contiguous ranges of requests (host CPU work only; the
    workers inherit the inputs and the GPU results through fork and never
    touch the GPU). Prints the rows checked and the tolerated flips."""
    import multiprocessing as mp
    global _JOB
    nb = w["B"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = 4
    nw = max(1, min(workers, cores, nb))
    bounds = np.linspace(0, nb, nw + 1).round().astype(int)
    jobs = [(int(bounds[i]), int(bounds[i + 1])) for i in range(nw) if bounds[i + 1] > bounds[i]]
    _JOB = (w, gpu, stats, label, filt)
    try:
        with mp.get_context("fork").Pool(len(jobs)) as pool:
            parts = pool.map(_compare_job, jobs)
    finally:
        _JOB = None
    hard = [h for p in parts for h in p[0]]
    flips = sum(p[1] for p in parts)
    rows = sum(p[2] for p in parts)
    print(f"{label}: {nb} requests, {rows} rows, {flips} tolerated flips, {len(hard)} hard mismatches", flush=True)
    assert not hard, f"{label}: {len(hard)} hard mismatches, first: {hard[:3]}"
    assert flips <= 1e-4 * rows, f"{label}: {flips} tolerated flips in {rows} rows"
    return rows, flips


def check_stats(gs, rs, label):
    gs = np.asarray(gs, dtype=np.float64)
    rs = np.asarray(rs, dtype=np.float64)
    np.testing.assert_allclose(gs[:, 0], rs[:, 0], rtol=1e-6, atol=1e-30, err_msg=label + " max(l/T)")
    np.testing.assert_allclose(gs[:, 1], rs[:, 1], rtol=0, atol=1e-5, err_msg=label + " ln Z")
    d = ~np.isnan(rs[:, 2])
    assert np.array_equal(np.isnan(gs[:, 2]), ~d), label + " p(x) NaN pattern"
    np.testing.assert_allclose(gs[d, 2], rs[d, 2], rtol=1e-5, atol=1e-30, err_msg=label + " p(x)")
    np.testing.assert_allclose(gs[:, 3], rs[:, 3], rtol=1e-5, atol=2e-6, err_msg=label + " R")
