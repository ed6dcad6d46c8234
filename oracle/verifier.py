"""Plain float64 reference of the speculative-sampling verifier (the oracle).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

It is written for clarity, not speed: one request at a time, one position at a
time, every quantity in float64, each step in the order the pages give it.

Sources, cited by page and section (no other text is used):

[COURSE]  tarrragon.github.io, course chapter on speculative decoding,
          section "演算法核心：sampling 階段的接受邏輯" (the simplified
          accept / replace / bonus procedure).
[GUIDE]   timinsight.com, "Speculative Decoding 實作指南：基準、驗證與取捨",
          section "Step 2: 導入 Draft Proposal 與 Target Verification"
          (one verification step as PyTorch pseudocode, including the
          residual-mass fallback) and section "最終驗證與回退判準"
          (how to validate: token-by-token under greedy, a pre-declared
          statistic on a small vocabulary under sampling).
[READING] bloss0m.com, "Speculative Decoding：用小模型打草稿、大模型一次驗，
          但 T5 加速比不代表所有推論堆疊", section "技術機制 / Technical
          mechanism": speculative sampling (paper §2.3), Algorithm 1,
          Eq. (1), Theorem 3.5 and Corollary 3.6; section "實驗如何讀":
          Table 1 and Table 2 (temp=0 is argmax decoding).
[VISUAL]  blog.vllbc.top, "Speculative Decoding：draft 先猜，target 一次验证":
          the Algorithm 1 walk-through (accept rule, recover / bonus token),
          the two-path argument that the output is distributed as p
          (paper App. A.1), the closed form of beta and alpha, Eq. (1), the
          vLLM verification path (cu_num_draft_tokens, accepted + recovered +
          bonus), and the note on paper §2.2 (temperature, top-k, top-p fold
          into the adjusted p and q; a greedy draft is a one-hot q).

Readings taken where the pages are silent or disagree (each is also listed in
the design notes of the repository):

* Accept rule. [READING] and [VISUAL] accept when r <= p(x)/q(x); [COURSE]
  and [GUIDE] write r < min(1, p/q). We take "<=" in product form,
  ``u * q(x) <= p(x)``, together with ``p(x) > 0``, for u in (0, 1].
  Then p(x) = 0 never accepts, p(x) >= q(x) always accepts, and no division
  is needed (q(x) = 0 with p(x) > 0 accepts).
* Uniforms. A request with g draft tokens owns g + 1 uniforms: entries
  0..g-1 are the accept uniforms r_1..r_g, entry g is the single sample
  uniform, used for whichever token (recovered or bonus) is emitted. The
  pages draw one r per position and "a sample", without saying from what.
* Sampling. ``sample_from_distribution`` is not defined by [GUIDE]. We use the
  inverse CDF in ascending token order: C = cumsum(w) in float64, and the
  token is the smallest k with ``C[k] >= u * C[-1]``.
* Residual fallback. [GUIDE] samples from p when the residual mass is not
  above 1e-8; we use the same constant with "<= 1e-8 -> p".
* Temperature applies to the target logits only; q arrives already adjusted
  ([VISUAL], paper §2.2). Temperature 0 means argmax decoding ([READING],
  Table 2), the argmax taking the lowest index on ties (pages silent).
* Output layout. A request emits n accepted drafts plus one token; the
  row is padded with -1 to g + 1 entries ([GUIDE] returns a variable-length
  tensor instead).
* top-k / top-p ([VISUAL] on paper §2.2: like the temperature, they fold into
  an adjusted p, and the same rejection sampling runs on it; [GUIDE] asks to
  keep them identical on both sides). The pages give no details; we take:
  the filters act on the temperature-scaled target, top-k first, then top-p
  on the renormalized top-k distribution; both are thresholds on the logit
  value, ties at the threshold kept: top-k keeps every token whose logit is
  at least the k-th largest logit (counted with multiplicity), top-p keeps
  every token whose logit is at least t, t the largest logit value whose
  tokens at or above it carry at least top_p of the mass; the kept tokens
  are renormalized. top_k <= 0 or >= V, and top_p >= 1, switch a filter off.
  q arrives already adjusted by the drafter.
"""

from __future__ import annotations

import numpy as np

# [GUIDE] Step 2: when the residual mass is not above this, sample from p.
SAMPLE_FALLBACK_MASS = 1e-8


def target_probs(logits_row, temperature: float) -> np.ndarray:
    """Target distribution p of one row, float64.

    T > 0: softmax(l / T) ([GUIDE] Step 2 applies a softmax to the target
    logits; [VISUAL] on paper §2.2 folds the temperature into p).
    T == 0: one-hot at argmax(l), lowest index on ties ([READING] Table 2
    reads temp=0 as argmax).
    """
    l = np.asarray(logits_row, dtype=np.float64)
    if temperature == 0.0:
        p = np.zeros_like(l)
        p[int(np.argmax(l))] = 1.0
        return p
    s = l / float(temperature)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def adjusted_target_probs(logits_row, temperature: float, top_k: int = 0, top_p: float = 1.0) -> np.ndarray:
    """Target distribution after top-k and top-p (see the module notes for the
    readings): the kept set is {l >= tau}, with tau the larger of the top-k
    and top-p thresholds, and p is renormalized over it. T > 0."""
    l = np.asarray(logits_row, dtype=np.float64)
    p = target_probs(l, temperature)
    keep = np.ones(len(l), dtype=bool)
    if 0 < top_k < len(l):
        kth = np.sort(l)[::-1][top_k - 1]  # the k-th largest logit, with multiplicity
        keep &= l >= kth
    if not keep.all():  # renormalized only when something was removed
        p = np.where(keep, p, 0.0)
        p = p / np.sum(p)
    if top_p < 1.0:
        vals = np.unique(l[keep])[::-1]  # kept logit values, descending
        t = vals[-1]
        for v in vals:  # the first (largest) value whose tokens at or above it reach top_p
            if np.sum(p[l >= v]) >= top_p:
                t = v
                break
        if np.any(l[keep] < t):
            keep &= l >= t
            p = np.where(keep, p, 0.0)
            p = p / np.sum(p)
    return p


def accept_draft(p_x: float, q_x: float, u: float) -> bool:
    """Accept test for one drafted token x.

    [READING] speculative sampling / Algorithm 1 and [VISUAL] Algorithm 1:
    keep x when r <= p(x)/q(x). Written without the division (see module
    notes), with p(x) > 0 required.
    """
    return bool(p_x > 0.0 and u * q_x <= p_x)


def residual_weights(p_row: np.ndarray, q_row: np.ndarray):
    """Unnormalised residual max(0, p - q) and its mass, with the fallback.

    [READING] and [VISUAL]: after the first rejection the replacement token is
    drawn from norm(max(0, p - q)). [GUIDE] Step 2: if the clamped mass is
    not above 1e-8, draw from p instead. Returns (w, mass, used_fallback),
    where mass is the residual mass before any fallback.
    """
    w = np.maximum(0.0, p_row - q_row)
    mass = float(np.cumsum(w)[-1])
    if mass <= SAMPLE_FALLBACK_MASS:
        return p_row, mass, True
    return w, mass, False


def inverse_cdf(w: np.ndarray, u: float) -> int:
    """Draw one token from the unnormalised weights w with the uniform u.

    Inverse CDF in ascending token order: smallest k with C[k] >= u * C[-1],
    C = cumsum(w) in float64. For u in (0, 1] the result is an index whose
    weight is positive.
    """
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return int(np.searchsorted(c, u * c[-1], side="left"))


def inverse_cdf_many(w: np.ndarray, us) -> np.ndarray:
    """inverse_cdf for many uniforms at once (one cumulative sum): the same
    C = cumsum(w) in float64 and the same smallest k with C[k] >= u * C[-1]
    for every u in `us`."""
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return np.searchsorted(c, np.asarray(us, dtype=np.float64) * c[-1], side="left").astype(np.int64)


def _onehot(v: int, x: int) -> np.ndarray:
    q = np.zeros(v, dtype=np.float64)
    q[x] = 1.0
    return q


def verify_request(p_rows, q_rows, draft_tokens, uniforms):
    """Verify one request: Algorithm 1's accept loop, then recover or bonus.

    p_rows:       g + 1 target distributions (float64, length V each).
    q_rows:       g draft distributions, or None for a one-hot draft at the
                  drafted token ([VISUAL], paper §2.2 note: a greedy draft is
                  a one-hot q).
    draft_tokens: the g drafted tokens x_1..x_g.
    uniforms:     g + 1 uniforms in (0, 1]: g accept uniforms, then the
                  sample uniform.

    Steps ([READING] Algorithm 1; [VISUAL] Algorithm 1; [COURSE] steps 3-4):
    scan positions in order and stop at the first rejection; n is the number
    of accepted drafts. If n < g, draw from the residual of position n + 1
    (0-based n); otherwise draw the bonus token from p_{g+1}.
    Returns (tokens, n) with tokens = x_1..x_n followed by the drawn token.
    """
    g = len(draft_tokens)
    v = len(p_rows[0])
    n = 0
    while n < g:
        x = int(draft_tokens[n])
        q_x = 1.0 if q_rows is None else float(q_rows[n][x])
        if accept_draft(float(p_rows[n][x]), q_x, float(uniforms[n])):
            n += 1
        else:
            break
    if n < g:
        q_row = _onehot(v, int(draft_tokens[n])) if q_rows is None else np.asarray(q_rows[n], dtype=np.float64)
        w, _, _ = residual_weights(p_rows[n], q_row)
    else:
        w = p_rows[g]
    t = inverse_cdf(w, float(uniforms[g]))
    return [int(x) for x in draft_tokens[:n]] + [t], n


def row_statistics(logits_row, temperature: float, q_row, x):
    """Per-row statistics {max(l/T), ln sum exp(l/T - max), p(x), R}.

    For a draft row, R is the residual mass sum max(0, p - q) of that row
    ([VISUAL]: it equals 1 - sum min(p, q)); q_row None means one-hot at x.
    For the bonus row (x None) p(x) is NaN and R is 1, the mass of p itself.
    Only defined for T > 0.
    """
    if not temperature > 0.0:
        raise ValueError("row statistics are defined for temperature > 0 only")
    l = np.asarray(logits_row, dtype=np.float64)
    s = l / float(temperature)
    m = float(np.max(s))
    lse = float(np.log(np.sum(np.exp(s - m))))
    p = target_probs(l, temperature)
    if x is None:
        return m, lse, float("nan"), 1.0
    q = _onehot(len(l), int(x)) if q_row is None else np.asarray(q_row, dtype=np.float64)
    r = float(np.cumsum(np.maximum(0.0, p - q))[-1])
    return m, lse, float(p[int(x)]), r


def verify_ragged(logits, draft_probs, draft_tokens, cu_num_draft_tokens, uniforms, temperature, with_stats=False,
                  top_k=0, top_p=1.0):
    """Ragged batch ([VISUAL], vLLM verification path: requests are scanned
    through cu_num_draft_tokens and each emits accepted + recovered + bonus).

    Layout (our reading; the page only names the offsets):
      cu_num_draft_tokens [B+1], cu[0] = 0, request b owns draft rows
      cu[b]..cu[b+1]-1 and target rows cu[b]+b .. cu[b+1]+b (the last one is
      its bonus row); logits [T_total + B, V]; draft_probs [T_total, V] or
      None (one-hot drafts); draft_tokens [T_total]; uniforms [T_total + B]
      in target-row layout.
    Returns (out_tokens [T_total + B] int64, -1 padded; num_accepted [B];
    row_stats [T_total + B, 4] or None). top_k / top_p adjust every target
    row (adjusted_target_probs; T > 0, no row statistics).
    """
    filtered = (0 < top_k) or top_p < 1.0
    if filtered and (temperature == 0.0 or with_stats):
        raise ValueError("top-k / top-p are defined here for T > 0 without row statistics")
    cu = np.asarray(cu_num_draft_tokens, dtype=np.int64)
    nreq = len(cu) - 1
    rows = int(cu[-1]) + nreq
    out = np.full(rows, -1, dtype=np.int64)
    nacc = np.zeros(nreq, dtype=np.int32)
    stats = np.full((rows, 4), np.nan, dtype=np.float64) if with_stats else None
    for b in range(nreq):
        d0, d1 = int(cu[b]), int(cu[b + 1])
        g = d1 - d0
        t0 = d0 + b
        if filtered:
            p_rows = [adjusted_target_probs(logits[t0 + i], temperature, top_k, top_p) for i in range(g + 1)]
        else:
            p_rows = [target_probs(logits[t0 + i], temperature) for i in range(g + 1)]
        q_rows = None if draft_probs is None else [draft_probs[d0 + i] for i in range(g)]
        x = draft_tokens[d0:d1]
        toks, n = verify_request(p_rows, q_rows, x, uniforms[t0:t0 + g + 1])
        out[t0:t0 + len(toks)] = toks
        nacc[b] = n
        if with_stats:
            for i in range(g + 1):
                q_row = None if (draft_probs is None or i == g) else draft_probs[d0 + i]
                xi = None if i == g else int(x[i])
                stats[t0 + i] = row_statistics(logits[t0 + i], temperature, q_row, xi)
    return out, nacc, stats


def verify_probs(logits, draft_probs, draft_tokens, uniforms, temperature, with_stats=False, top_k=0, top_p=1.0):
    """Dense batch: logits [B, g+1, V], draft_probs [B, g, V] or None,
    draft_tokens [B, g], uniforms [B, g+1]. The dense call is the ragged call
    with cu[b] = b * g. Returns (out_tokens [B, g+1], num_accepted [B],
    row_stats [B, g+1, 4] or None)."""
    nreq, g1, v = logits.shape
    g = g1 - 1
    cu = np.arange(nreq + 1, dtype=np.int64) * g
    q = None if draft_probs is None else np.asarray(draft_probs).reshape(nreq * g, v)
    out, nacc, stats = verify_ragged(
        np.asarray(logits).reshape(nreq * g1, v), q, np.asarray(draft_tokens).reshape(-1), cu,
        np.asarray(uniforms).reshape(-1), temperature, with_stats, top_k, top_p)
    return out.reshape(nreq, g1), nacc, (None if stats is None else stats.reshape(nreq, g1, 4))


def verify_greedy(logits, draft_tokens):
    """Greedy verification (temperature 0, [READING] Table 2 temp=0 and
    [GUIDE] validation: greedy output is compared token by token).

    A draft is accepted while it equals the target argmax (lowest index on
    ties); the emitted token is the argmax at the first mismatch, or at the
    bonus row. Returns (out_tokens [B, g+1], num_accepted [B]).
    """
    nreq, g1, _ = logits.shape
    g = g1 - 1
    out = np.full((nreq, g1), -1, dtype=np.int64)
    nacc = np.zeros(nreq, dtype=np.int32)
    for b in range(nreq):
        a = [int(np.argmax(np.asarray(logits[b, i], dtype=np.float64))) for i in range(g1)]
        n = 0
        while n < g and int(draft_tokens[b, n]) == a[n]:
            n += 1
        out[b, :n] = draft_tokens[b, :n]
        out[b, n] = a[n]
        nacc[b] = n
    return out, nacc
