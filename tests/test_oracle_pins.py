"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check is a closed form,
a value a page prints, an exact count over the fp32 uniform lattice
u = (j + 1) * 2**-24, a textbook library routine, or a statistical test with
its statistic and threshold fixed before the run (the validation method of
timinsight.com, "Speculative Decoding 實作指南", section "最終驗證與回退判準").
"""

import json
import os
import multiprocessing as mp

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import (accept_draft, inverse_cdf, residual_weights, row_statistics, target_probs,
                    verify_greedy, verify_probs, verify_ragged, verify_request)

N_LATTICE = 1 << 24
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def lattice_u(j):
    return (j + 1) * 2.0 ** -24


def lattice_segments(fn):
    """Partition the uniform lattice j = 0..2^24-1 into maximal runs on which
    fn(j) is constant, assuming fn is monotone (checked on a sample). Returns
    [(value, count), ...]. About 24 calls of fn per run."""
    rng = np.random.default_rng(0)
    probe = np.sort(rng.integers(0, N_LATTICE, 64))
    vals = [fn(int(j)) for j in probe]
    segs = []
    lo = 0
    while lo < N_LATTICE:
        v = fn(lo)
        a, b = lo, N_LATTICE - 1
        if fn(b) == v:
            hi = b
        else:
            while b - a > 1:  # fn(a) == v, fn(b) != v
                mid = (a + b) // 2
                if fn(mid) == v:
                    a = mid
                else:
                    b = mid
            hi = a
        segs.append((v, hi - lo + 1))
        lo = hi + 1
    # monotone: the probe values appear in segment order
    order = [s[0] for s in segs]
    pos = [order.index(v) for v in vals]
    assert pos == sorted(pos), "function is not monotone on the lattice"
    return segs


def lattice_freq(fn):
    freq = {}
    for v, c in lattice_segments(fn):
        freq[v] = freq.get(v, 0) + c
    return freq


# ----------------------------------------------------------------- softmax


def test_target_probs_closed_form():
    # softmax of (0, ln 2, ln 3) is (1, 2, 3) / 6; at T = 1/2 it is (1, 4, 9) / 14
    l = np.array([0.0, np.log(2.0), np.log(3.0)])
    np.testing.assert_allclose(target_probs(l, 1.0), np.array([1, 2, 3]) / 6.0, rtol=1e-15, atol=0)
    np.testing.assert_allclose(target_probs(l, 0.5), np.array([1, 4, 9]) / 14.0, rtol=1e-14, atol=0)
    # shift invariance: a large common offset must not change p (max is subtracted)
    np.testing.assert_allclose(target_probs(l + 1000.0, 1.0), np.array([1, 2, 3]) / 6.0, rtol=1e-13, atol=0)


def test_target_probs_vs_scipy_and_invariants():
    rng = np.random.default_rng(1)
    for v, t in [(32, 1.0), (1000, 0.7), (32000, 1.3)]:
        l = rng.normal(0, 4, v).astype(np.float32)
        p = target_probs(l, t)
        ref = scipy.special.softmax(l.astype(np.float64) / t)
        np.testing.assert_allclose(p, ref, rtol=1e-12, atol=0)
        assert abs(p.sum() - 1.0) < 1e-12
        i, j = 3, 17
        assert np.isclose(p[i] / p[j], np.exp((float(l[i]) - float(l[j])) / t), rtol=1e-12)


def test_target_probs_neg_inf_entries():
    l = np.array([-np.inf, 0.0, -np.inf, np.log(3.0)])
    np.testing.assert_allclose(target_probs(l, 1.0), [0, 0.25, 0, 0.75], rtol=1e-15, atol=0)


def test_argmax_lowest_index_on_ties():
    l = np.array([1.0, 5.0, 2.0, 5.0, 5.0], dtype=np.float32)
    np.testing.assert_array_equal(target_probs(l, 0.0), [0, 1, 0, 0, 0])
    assert np.argmax(target_probs(np.full(7, -np.inf), 0.0)) == 0


def test_row_statistics_vs_scipy_logsumexp():
    rng = np.random.default_rng(2)
    l = rng.normal(0, 3, 5000)
    q = scipy.special.softmax(rng.normal(0, 3, 5000))
    m, lse, px, r = row_statistics(l, 0.7, q, 11)
    assert m == pytest.approx(l.max() / 0.7, rel=1e-15)
    assert lse + m == pytest.approx(scipy.special.logsumexp(l / 0.7), rel=1e-13)
    p = scipy.special.softmax(l / 0.7)
    assert px == pytest.approx(p[11], rel=1e-12)
    # residual mass identity sum max(0, p - q) = 1 - sum min(p, q)
    assert r == pytest.approx(1.0 - np.minimum(p, q).sum(), abs=1e-12)


# ---------------------------------------------------------------- accept test


@pytest.mark.parametrize("p,q,expected", [
    (3 / 8, 1 / 2, (3 * N_LATTICE) // 4),   # ratio 3/4
    (1 / 8, 1 / 2, N_LATTICE // 4),
    (1 / 2, 1 / 2, N_LATTICE),              # p = q always accepts, u = 1 included
    (3 / 4, 1 / 2, N_LATTICE),              # p > q always accepts
    (0.0, 1 / 2, 0),                        # p = 0 never accepts
    (1 / 4, 0.0, N_LATTICE),                # q = 0 with p > 0 accepts
    (0.0, 0.0, 0),                          # a token the target cannot emit is never emitted
])
def test_accept_probability_lattice_exact(p, q, expected):
    freq = lattice_freq(lambda j: accept_draft(p, q, lattice_u(j)))
    assert freq.get(True, 0) == expected


def test_beta_is_sum_min_p_q():
    """P(accept) with x ~ q equals beta = sum_x min(p, q) (Theorem 3.5,
    Corollary 3.6 as the pages restate them), to the lattice resolution."""
    rng = np.random.default_rng(3)
    for _ in range(3):
        p = rng.dirichlet(np.ones(16) * 0.5)
        q = rng.dirichlet(np.ones(16) * 0.5)
        acc = 0.0
        for x in range(16):
            c = lattice_freq(lambda j: accept_draft(p[x], q[x], lattice_u(j))).get(True, 0)
            acc += q[x] * c / N_LATTICE
        assert acc == pytest.approx(np.minimum(p, q).sum(), abs=16 * 2.0 ** -24)


# ---------------------------------------------------------------- inverse CDF


def test_inverse_cdf_lattice_exact_dyadic():
    w = np.array([1.0, 2.0, 0.0, 1.0])  # CDF boundaries at 1/4, 3/4, 3/4, 1
    freq = lattice_freq(lambda j: inverse_cdf(w, lattice_u(j)))
    assert freq == {0: N_LATTICE // 4, 1: N_LATTICE // 2, 3: N_LATTICE // 4}


def test_inverse_cdf_lattice_counts_general():
    rng = np.random.default_rng(4)
    w = rng.random(16) * (rng.random(16) < 0.7)
    w[3] = 0.5
    c = np.cumsum(w) / w.sum()
    freq = lattice_freq(lambda j: inverse_cdf(w, lattice_u(j)))
    prev = 0
    for k in range(16):
        upto = int(np.floor(c[k] * N_LATTICE + 1e-9))  # lattice points with u <= c[k]
        assert abs(freq.get(k, 0) - (upto - prev)) <= 1
        assert (k in freq) == (w[k] > 0)  # zero weight is never drawn
        prev = upto


def test_inverse_cdf_boundaries():
    w = np.array([0.0, 1.0, 1.0, 0.0])
    assert inverse_cdf(w, 0.5) == 1      # on the boundary: the lower token
    assert inverse_cdf(w, 0.5 + 2 ** -24) == 2
    assert inverse_cdf(w, 1.0) == 2      # u = 1 gives the last positive weight
    assert inverse_cdf(w, 2 ** -24) == 1  # smallest u skips the zero-weight head


# ------------------------------------------------------------ residual branch


def test_residual_fallback_constant():
    p = np.array([0.5, 0.5])
    w, mass, fb = residual_weights(p, np.array([0.5 + 1e-9, 0.5 - 1e-9]))
    assert fb and np.array_equal(w, p) and mass == pytest.approx(1e-9, rel=1e-6)
    w, mass, fb = residual_weights(p, np.array([0.5 + 4e-8, 0.5 - 4e-8]))
    assert not fb and w[0] == 0.0 and w[1] == pytest.approx(4e-8, rel=1e-6)
    assert oracle.SAMPLE_FALLBACK_MASS == 1e-8


@pytest.mark.parametrize("m,fallback", [
    (0.5e-8, True), (0.99e-8, True), (1e-8, True),          # not above 1e-8: draw from p
    (float(np.nextafter(1e-8, 1.0)), False), (1.01e-8, False), (2e-8, False),
])
def test_residual_fallback_at_the_threshold(m, fallback):
    """[GUIDE] Step 2: the replacement is drawn from p when the residual mass
    is not above 1e-8. Rows built so that the residual mass is exactly m in
    float64: p = [m, 1 - m] against q = [0, 1] leaves max(0, p - q) = [m, 0]
    (the second difference is negative). The threshold itself (the float64
    nearest 1e-8) falls back, the next float above it does not."""
    p = np.array([m, 1.0 - m])
    w, mass, fb = residual_weights(p, np.array([0.0, 1.0]))
    assert mass == m
    assert fb is fallback
    assert np.array_equal(w, p if fallback else np.array([m, 0.0]))


@pytest.mark.parametrize("m,fallback", [(0.99e-8, True), (1e-8, True), (1.01e-8, False)])
def test_residual_fallback_decides_the_emitted_token(m, fallback):
    """The fallback seen through a whole request: one draft x = 2 with
    q(x) = 1/2 > p(x) = 1/2 - m, rejected at u = 1; the residual
    max(0, p - q) = [m, 0, 0] has mass m. Drawn from the residual, the sample
    uniform 0.75 gives token 0 (the only positive weight); drawn from p
    (C = [m, 1/2 + m, 1]) it gives token 2."""
    p1 = np.array([m, 0.5, 0.5 - m])
    q1 = np.array([0.0, 0.5, 0.5])
    bonus = np.array([0.25, 0.25, 0.5])
    toks, n = oracle.verify_request([p1, bonus], [q1], [2], [1.0, 0.75])
    assert n == 0
    assert toks == [2 if fallback else 0]


def test_recovered_token_never_the_rejected_draft():
    """A rejection needs p(x) < q(x), so max(0, p - q) is zero at x: the
    recovered token differs from the rejected draft (outside the fallback)."""
    rng = np.random.default_rng(5)
    seen = 0
    for _ in range(300):
        v, g = 8, 3
        p = [rng.dirichlet(np.ones(v)) for _ in range(g + 1)]
        q = [rng.dirichlet(np.ones(v)) for _ in range(g)]
        x = [int(rng.choice(v, p=qq)) for qq in q]
        u = rng.random(g + 1) * (1 - 2 ** -24) + 2 ** -24
        toks, n = verify_request(p, q, x, u)
        assert len(toks) == n + 1 and toks[:n] == x[:n]
        if n < g:
            seen += 1
            assert toks[n] != x[n]
    assert seen > 50


# ----------------------------------------------------------- alpha = 1 and 0


def test_alpha_one_when_q_equals_p():
    rng = np.random.default_rng(6)
    v, g = 50, 6
    for _ in range(200):
        p = [rng.dirichlet(np.ones(v)) for _ in range(g + 1)]
        x = [int(rng.choice(v, p=pp)) for pp in p[:g]]
        u = rng.random(g + 1) * (1 - 2 ** -24) + 2 ** -24
        u[0] = 1.0  # even the largest uniform accepts when q = p
        toks, n = verify_request(p, p[:g], x, u)
        assert n == g and toks[:g] == x


def test_alpha_zero_on_disjoint_support():
    """Target logits are -inf on the draft's support, so every draft is
    rejected at position 1 and the emitted token is distributed as p_1
    (the residual equals p_1), exactly on the lattice."""
    v, g = 8, 2
    rng = np.random.default_rng(7)
    tl = rng.normal(0, 1, (g + 1, v))
    tl[:, :4] = -np.inf                      # target lives on 4..7
    q = np.zeros((g, v))
    q[:, :4] = rng.dirichlet(np.ones(4), g)  # draft lives on 0..3
    p = [target_probs(r, 1.0) for r in tl]
    x = [1, 2]
    freq = lattice_freq(lambda j: verify_request(p, q, x, [0.5, 0.5, lattice_u(j)])[0][0])
    for k in range(v):
        assert freq.get(k, 0) / N_LATTICE == pytest.approx(p[0][k], abs=2 * 2.0 ** -24)
    assert verify_request(p, q, x, [2 ** -24, 2 ** -24, 0.5])[1] == 0


# ------------------------------------------------- output distribution == p


def _tables(rng, v, g):
    """Prefix-indexed target and draft tables: p[j][prefix] and q[j][prefix]."""
    p = [{(): rng.dirichlet(np.ones(v) * 0.7)}]
    q = [{(): rng.dirichlet(np.ones(v) * 0.7)}]
    for j in range(1, g + 1):
        prefixes = [tuple(int(d) for d in np.unravel_index(i, (v,) * j)) for i in range(v ** j)]
        p.append({pre: rng.dirichlet(np.ones(v) * 0.7) for pre in prefixes})
        if j < g:
            q.append({pre: rng.dirichlet(np.ones(v) * 0.7) for pre in prefixes})
    return p, q


def test_output_distribution_exact_v4_g2():
    """Paper App. A.1 as the pages restate it: the tokens a verifier call
    emits, continued by the target where the call stops short, follow the
    target's own sequence distribution. Exact enumeration over drafts, with
    every branch probability taken as a count over the uniform lattice by
    calling the oracle itself."""
    v, g = 4, 2
    rng = np.random.default_rng(8)
    p, q = _tables(rng, v, g)
    tiny, one = lattice_u(0), 1.0
    got = np.zeros((v, v, v))
    for x1 in range(v):
        for x2 in range(v):
            wx = q[0][()][x1] * q[1][(x1,)][x2]
            prows = [p[0][()], p[1][(x1,)], p[2][(x1, x2)]]
            qrows = [q[0][()], q[1][(x1,)]]
            call = lambda u1, u2, us: verify_request(prows, qrows, [x1, x2], [u1, u2, us])
            a1 = lattice_freq(lambda j: call(lattice_u(j), tiny, 0.5)[1] >= 1).get(True, 0) / N_LATTICE
            a2 = lattice_freq(lambda j: call(tiny, lattice_u(j), 0.5)[1] >= 2).get(True, 0) / N_LATTICE
            if a1 < 1:
                r1 = lattice_freq(lambda j: call(one, tiny, lattice_u(j))[0][0])
                for s1, c in r1.items():
                    got[s1] += wx * (1 - a1) * c / N_LATTICE * np.outer(p[1][(s1,)], np.ones(v)) * \
                        np.stack([p[2][(s1, s2)] for s2 in range(v)])
            if a1 > 0 and a2 < 1:
                r2 = lattice_freq(lambda j: call(tiny, one, lattice_u(j))[0][1])
                for s2, c in r2.items():
                    got[x1, s2] += wx * a1 * (1 - a2) * c / N_LATTICE * p[2][(x1, s2)]
            if a1 > 0 and a2 > 0:
                r3 = lattice_freq(lambda j: call(tiny, tiny, lattice_u(j))[0][2])
                for s3, c in r3.items():
                    got[x1, x2, s3] += wx * a1 * a2 * c / N_LATTICE
    want = np.einsum("a,ab,abc->abc", p[0][()],
                     np.stack([p[1][(a,)] for a in range(v)]),
                     np.stack([np.stack([p[2][(a, b)] for b in range(v)]) for a in range(v)]))
    assert np.abs(got - want).max() < 2e-6
    assert abs(got.sum() - 1.0) < 2e-6


def _chisq_trials(args):
    seed, n, v, g = args
    rng = np.random.default_rng(9)
    p, q = _tables(rng, v, g)   # same tables in every worker
    rs = np.random.default_rng(seed)
    first = np.zeros(v, dtype=np.int64)
    pair = np.zeros((v, v), dtype=np.int64)
    for _ in range(n):
        x = []
        for j in range(g):
            x.append(int(rs.choice(v, p=q[j][tuple(x)])))
        prows = [p[j][tuple(x[:j])] for j in range(g + 1)]
        qrows = [q[j][tuple(x[:j])] for j in range(g)]
        u = (rs.integers(0, N_LATTICE, g + 1) + 1) * 2.0 ** -24
        toks, _ = verify_request(prows, qrows, x, u)
        s1 = toks[0]
        s2 = toks[1] if len(toks) > 1 else int(rs.choice(v, p=p[1][(s1,)]))
        first[s1] += 1
        pair[s1, s2] += 1
    return first, pair


def test_output_distribution_chisquare_v16():
    """V = 16, gamma = 3, 10^6 verifier calls with fresh drafts and uniforms.
    Pre-declared statistic: Pearson chi-square of the first emitted token
    against p_1 (15 dof) and of the first two tokens, continued by the target
    where the call emitted one, against p_1 p_2 (255 dof); each must pass at
    significance 0.001."""
    v, g, total = 16, 3, 1_000_000
    workers = min(8, len(os.sched_getaffinity(0)))
    chunks = [(100 + i, total // workers, v, g) for i in range(workers)]
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_chisq_trials, chunks)
    first = sum(r[0] for r in res)
    pair = sum(r[1] for r in res)
    n = first.sum()
    p, _ = _tables(np.random.default_rng(9), v, g)
    e1 = n * p[0][()]
    stat1 = ((first - e1) ** 2 / e1).sum()
    e2 = n * np.outer(p[0][()], np.ones(v)) * np.stack([p[1][(a,)] for a in range(v)])
    stat2 = ((pair - e2) ** 2 / e2).sum()
    assert stat1 < scipy.stats.chi2.ppf(0.999, v - 1), stat1
    assert stat2 < scipy.stats.chi2.ppf(0.999, v * v - 1), stat2


# ------------------------------------------------------------------ Eq. (1)


def test_eq1_printed_values():
    """E[N] = sum_{k=0..gamma} alpha^k reproduces the speeds the pages print
    for drafts of negligible cost (tests/golden/eq1_printed_values.json)."""
    cases = json.load(open(os.path.join(GOLDEN, "eq1_printed_values.json")))["cases"]
    for c in cases:
        e = sum(c["alpha"] ** k for k in range(c["gamma"] + 1))
        assert round(e, c["digits"]) == pytest.approx(c["printed"], abs=10 ** -c["digits"] / 2 + 1e-12)


def test_eq1_accept_count_distribution_iid():
    """I.i.d. acceptance (the same p, q at every position, x ~ q): the number
    of accepted drafts n satisfies P(n >= k) = beta^k, so the mean number of
    emitted tokens is sum_k beta^k (Eq. (1)). Here beta = 0.9, gamma = 10,
    which the pages print as 6.86."""
    v, g, trials = 2, 10, 40_000
    p = np.array([0.9, 0.1])
    q = np.array([1.0, 0.0])                 # beta = sum min(p, q) = 0.9
    rs = np.random.default_rng(10)
    counts = np.zeros(g + 1, dtype=np.int64)
    for _ in range(trials):
        u = (rs.integers(0, N_LATTICE, g + 1) + 1) * 2.0 ** -24
        _, n = verify_request([p] * (g + 1), [q] * g, [0] * g, u)
        counts[n] += 1
    beta = np.floor(0.9 * N_LATTICE) / N_LATTICE
    want = np.array([beta ** k * (1 - beta) for k in range(g)] + [beta ** g])
    se = np.sqrt(want * (1 - want) / trials)
    assert np.all(np.abs(counts / trials - want) < 5 * se + 1e-12)
    mean_tokens = (np.arange(g + 1) + 1) @ counts / trials
    assert mean_tokens == pytest.approx(6.862, abs=0.05)


# --------------------------------------------------- batch-level semantics


def test_greedy_semantics_small():
    # argmax rows: 3, 1, 0 ; drafts (3, 2) -> first accepted, second rejected
    l = np.full((1, 3, 4), 0.0, dtype=np.float32)
    l[0, 0, 3] = 2.0
    l[0, 1, 1] = 2.0
    l[0, 2, [0, 2]] = 3.0  # tie: lowest index wins
    out, n = verify_greedy(l, np.array([[3, 2]]))
    assert out.tolist() == [[3, 1, -1]] and n.tolist() == [1]
    out, n = verify_greedy(l, np.array([[3, 1]]))
    assert out.tolist() == [[3, 1, 0]] and n.tolist() == [2]


def test_temperature_zero_probs_is_greedy():
    rng = np.random.default_rng(11)
    l = rng.normal(0, 1, (20, 4, 40)).astype(np.float32)
    a = l.argmax(-1)
    x = np.where(rng.random((20, 3)) < 0.6, a[:, :3], rng.integers(0, 40, (20, 3)))
    q = rng.dirichlet(np.ones(40), (20, 3))
    u = (rng.integers(0, N_LATTICE, (20, 4)) + 1) * 2.0 ** -24
    o1, n1, _ = verify_probs(l, q, x, u, 0.0)
    o2, n2 = verify_greedy(l, x)
    assert np.array_equal(o1, o2) and np.array_equal(n1, n2)


def test_ragged_zero_length_request_samples_p1():
    v = 8
    rng = np.random.default_rng(12)
    l = rng.normal(0, 1, (1, v))
    p = target_probs(l[0], 1.0)
    freq = lattice_freq(lambda j: int(verify_ragged(l, None, np.zeros(0, np.int64), [0, 0],
                                                    np.array([lattice_u(j)]), 1.0)[0][0]))
    for k in range(v):
        assert freq.get(k, 0) / N_LATTICE == pytest.approx(p[k], abs=2 * 2.0 ** -24)


def test_onehot_draft_accepts_with_probability_p_x():
    """One-hot q at x (a greedy draft, [VISUAL] on paper §2.2): the draft is
    accepted with probability p(x), and the residual is p without x."""
    p = np.array([0.125, 0.5, 0.375])
    c = lattice_freq(lambda j: verify_request([p, p], None, [2], [lattice_u(j), 0.5])[1]).get(1, 0)
    assert c == (3 * N_LATTICE) // 8
    freq = lattice_freq(lambda j: verify_request([p, p], None, [2], [1.0, lattice_u(j)])[0][0])
    assert freq == {0: N_LATTICE // 5, 1: N_LATTICE - N_LATTICE // 5} or \
        abs(freq[0] - N_LATTICE * 0.2) <= 1


# ------------------------------------------------------------ top-k / top-p adjusted p


def _sorted_prefix_filter(l, T, k, top_p):
    """For rows with distinct logits: keep the k largest, then the shortest
    prefix (by decreasing probability) whose cumulative probability reaches
    top_p, renormalize. Written without value thresholds."""
    order = np.argsort(-l, kind="stable")
    idx = order[:k] if 0 < k < len(l) else order
    w = np.exp((l[idx] - l[idx].max()) / T)
    w = w / w.sum()
    if top_p < 1.0:
        c = np.cumsum(w)
        n = int(np.argmax(c >= top_p)) + 1 if np.any(c >= top_p) else len(idx)
        idx = idx[:n]
    out = np.zeros(len(l))
    out[idx] = np.exp((l[idx] - l[idx].max()) / T)
    return out / out.sum()


def test_adjusted_probs_off_is_softmax():
    rng = np.random.default_rng(20)
    l = rng.normal(0, 3, 300)
    for T in (0.5, 1.0, 2.0):
        np.testing.assert_array_equal(oracle.adjusted_target_probs(l, T), target_probs(l, T))
        np.testing.assert_array_equal(oracle.adjusted_target_probs(l, T, top_k=300, top_p=1.0), target_probs(l, T))
        np.testing.assert_array_equal(oracle.adjusted_target_probs(l, T, top_k=0, top_p=1.0), target_probs(l, T))


def test_adjusted_probs_match_a_sorted_prefix_filter_on_distinct_logits():
    rng = np.random.default_rng(21)
    for _ in range(200):
        v = int(rng.integers(2, 80))
        l = rng.normal(0, 2.5, v)
        T = float(rng.choice([0.3, 0.7, 1.0, 1.6]))
        k = int(rng.integers(0, v + 3))
        top_p = float(rng.choice([1.0, 0.95, 0.8, 0.5, 0.1, 1e-9]))
        got = oracle.adjusted_target_probs(l, T, k, top_p)
        want = _sorted_prefix_filter(l, T, k, top_p)
        np.testing.assert_array_equal(got > 0, want > 0)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def test_adjusted_probs_closed_forms_and_ties():
    l = np.array([3.0, 3.0, 1.0, 0.0, 3.0, -2.0])
    third = np.array([1, 1, 0, 0, 1, 0]) / 3.0
    # top-k counts with multiplicity and keeps every token tied at the k-th value
    for k in (1, 2, 3):
        np.testing.assert_allclose(oracle.adjusted_target_probs(l, 1.0, top_k=k), third, rtol=1e-15)
    p4 = oracle.adjusted_target_probs(l, 1.0, top_k=4)
    assert list(p4 > 0) == [True, True, True, False, True, False]
    # a tiny top_p keeps the maximum's value group, a unique maximum alone
    np.testing.assert_allclose(oracle.adjusted_target_probs(l, 0.7, top_p=1e-12), third, rtol=1e-15)
    u = np.array([0.5, 2.0, -1.0, 1.9])
    np.testing.assert_array_equal(oracle.adjusted_target_probs(u, 1.0, top_k=1), [0, 1, 0, 0])
    np.testing.assert_array_equal(oracle.adjusted_target_probs(u, 1.0, top_p=1e-9), [0, 1, 0, 0])
    # top-p applies to the renormalized top-k distribution: with the two largest kept,
    # p = (e^2, e^1.9) / sum, and 0.5 of that mass is reached by the first alone
    assert list(oracle.adjusted_target_probs(u, 1.0, top_k=2, top_p=0.5) > 0) == [False, True, False, False]
    assert list(oracle.adjusted_target_probs(u, 1.0, top_k=2, top_p=0.6) > 0) == [False, True, False, True]


def test_adjusted_probs_invariants_with_ties():
    """Brute force over every candidate threshold on rows drawn from a few
    values: the kept set is {l >= tau}, tau the larger of the top-k threshold
    (largest value with at least k tokens at or above it) and the top-p one
    (largest kept value whose tokens at or above it carry >= top_p of the
    renormalized top-k mass), and that set is the smallest such."""
    rng = np.random.default_rng(22)
    for _ in range(300):
        v = int(rng.integers(1, 12))
        l = rng.choice([-1.0, 0.0, 0.5, 2.0, 2.5], v)
        T = float(rng.choice([0.5, 1.0]))
        k = int(rng.integers(0, v + 2))
        top_p = float(rng.choice([1.0, 0.9, 0.6, 0.3, 0.05]))
        cand = sorted(set(l.tolist()), reverse=True)
        tk = cand[-1]
        if 0 < k < v:
            tk = max(t for t in cand if np.sum(l >= t) >= k)
        base = np.where(l >= tk, np.exp((l - l.max()) / T), 0.0)
        base /= base.sum()
        tp = tk
        if top_p < 1.0:
            tp = max(t for t in cand if t >= tk and base[l >= t].sum() >= top_p)
        tau = max(tk, tp)
        want = np.where(l >= tau, np.exp((l - l.max()) / T), 0.0)
        want /= want.sum()
        got = oracle.adjusted_target_probs(l, T, k, top_p)
        np.testing.assert_array_equal(got > 0, l >= tau)
        np.testing.assert_allclose(got, want, rtol=1e-12)
        assert abs(got.sum() - 1.0) < 1e-12
        kept = sorted(set(l[got > 0].tolist()))
        if top_p < 1.0 and len(kept) > 1:  # minimal: without the smallest kept value, below top_p
            assert base[l > kept[0]].sum() < top_p


def test_filtered_batch_equals_per_request_adjusted_rows():
    rng = np.random.default_rng(23)
    B, g, V, T = 5, 3, 40, 0.9
    logits = rng.normal(0, 2, (B, g + 1, V))
    q = rng.dirichlet(np.ones(V), (B, g))
    x = np.array([[rng.choice(V, p=q[b, i]) for i in range(g)] for b in range(B)])
    u = (rng.integers(0, N_LATTICE, (B, g + 1)) + 1) * 2.0 ** -24
    out, nacc, _ = oracle.verify_probs(logits, q, x, u, T, top_k=7, top_p=0.8)
    for b in range(B):
        p_rows = [oracle.adjusted_target_probs(logits[b, i], T, 7, 0.8) for i in range(g + 1)]
        toks, n = verify_request(p_rows, list(q[b]), x[b], u[b])
        assert n == nacc[b] and list(out[b, : n + 1]) == toks


def test_top_p_boundary_is_inclusive():
    """When the tokens at or above a value carry exactly top_p of the mass,
    top-p stops there (reading: "at least top_p")."""
    l = np.array([5.0, 0.0, 5.0, 0.0, -1.0])
    for T in (1.0, 0.5):
        p = target_probs(l, T)
        top = float(np.sum(p[l >= 5.0]))  # the exact mass of the top value group
        got = oracle.adjusted_target_probs(l, T, top_p=top)
        assert list(got > 0) == [True, False, True, False, False]
        np.testing.assert_allclose(got[[0, 2]], [0.5, 0.5], rtol=1e-15)
        # just above it, the next value group joins
        assert list(oracle.adjusted_target_probs(l, T, top_p=np.nextafter(top, 2.0)) > 0) == [True, True, True, True,
                                                                                             False]


def test_inverse_cdf_many_equals_the_scalar_draw():
    rng = np.random.default_rng(31)
    for _ in range(20):
        v = int(rng.integers(1, 300))
        w = rng.random(v) * (rng.random(v) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        us = (rng.integers(0, N_LATTICE, 200) + 1) * 2.0 ** -24
        us[:2] = [2.0 ** -24, 1.0]
        got = oracle.inverse_cdf_many(w, us)
        assert got.tolist() == [oracle.inverse_cdf(w, float(u)) for u in us]
