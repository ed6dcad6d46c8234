"""Seeded synthetic inputs for the verifier (shared by tests and the bench).

This module only makes inputs: target logits, draft distributions, drafted
tokens, uniforms and ragged offsets. It holds none of the verifier's
arithmetic. The draft distribution q = softmax(draft logits) and the drafted
tokens x ~ q stand in for a draft model (a drafter's job, upstream of the
verifier); x is drawn with numpy's ``Generator.choice``. Greedy workloads need
the target argmax to plant drafts that match it; numpy's ``argmax`` supplies
it.

Every request is generated from its own stream,
``SeedSequence(1000 * recipe_id + seed, spawn_key=(b,))``, so requests are
produced in parallel threads with a result that does not depend on the thread
count, and a workload with fewer requests is a prefix of the larger one.

Recipes (sizes can be overridden for smaller parity cases):

  tiny        B=1, g=4, V=32, fp32 target ~N(0, 2^2), independent draft logits
              ~N(0, 2^2), q = softmax(draft logits), T=1.
  dense_f32   B=64, g=5, V=32000, fp32 target ~N(0, 3^2), draft logits =
              target[:, :g] + N(0, 1), T=1 (high overlap).
  peaked_bf16 B=256, g=7, V=128256, bf16 target = N(0, 4^2) plus 8 on
              floor(0.01 V) distinct random ids per row, draft logits =
              (bf16 target + N(0, 2^2)) / 0.7, T=0.7.
  ragged_bf16 B=512, g_b ~ U{1..8}, V=152064, bf16 target ~N(0, 3^2),
              independent draft logits ~N(0, 3^2), T=1 (low overlap).
  greedy_bf16 B=1024, g=4, V=128256, bf16 target ~N(0, 3^2), drafts equal the
              target argmax with probability 0.7, else uniform over the other
              ids; T=0, no q.
  onehot_bf16 the greedy_bf16 inputs with one-hot drafts (no q) and T=1.

Uniforms are ``(k + 1) * 2**-24`` with k uniform in [0, 2**24): exact in
fp32, inside (0, 1]. bf16 values are fp32 values rounded to nearest even.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

RECIPES = {
    "tiny": dict(rid=1, B=1, gamma=4, V=32, dtype="f32", T=1.0),
    "dense_f32": dict(rid=2, B=64, gamma=5, V=32000, dtype="f32", T=1.0),
    "peaked_bf16": dict(rid=3, B=256, gamma=7, V=128256, dtype="bf16", T=0.7),
    "ragged_bf16": dict(rid=4, B=512, gamma=8, V=152064, dtype="bf16", T=1.0),
    "greedy_bf16": dict(rid=5, B=1024, gamma=4, V=128256, dtype="bf16", T=0.0),
    "onehot_bf16": dict(rid=5, B=1024, gamma=4, V=128256, dtype="bf16", T=1.0),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest even; returns the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def lattice_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return ((k + 1).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _normal(rng, shape, sigma):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def _draft_rows(rng, z_rows):
    """Draft-model stand-in: q = softmax(z) per row (fp32) and x ~ q."""
    z64 = np.asarray(z_rows, dtype=np.float64)
    z64 = np.exp(z64 - z64.max(axis=-1, keepdims=True))
    z64 /= z64.sum(axis=-1, keepdims=True)
    v = z64.shape[-1]
    x = np.array([rng.choice(v, p=row / row.sum()) for row in z64], dtype=np.int64)
    return z64.astype(np.float32), x


def _exact(dtype, rows_f32):
    """Round to the storage type; returns (values as fp32, bf16 bits or None)."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(rows_f32)
        return bf16_bits_to_f32(bits), bits
    return np.ascontiguousarray(rows_f32, dtype=np.float32), None


def _request(name, rng, g, v, dtype):
    """One request's inputs: dict(logits, bits, q, x, u)."""
    if name == "tiny":
        lf, bits = _exact(dtype, _normal(rng, (g + 1, v), 2.0))
        q, x = _draft_rows(rng, _normal(rng, (g, v), 2.0))
    elif name == "dense_f32":
        lf, bits = _exact(dtype, _normal(rng, (g + 1, v), 3.0))
        q, x = _draft_rows(rng, lf[:g] + _normal(rng, (g, v), 1.0))
    elif name == "peaked_bf16":
        t = _normal(rng, (g + 1, v), 4.0)
        for i in range(g + 1):
            t[i, rng.choice(v, size=v // 100, replace=False)] += np.float32(8.0)
        lf, bits = _exact(dtype, t)
        q, x = _draft_rows(rng, (lf[:g] + _normal(rng, (g, v), 2.0)) / np.float32(0.7))
    elif name == "ragged_bf16":
        lf, bits = _exact(dtype, _normal(rng, (g + 1, v), 3.0))
        q, x = _draft_rows(rng, _normal(rng, (g, v), 3.0))
    elif name in ("greedy_bf16", "onehot_bf16"):
        lf, bits = _exact(dtype, _normal(rng, (g + 1, v), 3.0))
        a = np.argmax(lf[:g], axis=-1)
        other = rng.integers(0, v - 1, size=g)
        other = other + (other >= a)
        keep = rng.random(g) < 0.7
        x = np.where(keep, a, other).astype(np.int64)
        q = None
    else:
        raise KeyError(name)
    u = lattice_uniforms(rng, g + 1)
    return dict(logits=lf, bits=bits, q=q, x=x, u=u)


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def make_workload(name: str, seed: int = 0, B: int | None = None, V: int | None = None,
                  gamma: int | None = None) -> dict:
    """Build one seeded workload. ``B``, ``V`` and ``gamma`` override the
    recipe's sizes (same value distributions) for smaller parity cases.

    Dense workloads: logits [B, g+1, V] (fp32 values, exact for bf16),
    logits_bits [B, g+1, V] uint16 (bf16 only), draft_probs [B, g, V] fp32 or
    None, draft_tokens [B, g] int64, uniforms [B, g+1] fp32.
    Ragged (``ragged_bf16``): logits [T+B, V], draft_probs [T, V],
    draft_tokens [T], uniforms [T+B], cu [B+1] int32, max_gamma.
    """
    r = dict(RECIPES[name])
    rid = r["rid"]
    nb = r["B"] if B is None else B
    v = r["V"] if V is None else V
    gmax = r["gamma"] if gamma is None else gamma
    dtype, temp = r["dtype"], r["T"]
    ragged = name == "ragged_bf16"

    def one(b):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(1000 * rid + seed, spawn_key=(b,))))
        g = int(rng.integers(1, gmax + 1)) if ragged else gmax
        return _request(name, rng, g, v, dtype)

    w = dict(name=name, seed=seed, B=nb, V=v, temperature=temp, dtype=dtype)
    onehot = name in ("greedy_bf16", "onehot_bf16")
    if ragged:
        # draft lengths first (cheap, from each request's own stream) to size the outputs
        gb = np.array([int(np.random.Generator(np.random.PCG64(np.random.SeedSequence(
            1000 * rid + seed, spawn_key=(b,)))).integers(1, gmax + 1)) for b in range(nb)], dtype=np.int64)
        cu = np.zeros(nb + 1, dtype=np.int64)
        cu[1:] = np.cumsum(gb)
        ntok = int(cu[-1])
        w.update(kind="ragged", gamma=None, cu=cu.astype(np.int32), max_gamma=int(gb.max()) if nb else 0)
        trow = lambda b: slice(int(cu[b]) + b, int(cu[b + 1]) + b + 1)
        drow = lambda b: slice(int(cu[b]), int(cu[b + 1]))
        lshape, qshape, xshape, ushape = (ntok + nb, v), (ntok, v), (ntok,), (ntok + nb,)
    else:
        w.update(kind="dense", gamma=gmax, cu=None)
        trow = drow = (lambda b: b)
        lshape, qshape, xshape, ushape = (nb, gmax + 1, v), (nb, gmax, v), (nb, gmax), (nb, gmax + 1)
    w["logits"] = np.empty(lshape, dtype=np.float32)
    w["logits_bits"] = np.empty(lshape, dtype=np.uint16) if dtype == "bf16" else None
    w["draft_probs"] = None if onehot else np.empty(qshape, dtype=np.float32)
    w["draft_tokens"] = np.empty(xshape, dtype=np.int64)
    w["uniforms"] = np.empty(ushape, dtype=np.float32)

    def fill(b):
        rq = one(b)
        w["logits"][trow(b)] = rq["logits"]
        if rq["bits"] is not None:
            w["logits_bits"][trow(b)] = rq["bits"]
        if rq["q"] is not None:
            w["draft_probs"][drow(b)] = rq["q"]
        w["draft_tokens"][drow(b)] = rq["x"]
        w["uniforms"][trow(b)] = rq["u"]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nb)))
    return w


def make_dense_custom(seed: int, B: int, gamma: int, V: int, dtype: str, temperature: float,
                      logit_sigma: float = 3.0, q_kind: str = "noisy", q_sigma: float = 1.0) -> dict:
    """Free-form dense workload for edge-case parity tests.

    q_kind: "noisy" (q = softmax((target + N(0, q_sigma^2)) / T)),
    "independent" (q = softmax(N(0, logit_sigma^2))), or "onehot" (no q,
    drafted tokens uniform over the vocabulary).
    """
    rng = np.random.Generator(np.random.PCG64(777_000 + seed))
    w = dict(name="custom", seed=seed, B=B, V=V, gamma=gamma, temperature=temperature, dtype=dtype,
             kind="dense", cu=None)
    lf, bits = _exact(dtype, _normal(rng, (B * (gamma + 1), V), logit_sigma))
    w["logits"] = lf.reshape(B, gamma + 1, V)
    w["logits_bits"] = None if bits is None else bits.reshape(B, gamma + 1, V)
    if q_kind == "onehot" or gamma == 0:
        w["draft_probs"] = None
        w["draft_tokens"] = rng.integers(0, V, size=(B, gamma)).astype(np.int64)
    else:
        if q_kind == "noisy":
            z = w["logits"][:, :gamma] + _normal(rng, (B, gamma, V), q_sigma)
        else:
            z = _normal(rng, (B, gamma, V), logit_sigma)
        if temperature > 0:
            z = z / np.float32(temperature)
        q, x = _draft_rows(rng, z.reshape(B * gamma, V))
        w["draft_probs"] = q.reshape(B, gamma, V)
        w["draft_tokens"] = x.reshape(B, gamma)
    w["uniforms"] = lattice_uniforms(rng, (B, gamma + 1))
    return w


def dense_as_ragged(w: dict) -> dict:
    """View a dense workload in the ragged layout (cu[b] = b * g)."""
    nb, g, v = w["B"], w["gamma"], w["V"]
    r = dict(w)
    r["kind"] = "ragged"
    r["cu"] = (np.arange(nb + 1) * g).astype(np.int32)
    r["max_gamma"] = g
    r["logits"] = w["logits"].reshape(nb * (g + 1), v)
    if w.get("logits_bits") is not None:
        r["logits_bits"] = w["logits_bits"].reshape(nb * (g + 1), v)
    r["draft_probs"] = None if w["draft_probs"] is None else w["draft_probs"].reshape(nb * g, v)
    r["draft_tokens"] = w["draft_tokens"].reshape(-1)
    r["uniforms"] = w["uniforms"].reshape(-1)
    return r
