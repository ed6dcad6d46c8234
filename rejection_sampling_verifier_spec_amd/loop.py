"""Synthetic end-to-end speculative decoding loop with bigram target and draft.

Stands in for the models the pages run ([READING] "實驗如何讀" and "消融與設計
選擇", which note that even a bigram drafter speeds decoding up; [VISUAL] on
the expected number of tokens per target call, Eq. (1)): the "target" is a
random bigram table of logits (row = previous token, bf16 or fp32) and the
"drafter" a second bigram table, so no trained weights are needed. One step
of the loop, for B independent sequences:

  1. draft gamma tokens autoregressively from the draft table:
     q_i = softmax(draft[prev] / T) in fp32, x_i drawn from q_i by the
     inverse CDF with seeded uniforms;
  2. gather the target logit rows of the gamma + 1 contexts (prev, x_1 ..
     x_gamma) into a [B, gamma + 1, V] batch;
  3. verify the batch (by default through the C ABI, spec_verify_probs, or
     spec_verify_probs_filtered when top-k / top-p are set: the emitted
     tokens then follow the adjusted target, whatever the drafter's q);
  4. append x_1 .. x_n and the drawn token; the last one is the next context.

The loop keeps the bookkeeping the pages use: tokens emitted per target call
and accepted drafts per position. Two table kinds:

  "iid"   every context's target and draft rows are the same permutation of
          one base pair (target logits, draft logits), so the acceptance
          probability beta = sum_x min(p(x), q(x)) is the same at every
          position and acceptances are iid: the mean number of tokens per
          step is (1 - beta^(gamma + 1)) / (1 - beta) ([VISUAL], Eq. (1));
  "free"  independent random rows (draft = target + noise): the acceptance
          rate varies with the context (the non-iid case).

Draft sampling, gathers and bookkeeping use torch (workload plumbing, not
the verifier); the verifier runs in the library's kernels. The tables are
generated with numpy from a seed; a table has R <= V rows and context c uses
row c mod R (still a first-order Markov model; R = V for the checks of the
next-token distribution).
"""

from __future__ import annotations

import dataclasses
import time

import numpy as np
import torch

from . import api
from .workloads import bf16_bits_to_f32, f32_to_bf16_bits


@dataclasses.dataclass
class BigramPair:
    """Target and draft bigram logit tables, [R, V] each (context c uses row c mod R)."""

    target: torch.Tensor  # [R, V] bf16 or fp32
    draft: torch.Tensor  # [R, V] fp32
    temperature: float
    kind: str
    base_target: np.ndarray | None = None  # "iid": the base rows (fp32 values of the target)
    base_draft: np.ndarray | None = None


def make_bigram_pair(V: int, seed: int, kind: str = "iid", dtype: str = "bf16", temperature: float = 1.0,
                     target_sigma: float = 2.0, draft_noise: float = 1.0, rows: int | None = None,
                     device="cuda") -> BigramPair:
    R = min(V, 256) if rows is None else rows
    rng = np.random.default_rng(np.random.SeedSequence(9000 + seed))
    if kind == "iid":
        l0 = rng.normal(0.0, target_sigma, V).astype(np.float32)
        if dtype == "bf16":
            l0 = bf16_bits_to_f32(f32_to_bf16_bits(l0))
        d0 = (l0 + rng.normal(0.0, draft_noise, V)).astype(np.float32)
        perm = np.stack([rng.permutation(V).astype(np.int32) for _ in range(R)])
        tgt = l0[perm]
        drf = d0[perm]
        base_t, base_d = l0, d0
    elif kind == "free":
        tgt = rng.normal(0.0, target_sigma, (R, V)).astype(np.float32)
        if dtype == "bf16":
            tgt = bf16_bits_to_f32(f32_to_bf16_bits(tgt))
        drf = (tgt + rng.normal(0.0, draft_noise, (R, V))).astype(np.float32)
        base_t = base_d = None
    else:
        raise ValueError(f"unknown table kind {kind!r}")
    if dtype == "bf16":
        t = torch.from_numpy(f32_to_bf16_bits(tgt).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        t = torch.from_numpy(tgt).to(device)
    return BigramPair(t, torch.from_numpy(drf).to(device), float(temperature), kind, base_t, base_d)


def hip_verifier(workspace_rows: int, V: int, device, top_k: int = 0, top_p: float = 1.0):
    """The library's verifier with one workspace reused across steps (with
    top-k / top-p: the filtered entry point)."""
    ws = torch.zeros(api.workspace_size(workspace_rows, V), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)
    filtered = (0 < top_k < V) or top_p < 1.0

    def verify(logits, q, x, u, T):
        if filtered:
            out, nacc, _ = api.verify_probs_filtered(logits, q, x, u, T, top_k, top_p, workspace=ws, stream=stream)
        else:
            out, nacc, _, _ = api.verify_probs(logits, q, x, u, T, workspace=ws, stream=stream)
        return out, nacc

    return verify


def _lattice(gen: torch.Generator, shape, device) -> torch.Tensor:
    # (k + 1) 2^-24, k uniform in [0, 2^24): exact in fp32, inside (0, 1]
    k = torch.randint(0, 1 << 24, shape, generator=gen, device=device, dtype=torch.int64)
    return ((k + 1).to(torch.float64) * 2.0 ** -24).to(torch.float32)


def draft_step(pair: BigramPair, ctx: torch.Tensor, gamma: int, gen: torch.Generator):
    """gamma draft tokens per sequence and their fp32 distributions q."""
    B = ctx.shape[0]
    R, V = pair.draft.shape
    xs, qs = [], []
    prev = ctx
    for _ in range(gamma):
        q = torch.softmax(pair.draft[prev % R] / pair.temperature, dim=-1)  # fp32, the q the verifier gets
        cum = torch.cumsum(q.to(torch.float64), dim=-1)
        v = _lattice(gen, (B, 1), ctx.device).to(torch.float64)
        x = torch.searchsorted(cum, v * cum[:, -1:], right=False).clamp_(max=V - 1).squeeze(1)
        xs.append(x)
        qs.append(q)
        prev = x
    return torch.stack(xs, 1), torch.stack(qs, 1)


@dataclasses.dataclass
class LoopStats:
    steps: int = 0
    request_steps: int = 0
    tokens: int = 0
    accepted_hist: np.ndarray | None = None  # [gamma + 1]: how often n accepted drafts
    pair_counts: np.ndarray | None = None  # [V, V] (prev, next) counts of emitted tokens, when kept
    seconds: float = 0.0

    @property
    def tokens_per_step(self) -> float:
        return self.tokens / max(self.request_steps, 1)


def run(pair: BigramPair, B: int, gamma: int, steps: int, seed: int = 0, verify=None, keep_pairs: bool = False,
        device=None, top_k: int = 0, top_p: float = 1.0) -> LoopStats:
    """Run `steps` draft-and-verify steps for B sequences from random contexts
    (top_k / top_p: the library's filtered verifier, when `verify` is None)."""
    device = device or pair.target.device
    R, V = pair.target.shape
    gen = torch.Generator(device=device)
    gen.manual_seed(7919 * seed + 17)
    verify = verify or hip_verifier(B * (gamma + 1), V, device, top_k, top_p)
    ctx = torch.randint(0, V, (B,), generator=gen, device=device, dtype=torch.int64)
    st = LoopStats(accepted_hist=np.zeros(gamma + 1, dtype=np.int64),
                   pair_counts=np.zeros((V, V), dtype=np.int64) if keep_pairs else None)
    pos = torch.arange(gamma + 1, device=device)
    if device.type == "cuda":
        torch.cuda.synchronize(device)
    t0 = time.perf_counter()
    for _ in range(steps):
        x, q = draft_step(pair, ctx, gamma, gen)
        contexts = torch.cat([ctx[:, None], x], 1)  # [B, gamma + 1]: prev, x_1 .. x_gamma
        logits = pair.target[contexts % R]  # [B, gamma + 1, V]
        u = _lattice(gen, (B, gamma + 1), device)
        out, nacc = verify(logits, q.contiguous(), x.contiguous(), u, pair.temperature)
        nacc = nacc.to(torch.int64)
        st.accepted_hist += np.bincount(nacc.cpu().numpy(), minlength=gamma + 1)
        if keep_pairs:
            emitted = pos[None, :] <= nacc[:, None]  # x_1 .. x_n and the drawn token
            prevs = torch.cat([ctx[:, None], out[:, :-1]], 1)
            pc = (prevs[emitted] * V + out[emitted]).cpu().numpy()
            st.pair_counts += np.bincount(pc, minlength=V * V).reshape(V, V)
        st.tokens += int((nacc + 1).sum().item())
        ctx = out.gather(1, nacc[:, None]).squeeze(1)
        st.steps += 1
        st.request_steps += B
    if device.type == "cuda":
        torch.cuda.synchronize(device)
    st.seconds = time.perf_counter() - t0
    return st


def eq1_tokens_per_step(beta: float, gamma: int) -> tuple[float, float]:
    """Mean and variance of the tokens emitted per step when each draft is
    accepted independently with probability beta ([VISUAL], Eq. (1)): n
    accepted drafts has P(n = k) = beta^k (1 - beta) for k < gamma and
    P(n = gamma) = beta^gamma, and the step emits n + 1 tokens."""
    probs = np.array([beta ** k * (1.0 - beta) for k in range(gamma)] + [beta ** gamma])
    vals = np.arange(1, gamma + 2, dtype=np.float64)
    mean = float(np.sum(probs * vals))
    return mean, float(np.sum(probs * vals ** 2) - mean ** 2)
