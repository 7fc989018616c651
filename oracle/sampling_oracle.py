"""CPU oracle of the sampled verify (test infrastructure only): the target's
truncated distribution per verify row, draws from it, and the two accept rules
the pages describe for nonzero temperature.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call it. It shares no code
with the HIP library. Arithmetic is numpy float64; logits are taken as given
(fp32 inputs are converted exactly).

Sources (page titles and sections):
  [P1] "144 tok/s needs 502 GB/s, and Apple sells two M5 Max chips":
       section "Exact, up to top-32" (the target's distribution is temperature
       over its first top_k <= 32 entries, truncated by top_p and
       renormalised; acceptance is the speculative-sampling test u*q < p with
       a draw from max(p - q, 0) on rejection; a token outside a candidate set
       has probability zero) and section "What is actually open" (the check is
       distribution equivalence at temperature 1, top_k 32).
  [P2] "Beating Splash on an M5 Max": section "What actually moved the
       needle" (the sampler's truncation, its draw and the accept test all
       run on the GPU, which hands back only a compact result block).
  [P3] "Speculative decoding": section "Is it really lossless?" (with
       sampling, accepted drafts plus the resampled correction are an exact
       sample of the target).
  [P4] "lithos-metal ...": section "How DSpark is wired in" (the point-mass
       case: the drafter's argmax is accepted only when it equals the target's
       sampled token; the matched prefix plus the target's own token after it
       is committed).

Readings where the pages leave a step open (each is listed in the design doc):
  * Candidate order: logit descending, equal logits by lower token id; -0
    equals +0; NaN logits are never candidates. A row whose largest logit is
    not finite (all NaN, or an infinity on top) has no distribution: its draw
    is -1 and an accept scan stops there.
  * Temperature divides the logit difference to the row maximum:
    w_i = exp((z_i - z_max) / T) over the first top_k candidates.
  * top_p keeps the shortest prefix of the candidates whose mass reaches
    top_p of the top_k mass (the crossing candidate included, at least one);
    candidates of zero weight are never kept.
  * A draw with uniform u in [0, 1) picks the first kept candidate whose
    cumulative probability exceeds u (the last kept one if rounding leaves
    none).
  * Speculative sampling: the draft's distribution for verify row j is given
    as up to 16 (token id, probability) pairs (id -1 = empty; the first pair
    with a matching id counts; other tokens have probability zero). Draft j is
    accepted when u_accept[j] * q_j(d_j) < p_j(d_j). On the first rejection the
    token is drawn with u_draw[j] from max(p_j - q_j, 0) over the target's kept
    candidates, or from p_j itself if that residual has no mass. When every
    draft is accepted, the bonus is drawn from the last row's p with
    u_draw[R-1].
  * Point-mass (draft given as tokens only): row j's token is the draw from
    p_j with u_draw[j]; the scan is the greedy one on those draws.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "MAX_TOP_K", "DRAFT_CANDIDATES",
    "candidate_order", "target_distribution", "draw", "row_draws",
    "point_mass_accept", "draft_prob", "residual", "spec_accept",
]

MAX_TOP_K = 32         # [P1] "Exact, up to top-32": MAX_TOP_K is 32
DRAFT_CANDIDATES = 16  # [P1] "Exact, up to top-32": the draft contributes 16 per row


def candidate_order(row) -> np.ndarray:
    """Token ids of the non-NaN logits of one row, logit descending, equal
    logits by lower id (a stable sort of -z; -0 and +0 compare equal)."""
    z = np.asarray(row, dtype=np.float64)
    ids = np.flatnonzero(~np.isnan(z))
    order = np.argsort(-z[ids], kind="stable")
    return ids[order]


def target_distribution(row, temperature: float, top_k: int, top_p: float):
    """([P1] "Exact, up to top-32") The target's distribution for one verify
    row: temperature over the first top_k candidates, truncated by top_p,
    renormalised. Returns (ids, probs) of the kept candidates in candidate
    order; both empty when the row has no distribution (its largest logit is
    NaN or infinite)."""
    assert temperature > 0 and 1 <= top_k <= MAX_TOP_K and 0 < top_p <= 1
    z = np.asarray(row, dtype=np.float64)
    ids = candidate_order(z)[:top_k]
    if ids.size == 0 or not math.isfinite(z[ids[0]]):
        return np.empty(0, dtype=np.int64), np.empty(0)
    w = np.exp((z[ids] - z[ids[0]]) / temperature)
    total = w.sum()
    kept = 0
    mass = 0.0
    while kept < ids.size:
        mass += w[kept]
        kept += 1
        if mass >= top_p * total:
            break
    while kept > 1 and w[kept - 1] == 0.0:  # zero-weight candidates are not kept
        kept -= 1
    w = w[:kept]
    return ids[:kept].astype(np.int64), w / w.sum()


def draw(ids, probs, u: float) -> int:
    """Inverse-CDF draw: the first kept candidate whose cumulative probability
    exceeds u; the last one if none does; -1 for an empty distribution."""
    if len(ids) == 0:
        return -1
    c = np.cumsum(probs)
    hit = np.flatnonzero(c > u)
    return int(ids[hit[0]] if hit.size else ids[-1])


def row_draws(logits, temperature, top_k, top_p, u_draw):
    """Per row: the draw from the row's target distribution with u_draw[row]."""
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    u = np.asarray(u_draw, dtype=np.float64).reshape(-1)
    out = np.empty(lg.shape[0], dtype=np.int64)
    for r in range(lg.shape[0]):
        ids, p = target_distribution(lg[r], temperature, top_k, top_p)
        out[r] = draw(ids, p, float(u[r]))
    return out


def point_mass_accept(row_tokens, drafts):
    """([P4] "How DSpark is wired in") Point-mass accept per lane: row j's
    sampled token is compared with draft j; the matched prefix is accepted and
    the target's own token after it is the bonus. row_tokens [lanes][R],
    drafts [lanes][R-1]. Returns (accept_len[lanes], commit[lanes][R]) with -1
    after the committed tokens; a row without a draw (-1) matches nothing."""
    a = np.asarray(row_tokens, dtype=np.int64)
    d = np.asarray(drafts, dtype=np.int64).reshape(a.shape[0], a.shape[1] - 1)
    lanes, r = a.shape
    acc_len = np.empty(lanes, dtype=np.int64)
    commit = np.full((lanes, r), -1, dtype=np.int64)
    for l in range(lanes):
        acc = 0
        while acc < r - 1 and a[l, acc] >= 0 and a[l, acc] == d[l, acc]:
            acc += 1
        acc_len[l] = acc + 1
        commit[l, : acc + 1] = a[l, : acc + 1]
    return acc_len, commit


def draft_prob(q_ids, q_probs, token: int) -> float:
    """q(token) from the draft's (id, prob) pairs: the first matching pair, 0
    for a token outside the set ([P1] "Exact, up to top-32")."""
    for i, p in zip(np.asarray(q_ids).reshape(-1), np.asarray(q_probs, dtype=np.float64).reshape(-1)):
        if i >= 0 and int(i) == int(token):
            return float(p)
    return 0.0


def residual(ids, probs, q_ids, q_probs) -> np.ndarray:
    """max(p - q, 0) over the target's kept candidates (unnormalised)."""
    return np.array([max(float(p) - draft_prob(q_ids, q_probs, int(t)), 0.0) for t, p in zip(ids, probs)])


def spec_accept(dists, drafts, q_ids, q_probs, u_accept, u_draw):
    """([P1] "Exact, up to top-32"; [P3] "Is it really lossless?") Speculative
    sampling over one lane's R verify rows.

    dists: list of R (ids, probs) target distributions; drafts [R-1];
    q_ids / q_probs [R-1][16]; u_accept [R] (the first R-1 used); u_draw [R].
    Returns (accept_len, commit[R]) with -1 after the committed tokens."""
    r = len(dists)
    commit = np.full(r, -1, dtype=np.int64)
    for j in range(r - 1):
        ids, p = dists[j]
        d = int(drafts[j])
        if len(ids) == 0:  # no distribution: the scan stops, committing nothing here
            return j + 1, commit
        pd = draft_prob(ids, p, d)
        qd = draft_prob(q_ids[j], q_probs[j], d)
        if float(u_accept[j]) * qd < pd:
            commit[j] = d
            continue
        res = residual(ids, p, q_ids[j], q_probs[j])
        if res.sum() > 0.0:
            commit[j] = draw(ids, res / res.sum(), float(u_draw[j]))
        else:
            commit[j] = draw(ids, p, float(u_draw[j]))
        return j + 1, commit
    ids, p = dists[r - 1]
    commit[r - 1] = draw(ids, p, float(u_draw[r - 1]))
    return r, commit
