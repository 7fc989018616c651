"""Pins of the sampled-verify oracle (oracle/sampling_oracle.py) to what the
pages and the mathematics fix, independent of the oracle's own code:
library softmax, closed forms, the greedy special case, and distribution
equivalence of speculative sampling ("144 tok/s needs 502 GB/s ...", sections
"Exact, up to top-32" and "What is actually open")."""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle as O


def _rng(*key):
    return np.random.default_rng(list(key))


def test_top_k_one_is_the_greedy_argmax():
    rng = _rng(1)
    for _ in range(50):
        z = rng.normal(size=300)
        z[rng.integers(0, 300, 5)] = z.max()  # equal maxima: the lowest id wins
        ids, p = O.target_distribution(z, float(rng.uniform(0.1, 3)), 1, float(rng.uniform(0.05, 1)))
        assert list(ids) == [int(O.argmax_lowest(z[None])[0])] and p.tolist() == [1.0]
        assert O.draw(ids, p, float(rng.uniform())) == ids[0]


def test_full_support_matches_library_softmax():
    rng = _rng(2)
    for t in (0.3, 1.0, 2.5):
        z = rng.normal(scale=2.0, size=20)
        ids, p = O.target_distribution(z, t, 20, 1.0)
        ref = special.softmax(z / t)
        assert sorted(ids.tolist()) == list(range(20))
        np.testing.assert_allclose(p, ref[ids], rtol=1e-12, atol=0)
        assert np.all(np.diff(z[ids]) <= 0)


def test_top_p_truncation_closed_form():
    # probabilities 1/2, 1/4, 1/8, 1/8 at temperature 1
    z = np.log([0.125, 0.5, 0.125, 0.25])
    ids, p = O.target_distribution(z, 1.0, 4, 0.45)
    assert ids.tolist() == [1] and p.tolist() == [1.0]
    ids, p = O.target_distribution(z, 1.0, 4, 0.6)
    assert ids.tolist() == [1, 3]
    np.testing.assert_allclose(p, [2 / 3, 1 / 3], rtol=1e-12)
    ids, p = O.target_distribution(z, 1.0, 4, 0.8)
    assert ids.tolist() == [1, 3, 0]  # equal logits: lower id first
    np.testing.assert_allclose(p, [4 / 7, 2 / 7, 1 / 7], rtol=1e-12)
    ids, p = O.target_distribution(z, 1.0, 3, 1.0)  # top_k cuts before top_p
    assert ids.tolist() == [1, 3, 0]


def test_temperature_closed_form():
    # z = log p: at temperature T the weights are p**(1/T)
    base = np.array([0.6, 0.3, 0.1])
    for t in (0.5, 2.0, 4.0):
        ids, p = O.target_distribution(np.log(base), t, 3, 1.0)
        ref = base ** (1 / t)
        np.testing.assert_allclose(p, ref / ref.sum(), rtol=1e-12)


def test_special_rows():
    nan, inf = float("nan"), float("inf")
    assert O.target_distribution([nan, nan], 1.0, 4, 1.0)[0].size == 0
    assert O.target_distribution([1.0, inf, 0.0], 1.0, 4, 1.0)[0].size == 0
    assert O.target_distribution([-inf, -inf], 1.0, 4, 1.0)[0].size == 0
    ids, p = O.target_distribution([nan, 2.0, -inf, 2.0, -0.0, 0.0], 1.0, 6, 1.0)
    assert ids.tolist() == [1, 3, 4, 5]  # -inf has zero weight; -0 == +0 by id
    assert p[0] == p[1] and p[2] == p[3] and abs(p.sum() - 1) < 1e-15
    assert O.draw([], [], 0.5) == -1
    assert O.row_draws(np.array([[nan, nan]]), 1.0, 4, 1.0, [0.3]).tolist() == [-1]


def test_draw_is_inverse_cdf():
    ids, p = np.array([7, 3, 9]), np.array([0.25, 0.5, 0.25])
    assert O.draw(ids, p, 0.0) == 7 and O.draw(ids, p, 0.2499) == 7
    assert O.draw(ids, p, 0.25) == 3 and O.draw(ids, p, 0.7499) == 3
    assert O.draw(ids, p, 0.75) == 9 and O.draw(ids, p, 0.999999) == 9


def _target_and_draft(seed, v=64):
    rng = _rng(seed)
    z = rng.normal(scale=1.5, size=v)
    ids, p = O.target_distribution(z, 0.8, 32, 0.9)
    # draft: 16 candidates, half from the target's kept set, half outside it
    inside = rng.choice(ids, size=min(8, ids.size), replace=False)
    outside = rng.choice(np.setdiff1d(np.arange(v), ids), size=16 - inside.size, replace=False)
    q_ids = np.concatenate([inside, outside]).astype(np.int64)
    q = rng.dirichlet(np.ones(16))
    return ids, p, q_ids, q


def test_draw_distribution():
    ids, p, _, _ = _target_and_draft(3)
    rng = _rng(4)
    n = 40000
    counts = {int(t): 0 for t in ids}
    for u in rng.uniform(size=n):
        counts[O.draw(ids, p, float(u))] += 1
    obs = np.array([counts[int(t)] for t in ids])
    assert stats.chisquare(obs, n * p).pvalue > 1e-4


def _spec_first_tokens(seed, n):
    ids, p, q_ids, q = _target_and_draft(seed)
    rng = _rng(seed, 1)
    d = rng.choice(q_ids, size=n, p=q)  # the draft token is a sample of q
    u = rng.uniform(size=(n, 2))
    dists = [(ids, p), (ids, p)]
    out = np.empty(n, dtype=np.int64)
    acc = 0
    for i in range(n):
        a, c = O.spec_accept(dists, [d[i]], q_ids[None], q[None], u[i], u[i][::-1])
        out[i] = c[0]
        acc += a == 2
    return ids, p, q_ids, q, out, acc / n


def test_speculative_sampling_preserves_the_target_distribution():
    # the committed token after one draft is distributed as the target's p,
    # whatever the draft's q ("Exact, up to top-32"; "Is it really lossless?")
    n = 30000
    ids, p, q_ids, q, out, acc_rate = _spec_first_tokens(5, n)
    obs = np.array([(out == t).sum() for t in ids])
    assert obs.sum() == n  # never a token outside the target's kept set
    assert stats.chisquare(obs, n * p).pvalue > 1e-4
    # acceptance rate: sum over tokens of min(p, q)
    qd = np.array([O.draft_prob(q_ids, q, int(t)) for t in ids])
    expect = np.minimum(p, qd).sum()
    assert abs(acc_rate - expect) < 5 * math.sqrt(expect * (1 - expect) / n) + 1e-9


def test_distribution_check_detects_a_wrong_residual(monkeypatch):
    # a planted mistake (drawing the rejected case from p instead of
    # max(p - q, 0)) must fail the same check: the test has the power to see it
    monkeypatch.setattr(O.sampling_oracle, "residual", lambda ids, probs, qi, qp: np.asarray(probs, dtype=float))
    n = 30000
    ids, p, _, _, out, _ = _spec_first_tokens(5, n)
    obs = np.array([(out == t).sum() for t in ids])
    assert stats.chisquare(obs, n * p).pvalue < 1e-6


def test_draft_equal_to_target_is_always_accepted():
    ids, p, _, _ = _target_and_draft(6)
    rng = _rng(7)
    for _ in range(500):
        d = int(rng.choice(ids, p=p))
        a, c = O.spec_accept([(ids, p), (ids, p)], [d], ids[None], p[None], rng.uniform(size=2), rng.uniform(size=2))
        assert a == 2 and c[0] == d


def test_top_k_one_reduces_both_rules_to_greedy():
    rng = _rng(8)
    lanes, r, v = 4, 8, 50
    for _ in range(20):
        z = rng.normal(size=(lanes * r, v))
        am = O.argmax_lowest(z).reshape(lanes, r)
        drafts = np.where(rng.uniform(size=(lanes, r - 1)) < 0.7, am[:, :-1], rng.integers(0, v, (lanes, r - 1)))
        g_len, g_commit = O.greedy_accept(am, drafts)
        toks = O.row_draws(z, 1.3, 1, 1.0, rng.uniform(size=lanes * r)).reshape(lanes, r)
        p_len, p_commit = O.point_mass_accept(toks, drafts)
        assert np.array_equal(p_len, g_len) and np.array_equal(p_commit, g_commit)
        for l in range(lanes):
            dists = [O.target_distribution(z[l * r + j], 1.3, 1, 1.0) for j in range(r)]
            q_ids = rng.integers(0, v, (r - 1, 16))
            q = rng.dirichlet(np.ones(16), size=r - 1) * 0.9
            a, c = O.spec_accept(dists, drafts[l], q_ids, q, rng.uniform(size=r), rng.uniform(size=r))
            assert a == g_len[l] and np.array_equal(c, g_commit[l])


def test_row_without_distribution_stops_the_scan():
    nan = float("nan")
    dists = [(np.array([4]), np.array([1.0])), (np.empty(0, dtype=np.int64), np.empty(0)), (np.array([2]), np.array([1.0]))]
    a, c = O.spec_accept(dists, [4, 2], np.full((2, 16), -1), np.zeros((2, 16)), [0.0, 0.0, 0.0], [0.5, 0.5, 0.5])
    assert a == 2 and c.tolist() == [4, -1, -1]
    toks = O.row_draws(np.array([[0.0, 1.0], [nan, nan], [1.0, 0.0]]), 1.0, 2, 1.0, [0.99, 0.5, 0.5])
    assert toks.tolist() == [0, -1, 0]
    a, c = O.point_mass_accept(toks[None], np.array([[0, -1]]))
    assert a.tolist() == [2] and c.tolist() == [[0, -1, -1]]
