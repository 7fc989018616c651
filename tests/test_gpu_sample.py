"""GPU parity of the sampled verify (vq_sample_accept) against the oracle
(oracle/sampling_oracle.py), through the C ABI.

Both sides read the same fp32 logits and uniforms (seeded host inputs). The
candidate lists are compared exactly (the order is fixed by the exact logit
values and token ids). Probabilities are compared to 1e-5. Decisions that
floating point takes -- how many candidates top_p keeps, which candidate a
uniform lands on, u*q < p -- are compared exactly except where the oracle's
fp64 margin is below 1e-5: there fp32 may legitimately decide the other way
(the tie class), and the lane is left out (their number is bounded).

"144 tok/s needs 502 GB/s ...", sections "Exact, up to top-32" and "What is
actually open" (the distribution check); "lithos-metal ...", section "How
DSpark is wired in" (the point-mass rule).
"""
import math

import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs, ops
from gpu_helpers import say

pytestmark = pytest.mark.gpu

EPS = 1e-5        # decision margin below which fp32 may differ from fp64
PROB_ATOL = 1e-5  # fp32 probabilities vs fp64


def _dev():
    import torch
    return torch, torch.device("cuda:0")


def _f32(a):
    torch, dev = _dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def _i32(a):
    torch, dev = _dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def run_gpu(logits, lanes, R, t, k, tp, u_draw, draft=None, q=None, u_accept=None, ws=None):
    torch, dev = _dev()
    M, V = logits.shape
    lg = _f32(logits)
    out = dict(tok=torch.full((M,), -7, dtype=torch.int32, device=dev),
               acc=torch.full((lanes,), -7, dtype=torch.int32, device=dev),
               commit=torch.full((lanes, R), -7, dtype=torch.int32, device=dev),
               cand=torch.full((M, 32), -7, dtype=torch.int32, device=dev),
               prob=torch.full((M, 32), -7.0, dtype=torch.float32, device=dev))
    if ws is None:
        ws = ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev)
    ops.vq_sample_accept(lg, lanes, R, t, k, tp, _f32(u_draw), out["acc"],
                         draft=None if draft is None else _i32(draft),
                         draft_ids=None if q is None else _i32(q[0]),
                         draft_probs=None if q is None else _f32(q[1]),
                         u_accept=None if u_accept is None else _f32(u_accept),
                         token_out=out["tok"], commit_out=out["commit"], cand_out=out["cand"],
                         prob_out=out["prob"], workspace=ws)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


# ---------------------------------------------------------------- tie class

def count_margin(z, t, k, tp):
    """fp64 margin of the top_p decision (inf when top_p = 1 or no choice)."""
    ids = O.candidate_order(z)[:k]
    if ids.size == 0 or not math.isfinite(z[ids[0]]) or tp >= 1.0:
        return math.inf
    w = np.exp((np.asarray(z, dtype=np.float64)[ids] - z[ids[0]]) / t)
    c = np.cumsum(w) / w.sum()
    return float(np.min(np.abs(c - tp)))


def draw_margin(probs, u):
    if len(probs) == 0:
        return math.inf
    return float(np.min(np.abs(np.cumsum(probs)[:-1] - u))) if len(probs) > 1 else math.inf


def check_rows(logits, t, k, tp, u_draw, got):
    """Per-row candidates, probabilities and draws; returns the set of rows
    whose decisions are clear of the tie class."""
    clear = set()
    for r in range(logits.shape[0]):
        ids, p = O.target_distribution(logits[r], t, k, tp)
        full = O.candidate_order(logits[r])[:k]
        n = ids.size
        if count_margin(logits[r], t, k, tp) <= EPS:
            # the kept count may differ; the candidates before it still agree
            m = min(n, int((got["cand"][r] >= 0).sum()))
            assert np.array_equal(got["cand"][r][:m], full[:m]), r
            continue
        assert np.array_equal(got["cand"][r][:n], ids), (r, got["cand"][r][:n], ids)
        assert np.all(got["cand"][r][n:] == -1) and np.all(got["prob"][r][n:] == 0.0), r
        np.testing.assert_allclose(got["prob"][r][:n], p, rtol=0, atol=PROB_ATOL, err_msg=f"row {r}")
        want = O.draw(ids, p, float(u_draw[r]))
        if draw_margin(p, float(u_draw[r])) <= EPS:
            j = int(np.flatnonzero(ids == want)[0])
            assert got["tok"][r] in ids[max(0, j - 1): j + 2], r
            continue
        assert got["tok"][r] == want, (r, got["tok"][r], want)
        clear.add(r)
    return clear


def lanes_clear_point_mass(rows_clear, toks, drafts, lanes, R):
    """Lanes whose oracle scan only passes rows outside the tie class."""
    out = []
    for l in range(lanes):
        stop = 0
        while stop < R - 1 and toks[l * R + stop] >= 0 and toks[l * R + stop] == drafts[l][stop]:
            stop += 1
        if all((l * R + j) in rows_clear or toks[l * R + j] < 0 for j in range(stop + 1)):
            out.append(l)
    return out


# ------------------------------------------------------------------- inputs

def structured_logits(key, lanes, R, V):
    z = inputs.logits_f32(key, lanes * R, V)
    nan, inf = np.float32("nan"), np.float32("inf")
    z[1, ::7] = nan                      # scattered NaN
    z[2, :] = nan                        # no distribution
    z[3, 5] = inf                        # +inf on top: no distribution
    z[4, :] = -inf                       # all -inf: no distribution
    z[5, [3, 11, V - 1]] = z[5].max() + 1  # exact ties at the top: lower id first
    z[6, 100:140] = 0.0                  # a block of equal values with -0 mixed in
    z[6, 100:140:2] = -0.0
    z[6, :100] = -5.0
    z[6, 140:] = -5.0
    z[7, 9] = -inf
    return z


def point_mass_drafts(key, logits, lanes, R, t, k, tp, u_draw):
    """Drafts that match the oracle's draws with probability 0.7 (so scans
    run long), else a uniform id."""
    toks = O.row_draws(logits, t, k, tp, u_draw).reshape(lanes, R)
    return inputs.drafts(key, np.where(toks >= 0, toks, 0), logits.shape[1])


# -------------------------------------------------------------------- tests

PARAMS = [(1.0, 32, 1.0), (0.7, 20, 0.9), (1.6, 5, 0.5), (1.0, 1, 1.0), (0.3, 32, 0.95)]


@pytest.mark.parametrize("t,k,tp", PARAMS)
@pytest.mark.parametrize("lanes,R,V", [(4, 8, 20000), (1, 8, 8193), (3, 5, 333), (2, 1, 70000)])
def test_point_mass(lanes, R, V, t, k, tp):
    say(f"case point-mass lanes={lanes} R={R} V={V} T={t} top_k={k} top_p={tp}")
    M = lanes * R
    key = (41, lanes, R, V)
    z = structured_logits(key, lanes, R, V) if M >= 8 else inputs.logits_f32(key, M, V)
    u = inputs.uniforms(key, M)
    d = point_mass_drafts(key, z, lanes, R, t, k, tp, u) if R > 1 else None
    got = run_gpu(z, lanes, R, t, k, tp, u, draft=d)
    clear = check_rows(z, t, k, tp, u, got)
    toks = O.row_draws(z, t, k, tp, u)
    want_len, want_commit = O.point_mass_accept(toks.reshape(lanes, R),
                                                d if d is not None else np.zeros((lanes, 0), np.int32))
    ok = lanes_clear_point_mass(clear, toks, d if d is not None else np.zeros((lanes, 0)), lanes, R)
    for l in ok:
        assert got["acc"][l] == want_len[l] and np.array_equal(got["commit"][l], want_commit[l]), l
    say(f"  rows clear {len(clear)}/{M}, lanes compared {len(ok)}/{lanes}, accept {got['acc'].tolist()}")
    assert len(ok) >= lanes - 1


def _spec_inputs(key, z, lanes, R, t, k, tp):
    V = z.shape[1]
    pref = np.full((lanes * (R - 1), 32), -1, dtype=np.int64)
    for l in range(lanes):
        for j in range(R - 1):
            ids, _ = O.target_distribution(z[l * R + j], t, k, tp)
            pref[l * (R - 1) + j, : ids.size] = ids
    q_ids, q_p, d = inputs.draft_distributions(key, pref, V)
    return (q_ids.reshape(lanes, R - 1, 16), q_p.reshape(lanes, R - 1, 16)), d.reshape(lanes, R - 1)


def spec_lane_clear(dists, drafts, q_ids, q_p, ua, ud):
    """True when every decision on the oracle's path is outside the tie class."""
    R = len(dists)
    for j in range(R - 1):
        ids, p = dists[j]
        if len(ids) == 0:
            return True
        pd = O.draft_prob(ids, p, int(drafts[j]))
        qd = O.draft_prob(q_ids[j], q_p[j], int(drafts[j]))
        if abs(float(ua[j]) * qd - pd) <= EPS:
            return False
        if float(ua[j]) * qd < pd:
            continue
        res = O.residual(ids, p, q_ids[j], q_p[j])
        if res.sum() > 0:
            return draw_margin(res / res.sum(), float(ud[j])) > EPS and res.sum() > EPS
        return draw_margin(p, float(ud[j])) > EPS
    ids, p = dists[R - 1]
    return draw_margin(p, float(ud[R - 1])) > EPS


@pytest.mark.parametrize("t,k,tp", PARAMS)
@pytest.mark.parametrize("lanes,R,V", [(4, 8, 20000), (2, 3, 5000), (1, 8, 248320)])
def test_speculative_sampling(lanes, R, V, t, k, tp):
    say(f"case speculative lanes={lanes} R={R} V={V} T={t} top_k={k} top_p={tp}")
    M = lanes * R
    key = (43, lanes, R, V)
    z = structured_logits(key, lanes, R, V) if M >= 8 else inputs.logits_f32(key, M, V)
    ud = inputs.uniforms(key, M)
    ua = inputs.uniforms(key + (1,), M)
    q, d = _spec_inputs(key, z, lanes, R, t, k, tp)
    got = run_gpu(z, lanes, R, t, k, tp, ud, draft=d, q=q, u_accept=ua)
    clear_rows = check_rows(z, t, k, tp, ud, got)
    compared = 0
    for l in range(lanes):
        dists = [O.target_distribution(z[l * R + j], t, k, tp) for j in range(R)]
        rows = range(l * R, l * R + R)
        if any(count_margin(z[r], t, k, tp) <= EPS for r in rows):
            continue
        if not spec_lane_clear(dists, d[l], q[0][l], q[1][l], ua[l * R:(l + 1) * R], ud[l * R:(l + 1) * R]):
            continue
        a, c = O.spec_accept(dists, d[l], q[0][l], q[1][l], ua[l * R:(l + 1) * R], ud[l * R:(l + 1) * R])
        assert got["acc"][l] == a and np.array_equal(got["commit"][l], c), (l, got["acc"][l], a, got["commit"][l], c)
        compared += 1
    say(f"  rows clear {len(clear_rows)}/{M}, lanes compared {compared}/{lanes}, accept {got['acc'].tolist()}")
    assert compared >= lanes - 1


def test_point_mass_full_acceptance():
    # every draft equals the target's draw: each lane commits R tokens, the
    # last being the bonus drawn at row R-1
    lanes, R, V = 4, 8, 50000
    key = (67,)
    z = inputs.logits_f32(key, lanes * R, V)
    u = inputs.uniforms(key, lanes * R)
    toks = O.row_draws(z, 0.8, 32, 0.95, u)
    d = toks.reshape(lanes, R)[:, : R - 1].astype(np.int32)
    say("case point-mass full acceptance")
    got = run_gpu(z, lanes, R, 0.8, 32, 0.95, u, draft=d)
    clear = check_rows(z, 0.8, 32, 0.95, u, got)
    ok = lanes_clear_point_mass(clear, toks, d, lanes, R)
    for l in ok:
        assert got["acc"][l] == R and np.array_equal(got["commit"][l], toks[l * R:(l + 1) * R])
    assert len(ok) >= lanes - 1


def _close_drafts(key, z, lanes, R, t, k, tp, under=False):
    """Draft distributions close to the target's: its 16 most likely kept
    candidates with probabilities perturbed by up to 30 % and renormalised
    (about half of the drafts are accepted), or, with `under`, scaled by
    0.85-1.0 without renormalising (q <= p: every draft is accepted and the
    scan ends in the bonus draw). Draft tokens are drawn from them."""
    g = np.random.default_rng([71, *key])
    q_ids = np.full((lanes, R - 1, 16), -1, dtype=np.int32)
    q_p = np.zeros((lanes, R - 1, 16), dtype=np.float32)
    d = np.zeros((lanes, R - 1), dtype=np.int32)
    for l in range(lanes):
        for j in range(R - 1):
            ids, p = O.target_distribution(z[l * R + j], t, k, tp)
            n = min(16, ids.size)
            if under:
                w = (p[:n] * g.uniform(0.85, 1.0, size=n)).astype(np.float32)
            else:
                w = p[:n] * g.uniform(0.7, 1.3, size=n)
                w = (w / w.sum()).astype(np.float32)
            q_ids[l, j, :n] = ids[:n]
            q_p[l, j, :n] = w
            d[l, j] = ids[g.choice(n, p=w.astype(np.float64) / w.astype(np.float64).sum())]
    return (q_ids, q_p), d


@pytest.mark.parametrize("under", [False, True])
@pytest.mark.parametrize("t,k,tp", [(1.0, 32, 1.0), (0.7, 16, 0.9), (0.25, 8, 0.99)])
def test_speculative_sampling_close_draft(t, k, tp, under):
    lanes, R, V = 4, 8, 40000
    key = (73, int(t * 100), k)
    z = inputs.logits_f32(key, lanes * R, V)
    ud = inputs.uniforms(key, lanes * R)
    ua = inputs.uniforms(key + (1,), lanes * R)
    q, d = _close_drafts(key, z, lanes, R, t, k, tp, under)
    say(f"case speculative close draft T={t} top_k={k} top_p={tp} q<=p {under}")
    got = run_gpu(z, lanes, R, t, k, tp, ud, draft=d, q=q, u_accept=ua)
    check_rows(z, t, k, tp, ud, got)
    compared = 0
    for l in range(lanes):
        dists = [O.target_distribution(z[l * R + j], t, k, tp) for j in range(R)]
        if any(count_margin(z[r], t, k, tp) <= EPS for r in range(l * R, l * R + R)):
            continue
        if not spec_lane_clear(dists, d[l], q[0][l], q[1][l], ua[l * R:(l + 1) * R], ud[l * R:(l + 1) * R]):
            continue
        a, c = O.spec_accept(dists, d[l], q[0][l], q[1][l], ua[l * R:(l + 1) * R], ud[l * R:(l + 1) * R])
        assert got["acc"][l] == a and np.array_equal(got["commit"][l], c), (l, got["acc"][l], a)
        if under:
            assert a == R
        compared += 1
    say(f"  lanes compared {compared}/{lanes}, accept {got['acc'].tolist()}")
    assert compared >= lanes - 1


def test_full_vocabulary_point_mass_m32():
    lanes, R, V = 4, 8, 248320
    say(f"case point-mass full vocabulary lanes={lanes} R={R} V={V}")
    key = (47,)
    z = inputs.logits_f32(key, lanes * R, V)
    u = inputs.uniforms(key, lanes * R)
    d = point_mass_drafts(key, z, lanes, R, 1.0, 32, 0.95, u)
    got = run_gpu(z, lanes, R, 1.0, 32, 0.95, u, draft=d)
    clear = check_rows(z, 1.0, 32, 0.95, u, got)
    toks = O.row_draws(z, 1.0, 32, 0.95, u)
    want_len, want_commit = O.point_mass_accept(toks.reshape(lanes, R), d)
    for l in lanes_clear_point_mass(clear, toks, d, lanes, R):
        assert got["acc"][l] == want_len[l] and np.array_equal(got["commit"][l], want_commit[l])
    assert len(clear) >= lanes * R - 1


def test_adversarial_candidates_in_one_lane():
    # the 32 largest logits of a chunk all sit in one lane's stride (the
    # worst case for the lane-maxima bound: 32 merge rounds), and a row whose
    # logits increase with the id
    lanes, R, V = 1, 2, 16384
    z = inputs.logits_f32((53,), lanes * R, V) * np.float32(0.1)
    z[0, 7 + 64 * np.arange(32)] = np.linspace(5, 9, 32, dtype=np.float32)
    z[1] = np.linspace(-3, 3, V, dtype=np.float32)
    u = inputs.uniforms((53,), lanes * R)
    say("case adversarial lists")
    got = run_gpu(z, lanes, R, 1.0, 32, 1.0, u, draft=np.array([[0]], np.int32))
    check_rows(z, 1.0, 32, 1.0, u, got)
    assert got["cand"][0][:32].tolist() == (7 + 64 * np.arange(32))[::-1].tolist()
    assert got["cand"][1][:32].tolist() == list(range(V - 1, V - 33, -1))


def test_head_logits_then_sample():
    # the end of the pass at nonzero temperature: the vocabulary head writes
    # fp32 logits and the sampled verify reads them. The oracle starts from
    # its own fp64 product; where the fp32 logits of two candidates lie within
    # the accumulation error of each other the order is the tie class.
    from gpu_helpers import to_dev_bf16, to_dev_u8
    torch, dev = _dev()
    lanes, R, V, K, t, k, tp = 2, 8, 20000, 1024, 1.0, 32, 0.9
    M = lanes * R
    key = (79,)
    h = inputs.x_bf16(key, M, K)
    codes, scales = inputs.nvfp4_weights(key, V, K)
    ref = O.gemm_nvfp4(h, codes, scales, 1.0)
    u = inputs.uniforms(key, M)
    toks_ref = O.row_draws(ref, t, k, tp, u)
    d = inputs.drafts(key, np.where(toks_ref >= 0, toks_ref, 0).reshape(lanes, R), V)
    say(f"case head logits -> sampled verify M={M} V={V} K={K}")
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    lg = torch.empty((M, V), dtype=torch.float32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    al = torch.empty(lanes, dtype=torch.int32, device=dev)
    ops.vq_lmhead_argmax_accept(to_dev_bf16(h), w, 1.0, V, _i32(d), lanes, R, am, al, logits_out=lg,
                                workspace=ops.workspace(ops.VQ_OP_LMHEAD, M, V, K, dev))
    out = dict(tok=torch.empty(M, dtype=torch.int32, device=dev), acc=torch.empty(lanes, dtype=torch.int32, device=dev),
               cand=torch.empty((M, 32), dtype=torch.int32, device=dev),
               prob=torch.empty((M, 32), dtype=torch.float32, device=dev))
    ops.vq_sample_accept(lg, lanes, R, t, k, tp, _f32(u), out["acc"], draft=_i32(d), token_out=out["tok"],
                         cand_out=out["cand"], prob_out=out["prob"],
                         workspace=ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev))
    torch.cuda.synchronize()
    got = {k_: v.cpu().numpy() for k_, v in out.items()}
    # the GEMM's own bound (asserted by the GEMM tests): every fp32 logit is
    # within 1e-5 * max|logit| of the fp64 one. Two candidates closer than
    # twice that may swap; probabilities move by at most ~4x that / T.
    tol_z = 1e-5 * float(np.max(np.abs(ref)))
    assert float(np.max(np.abs(lg.cpu().numpy() - ref))) <= tol_z
    tol_p = 4 * tol_z / t
    clear = 0
    for r in range(M):
        top = np.sort(ref[r])[::-1][: k + 1]
        if np.min(-np.diff(top)) <= 2 * tol_z or count_margin(ref[r], t, k, tp) <= tol_p:
            continue
        ids, p = O.target_distribution(ref[r], t, k, tp)
        assert np.array_equal(got["cand"][r][: ids.size], ids), r
        np.testing.assert_allclose(got["prob"][r][: ids.size], p, rtol=0, atol=tol_p)
        if draw_margin(p, float(u[r])) > tol_p:
            assert got["tok"][r] == toks_ref[r], r
            clear += 1
    say(f"  rows compared {clear}/{M}")
    assert clear >= M // 2  # the rest sit in the tie class (about one row in six here)


def test_repeat_calls_reuse_workspace_and_are_deterministic():
    torch, dev = _dev()
    lanes, R, V = 4, 8, 30000
    z = inputs.logits_f32((59,), lanes * R, V)
    u = inputs.uniforms((59,), lanes * R)
    ua = inputs.uniforms((59, 1), lanes * R)
    q, d = _spec_inputs((59,), z, lanes, R, 0.9, 32, 0.9)
    ws = ops.workspace(ops.VQ_OP_SAMPLE, lanes * R, V, 0, dev)
    say("case repeat calls")
    first = run_gpu(z, lanes, R, 0.9, 32, 0.9, u, draft=d, q=q, u_accept=ua, ws=ws)
    for _ in range(5):
        again = run_gpu(z, lanes, R, 0.9, 32, 0.9, u, draft=d, q=q, u_accept=ua, ws=ws)
        for key_ in first:
            assert np.array_equal(first[key_], again[key_]), key_
        pm = run_gpu(z, lanes, R, 0.9, 32, 0.9, u, draft=d, ws=ws)  # other rule, same workspace
        assert np.array_equal(pm["tok"], first["tok"])


def test_distribution_equivalence_on_gpu():
    # the pages' check: draws from the GPU follow the target distribution at
    # temperature 1, top_k 32 (chi-square against the oracle's probabilities)
    from scipy import stats
    torch, dev = _dev()
    lanes, R, V = 4, 8, 4096
    M = lanes * R
    row = inputs.logits_f32((61,), 1, V)[0] * np.float32(0.6)
    z = np.repeat(row[None], M, axis=0)
    ids, p = O.target_distribution(row, 1.0, 32, 1.0)
    ws = ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev)
    lg = _f32(z)
    tok = torch.empty(M, dtype=torch.int32, device=dev)
    acc = torch.empty(lanes, dtype=torch.int32, device=dev)
    d = _i32(np.zeros((lanes, R - 1)))
    draws = []
    say("case distribution equivalence (600 calls x 32 rows)")
    u_all = _f32(inputs.uniforms((61,), 600, M))
    for c in range(600):
        ops.vq_sample_accept(lg, lanes, R, 1.0, 32, 1.0, u_all[c], acc, draft=d, token_out=tok, workspace=ws)
        draws.append(tok.clone())
    got = torch.cat(draws).cpu().numpy()
    obs = np.array([(got == t).sum() for t in ids])
    assert obs.sum() == got.size
    pv = stats.chisquare(obs, got.size * p).pvalue
    say(f"  {got.size} draws over {ids.size} candidates, chi-square p-value {pv:.3g}")
    assert pv > 1e-4


def test_binding_rejections():
    torch, dev = _dev()
    lg = torch.zeros((8, 100), dtype=torch.float32, device=dev)
    u = torch.zeros(8, dtype=torch.float32, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        ops.vq_sample_accept(lg, 2, 8, 1.0, 32, 1.0, u, acc)
    with pytest.raises(ops.VerifyError):  # top_k above 32
        ops.vq_sample_accept(lg, 1, 8, 1.0, 40, 1.0, u, acc, draft=torch.zeros(7, dtype=torch.int32, device=dev),
                             workspace=ops.workspace(ops.VQ_OP_SAMPLE, 8, 100, 0, dev))
    with pytest.raises(ops.VerifyError):  # no workspace
        ops.vq_sample_accept(lg, 1, 8, 1.0, 32, 1.0, u, acc, draft=torch.zeros(7, dtype=torch.int32, device=dev))


def test_graph_replay_matches_eager():
    # the sampler inside a captured graph, replayed with eager calls on the
    # same workspace in between: every replay equals the eager result (the
    # per-lane counters are reset by the lane's last row each time)
    torch, dev = _dev()
    lanes, R, V = 4, 8, 40000
    M = lanes * R
    z = inputs.logits_f32((83,), M, V)
    u = inputs.uniforms((83,), M)
    ua = inputs.uniforms((83, 1), M)
    q, d = _spec_inputs((83,), z, lanes, R, 0.8, 32, 0.9)
    ws = ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev)
    say("case graph replay")
    eager = run_gpu(z, lanes, R, 0.8, 32, 0.9, u, draft=d, q=q, u_accept=ua, ws=ws)
    lg, uu, uaa = _f32(z), _f32(u), _f32(ua)
    dd, qi, qp = _i32(d), _i32(q[0]), _f32(q[1])
    tok = torch.full((M,), -7, dtype=torch.int32, device=dev)
    acc = torch.full((lanes,), -7, dtype=torch.int32, device=dev)
    commit = torch.full((lanes, R), -7, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ops.vq_sample_accept(lg, lanes, R, 0.8, 32, 0.9, uu, acc, draft=dd, draft_ids=qi, draft_probs=qp,
                                 u_accept=uaa, token_out=tok, commit_out=commit, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    for i in range(4):
        tok.fill_(-7)
        acc.fill_(-7)
        commit.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), eager["tok"]), i
        assert np.array_equal(acc.cpu().numpy(), eager["acc"]), i
        assert np.array_equal(commit.cpu().numpy(), eager["commit"]), i
        run_gpu(z, lanes, R, 0.8, 32, 0.9, u, draft=d, ws=ws)  # eager work between replays
