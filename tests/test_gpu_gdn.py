"""GPU parity of the Gated DeltaNet state stream (vq_gdn_verify, vq_gdn_commit)
against the fp64 oracle, through the C ABI.

Recurrence: the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta
Networks: Improving Mamba2 with Delta Rule", ICLR 2025) in the (dk, dv) layout
of "lithos-metal ...", section "What one token costs the bus"; double-buffered
commit: "Beating Splash on an M5 Max ...", section "What actually moved the
needle" (for every number of kept tokens the state must equal a reference scan
exactly), and "lithos-metal ...", section "How DSpark is wired in".

Gate: max|gpu - oracle| / max|oracle| <= GDN_TOL(T) for the state and the
outputs, where GDN_TOL(T) = 2 T (dk + 2) 2^-24: each row adds one fp32 rounding
of a dk-term dot product and two of the update to every state element, and the
errors of T rows add up. Rollback: the commit's state is bitwise the state a
verify call over the same kept rows writes.
"""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import rel_err, say, torch_dev

pytestmark = pytest.mark.gpu


def gdn_tol(T):
    return 2 * T * (128 + 2) * 2.0 ** -24


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def _dev(arrays):
    torch, dev = torch_dev()
    return [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in arrays]


def _check(gpu, ref, T, what):
    e = rel_err(gpu, ref)
    say(f"  parity {what}: max|gpu-oracle|/max|oracle| = {e:.3e} (gate {gdn_tol(T):.3e})")
    assert e <= gdn_tol(T), (what, e)


@pytest.mark.parametrize("B,T,H,Hk", [(1, 8, 48, 16), (2, 1, 4, 4), (3, 5, 6, 2), (4, 16, 3, 1), (2, 8, 2, 1),
                                      (4, 16, 48, 16)])
def test_gdn_verify_matches_oracle(B, T, H, Hk):
    say(f"case: gdn verify B={B} T={T} H={H} Hk={Hk}")
    torch, dev = torch_dev()
    host = inputs.gdn_inputs((700, B, T, H, Hk), B, T, H, Hk)
    st_ref, o_ref = O.gdn_scan(*host)
    state, q, k, v, a, b = _dev(host)
    out = torch.empty_like(state)
    o = torch.empty_like(v)
    _ops().vq_gdn_verify(state, out, q, k, v, a, b, o)
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), st_ref, T, "state")
    _check(o.cpu().numpy(), o_ref, T, "outputs")
    assert torch.equal(state.cpu(), torch.from_numpy(host[0])), "state_in was written"


def test_gdn_writes_nothing_outside_its_outputs():
    torch, dev = torch_dev()
    B, T, H, Hk = 2, 3, 4, 2
    host = inputs.gdn_inputs((701,), B, T, H, Hk)
    state, q, k, v, a, b = _dev(host)
    n_s, n_o = state.numel(), v.numel()
    pad = 4096
    s_buf = torch.full((n_s + 2 * pad,), 7.0, device=dev)
    o_buf = torch.full((n_o + 2 * pad,), 7.0, device=dev)
    out = s_buf[pad:pad + n_s].view(state.shape)
    o = o_buf[pad:pad + n_o].view(v.shape)
    _ops().vq_gdn_verify(state, out, q, k, v, a, b, o)
    acc = torch.tensor([1, 2], dtype=torch.int32, device=dev)
    _ops().vq_gdn_commit(state, out, q, k, v, a, b, acc, lanes=2)
    torch.cuda.synchronize()
    for buf, n in ((s_buf, n_s), (o_buf, n_o)):
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)


def test_gdn_rows_do_not_depend_on_batch():
    torch, dev = torch_dev()
    B, T, H, Hk = 5, 8, 6, 3
    state, q, k, v, a, b = _dev(inputs.gdn_inputs((702,), B, T, H, Hk))
    out = torch.empty_like(state)
    o = torch.empty_like(v)
    _ops().vq_gdn_verify(state, out, q, k, v, a, b, o)
    for e in range(B):
        sl = lambda x: x[e:e + 1].contiguous()  # noqa: E731
        out1 = torch.empty_like(sl(state))
        o1 = torch.empty_like(sl(v))
        _ops().vq_gdn_verify(sl(state), out1, sl(q), sl(k), sl(v), sl(a), sl(b), o1)
        torch.cuda.synchronize()
        assert torch.equal(out1[0], out[e]) and torch.equal(o1[0], o[e]), e


def _verify_rows(state, q, k, v, a, b, c):
    """vq_gdn_verify over the first c rows (c >= 1) of every entry."""
    torch, _ = torch_dev()
    cut = lambda x: x[:, :c].contiguous()  # noqa: E731
    out = torch.empty_like(state)
    _ops().vq_gdn_verify(state, out, cut(q), cut(k), cut(v), cut(a), cut(b))
    return out


@pytest.mark.parametrize("lanes,layers", [(1, 3), (2, 2), (4, 1)])
def test_gdn_commit_rollback_is_bitwise_for_every_kept_count(lanes, layers):
    # every accept length of every lane (and out-of-range ones, clamped):
    # lanes that kept all T rows keep the verify's slot, the others get the
    # re-scan of their kept rows, bitwise what a verify over them writes
    torch, dev = torch_dev()
    B, T, H, Hk = lanes * layers, 8, 6, 2
    host = inputs.gdn_inputs((703, lanes), B, T, H, Hk)
    state, q, k, v, a, b = _dev(host)
    verified = torch.empty_like(state)
    _ops().vq_gdn_verify(state, verified, q, k, v, a, b)
    ref_rows = {c: _verify_rows(state, q, k, v, a, b, c) for c in range(1, T + 1)}
    torch.cuda.synchronize()
    patterns = [[(c + l) % (T + 1) for l in range(lanes)] for c in range(T + 1)] + [[T + 3] * lanes, [-1] * lanes]
    for acc in patterns:
        say(f"case: gdn commit lanes={lanes} layers={layers} accept={acc}")
        slot = verified.clone()
        acc_d = torch.tensor(acc, dtype=torch.int32, device=dev)
        _ops().vq_gdn_commit(state, slot, q, k, v, a, b, acc_d, lanes=lanes)
        torch.cuda.synchronize()
        for e in range(B):
            c = min(max(acc[e % lanes], 0), T)
            want = verified[e] if c == T else (state[e] if c == 0 else ref_rows[c][e])
            assert torch.equal(slot[e], want), (acc, e, c)
    # the committed states against the oracle's commit
    acc = [(3 + l) % (T + 1) for l in range(lanes)]
    slot = verified.clone()
    _ops().vq_gdn_commit(state, slot, q, k, v, a, b, torch.tensor(acc, dtype=torch.int32, device=dev), lanes=lanes)
    torch.cuda.synchronize()
    st_ref, _ = O.gdn_scan(*host)
    want = O.gdn_commit(host[0], st_ref, *host[1:], acc, lanes)
    _check(slot.cpu().numpy(), want, T, "committed state")


def test_gdn_full_pass_state_stream_sampled():
    # the pass's shape: 48 GDN layers x 1 lane, 48 value heads sharing 16 key
    # heads, 8 verify rows; one verify call per layer and one commit call over
    # all layers with accept length 3, checked against the oracle on sampled
    # layers and bitwise against a 3-row verify everywhere
    torch, dev = torch_dev()
    L, T, H, Hk = 48, 8, 48, 16
    state, q, k, v, a, b = inputs.device_gdn_inputs((704,), L, T, H, Hk, dev)
    slot = torch.empty_like(state)
    o = torch.empty_like(v)
    for layer in range(L):
        sl = slice(layer, layer + 1)
        _ops().vq_gdn_verify(state[sl], slot[sl], q[sl], k[sl], v[sl], a[sl], b[sl], o[sl])
    acc = torch.tensor([3], dtype=torch.int32, device=dev)
    verified = slot.clone()
    _ops().vq_gdn_commit(state, slot, q, k, v, a, b, acc, lanes=1)
    three = _verify_rows(state, q, k, v, a, b, 3)
    torch.cuda.synchronize()
    assert torch.equal(slot, three)
    for layer in (0, 17, 47):
        say(f"case: gdn full-size layer {layer}")
        host = [x[layer:layer + 1].cpu().numpy() for x in (state, q, k, v, a, b)]
        st_ref, o_ref = O.gdn_scan(*host)
        _check(verified[layer:layer + 1].cpu().numpy(), st_ref, T, f"layer {layer} state")
        _check(o[layer:layer + 1].cpu().numpy(), o_ref, T, f"layer {layer} outputs")
        st3, _ = O.gdn_scan(*host, rows=[3])
        _check(slot[layer:layer + 1].cpu().numpy(), st3, 3, f"layer {layer} committed")


def test_gdn_graph_replay_matches_eager():
    torch, dev = torch_dev()
    B, T, H, Hk = 4, 8, 48, 16
    state, q, k, v, a, b = inputs.device_gdn_inputs((705,), B, T, H, Hk, dev)
    acc = torch.tensor([2, 8], dtype=torch.int32, device=dev)
    ops = _ops()
    ye, oe = torch.empty_like(state), torch.empty_like(v)
    ops.vq_gdn_verify(state, ye, q, k, v, a, b, oe)
    ops.vq_gdn_commit(state, ye, q, k, v, a, b, acc, lanes=2)
    torch.cuda.synchronize()
    eager_s, eager_o = ye.clone(), oe.clone()
    y, o = torch.zeros_like(state), torch.zeros_like(v)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ops.vq_gdn_verify(state, y, q, k, v, a, b, o)
            ops.vq_gdn_commit(state, y, q, k, v, a, b, acc, lanes=2)
    torch.cuda.current_stream().wait_stream(st)
    for i in range(4):
        y.zero_()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager_s) and torch.equal(o, eager_o), i
        ops.vq_gdn_verify(state, ye, q, k, v, a, b, oe)
        torch.cuda.synchronize()


def test_head_accept_length_drives_the_commit_on_device():
    # the accept lengths the vocabulary head writes on the device are the
    # counts the GDN commit reads: the two calls chain with no host round
    # trip, and the committed state equals the oracle's commit at the
    # oracle's accept lengths (seeded inputs without tie-class rows)
    from tests.gpu_helpers import to_dev_bf16, to_dev_u8
    torch, dev = torch_dev()
    ops = _ops()
    lanes, R, V, K = 2, 8, 4096, 512
    M = lanes * R
    hb = inputs.x_bf16((710,), M, K)
    codes, scales = inputs.nvfp4_weights((710,), V, K)
    logits = O.gemm_nvfp4(hb, codes, scales, 1.0)
    assert O.top2_gap(logits).min() > 1e-3
    am = O.argmax_lowest(logits).reshape(lanes, R)
    dr = inputs.drafts((710,), am, V)
    acc_ref, _ = O.greedy_accept(am, dr)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    am_d = torch.empty(M, dtype=torch.int32, device=dev)
    acc_d = torch.full((lanes,), -7, dtype=torch.int32, device=dev)
    layers, T, H, Hk = 3, R, 6, 2
    host = inputs.gdn_inputs((711,), layers * lanes, T, H, Hk)
    state, q, k, v, a, b = _dev(host)
    slot = torch.empty_like(state)
    ops.vq_gdn_verify(state, slot, q, k, v, a, b)
    ops.vq_lmhead_argmax_accept(to_dev_bf16(hb), w, 1.0, V, torch.from_numpy(dr).to(dev), lanes, R, am_d, acc_d,
                                workspace=ops.workspace(ops.VQ_OP_LMHEAD, M, V, K, dev))
    ops.vq_gdn_commit(state, slot, q, k, v, a, b, acc_d, lanes=lanes)
    torch.cuda.synchronize()
    assert np.array_equal(acc_d.cpu().numpy(), acc_ref), (acc_d.cpu().numpy(), acc_ref)
    st_ref, _ = O.gdn_scan(*host)
    want = O.gdn_commit(host[0], st_ref, *host[1:], acc_ref, lanes)
    _check(slot.cpu().numpy(), want, T, "commit driven by the head's accept lengths")


def _min_decision_margin(z, u, t, k, tp):
    # fp64 margins of the top_p cut and of the inverse-CDF draw per row
    out = np.inf
    for r in range(z.shape[0]):
        ids = O.candidate_order(z[r])[:k]
        w = np.exp((z[r][ids].astype(np.float64) - z[r][ids[0]]) / t)
        out = min(out, float(np.min(np.abs(np.cumsum(w) / w.sum() - tp))))
        _, p = O.target_distribution(z[r], t, k, tp)
        if len(p) > 1:
            out = min(out, float(np.min(np.abs(np.cumsum(p)[:-1] - u[r]))))
    return out


def test_sampled_accept_length_drives_the_commit_on_device():
    # the point-mass sampled verify writes its accept lengths on the device and
    # the GDN commit reads them: lane 0 keeps 4 rows (re-scanned), lane 1 all 8
    # (its slot is kept); seeded inputs whose decisions all clear the fp32/fp64
    # tie margin, so the accept lengths are exact
    torch, dev = torch_dev()
    ops = _ops()
    lanes, R, V = 2, 8, 8192
    M = lanes * R
    z = inputs.logits_f32((712,), M, V)
    u = inputs.uniforms((712,), M)
    assert _min_decision_margin(z, u, 1.0, 32, 0.95) > 1e-5
    toks = O.row_draws(z, 1.0, 32, 0.95, u).reshape(lanes, R)
    dr = toks[:, :R - 1].copy().astype(np.int32)
    dr[0, 3] = (dr[0, 3] + 1) % V
    acc_ref, _ = O.point_mass_accept(toks, dr)
    assert list(acc_ref) == [4, 8]
    layers, T, H, Hk = 2, R, 6, 2
    host = inputs.gdn_inputs((713,), layers * lanes, T, H, Hk)
    state, q, k, v, a, b = _dev(host)
    slot = torch.empty_like(state)
    ops.vq_gdn_verify(state, slot, q, k, v, a, b)
    acc_d = torch.full((lanes,), -7, dtype=torch.int32, device=dev)
    ops.vq_sample_accept(torch.from_numpy(z).to(dev), lanes, R, 1.0, 32, 0.95, torch.from_numpy(u).to(dev), acc_d,
                         draft=torch.from_numpy(dr).to(dev), workspace=ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev))
    ops.vq_gdn_commit(state, slot, q, k, v, a, b, acc_d, lanes=lanes)
    torch.cuda.synchronize()
    assert np.array_equal(acc_d.cpu().numpy(), acc_ref)
    st_ref, _ = O.gdn_scan(*host)
    want = O.gdn_commit(host[0], st_ref, *host[1:], acc_ref, lanes)
    _check(slot.cpu().numpy(), want, T, "commit driven by the sampled accept lengths")
