"""Pins of the Gated DeltaNet state-stream oracle.

The recurrence is the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated
Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025) in the
(dk, dv) state layout of "lithos-metal ...", section "What one token costs
the bus"; the double-buffered commit follows "Beating Splash on an M5 Max
...", section "What actually moved the needle", and "lithos-metal ...",
section "How DSpark is wired in".

Each pin checks a property the rule fixes without restating its formula:
pure decay when nothing is written, the delta rule's read-back of the value
written at a unit key, the projection form for orthonormal keys, the split of
one row into the key direction and its orthogonal complement, linearity in
(state, values), head sharing, and the rollback identity (re-scanning the
first c rows gives the state the full scan had after c rows).
"""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs


def _unit(g, *shape):
    x = g.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_no_write_is_pure_decay():
    B, T, H, Hk = 2, 5, 3, 3
    state, q, k, v, a, b = inputs.gdn_inputs((600,), B, T, H, Hk)
    b = np.zeros_like(b)
    st, o = O.gdn_scan(state, q, k, v, a, b)
    decay = np.cumprod(a.astype(np.float64), axis=1)  # [B][T][H]
    want = state.astype(np.float64) * decay[:, -1, :, None, None]
    assert np.allclose(st, want, rtol=1e-13, atol=0)
    for t in range(T):
        want_o = np.einsum("ehij,ehi->ehj", state.astype(np.float64), q[:, t].astype(np.float64)) * decay[:, t, :, None]
        assert np.allclose(o[:, t], want_o, rtol=1e-12, atol=1e-14)


def test_unit_key_full_write_reads_back_the_value():
    # a = 1, b = 1, |k| = 1: after the row the state maps k to v exactly,
    # and the output (which reads the updated state) with q = k is v
    g = np.random.default_rng(601)
    B, T, H = 1, 6, 2
    state = g.standard_normal((B, H, 128, 128))
    k = _unit(g, B, T, H, 128)
    v = g.standard_normal((B, T, H, 128))
    one = np.ones((B, T, H))
    st, o, per_row = O.gdn_scan(state, k, k, v, one, one, keep_states=True)
    for t in range(T):
        for h in range(H):
            S = per_row[0][t][h]
            assert np.allclose(S.T @ k[0, t, h], v[0, t, h], atol=1e-12)
    assert np.allclose(o, v, atol=1e-12)


def test_orthonormal_keys_project_out_and_write():
    # with a = b = 1 and orthonormal keys k_1..k_T the scan is the projection
    # (I - K K^T) S_0 + K V^T
    g = np.random.default_rng(602)
    T, dk, dv = 7, 128, 128
    Kmat, _ = np.linalg.qr(g.standard_normal((dk, T)))
    S0 = g.standard_normal((dk, dv))
    V = g.standard_normal((dv, T))
    k = Kmat.T[None, :, None, :]           # [1][T][1][dk]
    v = V.T[None, :, None, :]
    one = np.ones((1, T, 1))
    st, _ = O.gdn_scan(S0[None, None], k, k, v, one, one)
    want = (np.eye(dk) - Kmat @ Kmat.T) @ S0 + Kmat @ V.T
    assert np.allclose(st[0, 0], want, atol=1e-12)


@pytest.mark.parametrize("a,b", [(1.0, 0.3), (0.9, 1.0), (0.75, 0.5), (0.5, 0.0)])
def test_one_row_splits_into_key_direction_and_complement(a, b):
    # for unit k: directions orthogonal to k only decay (x^T S' = a x^T S), and
    # the key direction moves towards v: k^T S' = a (1 - b) k^T S + b v^T
    g = np.random.default_rng(603)
    dk, dv = 128, 128
    S = g.standard_normal((dk, dv))
    k = _unit(g, dk)
    v = g.standard_normal(dv)
    q = _unit(g, dk)
    S1, o = O.gdn_step(S, q, k, v, a, b)
    x = g.standard_normal((dk, 5))
    x -= np.outer(k, k @ x)                # orthogonal to k
    assert np.allclose(x.T @ S1, a * (x.T @ S), atol=1e-12)
    assert np.allclose(k @ S1, a * (1 - b) * (k @ S) + b * v, atol=1e-12)
    assert np.allclose(o, S1.T @ q, atol=1e-12)


def test_linear_in_state_and_values():
    B, T, H, Hk = 2, 4, 4, 2
    state, q, k, v, a, b = inputs.gdn_inputs((604,), B, T, H, Hk)
    full, of = O.gdn_scan(state, q, k, v, a, b)
    s0, o0 = O.gdn_scan(state, q, k, np.zeros_like(v), a, b)
    sv, ov = O.gdn_scan(np.zeros_like(state), q, k, v, a, b)
    assert np.allclose(full, s0 + sv, atol=1e-12)
    assert np.allclose(of, o0 + ov, atol=1e-12)


def test_value_heads_share_key_heads_in_consecutive_groups():
    B, T, H, Hk = 1, 3, 6, 2
    state, q, k, v, a, b = inputs.gdn_inputs((605,), B, T, H, Hk)
    idx = [0, 0, 0, 1, 1, 1]
    st, o = O.gdn_scan(state, q, k, v, a, b)
    st2, o2 = O.gdn_scan(state, q[:, :, idx], k[:, :, idx], v, a, b)
    assert np.array_equal(st, st2) and np.array_equal(o, o2)
    # a wrong grouping (h % Hk) would pair head 1 with key head 1
    st3, _ = O.gdn_scan(state, q[:, :, [0, 1, 0, 1, 0, 1]], k[:, :, [0, 1, 0, 1, 0, 1]], v, a, b)
    assert not np.allclose(st[0, 1], st3[0, 1])


def test_rollback_rescan_equals_the_full_scan_prefix():
    # every kept count c: scanning the first c rows from the read slot gives
    # bitwise the state the full scan held after c rows; continuing from it
    # over the rest gives the full scan
    B, T, H, Hk = 2, 8, 3, 1
    state, q, k, v, a, b = inputs.gdn_inputs((606,), B, T, H, Hk)
    full, o_full, per_row = O.gdn_scan(state, q, k, v, a, b, keep_states=True)
    for c in range(0, T + 1):
        st, o = O.gdn_scan(state, q, k, v, a, b, rows=[c] * B)
        for e in range(B):
            want = state[e].astype(np.float64) if c == 0 else per_row[e][c - 1]
            assert np.array_equal(st[e], want), c
        assert np.array_equal(o[:, :c], o_full[:, :c]) and not o[:, c:].any()
        rest, _ = O.gdn_scan(st, q[:, c:], k[:, c:], v[:, c:], a[:, c:], b[:, c:]) if c < T else (st, None)
        assert np.array_equal(rest, full), c


def test_commit_keeps_full_accepts_and_rescans_the_rest():
    lanes, layers, T, H, Hk = 3, 2, 8, 2, 1
    B = lanes * layers
    state, q, k, v, a, b = inputs.gdn_inputs((607,), B, T, H, Hk)
    written, _ = O.gdn_scan(state, q, k, v, a, b)
    marker = written.copy()
    for acc in ([8, 3, 1], [0, 9, -2], [5, 5, 5]):
        new = O.gdn_commit(state, marker, q, k, v, a, b, acc, lanes)
        for e in range(B):
            c = min(max(acc[e % lanes], 0), T)
            if c == T:
                assert np.array_equal(new[e], marker[e])
            else:
                want, _ = O.gdn_scan(state[e:e + 1], q[e:e + 1], k[e:e + 1], v[e:e + 1], a[e:e + 1], b[e:e + 1],
                                     rows=[c])
                assert np.array_equal(new[e], want[0])
                if c == 0:
                    assert np.array_equal(new[e], state[e].astype(np.float64))
