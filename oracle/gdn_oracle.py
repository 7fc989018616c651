"""Plain fp64 CPU oracle of the Gated DeltaNet state stream of the verify pass:
the delta recurrence over a lane's verify rows, written out of place from one
parity slot to the other, and the commit re-scan over the accepted rows only.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call it. It shares no code
with the HIP library and imports nothing from it.

What the pages fix:
  [P2] "Beating Splash on an M5 Max: where the tokens per second actually
       were", section "What actually moved the needle": the fused GDN step
       writes the state out of place from parity buffer A to B; a fully
       accepted round flips the parity; a partly rejected round re-scans only
       the committed rows from the untouched previous parity; for every
       possible number of kept tokens the state must equal a reference scan
       exactly.
  [P4] "lithos-metal: per-layer megakernels for Qwen3.8-27B on an M5 Max, and
       where the 200 tok/s comes from", section "What one token costs the
       bus": the state is fp32 with shape (v_heads, dk, dv) = (48, 128, 128)
       per GDN layer, 48 layers, read and written once per pass; section "How
       DSpark is wired in": the verify pass reads one slot and writes the
       other, and the commit pass recomputes the recurrence from the slot the
       verify read over the committed tokens only (their count is what the
       accept scan wrote).

What the pages leave open (each reading is listed in the design doc):
  * The recurrence itself. The pages name the "delta recurrence" of Gated
    DeltaNet but print no equation. The reading is the gated delta rule as
    published in S. Yang, J. Kautz, A. Hatamizadeh, "Gated Delta Networks:
    Improving Mamba2 with Delta Rule" (ICLR 2025), written in the (dk, dv)
    layout of [P4]: per value head, with decay a_t in (0, 1] and write
    strength b_t,
        S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
        o_t = S_t^T q_t                      (the updated state is read)
    q_t, k_t in R^dk, v_t, o_t in R^dv, S in R^{dk x dv}.
  * Gates, convolution and norms. a_t, b_t and the (already convolved and
    normalised) q_t, k_t, v_t are inputs; the 4-tap convolution window, the
    Q/K norm and the gate formulas are not part of this stream.
  * Head sharing. With Hk key heads and H value heads (Hk divides H), value
    head h reads the query and key of key head h // (H / Hk): consecutive
    value heads share a key head.
  * Commit count. The commit for a lane re-scans the first c rows, c = the
    lane's accept length clamped to [0, T]; when c = T the verify's output
    slot already holds that state and nothing is recomputed.

Array layouts (B independent entries, e.g. layers x lanes, entry-major):
  state [B][H][dk][dv]; q, k [B][T][Hk][dk]; v, o [B][T][H][dv];
  a, b [B][T][H].
"""
from __future__ import annotations

import numpy as np

__all__ = ["gdn_step", "gdn_scan", "gdn_commit"]


def gdn_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, a: float, b: float):
    """One row of the gated delta rule for one value head (fp64).

    S (dk, dv) is the state before the row; returns (S_t, o_t). The update is
    the published form a (I - b k k^T) S + b k v^T: first the decayed state
    a S, then the delta correction along k towards v.
    """
    S = np.asarray(S, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kS = k @ S                          # k^T S, shape (dv,)
    S_new = a * (S - b * np.outer(k, kS)) + b * np.outer(k, v)
    o = S_new.T @ q                     # read of the updated state
    return S_new, o


def gdn_scan(state, q, k, v, a, b, rows=None, keep_states=False):
    """The recurrence over the first `rows[e]` rows of every entry e (default:
    all T rows), from `state`.

    Returns (state_after, o) with o[e, t] = 0 for rows not scanned; with
    keep_states=True also the list of per-row states (states[e][t] is the
    state after rows 0..t of entry e).
    """
    state = np.asarray(state, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    B, H, dk, dv = state.shape
    T, Hk = q.shape[1], q.shape[2]
    assert q.shape == (B, T, Hk, dk) and k.shape == q.shape
    assert v.shape == (B, T, H, dv) and a.shape == (B, T, H) and b.shape == (B, T, H)
    assert H % Hk == 0
    group = H // Hk
    out = state.copy()
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    per_row = [[None] * T for _ in range(B)] if keep_states else None
    for e in range(B):
        n = T if rows is None else int(rows[e])
        for h in range(H):
            kh = h // group
            S = state[e, h]
            for t in range(n):
                S, o[e, t, h] = gdn_step(S, q[e, t, kh], k[e, t, kh], v[e, t, h], a[e, t, h], b[e, t, h])
                if keep_states:
                    if per_row[e][t] is None:
                        per_row[e][t] = np.zeros((H, dk, dv))
                    per_row[e][t][h] = S
            out[e, h] = S
    if keep_states:
        return out, o, per_row
    return out, o


def gdn_commit(slot_read, slot_written, q, k, v, a, b, accept_len, lanes: int):
    """The commit pass ([P4] "How DSpark is wired in"): entry e belongs to lane
    e % lanes; c = clamp(accept_len[lane], 0, T). Entries with c = T keep the
    verify's output `slot_written`; the others get the scan of their first c
    rows from `slot_read` (c = 0 copies the read slot). Returns the new
    contents of the written slot."""
    slot_written = np.asarray(slot_written, dtype=np.float64).copy()
    B, T = np.asarray(q).shape[:2]
    counts = [min(max(int(accept_len[e % lanes]), 0), T) for e in range(B)]
    redo = [e for e in range(B) if counts[e] < T]
    if redo:
        sub = lambda x: np.asarray(x)[redo]  # noqa: E731
        st, _ = gdn_scan(sub(slot_read), sub(q), sub(k), sub(v), sub(a), sub(b), rows=[counts[e] for e in redo])
        slot_written[redo] = st
    return slot_written
