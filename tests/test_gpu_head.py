"""GPU parity of vq_lmhead_argmax_accept: vocabulary-head GEMM, per-row argmax
(bit-exact outside the tie class) and the greedy accept length / commit
tokens (integer, bit-exact unless a tie-class row decides them)."""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import TIE_GAP, check_f32, say, to_dev_bf16, to_dev_u8, torch_dev

pytestmark = pytest.mark.gpu


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def run_head(h_bits, codes, scales, ts, drafts, lanes, R, want_logits=True, ws=None, reps=1):
    torch, dev = torch_dev()
    ops = _ops()
    M, K = h_bits.shape
    V = codes.shape[0]
    h = to_dev_bf16(h_bits)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    d = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).to(dev) if R > 1 else None
    ws = ws if ws is not None else ops.workspace(ops.VQ_OP_LMHEAD, M, V, K, dev)
    outs = []
    for _ in range(reps):
        am = torch.full((M,), -7, dtype=torch.int32, device=dev)
        mx = torch.empty((M,), dtype=torch.float32, device=dev)
        al = torch.full((lanes,), -7, dtype=torch.int32, device=dev)
        cm = torch.full((lanes, R), -7, dtype=torch.int32, device=dev)
        lg = torch.empty((M, V), dtype=torch.float32, device=dev) if want_logits else None
        ops.vq_lmhead_argmax_accept(h, w, ts, V, d, lanes, R, am, al, maxlogit_out=mx, commit_out=cm,
                                    logits_out=lg, workspace=ws)
        torch.cuda.synchronize()
        outs.append(dict(argmax=am.cpu().numpy(), maxlogit=mx.cpu().numpy(), accept=al.cpu().numpy(),
                         commit=cm.cpu().numpy(), logits=lg.cpu().numpy() if lg is not None else None))
    return outs if reps > 1 else outs[0]


def check_head(out, logits_ref, drafts, lanes, R):
    am_ref = O.argmax_lowest(logits_ref)
    gap = O.top2_gap(logits_ref)
    tie = gap <= TIE_GAP
    say(f"  rows {len(am_ref)}, tie-class rows {int(tie.sum())}")
    ok = (out["argmax"] == am_ref) | tie
    assert ok.all(), (out["argmax"], am_ref, gap)
    valid = am_ref >= 0
    if valid.any():
        mref = np.array([logits_ref[r, am_ref[r]] for r in range(len(am_ref)) if valid[r]])
        check_f32(out["maxlogit"][valid], mref, what="max logit")
    assert np.all(np.isnan(out["maxlogit"][~valid]))
    a = am_ref.reshape(lanes, R)
    d = np.asarray(drafts).reshape(lanes, R - 1) if R > 1 else np.zeros((lanes, 0), np.int64)
    ln_ref, cm_ref = O.greedy_accept(a, d)
    g_ln, g_cm = O.greedy_accept(out["argmax"].reshape(lanes, R), d)
    assert np.array_equal(out["accept"], g_ln) and np.array_equal(out["commit"], g_cm)  # kernel's own scan
    tie_l = tie.reshape(lanes, R)
    for l in range(lanes):
        first_tie = int(np.argmax(tie_l[l])) if tie_l[l].any() else R
        if first_tie > ln_ref[l] - 1:
            assert out["accept"][l] == ln_ref[l], (l, out["accept"][l], ln_ref[l])
            assert np.array_equal(out["commit"][l], cm_ref[l])
        else:
            upto = first_tie
            assert np.array_equal(out["commit"][l][:upto], cm_ref[l][:upto])
    assert out["accept"].min() >= 1 and out["accept"].max() <= R


@pytest.mark.parametrize("lanes,R,V,K,ts", [
    (1, 8, 5000, 512, 1.0), (4, 8, 3001, 256, 0.5), (2, 5, 777, 1024, 1.0), (3, 1, 100, 128, 1.0),
    (1, 2, 64, 128, 2.0), (4, 3, 20000, 384, 1.0), (2, 4, 1111, 640, 1.0),
    # >= 2,048 tiles at M > 8: tile pairs, the second with an odd tile count
    (2, 8, 64 * 2050, 128, 1.0), (4, 8, 64 * 2049 - 11, 256, 0.5), (3, 8, 64 * 2049 - 11, 128, 1.0),
])
def test_head_random(lanes, R, V, K, ts):
    say(f"case: head lanes={lanes} R={R} V={V} K={K}")
    M = lanes * R
    key = (200, lanes, R, V, K)
    h = inputs.x_bf16(key, M, K)
    codes, scales = inputs.nvfp4_weights(key, V, K)
    logits_ref = O.gemm_nvfp4(h, codes, scales, ts)
    drafts = inputs.drafts(key, O.argmax_lowest(logits_ref).reshape(lanes, R), V) if R > 1 else np.zeros((lanes, 0), np.int32)
    out = run_head(h, codes, scales, ts, drafts, lanes, R)
    check_f32(out["logits"], logits_ref, what="logits")
    check_head(out, logits_ref, drafts, lanes, R)


def test_head_exact_ties_break_to_lowest_index():
    # integer-valued activations and weights: every logit is exact in fp32 in
    # any summation order, so duplicated weight rows give exact ties.
    lanes, R, V, K = 2, 8, 700, 128
    M = lanes * R
    g = np.random.default_rng(7)
    hv = g.integers(-3, 4, size=(M, K)).astype(np.float32)
    import torch
    h = torch.from_numpy(hv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes = g.integers(0, 256, size=(V, K // 2), dtype=np.uint8)
    scales = np.full((V, K // 16), 0x38, dtype=np.uint8)          # 1.0
    # copy each row's best weight row to two other columns (exact ties), and
    # row 9's best to columns 100, 400 and 650
    logits0 = O.gemm_nvfp4(h, codes, scales, 1.0)
    for r in range(M):
        best = int(O.argmax_lowest(logits0[r:r + 1])[0])
        for dup in (best + 1 + r, V - 1 - r):
            if 0 <= dup < V and dup != best:
                codes[dup] = codes[best]
    b9 = int(O.argmax_lowest(O.gemm_nvfp4(h, codes, scales, 1.0)[9:10])[0])
    codes[[100, 400, 650]] = codes[b9]
    logits_ref = O.gemm_nvfp4(h, codes, scales, 1.0)
    am = O.argmax_lowest(logits_ref)
    assert (O.top2_gap(logits_ref) == 0).sum() >= 1
    drafts = am.reshape(lanes, R)[:, : R - 1].copy()
    drafts[1, 3] = -5                                             # out of range: never matches
    out = run_head(h, codes, scales, 1.0, drafts, lanes, R)
    assert np.array_equal(out["argmax"], am)                      # exact ties -> lowest index
    assert list(out["accept"]) == [8, 4]
    assert np.array_equal(out["logits"], logits_ref.astype(np.float32))


def test_head_nan_rows_and_zero_logits():
    lanes, R, V, K = 1, 4, 300, 128
    M = lanes * R
    h = inputs.x_bf16((201,), M, K)
    h[1, :] = 0x7FC0           # NaN row -> every logit NaN -> argmax -1
    h[2, :] = 0x8000           # -0 row -> every logit is a zero -> argmax 0
    codes, scales = inputs.nvfp4_weights((201,), V, K)
    scales[17, 2] = 0x7F       # one NaN column
    logits_ref = O.gemm_nvfp4(h, codes, scales, 1.0)
    am = O.argmax_lowest(logits_ref)
    assert am[1] == -1 and am[2] == 0
    drafts = np.array([[am[0], am[1], 5]], dtype=np.int32)
    out = run_head(h, codes, scales, 1.0, drafts, lanes, R)
    assert out["argmax"][1] == -1 and np.isnan(out["maxlogit"][1])
    assert out["argmax"][2] == 0 and out["maxlogit"][2] == 0.0
    check_head(out, logits_ref, drafts, lanes, R)


def test_head_repeat_calls_reuse_workspace():
    torch, dev = torch_dev()
    ops = _ops()
    lanes, R, V, K = 4, 8, 9000, 512
    key = (202,)
    h = inputs.x_bf16(key, lanes * R, K)
    codes, scales = inputs.nvfp4_weights(key, V, K)
    logits_ref = O.gemm_nvfp4(h, codes, scales, 1.0)
    drafts = inputs.drafts(key, O.argmax_lowest(logits_ref).reshape(lanes, R), V)
    ws = ops.workspace(ops.VQ_OP_LMHEAD, lanes * R, V, K, dev)
    outs = run_head(h, codes, scales, 1.0, drafts, lanes, R, want_logits=False, ws=ws, reps=3)
    for o in outs[1:]:
        for k in ("argmax", "accept", "commit"):
            assert np.array_equal(o[k], outs[0][k])
        assert np.array_equal(o["maxlogit"], outs[0]["maxlogit"])
    check_head(outs[2], logits_ref, drafts, lanes, R)


def test_head_m8_vocab_248320_full_size():
    say("case: vocabulary head V=248320 K=5120 M=8 (device-generated weights)")
    torch, dev = torch_dev()
    lanes, R, V, K = 1, 8, 248320, 5120
    key = (4,)
    c_d, s_d = inputs.device_nvfp4_weights(key, V, K, dev)
    h_d = inputs.device_x_bf16(key, lanes * R, K, dev)
    codes, scales = c_d.cpu().numpy(), s_d.cpu().numpy()
    h = h_d.view(torch.int16).cpu().numpy().view(np.uint16)
    say("  oracle logits ...")
    logits_ref = O.gemm_nvfp4(h, codes, scales, 1.0)
    drafts = inputs.drafts(key, O.argmax_lowest(logits_ref).reshape(lanes, R), V)
    say(f"  drafts {drafts.tolist()}")
    out = run_head(h, codes, scales, 1.0, drafts, lanes, R)
    check_f32(out["logits"], logits_ref, what="logits")
    check_head(out, logits_ref, drafts, lanes, R)
    say(f"  accept_len {out['accept'].tolist()} commit {out['commit'].tolist()}")
