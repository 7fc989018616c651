"""GPU parity of the affine 4-bit path (vq_pack_affine_q4, vq_gemm_affine_q4)
against the fp64 oracle, through the C ABI ("144 tok/s needs 502 GB/s ...",
section "The engine hard-codes the model": scale and bias per 64 inputs).

fp32-mode outputs are gated at max|gpu-oracle|/max|oracle| <= 2e-3; bf16
stores must equal RNE of the fp32 store bitwise and lie in the flip class
otherwise. The packed layout is checked byte for byte against a numpy
packer written from the header's description.
"""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import (bf16_to_bits, check_bf16_store, check_f32, pack_affine_np, say, to_dev_bf16,
                               to_dev_u8, torch_dev)

pytestmark = pytest.mark.gpu


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def _dev_i16(bits):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def pack(codes, sb, bb, gate_up=False):
    return _ops().pack_affine_q4(to_dev_u8(codes), _dev_i16(sb), _dev_i16(bb), gate_up=gate_up)


def run_affine(x_bits, codes, sb, bb, n_out, epi=0, out="both", w=None):
    torch, dev = torch_dev()
    ops = _ops()
    x = to_dev_bf16(x_bits)
    w = w if w is not None else pack(codes, sb, bb, gate_up=bool(epi))
    m, k = x_bits.shape
    op = ops.VQ_OP_AFFINE_Q4_SILU_MUL if epi else ops.VQ_OP_AFFINE_Q4
    ws = ops.workspace(op, m, n_out, k, dev)
    y32 = torch.empty((m, n_out), dtype=torch.float32, device=dev)
    ops.vq_gemm_affine_q4(x, w, y32, epilogue=epi, workspace=ws)
    res = {"f32": y32.cpu().numpy()}
    if out == "both":
        yb = torch.empty((m, n_out), dtype=torch.bfloat16, device=dev)
        ops.vq_gemm_affine_q4(x, w, yb, epilogue=epi, workspace=ws)
        res["bf16"] = bf16_to_bits(yb)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("rows,k,gate_up", [(100, 384, False), (64, 128, False), (140, 256, True),
                                           (2, 128, True), (1, 512, False)])
def test_pack_affine_layout(rows, k, gate_up):
    say(f"case: pack affine rows={rows} K={k} gate_up={gate_up}")
    codes, sb, bb = inputs.affine_weights((400, rows, k), rows, k)
    got = pack(codes, sb, bb, gate_up).cpu().numpy()
    want = pack_affine_np(codes, sb, bb, gate_up)
    assert got.shape == want.shape and np.array_equal(got, want)


@pytest.mark.parametrize("m,n,k", [(8, 1000, 512), (1, 64, 128), (5, 130, 256), (16, 700, 384), (24, 333, 640),
                                   (32, 2048, 1024), (8, 512, 17408), (17, 96, 5120), (3, 4097, 128)])
def test_affine_gemm(m, n, k):
    say(f"case: affine GEMM M={m} N={n} K={k}")
    key = (410, m, n, k)
    x = inputs.x_bf16(key, m, k)
    codes, sb, bb = inputs.affine_weights(key, n, k)
    ref = O.gemm_affine_q4(x, codes, sb, bb)
    res = run_affine(x, codes, sb, bb, n)
    check_f32(res["f32"], ref, what="affine fp32")
    check_bf16_store(res["bf16"], res["f32"], ref)


@pytest.mark.parametrize("m,inter,k", [(8, 512, 1024), (32, 320, 256), (12, 96, 5120)])
def test_affine_silu_mul(m, inter, k):
    say(f"case: affine [gate; up] + SiLU*up M={m} N={inter} K={k}")
    key = (420, m, inter, k)
    x = inputs.x_bf16(key, m, k)
    codes, sb, bb = inputs.affine_weights(key, 2 * inter, k)
    h, _ = O.mlp_silu_mul_affine(x, codes, sb, bb, inter)
    res = run_affine(x, codes, sb, bb, inter, epi=1)
    check_f32(res["f32"], h, what="affine SiLU*up fp32")
    check_bf16_store(res["bf16"], res["f32"], h)


def test_affine_special_weights():
    # zero scales (the bias alone), codes 0 and 15, one-hot activations
    m, n, k = 8, 192, 256
    g = np.random.default_rng(430)
    codes = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    codes[:64] = 0x00
    codes[64:128] = 0xFF
    _, sb, bb = inputs.affine_weights((430,), n, k)
    sb[:32] = 0                      # +0 scale: bias only
    sb[32:48] = 0x8000               # -0 scale
    x = np.zeros((m, k), dtype=np.float32)
    for i in range(m):
        x[i, (37 * i + 5) % k] = 1.0
    x[7] = g.standard_normal(k).astype(np.float32)
    import torch
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = O.gemm_affine_q4(xb, codes, sb, bb)
    res = run_affine(xb, codes, sb, bb, n)
    # one-hot rows pick single weights s*q + b: exact in fp32
    assert np.array_equal(res["f32"][:7].astype(np.float64), ref[:7])
    check_f32(res["f32"], ref, what="affine special")


def test_affine_rows_do_not_depend_on_m():
    # 16 activation rows per row group, shares summed in a fixed order: a row's
    # result is bit-identical whatever M is
    n, k = 1000, 1024
    codes, sb, bb = inputs.affine_weights((440,), n, k)
    x32 = inputs.x_bf16((440,), 32, k)
    w = pack(codes, sb, bb)
    full = run_affine(x32, None, None, None, n, out="f32", w=w)["f32"]
    for m in (1, 8, 16, 24):
        part = run_affine(x32[:m], None, None, None, n, out="f32", w=w)["f32"]
        assert np.array_equal(part, full[:m]), m


def test_affine_full_size_down_projection_sampled_columns():
    # the MLP down projection's shape (5,120 x 17,408) at M = 8 and 32, checked
    # on sampled output columns (the oracle computes those rows only)
    n, k = 5120, 17408
    codes, sb, bb = inputs.affine_weights((450,), n, k)
    w = pack(codes, sb, bb)
    cols = np.random.default_rng(450).choice(n, size=96, replace=False)
    for m in (8, 32):
        say(f"case: affine full-size down M={m}")
        x = inputs.x_bf16((450, m), m, k)
        res = run_affine(x, None, None, None, n, out="f32", w=w)
        ref = O.gemm_affine_q4(x, codes, sb, bb, rows=cols)
        check_f32(res["f32"][:, cols], ref, what=f"affine down M={m}")


def test_affine_graph_replay_matches_eager():
    torch, dev = torch_dev()
    ops = _ops()
    m, inter, k = 8, 1024, 2048
    x = inputs.x_bf16((460,), m, k)
    codes, sb, bb = inputs.affine_weights((460,), 2 * inter, k)
    w = pack(codes, sb, bb, gate_up=True)
    xd = to_dev_bf16(x)
    ws = ops.workspace(ops.VQ_OP_AFFINE_Q4_SILU_MUL, m, inter, k, dev)
    ye = torch.empty((m, inter), dtype=torch.float32, device=dev)
    ops.vq_gemm_affine_q4(xd, w, ye, epilogue=ops.VQ_EPI_SILU_MUL, workspace=ws)
    eager = ye.cpu().numpy()
    y = torch.zeros_like(ye)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ops.vq_gemm_affine_q4(xd, w, y, epilogue=ops.VQ_EPI_SILU_MUL, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    for i in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager), i
        ops.vq_gemm_affine_q4(xd, w, ye, epilogue=ops.VQ_EPI_SILU_MUL, workspace=ws)
        torch.cuda.synchronize()
