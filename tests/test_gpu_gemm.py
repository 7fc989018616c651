"""GPU parity of vq_gemm_nvfp4 / vq_gemm_fp8 against the fp64 oracle.

Every case calls the HIP library through its C ABI (ops.py is argument
marshalling only) and compares with the oracle element by element on the same
seeded inputs. fp32-mode outputs are gated at max|gpu-oracle|/max|oracle| <=
2e-3; bf16 stores must equal RNE of the fp32 store bitwise and may differ from
RNE(oracle) only in the flip class.
"""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import (bf16_to_bits, check_bf16_store, check_f32, pack_fp8_np, pack_nvfp4_np, say,
                               to_dev_bf16, to_dev_u8, torch_dev)

pytestmark = pytest.mark.gpu


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def run_nvfp4(x_bits, codes, scales, ts, n_out, epi=0, out="both", ws=None):
    torch, dev = torch_dev()
    ops = _ops()
    x = to_dev_bf16(x_bits)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales), gate_up=bool(epi))
    m, k = x_bits.shape
    op = ops.VQ_OP_NVFP4_SILU_MUL if epi else ops.VQ_OP_NVFP4
    ws = ws if ws is not None else ops.workspace(op, m, n_out, k, dev)
    y32 = torch.empty((m, n_out), dtype=torch.float32, device=dev)
    ops.vq_gemm_nvfp4(x, w, ts, y32, epilogue=epi, workspace=ws)
    res = {"f32": y32.cpu().numpy()}
    if out == "both":
        yb = torch.empty((m, n_out), dtype=torch.bfloat16, device=dev)
        ops.vq_gemm_nvfp4(x, w, ts, yb, epilogue=epi, workspace=ws)
        res["bf16"] = bf16_to_bits(yb)
    torch.cuda.synchronize()
    return res


def run_fp8(x_bits, w, wscale, out="both"):
    torch, dev = torch_dev()
    ops = _ops()
    x = to_dev_bf16(x_bits)
    wd = ops.pack_fp8(to_dev_u8(w))
    m, k = x_bits.shape
    n = w.shape[0]
    ws = ops.workspace(ops.VQ_OP_FP8, m, n, k, dev)
    y32 = torch.empty((m, n), dtype=torch.float32, device=dev)
    ops.vq_gemm_fp8(x, wd, wscale, y32, workspace=ws)
    res = {"f32": y32.cpu().numpy()}
    if out == "both":
        yb = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ops.vq_gemm_fp8(x, wd, wscale, yb, workspace=ws)
        res["bf16"] = bf16_to_bits(yb)
    torch.cuda.synchronize()
    return res


# ------------------------------------------------------------- packing

@pytest.mark.parametrize("rows,k,gate_up", [(100, 384, False), (64, 128, False), (140, 256, True),
                                           (2, 128, True), (1, 512, False)])
def test_pack_nvfp4_layout(rows, k, gate_up):
    say(f"case: pack NVFP4 rows={rows} K={k} gate_up={gate_up}")
    ops = _ops()
    codes, scales = inputs.nvfp4_weights((300, rows, k), rows, k)
    got = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales), gate_up=gate_up).cpu().numpy()
    want = pack_nvfp4_np(codes, scales, gate_up)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,k", [(130, 512), (64, 128), (1, 256)])
def test_pack_fp8_layout(rows, k):
    say(f"case: pack FP8 rows={rows} K={k}")
    ops = _ops()
    w = np.random.default_rng(rows).integers(0, 256, size=(rows, k), dtype=np.uint8)
    got = ops.pack_fp8(to_dev_u8(w)).cpu().numpy()
    want = pack_fp8_np(w)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


# ------------------------------------------------------------------- NVFP4

def test_nvfp4_single_gemm_m8_k512_n1024():
    say("case: NVFP4 M=8 K=512 N=1024 (seed 0 recipe)")
    x = inputs.x_bf16((1,), 8, 512)
    codes, scales = inputs.nvfp4_weights((1,), 1024, 512)
    ref = O.gemm_nvfp4(x, codes, scales, 1.0)
    r = run_nvfp4(x, codes, scales, 1.0, 1024)
    check_f32(r["f32"], ref, what="cfg1 f32")
    check_bf16_store(r["bf16"], r["f32"], ref)


@pytest.mark.parametrize("m,n,k,ts", [
    (1, 1, 128, 1.0), (3, 33, 384, 0.37), (8, 100, 512, 1.0), (13, 257, 640, 2.5),
    (24, 64, 1024, 1.0), (32, 200, 256, 0.125), (8, 4096, 2048, 1.0), (5, 1000, 5120, 1.0),
    (16, 2, 128, 1.0), (8, 65, 128, 1.0), (9, 130, 768, 1.0), (7, 3000, 17408, 1.0),
    (17, 70, 384, 1.0), (29, 130, 640, 0.5),
    # >= 2,048 tiles at M > 8: tile pairs (an odd tile count, then an even one)
    (13, 64 * 2049 - 5, 128, 1.0), (32, 64 * 2050, 256, 0.5),
])
def test_nvfp4_shapes(m, n, k, ts):
    say(f"case: NVFP4 M={m} N={n} K={k} ts={ts}")
    x = inputs.x_bf16((100, m, n, k), m, k)
    codes, scales = inputs.nvfp4_weights((100, m, n, k), n, k)
    ref = O.gemm_nvfp4(x, codes, scales, ts)
    r = run_nvfp4(x, codes, scales, ts, n)
    check_f32(r["f32"], ref, what=f"M{m} N{n} K{k}")
    check_bf16_store(r["bf16"], r["f32"], ref)


def test_nvfp4_one_hot_is_bit_exact():
    # Y[0, n] = W[n, k] * 1.0 exactly: pins the decode, the nibble order, the
    # scale-block mapping and the operand roles.
    n, k, ts = 130, 384, 0.75
    codes, scales = inputs.nvfp4_weights((101,), n, k)
    w = O.dequant_nvfp4(codes, scales, ts)
    for kk in (0, 1, 7, 8, 15, 16, 31, 32, 63, 64, 100, 127, 128, 255, 256, 383):
        say(f"case: one-hot k={kk}")
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, kk] = 0x3F80
        r = run_nvfp4(x, codes, scales, ts, n, out="f32")
        assert np.array_equal(r["f32"][0].astype(np.float64), w[:, kk].astype(np.float32).astype(np.float64)), kk


def test_nvfp4_special_values():
    m, n, k = 4, 96, 256
    x = inputs.x_bf16((102,), m, k)
    codes, scales = inputs.nvfp4_weights((102,), n, k)
    # zero block scales, NaN block scales on two rows, all-(-0) codes on a row
    scales[:, 3] = 0
    scales[5, 7] = 0x7F
    scales[90, 0] = 0xFF
    codes[10, :] = 0x88
    scales[10, :] = 0x38  # 1.0
    ref = O.gemm_nvfp4(x, codes, scales, 1.0)
    r = run_nvfp4(x, codes, scales, 1.0, n)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(r["f32"]), nan_ref)
    assert nan_ref[:, 5].all() and nan_ref[:, 90].all()
    fin = ~nan_ref
    check_f32(np.where(fin, r["f32"], 0), np.where(fin, ref, 0), what="finite part")
    assert np.all(r["f32"][:, 10] == 0.0)


def test_nvfp4_silu_mul_small():
    m, inter, k = 8, 300, 512
    x = inputs.x_bf16((103,), m, k)
    codes, scales = inputs.nvfp4_weights((103,), 2 * inter, k)
    h, hb = O.mlp_silu_mul(x, codes, scales, 1.0, inter)
    r = run_nvfp4(x, codes, scales, 1.0, inter, epi=1)
    check_f32(r["f32"], h, what="silu*up f32")
    check_bf16_store(r["bf16"], r["f32"], h)


def test_nvfp4_silu_mul_tile_pairs():
    # M > 8 on >= 2,048 tiles: tile pairs, the last one alone (odd count)
    m, inter, k = 16, 32 * 2049, 128
    x = inputs.x_bf16((116,), m, k)
    codes, scales = inputs.nvfp4_weights((116,), 2 * inter, k)
    h, hb = O.mlp_silu_mul(x, codes, scales, 1.0, inter)
    r = run_nvfp4(x, codes, scales, 1.0, inter, epi=1)
    check_f32(r["f32"], h, what="silu*up f32 (tile pairs)")
    check_bf16_store(r["bf16"], r["f32"], h)


def test_tile_pair_rows_independent_of_m():
    # the scaled family's tile-pair split depends on (N, K) only: rows shared
    # by calls at M = 9..32 are bitwise equal
    torch, dev = torch_dev()
    ops = _ops()
    n, k = 64 * 2050, 256
    codes, scales = inputs.nvfp4_weights((117,), n, k)
    x32 = inputs.x_bf16((117,), 32, k)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    ws = ops.workspace(ops.VQ_OP_NVFP4, 32, n, k, dev)
    outs = {}
    for m in (32, 9, 16, 24):
        say(f"case: tile pairs M={m}")
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        ops.vq_gemm_nvfp4(to_dev_bf16(x32[:m]), w, 1.0, y, workspace=ws)
        outs[m] = y.cpu().numpy()
    for m in (9, 16, 24):
        assert np.array_equal(outs[m], outs[32][:m]), m
    check_f32(outs[32], O.gemm_nvfp4(x32, codes, scales, 1.0), what="tile pairs M=32")


def test_mlp_layer_m8_full_size():
    say("case: MLP layer M=8: [gate;up] 34816x5120 + SiLU*up, down 5120x17408")
    m, hid, inter = 8, 5120, 17408
    x = inputs.x_bf16((2,), m, hid)
    gu_c, gu_s = inputs.nvfp4_weights((2, 0), 2 * inter, hid)
    dn_c, dn_s = inputs.nvfp4_weights((2, 1), hid, inter)
    h_ref, h_bits = O.mlp_silu_mul(x, gu_c, gu_s, 1.0, inter)
    r1 = run_nvfp4(x, gu_c, gu_s, 1.0, inter, epi=1)
    check_f32(r1["f32"], h_ref, what="h = silu(gate)*up")
    check_bf16_store(r1["bf16"], r1["f32"], h_ref)
    # down projection on the GPU's own bf16 h and, for the oracle, the same bits
    y_ref = O.gemm_nvfp4(r1["bf16"], dn_c, dn_s, 1.0)
    r2 = run_nvfp4(r1["bf16"], dn_c, dn_s, 1.0, hid)
    check_f32(r2["f32"], y_ref, what="down")
    check_bf16_store(r2["bf16"], r2["f32"], y_ref)
    # and the whole layer against the oracle's own chain (h rounded once to bf16)
    y_chain = O.gemm_nvfp4(h_bits, dn_c, dn_s, 1.0)
    check_f32(r2["f32"], y_chain, what="layer vs oracle chain")


# --------------------------------------------------------------------- FP8

@pytest.mark.parametrize("m,n,k,ws", [
    (1, 1, 128, 1.0), (8, 100, 512, 0.37), (13, 257, 640, 0.125), (32, 64, 1024, 1.0), (8, 1000, 6144, 1.0),
    (24, 3000, 5120, 1.0), (17, 70, 384, 1.0), (29, 130, 640, 0.5),
])
def test_fp8_shapes(m, n, k, ws):
    say(f"case: FP8 M={m} N={n} K={k} scale={ws}")
    x = inputs.x_bf16((104, m, n, k), m, k)
    w = inputs.fp8_weights((104, m, n, k), n, k)
    ref = O.gemm_fp8(x, w, ws)
    r = run_fp8(x, w, ws)
    check_f32(r["f32"], ref, what=f"fp8 M{m} N{n} K{k}")
    check_bf16_store(r["bf16"], r["f32"], ref)


def test_fp8_all_codes_one_hot():
    # every E4M3 code (NaN codes included) decoded exactly by the kernel
    n, k = 256, 128
    w = np.zeros((n, k), dtype=np.uint8)
    w[:, 5] = np.arange(256, dtype=np.uint8)
    x = np.zeros((1, k), dtype=np.uint16)
    x[0, 5] = 0x3F80
    r = run_fp8(x, w, 1.0, out="f32")
    ref = O.E4M3FN_TABLE
    got = r["f32"][0].astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("m", [32, 24, 17, 16, 9, 8, 5])
def test_wide_rows_one_hot_row_map(m):
    # Row r of X is one-hot at k_r (k_r spread over both 128-B lines of an
    # iteration, every 16-B segment and both row halves of a 16-row group), so
    # Y[r] must be exactly column k_r of the decoded weights: pins which
    # activation row and k reach each MFMA lane when the kernels read whole
    # lines and reorder them in LDS (every NVFP4 and FP8 kernel except FP8 at
    # M = 9-16), including the two-block A operand of NVFP4 at M <= 8.
    n, k = 96, 256
    ks = [(37 * r + 5) % k for r in range(m)]
    x = np.zeros((m, k), dtype=np.uint16)
    for r, kk in enumerate(ks):
        x[r, kk] = 0x3F80
    say(f"case: one-hot rows NVFP4 M={m}")
    codes, scales = inputs.nvfp4_weights((115, m), n, k)
    wdq = O.dequant_nvfp4(codes, scales, 1.0).astype(np.float32)
    got = run_nvfp4(x, codes, scales, 1.0, n, out="f32")["f32"]
    for r, kk in enumerate(ks):
        assert np.array_equal(got[r], wdq[:, kk]), (r, kk)
    say(f"case: one-hot rows FP8 M={m}")
    w8 = inputs.fp8_weights((115, m), n, k)
    got = run_fp8(x, w8, 1.0, out="f32")["f32"]
    for r, kk in enumerate(ks):
        assert np.array_equal(got[r].astype(np.float64), O.E4M3FN_TABLE[w8[:, kk]]), (r, kk)


# ---------------------------------------------- properties of the schedule

def test_rows_independent_of_m_and_deterministic():
    # the K partition and the reduction order depend only on (N, K) and the
    # NVFP4 compute family (M <= 8: block scale after the MFMA; M > 8: weights
    # scaled before it): rows shared by calls of one family are bitwise equal.
    torch, dev = torch_dev()
    ops = _ops()
    n, k = 5120, 17408        # the narrow, long-K down projection shape
    codes, scales = inputs.nvfp4_weights((105,), n, k)
    x32 = inputs.x_bf16((105,), 32, k)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    ws = ops.workspace(ops.VQ_OP_NVFP4, 32, n, k, dev)
    outs = {}
    for m in (32, 8, 1, 24, 16, 5, 9):
        say(f"case: down projection M={m}")
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        ops.vq_gemm_nvfp4(to_dev_bf16(x32[:m]), w, 1.0, y, workspace=ws)
        outs[m] = y.cpu().numpy()
    for m in (1, 5):
        assert np.array_equal(outs[m], outs[8][:m]), m
    for m in (9, 16, 24):
        assert np.array_equal(outs[m], outs[32][:m]), m
    y2 = torch.empty((32, n), dtype=torch.float32, device=dev)
    ops.vq_gemm_nvfp4(to_dev_bf16(x32), w, 1.0, y2, workspace=ws)
    assert np.array_equal(y2.cpu().numpy(), outs[32])
    ref = O.gemm_nvfp4(x32, codes, scales, 1.0)
    check_f32(outs[8], ref[:8], what="down M=8")
    check_f32(outs[32], ref, what="down M=32")


def test_fp8_rows_independent_of_m():
    torch, dev = torch_dev()
    ops = _ops()
    n, k = 1000, 6144
    w = ops.pack_fp8(to_dev_u8(inputs.fp8_weights((107,), n, k)))
    x32 = inputs.x_bf16((107,), 32, k)
    ws = ops.workspace(ops.VQ_OP_FP8, 32, n, k, dev)
    outs = {}
    for m in (32, 8, 17):
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        ops.vq_gemm_fp8(to_dev_bf16(x32[:m]), w, 0.5, y, workspace=ws)
        outs[m] = y.cpu().numpy()
    for m in (8, 17):
        assert np.array_equal(outs[m], outs[32][:m]), m


def test_graph_capture_and_replay():
    torch, dev = torch_dev()
    ops = _ops()
    m, n, k = 8, 2048, 1024
    x = inputs.x_bf16((106,), m, k)
    codes, scales = inputs.nvfp4_weights((106,), n, k)
    xd = to_dev_bf16(x)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    ws = ops.workspace(ops.VQ_OP_NVFP4, m, n, k, dev)
    y_eager = torch.empty((m, n), dtype=torch.float32, device=dev)
    ops.vq_gemm_nvfp4(xd, w, 1.0, y_eager, workspace=ws)
    eager = y_eager.cpu().numpy()
    y = torch.zeros((m, n), dtype=torch.float32, device=dev)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ops.vq_gemm_nvfp4(xd, w, 1.0, y, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    for i in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager), i
        ops.vq_gemm_nvfp4(xd, w, 1.0, y_eager, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()


def test_binding_rejects_short_workspace():
    torch, dev = torch_dev()
    ops = _ops()
    x = torch.zeros((8, 512), dtype=torch.bfloat16, device=dev)
    w = torch.zeros(ops.packed_bytes(ops.VQ_PACK_NVFP4, 1024, 512), dtype=torch.uint8, device=dev)
    y = torch.empty((8, 1024), dtype=torch.float32, device=dev)
    ws = torch.zeros(64, dtype=torch.uint8, device=dev)
    with pytest.raises(ops.VerifyError) as ei:
        ops.vq_gemm_nvfp4(x, w, 1.0, y, workspace=ws)
    assert ei.value.status == ops.VQ_ERR_WORKSPACE
    # packed weights one block short of the shape
    ws = ops.workspace(ops.VQ_OP_NVFP4, 8, 1024, 512, dev)
    with pytest.raises(ops.VerifyError) as ei:
        ops.vq_gemm_nvfp4(x, w[:-4608], 1.0, y, workspace=ws)
    assert ei.value.status == ops.VQ_ERR_SHAPE


# ------------------------------------------- model shapes, as bench.py runs them

@pytest.mark.parametrize("n,k", [(16384, 5120), (14336, 5120), (5120, 6144)])
@pytest.mark.parametrize("m", [8, 32])
def test_fp8_model_shapes_full_size(n, k, m):
    # GDN in-projection (256 workgroups, one tile each), attention q+gate+k+v
    # (224, one tile each) and the out-projections (240, three per tile)
    say(f"case: FP8 full size M={m} N={n} K={k}")
    key = (110, n, k)
    x = inputs.x_bf16(key + (m,), m, k)
    w = inputs.fp8_weights(key, n, k)
    ref = O.gemm_fp8(x, w, 0.75)
    r = run_fp8(x, w, 0.75)
    check_f32(r["f32"], ref, what=f"fp8 {n}x{k} M{m}")
    check_bf16_store(r["bf16"], r["f32"], ref)


@pytest.mark.parametrize("m", [16, 32])
def test_mlp_gate_up_full_size_wide_rows(m):
    # the weights-scaled-in-registers NVFP4 family (M > 8) on the [gate; up] shape
    say(f"case: [gate;up] 34816x5120 + SiLU*up at M={m}")
    inter, hid = 17408, 5120
    x = inputs.x_bf16((111, m), m, hid)
    gu_c, gu_s = inputs.nvfp4_weights((2, 0), 2 * inter, hid)
    h_ref, _ = O.mlp_silu_mul(x, gu_c, gu_s, 1.0, inter)
    r = run_nvfp4(x, gu_c, gu_s, 1.0, inter, epi=1)
    check_f32(r["f32"], h_ref, what=f"h M{m}")
    check_bf16_store(r["bf16"], r["f32"], h_ref)


# ----------------------------------------- every E4M3 block-scale code, both families

def _all_scale_codes_case(m):
    """K = 128 (8 scale blocks per row), 32 weight rows: the 32 x 8 block
    scales take every finite E4M3FN code once (0x00-0x7E and 0x80-0xFE, 254
    codes, two repeated) and every code nibble is non-zero, so each scale's
    decode reaches the output. Activation row i is one-hot at k = 16 (i % 8)
    + 2 (i // 8) + 1: rows 0-7 hit the 8 scale blocks, rows 8-15 the same
    blocks at other k. Y[i, n] = E2M1(code[n, k_i]) * E4M3(scale[n, k_i / 16])
    * ts exactly (every such product is exact in bf16 and fp32)."""
    n, k, ts = 32, 128, 0.75
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    scales = np.concatenate([finite, finite[:2]]).reshape(n, k // 16)
    g = np.random.default_rng(1234)
    lo = g.integers(1, 16, size=(n, k // 2), dtype=np.uint8)
    hi = g.integers(1, 16, size=(n, k // 2), dtype=np.uint8)
    lo[lo == 8] = 9  # 8 is -0
    hi[hi == 8] = 9
    codes = (lo | (hi << 4)).astype(np.uint8)
    ks = [16 * (i % 8) + 2 * (i // 8) + 1 for i in range(m)]
    x = np.zeros((m, k), dtype=np.uint16)
    for i, kk in enumerate(ks):
        x[i, kk] = 0x3F80
    w = O.dequant_nvfp4(codes, scales, ts)
    want = np.stack([w[:, kk] for kk in ks]).astype(np.float32).astype(np.float64)
    return x, codes, scales, ts, n, want


@pytest.mark.parametrize("m", [8, 16])
def test_nvfp4_every_block_scale_code_bit_exact(m):
    # m = 8: the block-scale-after-MFMA family; m = 16: weights scaled in registers
    say(f"case: every finite E4M3 block-scale code, one-hot activations, M={m}")
    x, codes, scales, ts, n, want = _all_scale_codes_case(m)
    r = run_nvfp4(x, codes, scales, ts, n, out="f32")
    got = r["f32"].astype(np.float64)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]
    # the decoded scales span the whole E4M3FN range, subnormals included
    used = O.E4M3FN_TABLE[scales]
    assert np.nanmax(used) == 448.0 and np.min(np.abs(used[used != 0])) == 2.0 ** -9


# ------------------------------------------------- FP8 accumulating entry point

def run_fp8_acc(x_bits, w, wscale, y0=None, reps=1):
    """vq_gemm_fp8_accumulate into an fp32 output holding zeros (or y0)."""
    torch, dev = torch_dev()
    ops = _ops()
    x = to_dev_bf16(x_bits)
    wd = ops.pack_fp8(to_dev_u8(w))
    m, n = x_bits.shape[0], w.shape[0]
    outs = []
    for _ in range(reps):
        y = torch.zeros((m, n), dtype=torch.float32, device=dev)
        if y0 is not None:
            y.copy_(torch.from_numpy(y0))
        ops.vq_gemm_fp8_accumulate(x, wd, wscale, y)
        outs.append(y.cpu().numpy())
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("m,n,k,ws", [
    (1, 1, 128, 1.0), (8, 100, 512, 0.37), (13, 257, 640, 0.125), (32, 64, 1024, 1.0), (8, 5000, 6144, 1.0),
    (24, 3000, 5120, 1.0), (8, 5120, 6144, 0.75), (32, 5120, 6144, 0.75), (8, 16384, 5120, 1.0),
])
def test_fp8_accumulate_matches_oracle_and_is_deterministic(m, n, k, ws):
    # three workgroups per 64 columns up to N = 5,440 (each 32-column unit
    # shared by two), one unit or more per workgroup beyond
    say(f"case: FP8 accumulate M={m} N={n} K={k} scale={ws}")
    x = inputs.x_bf16((112, m, n, k), m, k)
    w = inputs.fp8_weights((112, m, n, k), n, k)
    ref = O.gemm_fp8(x, w, ws)
    outs = run_fp8_acc(x, w, ws, reps=3)
    check_f32(outs[0], ref, what=f"fp8 accumulate M{m} N{n} K{k}")
    # elementwise within the fp32-accumulation bound, like the standard entry
    assert np.max(np.abs(outs[0] - ref)) <= 1e-5 * np.max(np.abs(ref))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "two calls from zero differ"
    std = run_fp8(x, w, ws, out="f32")["f32"]
    assert np.max(np.abs(outs[0] - std)) <= 1e-5 * np.max(np.abs(ref))


def test_fp8_accumulate_adds_into_y():
    m, n, k = 8, 300, 768
    x = inputs.x_bf16((113,), m, k)
    w = inputs.fp8_weights((113,), n, k)
    y0 = np.random.default_rng(113).standard_normal((m, n)).astype(np.float32)
    ref = O.gemm_fp8(x, w, 0.5)
    got = run_fp8_acc(x, w, 0.5, y0=y0)[0]
    check_f32(got - y0.astype(np.float64), ref, what="accumulate onto y0")
    assert np.max(np.abs(got - (y0 + ref))) <= 1e-5 * np.max(np.abs(y0 + ref))


def test_fp8_accumulate_all_codes_one_hot():
    # every E4M3 code through the accumulating path: the unit's other share
    # adds an exact zero, so the output is the decoded code (+0 for -0: y
    # starts at +0)
    n, k = 256, 384
    w = np.zeros((n, k), dtype=np.uint8)
    w[:, 5] = np.arange(256, dtype=np.uint8)
    x = np.zeros((1, k), dtype=np.uint16)
    x[0, 5] = 0x3F80
    got = run_fp8_acc(x, w, 1.0)[0][0].astype(np.float64)
    ref = O.E4M3FN_TABLE
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_fp8_accumulate_rows_independent_of_m():
    # the K partition and the two-share split depend only on (N, K), and
    # 0 + a + b does not depend on the order: rows are bitwise the same for
    # every M
    torch, dev = torch_dev()
    ops = _ops()
    n, k = 5120, 6144
    w = ops.pack_fp8(to_dev_u8(inputs.fp8_weights((114,), n, k)))
    x32 = inputs.x_bf16((114,), 32, k)
    outs = {}
    for m in (32, 8, 1, 17):
        say(f"case: FP8 accumulate out-projection M={m}")
        y = torch.zeros((m, n), dtype=torch.float32, device=dev)
        ops.vq_gemm_fp8_accumulate(to_dev_bf16(x32[:m]), w, 1.0, y)
        outs[m] = y.cpu().numpy()
    for m in (8, 1, 17):
        assert np.array_equal(outs[m], outs[32][:m]), m


def test_fp8_accumulate_graph_replay():
    # captured with the zero fill (a kernel, not a memset node) in front of
    # it; every replay, with eager work between them, equals the eager call
    torch, dev = torch_dev()
    ops = _ops()
    m, n, k = 8, 5120, 6144
    xd = to_dev_bf16(inputs.x_bf16((115,), m, k))
    w = ops.pack_fp8(to_dev_u8(inputs.fp8_weights((115,), n, k)))
    y = torch.zeros((m, n), dtype=torch.float32, device=dev)
    ops.vq_gemm_fp8_accumulate(xd, w, 1.0, y)
    eager = y.cpu().numpy()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            y.zero_()
            ops.vq_gemm_fp8_accumulate(xd, w, 1.0, y)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        y.fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager), rep
        ops.vq_gemm_fp8_accumulate(xd, w, 1.0, torch.zeros_like(y))  # eager work between replays
