"""GPU test of vq_gemm_nvfp4_noalloc, the allocation-free variant of
vq_gemm_nvfp4 (static per-device scratch instead of a workspace): its outputs
must equal vq_gemm_nvfp4's bit for bit (same kernels and schedule) on calls
of different shapes in a row on the shared scratch -- a large one, then
smaller ones, then the large one again -- and match the oracle; it must work
under graph capture, and reject shapes beyond the scratch on the host."""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import check_f32, say, to_dev_bf16, to_dev_u8, torch_dev

pytestmark = pytest.mark.gpu


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def _pair(x, w, ts, n, m, epi, dtype):
    """(no-alloc output, workspace output) of the same call."""
    torch, dev = torch_dev()
    ops = _ops()
    k = x.shape[1]
    y0 = torch.full((m, n), float("nan"), dtype=dtype, device=dev)
    y1 = torch.full((m, n), float("nan"), dtype=dtype, device=dev)
    ops.vq_gemm_nvfp4_noalloc(x, w, ts, y0, epilogue=epi)
    op = ops.VQ_OP_NVFP4_SILU_MUL if epi else ops.VQ_OP_NVFP4
    ops.vq_gemm_nvfp4(x, w, ts, y1, epilogue=epi, workspace=ops.workspace(op, m, n, k, dev))
    torch.cuda.synchronize()
    return y0, y1


def _same(a, b):
    import torch
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_noalloc_matches_workspace_entry_point_across_shapes():
    torch, dev = torch_dev()
    ops = _ops()
    bf, f32 = torch.bfloat16, torch.float32

    # 1. the full-size [gate; up] + SiLU*up at M = 8 (272 partial-sum slots' worth of workgroups)
    say("case: no-alloc [gate;up] 34816x5120 + SiLU*up, M=8, bf16")
    inter, hid = 17408, 5120
    c1, s1 = inputs.device_nvfp4_weights((500, 1), 2 * inter, hid, dev)
    w1 = ops.pack_nvfp4(c1, s1, gate_up=True)
    x1 = inputs.device_x_bf16((500, 1), 8, hid, dev)
    a1, b1 = _pair(x1, w1, 1.0, inter, 8, ops.VQ_EPI_SILU_MUL, bf)
    assert _same(a1, b1)
    first = a1.clone()

    # 2. a smaller call on the same scratch: M = 3, N = 1000, K = 512, fp32, against the oracle too
    say("case: no-alloc M=3 N=1000 K=512 fp32, then the oracle")
    xh = inputs.x_bf16((500, 2), 3, 512)
    ch, sh = inputs.nvfp4_weights((500, 2), 1000, 512)
    w2 = ops.pack_nvfp4(to_dev_u8(ch), to_dev_u8(sh))
    a2, b2 = _pair(to_dev_bf16(xh), w2, 0.37, 1000, 3, ops.VQ_EPI_NONE, f32)
    assert _same(a2, b2)
    check_f32(a2.cpu().numpy(), O.gemm_nvfp4(xh, ch, sh, 0.37), what="no-alloc M=3")

    # 3. the scaled family (M = 16) on the down shape, all tiles split over three workgroups
    say("case: no-alloc down 5120x17408 at M=16, fp32")
    c3, s3 = inputs.device_nvfp4_weights((500, 3), hid, inter, dev)
    w3 = ops.pack_nvfp4(c3, s3)
    x3 = inputs.device_x_bf16((500, 3), 16, inter, dev)
    a3, b3 = _pair(x3, w3, 1.0, hid, 16, ops.VQ_EPI_NONE, f32)
    assert _same(a3, b3)
    rows = np.arange(0, hid, 37)
    ref = O.gemm_nvfp4(x3.view(torch.int16).cpu().numpy().view(np.uint16), c3.cpu().numpy()[rows],
                       s3.cpu().numpy()[rows], 1.0)
    check_f32(a3.cpu().numpy()[:, rows], ref, what="no-alloc down M=16 (sampled columns)")

    # 3b. tile pairs (the scaled family on >= 2,048 tiles, an odd count) at M = 24
    say("case: no-alloc tile pairs N=131131 K=256 at M=24, fp32")
    n5, k5 = 64 * 2049 - 5, 256
    x5 = inputs.x_bf16((500, 5), 24, k5)
    c5, s5 = inputs.nvfp4_weights((500, 5), n5, k5)
    w5 = ops.pack_nvfp4(to_dev_u8(c5), to_dev_u8(s5))
    a5, b5 = _pair(to_dev_bf16(x5), w5, 1.0, n5, 24, ops.VQ_EPI_NONE, f32)
    assert _same(a5, b5)
    check_f32(a5.cpu().numpy(), O.gemm_nvfp4(x5, c5, s5, 1.0), what="no-alloc tile pairs M=24")

    # 4. the first shape again: the counters the smaller calls used were left at zero
    say("case: no-alloc [gate;up] again after the other shapes")
    a4, _ = _pair(x1, w1, 1.0, inter, 8, ops.VQ_EPI_SILU_MUL, bf)
    assert _same(a4, first)


def test_noalloc_under_graph_capture():
    torch, dev = torch_dev()
    ops = _ops()
    say("case: no-alloc calls captured in a graph (two shapes), replayed with eager work between")
    x = inputs.x_bf16((501,), 8, 1024)
    c, s = inputs.nvfp4_weights((501,), 2 * 640, 1024)
    w = ops.pack_nvfp4(to_dev_u8(c), to_dev_u8(s), gate_up=True)
    c2, s2 = inputs.nvfp4_weights((502,), 1000, 640)
    w2 = ops.pack_nvfp4(to_dev_u8(c2), to_dev_u8(s2))
    xd = to_dev_bf16(x)
    h = torch.empty((8, 640), dtype=torch.bfloat16, device=dev)
    y = torch.empty((8, 1000), dtype=torch.float32, device=dev)

    def run():
        ops.vq_gemm_nvfp4_noalloc(xd, w, 1.0, h, epilogue=ops.VQ_EPI_SILU_MUL)
        ops.vq_gemm_nvfp4_noalloc(h, w2, 1.0, y)

    run()
    torch.cuda.synchronize()
    eh, ey = h.clone(), y.clone()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for i in range(3):
        h.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(h, eh) and _same(y, ey), i
        run()  # eager calls on the same scratch between replays
        torch.cuda.synchronize()
    hb = h.view(torch.int16).cpu().numpy().view(np.uint16)
    hr, _ = O.mlp_silu_mul(x, c, s, 1.0, 640)
    check_f32(O.bf16_bits_to_f64(hb), hr, tol=4e-3, what="graph h (bf16)")
    check_f32(y.cpu().numpy(), O.gemm_nvfp4(hb, c2, s2, 1.0), what="graph y")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    torch, dev = torch_dev()
    ops = _ops()
    x = torch.zeros((8, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros(16, dtype=torch.uint8, device=dev)
    y = torch.empty((8, 4194305), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ops.VerifyError) as ei:
        ops.vq_gemm_nvfp4_noalloc(x, w, 1.0, y)
    assert ei.value.status == ops.VQ_ERR_SHAPE
