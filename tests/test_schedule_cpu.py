"""The GEMM schedules on the host (no GPU): vq_schedule_info reports how a
call is split, and the properties the kernels' reductions rely on hold for
every shape tried.

Split-K / stream-K on the narrow projections: "Beating Splash on an M5 Max
...", section "The kernels were not the gap". Workgroup g of G owns the
iterations [g W / G, (g + 1) W / G) of the unit-major (unit, k-iteration)
space, W = units * K / 128.

* Every schedule: at least one workgroup and at most one per CU (256), and
  the reduction slots suffice: a workgroup shares at most two units (the
  first and the last it touches) with other workgroups.
* The accumulating FP8 entry: no unit has more than two workgroup shares,
  which is what makes its fp32 additions order-independent from zero
  (0 + a + b = 0 + b + a; three shares would not be).
* The pass's shapes get the splits the measurements are quoted on.
"""
import os

import numpy as np
import pytest

from bit_block_scaled_vq_amd import ops

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="libverify.so not built")

GEMM_OPS = [ops.VQ_OP_NVFP4, ops.VQ_OP_NVFP4_SILU_MUL, ops.VQ_OP_FP8, ops.VQ_OP_LMHEAD, ops.VQ_OP_AFFINE_Q4,
            ops.VQ_OP_AFFINE_Q4_SILU_MUL, ops.VQ_OP_FP8_ACCUMULATE]
NS = [1, 31, 32, 64, 96, 100, 1000, 5000, 5120, 5440, 5441, 5504, 14336, 16384, 17408, 65536, 248320]
KS = [128, 256, 384, 640, 5120, 6144, 17408]


def shares_per_unit(units, iters, wgs):
    """Number of workgroups whose range meets each unit."""
    W = units * iters
    bounds = np.unique((np.arange(1, wgs, dtype=np.int64) * W) // wgs)
    starts = np.arange(units, dtype=np.int64) * iters
    # boundaries strictly inside unit u: starts[u] < b < starts[u] + iters
    lo = np.searchsorted(bounds, starts, side="right")
    hi = np.searchsorted(bounds, starts + iters, side="left")
    return 1 + (hi - lo)


@pytest.mark.parametrize("op", GEMM_OPS)
def test_schedules_fit_the_chip_and_the_reduction_slots(op):
    for n in NS:
        for k in KS:
            units, iters, wgs = ops.schedule_info(op, n, k)
            assert iters == k // 128
            assert 1 <= wgs <= 256, (op, n, k, wgs)
            W = units * iters
            b = (np.arange(wgs + 1, dtype=np.int64) * W) // wgs
            assert b[0] == 0 and b[-1] == W and np.all(np.diff(b) >= 0)
            # units a workgroup shares with others: at most its first and its last
            sh = shares_per_unit(units, iters, wgs)
            for g in range(0, wgs, max(1, wgs // 16)):
                if b[g] == b[g + 1]:
                    continue
                u0, u1 = b[g] // iters, (b[g + 1] - 1) // iters
                inner = [u for u in range(u0 + 1, u1) if sh[u] > 1]
                assert not inner, (op, n, k, g, inner[:4])


def test_accumulating_schedule_gives_every_unit_at_most_two_shares():
    for n in NS:
        for k in KS:
            units, iters, wgs = ops.schedule_info(ops.VQ_OP_FP8_ACCUMULATE, n, k)
            assert units == 2 * ((n + 63) // 64)  # both halves of every 64-row tile
            sh = shares_per_unit(units, iters, wgs)
            assert sh.max() <= 2, (n, k, units, iters, wgs, int(sh.max()))


def test_the_pass_shapes_get_their_documented_splits():
    # (op, N, K) -> (units, iterations per unit, workgroups)
    want = {
        (ops.VQ_OP_FP8, 16384, 5120): (256, 40, 256),               # GDN in: one tile per workgroup
        (ops.VQ_OP_FP8, 14336, 5120): (224, 40, 224),               # attention q+gate+k+v
        (ops.VQ_OP_FP8_ACCUMULATE, 5120, 6144): (160, 48, 240),     # out-projections: 3 per 64 columns
        (ops.VQ_OP_NVFP4_SILU_MUL, 17408, 5120): (544, 40, 248),    # [gate; up]: stream-K
        (ops.VQ_OP_NVFP4, 5120, 17408): (80, 136, 240),             # down: 3 per tile
        (ops.VQ_OP_LMHEAD, 248320, 5120): (3880, 40, 248),          # vocabulary head: stream-K
    }
    for (op, n, k), w in want.items():
        assert ops.schedule_info(op, n, k) == w, (op, n, k)
        assert ops.schedule_info(op, n, k, M=1) == w, (op, n, k)
    # M > 8: the NVFP4 ops on outputs of >= 2,048 tiles (the vocabulary head)
    # stream tile pairs (one activation load feeds 128 columns); narrower
    # NVFP4 and every FP8 split stay as at M <= 8
    wide = {(ops.VQ_OP_LMHEAD, 248320, 5120): (1940, 40, 248)}
    for m in (9, 16, 24, 32):
        for (op, n, k), w in want.items():
            assert ops.schedule_info(op, n, k, M=m) == wide.get((op, n, k), w), (op, n, k, m)
    # an odd tile count: the last pair is one tile
    assert ops.schedule_info(ops.VQ_OP_NVFP4, 64 * 2049 - 5, 256, M=16)[0] == 1025
    assert ops.schedule_info(ops.VQ_OP_NVFP4_SILU_MUL, 32 * 2049, 256, M=9)[0] == 1025
    assert ops.schedule_info(ops.VQ_OP_NVFP4, 64 * 2047, 256, M=16)[0] == 2047  # below 2,048 tiles: tiles
    # the out-projections' units: exactly two shares each
    sh = shares_per_unit(160, 48, 240)
    assert sh.min() == 2 and sh.max() == 2


def test_workspace_serves_both_nvfp4_families():
    # one workspace of (op, N, K) for every M: sized for the larger of the
    # M <= 8 (tiles) and M > 8 (tile pairs) layouts
    L = ops.lib()
    for op, n, k in ((ops.VQ_OP_NVFP4_SILU_MUL, 17408, 5120), (ops.VQ_OP_LMHEAD, 248320, 5120),
                     (ops.VQ_OP_NVFP4, 64 * 2049 - 5, 256)):
        sizes = {L.vq_workspace_bytes(op, m, n, k) for m in (1, 8, 9, 32)}
        assert len(sizes) == 1 and sizes.pop() > 0, (op, n, k)


def test_schedule_info_validates():
    import ctypes
    L = ops.lib()
    x = ctypes.c_int32()
    p = ctypes.byref(x)
    assert L.vq_schedule_info(ops.VQ_OP_FP8, 8, 64, 128, None, p, p) == ops.VQ_ERR_NULL
    assert L.vq_schedule_info(ops.VQ_OP_FP8, 8, 0, 128, p, p, p) == ops.VQ_ERR_SHAPE
    assert L.vq_schedule_info(ops.VQ_OP_FP8, 8, 64, 100, p, p, p) == ops.VQ_ERR_SHAPE
    assert L.vq_schedule_info(ops.VQ_OP_SAMPLE, 8, 64, 128, p, p, p) == ops.VQ_ERR_VALUE
    assert L.vq_schedule_info(99, 8, 64, 128, p, p, p) == ops.VQ_ERR_VALUE
    assert L.vq_schedule_info(ops.VQ_OP_NVFP4, 0, 64, 128, p, p, p) == ops.VQ_ERR_SHAPE
    assert L.vq_schedule_info(ops.VQ_OP_NVFP4, 33, 64, 128, p, p, p) == ops.VQ_ERR_SHAPE
