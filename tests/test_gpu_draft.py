"""GPU parity of the draft-side shapes ("144 tok/s needs 502 GB/s ...",
section "The engine hard-codes the model", geometry table: the 5-layer draft
at hidden 5,120 with qkv 6,144, dynamic 1,280, attention 4,096 and SwiGLU
17,408, and the 5,120 x 25,600 context projection). Same kernels as the
verify pass; the shapes add N = 1,280 and K = 4,096 / 25,600 schedules."""
import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import check_f32, say, to_dev_bf16, to_dev_u8, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k", [(8, 1280, 5120), (8, 8704, 5120), (8, 5120, 4096), (16, 1280, 5120),
                                   (8, 5120, 25600), (32, 5120, 25600)])
def test_draft_shapes_nvfp4(m, n, k):
    from bit_block_scaled_vq_amd import ops
    torch, dev = torch_dev()
    say(f"case: draft shape NVFP4 M={m} N={n} K={k}")
    key = (500, m, n, k)
    x = inputs.x_bf16(key, m, k)
    codes, scales = inputs.nvfp4_weights(key, n, k)
    w = ops.pack_nvfp4(to_dev_u8(codes), to_dev_u8(scales))
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    ops.vq_gemm_nvfp4(to_dev_bf16(x), w, 0.75, y, workspace=ops.workspace(ops.VQ_OP_NVFP4, m, n, k, dev))
    torch.cuda.synchronize()
    cols = np.random.default_rng(500).choice(n, size=min(n, 160), replace=False)
    ref = O.gemm_nvfp4(x, codes, scales, 0.75, rows=cols)
    check_f32(y.cpu().numpy()[:, cols], ref, what=f"draft M={m} N={n} K={k}")
