"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call.

No test here launches anything: every call either fails validation or, on a
host without a GPU, stops at the device check. The one call that would pass
validation is skipped when a GPU is visible.
"""
import ctypes
import os
import re

import pytest

from bit_block_scaled_vq_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="libverify.so not built")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "libverify.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int32_t|size_t)\s+(vq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    L = ops.lib()
    names = _header_functions()
    assert set(names) == set(ops.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = ops.lib()
    assert L.vq_abi_version() == 8
    assert ops.status_str(ops.VQ_OK) == "VQ_OK"
    assert ops.status_str(ops.VQ_ERR_WORKSPACE) == "VQ_ERR_WORKSPACE"
    assert ops.status_str(99) == "VQ_ERR_UNKNOWN"


A = 1 << 20  # a fake, 16-byte-aligned address: never dereferenced (validation fails first)


def _nvfp4(x=A, w=A, wn=1 << 30, y=A, yd=0, M=8, N=1024, K=512, epi=0, ws=A, wsn=1 << 30):
    return ops.lib().vq_gemm_nvfp4(x, w, wn, 1.0, y, yd, M, N, K, epi, ws, wsn, None)


def test_gemm_nvfp4_validation():
    assert _nvfp4(x=None) == ops.VQ_ERR_NULL
    assert _nvfp4(y=None) == ops.VQ_ERR_NULL
    assert _nvfp4(M=0) == ops.VQ_ERR_SHAPE
    assert _nvfp4(M=33) == ops.VQ_ERR_SHAPE
    assert _nvfp4(N=0) == ops.VQ_ERR_SHAPE
    assert _nvfp4(K=32) == ops.VQ_ERR_SHAPE
    assert _nvfp4(K=96) == ops.VQ_ERR_SHAPE
    assert _nvfp4(K=192) == ops.VQ_ERR_SHAPE
    assert _nvfp4(yd=5) == ops.VQ_ERR_VALUE
    assert _nvfp4(epi=3) == ops.VQ_ERR_VALUE
    assert _nvfp4(x=A + 8) == ops.VQ_ERR_ALIGN
    assert _nvfp4(w=None) == ops.VQ_ERR_NULL
    assert _nvfp4(w=A + 4) == ops.VQ_ERR_ALIGN
    need = ops.packed_bytes(ops.VQ_PACK_NVFP4, 1024, 512)
    assert _nvfp4(wn=need - 1) == ops.VQ_ERR_SHAPE
    need_gu = ops.packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, 2048, 512)
    assert _nvfp4(epi=1, wn=need_gu - 16) == ops.VQ_ERR_SHAPE
    assert _nvfp4(y=A + 1) == ops.VQ_ERR_ALIGN
    assert _nvfp4(ws=None) == ops.VQ_ERR_WORKSPACE
    assert _nvfp4(wsn=16) == ops.VQ_ERR_WORKSPACE
    assert "workspace" in ops.last_error()


def test_gemm_fp8_validation():
    L = ops.lib()
    big = 1 << 30
    assert L.vq_gemm_fp8(None, A, big, 1.0, A, 0, 8, 64, 128, A, big, None) == ops.VQ_ERR_NULL
    assert L.vq_gemm_fp8(A, A, big, 1.0, A, 0, 8, 64, 100, A, big, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8(A, A, big, 1.0, A, 0, 8, 64, 64, A, big, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8(A, A + 2, big, 1.0, A, 0, 8, 64, 128, A, big, None) == ops.VQ_ERR_ALIGN
    assert L.vq_gemm_fp8(A, A, 8191, 1.0, A, 0, 8, 64, 128, A, big, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8(A, A, big, 1.0, A, 0, 8, 64, 128, A, 0, None) == ops.VQ_ERR_WORKSPACE


def test_gemm_fp8_accumulate_validation():
    L = ops.lib()
    big = 1 << 30
    assert L.vq_gemm_fp8_accumulate(None, A, big, 1.0, A, 8, 64, 128, None) == ops.VQ_ERR_NULL
    assert L.vq_gemm_fp8_accumulate(A, None, big, 1.0, A, 8, 64, 128, None) == ops.VQ_ERR_NULL
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, None, 8, 64, 128, None) == ops.VQ_ERR_NULL
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, A, 0, 64, 128, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, A, 33, 64, 128, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, A, 8, 0, 128, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, A, 8, 64, 100, None) == ops.VQ_ERR_SHAPE
    assert L.vq_gemm_fp8_accumulate(A + 8, A, big, 1.0, A, 8, 64, 128, None) == ops.VQ_ERR_ALIGN
    assert L.vq_gemm_fp8_accumulate(A, A + 2, big, 1.0, A, 8, 64, 128, None) == ops.VQ_ERR_ALIGN
    assert L.vq_gemm_fp8_accumulate(A, A, big, 1.0, A + 2, 8, 64, 128, None) == ops.VQ_ERR_ALIGN
    need = ops.packed_bytes(ops.VQ_PACK_FP8, 64, 128)
    assert L.vq_gemm_fp8_accumulate(A, A, need - 1, 1.0, A, 8, 64, 128, None) == ops.VQ_ERR_SHAPE
    assert "packed weights" in ops.last_error()


def test_fp8_accumulate_binding_refuses_host_and_wrong_dtypes():
    import torch
    x = torch.zeros((8, 128), dtype=torch.bfloat16)
    w = torch.zeros(8192, dtype=torch.uint8)
    with pytest.raises(ValueError):  # host tensors are refused before any library call
        ops.vq_gemm_fp8_accumulate(x, w, 1.0, torch.zeros((8, 64), dtype=torch.float32))
    with pytest.raises(TypeError):  # the output must be fp32
        ops.vq_gemm_fp8_accumulate(x.float(), w, 1.0, torch.zeros((8, 64), dtype=torch.bfloat16))


def _head(h=A, draft=A, lanes=1, R=8, V=1000, K=256, am=A, al=A, logits=None, ld=1, ws=A, wsn=1 << 30):
    return ops.lib().vq_lmhead_argmax_accept(h, A, 1 << 30, 1.0, draft, lanes, R, V, K, am, None, al, None,
                                             logits, ld, ws, wsn, None)


def test_lmhead_validation():
    assert _head(h=None) == ops.VQ_ERR_NULL
    assert _head(am=None) == ops.VQ_ERR_NULL
    assert _head(draft=None) == ops.VQ_ERR_NULL
    assert _head(lanes=0) == ops.VQ_ERR_SHAPE
    assert _head(lanes=5) == ops.VQ_ERR_SHAPE
    assert _head(R=9) == ops.VQ_ERR_SHAPE
    assert _head(V=0) == ops.VQ_ERR_SHAPE
    assert _head(am=A + 2) == ops.VQ_ERR_ALIGN
    assert _head(logits=A, ld=7) == ops.VQ_ERR_VALUE
    assert _head(wsn=8) == ops.VQ_ERR_WORKSPACE


def _sample(lg=A, lanes=1, R=8, V=1000, t=1.0, k=32, tp=0.9, draft=A, qi=None, qp=None, ua=None, ud=A,
            al=A, ws=A, wsn=1 << 30):
    return ops.lib().vq_sample_accept(lg, lanes, R, V, t, k, tp, draft, qi, qp, ua, ud, None, al, None, None,
                                      None, ws, wsn, None)


def test_sample_validation():
    nan, inf = float("nan"), float("inf")
    assert _sample(lg=None) == ops.VQ_ERR_NULL
    assert _sample(ud=None) == ops.VQ_ERR_NULL
    assert _sample(al=None) == ops.VQ_ERR_NULL
    assert _sample(draft=None) == ops.VQ_ERR_NULL
    assert _sample(qi=A) == ops.VQ_ERR_NULL          # ids without probs
    assert _sample(qi=A, qp=A) == ops.VQ_ERR_NULL    # speculative rule without u_accept
    assert _sample(lanes=5) == ops.VQ_ERR_SHAPE
    assert _sample(R=0) == ops.VQ_ERR_SHAPE
    assert _sample(V=0) == ops.VQ_ERR_SHAPE
    assert _sample(V=(1 << 20) + 1) == ops.VQ_ERR_SHAPE
    for t in (0.0, -1.0, nan, inf):
        assert _sample(t=t) == ops.VQ_ERR_VALUE
    assert _sample(k=0) == ops.VQ_ERR_VALUE and _sample(k=33) == ops.VQ_ERR_VALUE
    for tp in (0.0, 1.5, nan):
        assert _sample(tp=tp) == ops.VQ_ERR_VALUE
    assert _sample(lg=A + 2) == ops.VQ_ERR_ALIGN
    assert _sample(ws=None) == ops.VQ_ERR_WORKSPACE
    assert _sample(wsn=64) == ops.VQ_ERR_WORKSPACE
    assert _sample(R=1, draft=None, ws=None) == ops.VQ_ERR_WORKSPACE  # R = 1 needs no draft


def test_sample_workspace_bytes():
    L = ops.lib()
    assert L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 0, 1000, 0) == 0
    assert L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 33, 1000, 0) == 0
    assert L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 8, (1 << 20) + 1, 0) == 0
    # chunk candidate lists: ceil(V / 8192) chunks x 4 waves x 32 keys of 8 bytes per row
    assert L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 8, 248320, 0) >= 8 * 31 * 4 * 32 * 8
    assert L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 32, 248320, 0) > L.vq_workspace_bytes(ops.VQ_OP_SAMPLE, 8, 248320, 0)


def test_workspace_bytes():
    L = ops.lib()
    assert L.vq_workspace_bytes(ops.VQ_OP_NVFP4, 0, 10, 128) == 0
    assert L.vq_workspace_bytes(ops.VQ_OP_NVFP4, 8, 10, 64) == 0
    assert L.vq_workspace_bytes(ops.VQ_OP_NVFP4, 8, 10, 128) > 0
    assert L.vq_workspace_bytes(9, 8, 10, 64) == 0
    for op in (ops.VQ_OP_NVFP4, ops.VQ_OP_NVFP4_SILU_MUL, ops.VQ_OP_FP8, ops.VQ_OP_LMHEAD):
        sizes = {L.vq_workspace_bytes(op, m, 17408, 5120) for m in (1, 8, 16, 24, 32)}
        assert len(sizes) == 1 and sizes.pop() > 0          # M-independent
    assert L.vq_workspace_bytes(ops.VQ_OP_LMHEAD, 8, 248320, 5120) > L.vq_workspace_bytes(ops.VQ_OP_NVFP4, 8, 248320, 5120)


def test_packed_bytes():
    L = ops.lib()
    # 64-row tiles x 128-K iterations; NVFP4 blocks 4096 B of codes + 512 B of
    # scales (9 bytes per 16 weights), FP8 blocks 8192 B (one byte per weight)
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4, 64, 128) == 4608 == 64 * 128 * 9 // 16
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4, 65, 256) == 2 * 2 * 4608
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, 64, 128) == 4608
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, 66, 128) == 2 * 4608
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, 63, 128) == 0
    assert L.vq_packed_bytes(ops.VQ_PACK_FP8, 130, 384) == 3 * 3 * 8192
    assert L.vq_packed_bytes(ops.VQ_PACK_FP8, 0, 128) == 0
    assert L.vq_packed_bytes(ops.VQ_PACK_FP8, 64, 100) == 0
    assert L.vq_packed_bytes(7, 64, 128) == 0
    # the model's matrices pack without padding (row counts are multiples of 64)
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, 2 * 17408, 5120) == 2 * 17408 * 5120 * 9 // 16
    assert L.vq_packed_bytes(ops.VQ_PACK_NVFP4, 248320, 5120) == 248320 * 5120 * 9 // 16


def test_affine_validation():
    L = ops.lib()
    n = 1 << 30
    assert L.vq_pack_affine_q4(A, A, None, 64, 128, 0, A, n, None) == ops.VQ_ERR_NULL
    assert L.vq_pack_affine_q4(A, A, A, 64, 128, 2, A, n, None) == ops.VQ_ERR_VALUE
    assert L.vq_pack_affine_q4(A, A, A, 63, 128, 1, A, n, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_affine_q4(A, A, A, 64, 64, 0, A, n, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_affine_q4(A, A, A + 2, 64, 128, 0, A, n, None) == ops.VQ_ERR_ALIGN
    assert L.vq_pack_affine_q4(A, A, A, 64, 128, 0, A, 4607, None) == ops.VQ_ERR_SHAPE
    g = L.vq_gemm_affine_q4
    assert g(None, A, n, A, 0, 8, 64, 128, 0, A, n, None) == ops.VQ_ERR_NULL
    assert g(A, A, n, A, 3, 8, 64, 128, 0, A, n, None) == ops.VQ_ERR_VALUE
    assert g(A, A, n, A, 0, 8, 64, 128, 2, A, n, None) == ops.VQ_ERR_VALUE
    assert g(A, A, n, A, 0, 33, 64, 128, 0, A, n, None) == ops.VQ_ERR_SHAPE
    assert g(A, A, n, A, 0, 8, 64, 192, 0, A, n, None) == ops.VQ_ERR_SHAPE
    assert g(A, A, 4607, A, 0, 8, 64, 128, 0, A, n, None) == ops.VQ_ERR_SHAPE
    assert g(A, A, n, A, 0, 8, 64, 128, 0, A, 8, None) == ops.VQ_ERR_WORKSPACE
    # same packed sizes as NVFP4: 9 bytes per 16 weights
    for rows, k in ((64, 128), (130, 512), (2 * 17408, 5120)):
        assert L.vq_packed_bytes(ops.VQ_PACK_AFFINE_Q4, rows, k) == L.vq_packed_bytes(ops.VQ_PACK_NVFP4, rows, k)
        assert L.vq_packed_bytes(ops.VQ_PACK_AFFINE_Q4_GATE_UP, rows, k) == \
            L.vq_packed_bytes(ops.VQ_PACK_NVFP4_GATE_UP, rows, k)
    assert L.vq_workspace_bytes(ops.VQ_OP_AFFINE_Q4, 8, 5120, 17408) == L.vq_workspace_bytes(ops.VQ_OP_NVFP4, 8, 5120, 17408)


def test_pack_validation():
    L = ops.lib()
    n = 1 << 30
    assert L.vq_pack_nvfp4(None, A, 64, 128, 0, A, n, None) == ops.VQ_ERR_NULL
    assert L.vq_pack_nvfp4(A, A, 64, 128, 2, A, n, None) == ops.VQ_ERR_VALUE
    assert L.vq_pack_nvfp4(A, A, 63, 128, 1, A, n, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_nvfp4(A, A, 64, 96, 0, A, n, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_nvfp4(A, A + 1, 64, 128, 0, A, n, None) == ops.VQ_ERR_ALIGN
    assert L.vq_pack_nvfp4(A, A, 64, 128, 0, A, 4607, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_fp8(A, 64, 128, None, n, None) == ops.VQ_ERR_NULL
    assert L.vq_pack_fp8(A, 0, 128, A, n, None) == ops.VQ_ERR_SHAPE
    assert L.vq_pack_fp8(A, 64, 128, A + 8, n, None) == ops.VQ_ERR_ALIGN
    assert L.vq_pack_fp8(A, 64, 128, A, 8191, None) == ops.VQ_ERR_SHAPE


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


S0 = 1 << 32           # fake state slots, far enough apart not to overlap
S1 = S0 + (1 << 31)


def _gdn(si=S0, so=S1, q=A, k=A, v=A, a=A, b=A, o=A, B=2, T=8, H=48, Hk=16):
    return ops.lib().vq_gdn_verify(si, so, q, k, v, a, b, o, B, T, H, Hk, None)


def _commit(acc=A, lanes=2, B=4, T=8, H=48, Hk=16, si=S0, so=S1):
    return ops.lib().vq_gdn_commit(si, so, A, A, A, A, A, acc, lanes, B, T, H, Hk, None)


def test_gdn_validation():
    assert _gdn(si=None) == ops.VQ_ERR_NULL
    assert _gdn(k=None) == ops.VQ_ERR_NULL
    assert _gdn(b=None) == ops.VQ_ERR_NULL
    assert _gdn(B=0) == ops.VQ_ERR_SHAPE
    assert _gdn(T=0) == ops.VQ_ERR_SHAPE
    assert _gdn(T=17) == ops.VQ_ERR_SHAPE
    assert _gdn(Hk=0) == ops.VQ_ERR_SHAPE
    assert _gdn(H=48, Hk=96) == ops.VQ_ERR_SHAPE
    assert _gdn(H=48, Hk=5) == ops.VQ_ERR_SHAPE
    assert _gdn(q=A + 4) == ops.VQ_ERR_ALIGN
    assert _gdn(k=A + 8) == ops.VQ_ERR_ALIGN
    assert _gdn(v=A + 2) == ops.VQ_ERR_ALIGN
    assert _gdn(o=A + 1) == ops.VQ_ERR_ALIGN
    # the two slots must not overlap: 2 entries x 48 heads x 64 KiB = 6 MiB
    assert _gdn(so=S0 + (6 << 20) - 4) == ops.VQ_ERR_VALUE
    assert _gdn(si=S1, so=S1) == ops.VQ_ERR_VALUE
    assert _commit(acc=None) == ops.VQ_ERR_NULL
    assert _commit(lanes=0) == ops.VQ_ERR_SHAPE
    assert _commit(lanes=5, B=5) == ops.VQ_ERR_SHAPE
    assert _commit(lanes=3, B=4) == ops.VQ_ERR_SHAPE
    assert _commit(acc=A + 2) == ops.VQ_ERR_ALIGN
    assert "lanes" in (_commit(lanes=3, B=4) and ops.last_error())


@pytest.mark.skipif(_gpu_visible(), reason="would pass validation and launch with fake pointers")
def test_valid_call_without_gpu_reports_device_error():
    assert _nvfp4() == ops.VQ_ERR_DEVICE
    assert ops.lib().vq_pack_fp8(A, 64, 128, A, 1 << 30, None) == ops.VQ_ERR_DEVICE
    assert ops.lib().vq_probe_copy(A, A, 1024, None) == ops.VQ_ERR_DEVICE
    assert _sample() == ops.VQ_ERR_DEVICE
    assert _gdn(so=S0 + (6 << 20)) == ops.VQ_ERR_DEVICE  # adjacent slots do not overlap
    assert _gdn(o=None) == ops.VQ_ERR_DEVICE
    assert _commit() == ops.VQ_ERR_DEVICE


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        ops.lib()


def _noalloc(x=A, w=A, wn=1 << 30, y=A, yd=0, M=8, N=1024, K=512, epi=0):
    return ops.lib().vq_gemm_nvfp4_noalloc(x, w, wn, 1.0, y, yd, M, N, K, epi, None)


def test_gemm_nvfp4_noalloc_validation():
    # the allocation-free variant checks the same arguments, plus the size its
    # static scratch holds (65,536 tiles: N <= 4,194,304, or 2,097,152 with
    # SILU_MUL), before any HIP call
    assert _noalloc(x=None) == ops.VQ_ERR_NULL
    assert _noalloc(w=None) == ops.VQ_ERR_NULL
    assert _noalloc(M=0) == ops.VQ_ERR_SHAPE
    assert _noalloc(M=33) == ops.VQ_ERR_SHAPE
    assert _noalloc(K=96) == ops.VQ_ERR_SHAPE
    assert _noalloc(yd=2) == ops.VQ_ERR_VALUE
    assert _noalloc(epi=2) == ops.VQ_ERR_VALUE
    assert _noalloc(N=4194305) == ops.VQ_ERR_SHAPE
    assert "scratch" in ops.last_error()
    assert _noalloc(N=2097153, epi=1) == ops.VQ_ERR_SHAPE
    assert _noalloc(x=A + 8) == ops.VQ_ERR_ALIGN
    assert _noalloc(wn=100) == ops.VQ_ERR_SHAPE
