"""Thin Python binding of libverify (include/libverify.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype/shape/contiguity, and passes raw device
pointers and the current HIP stream to the C ABI. All arithmetic runs in the
HIP kernels of libverify.so; there is no fallback of any kind, and a missing
library raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libverify.so")

VQ_OK = 0
VQ_ERR_NULL = 1
VQ_ERR_SHAPE = 2
VQ_ERR_ALIGN = 3
VQ_ERR_WORKSPACE = 4
VQ_ERR_DEVICE = 5
VQ_ERR_LAUNCH = 6
VQ_ERR_VALUE = 7

VQ_OUT_BF16 = 0
VQ_OUT_F32 = 1
VQ_EPI_NONE = 0
VQ_EPI_SILU_MUL = 1
VQ_OP_NVFP4 = 0
VQ_OP_NVFP4_SILU_MUL = 1
VQ_OP_FP8 = 2
VQ_OP_LMHEAD = 3
VQ_OP_SAMPLE = 4
VQ_OP_AFFINE_Q4 = 5
VQ_OP_AFFINE_Q4_SILU_MUL = 6
VQ_OP_FP8_ACCUMULATE = 7
VQ_PACK_NVFP4 = 0
VQ_PACK_NVFP4_GATE_UP = 1
VQ_PACK_FP8 = 2
VQ_PACK_AFFINE_Q4 = 3
VQ_PACK_AFFINE_Q4_GATE_UP = 4

EXPORTS = [
    "vq_packed_bytes", "vq_pack_nvfp4", "vq_pack_fp8", "vq_pack_affine_q4", "vq_gemm_affine_q4",
    "vq_gemm_nvfp4", "vq_gemm_nvfp4_noalloc", "vq_gemm_fp8", "vq_gemm_fp8_accumulate", "vq_lmhead_argmax_accept",
    "vq_sample_accept", "vq_gdn_verify", "vq_gdn_commit", "vq_workspace_bytes", "vq_schedule_info",
    "vq_status_str", "vq_last_error", "vq_abi_version", "vq_probe_copy", "vq_probe_read",
]


class VerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libverify.so (built in-tree by bit_block_scaled_vq_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libverify.so is not built ({LIB_PATH}); run `python -m bit_block_scaled_vq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    L.vq_packed_bytes.argtypes = [i32, i32, i32]
    L.vq_packed_bytes.restype = sz
    L.vq_pack_nvfp4.argtypes = [vp, vp, i32, i32, i32, vp, sz, vp]
    L.vq_pack_nvfp4.restype = i32
    L.vq_pack_fp8.argtypes = [vp, i32, i32, vp, sz, vp]
    L.vq_pack_fp8.restype = i32
    L.vq_gemm_nvfp4.argtypes = [vp, vp, sz, f32, vp, i32, i32, i32, i32, i32, vp, sz, vp]
    L.vq_gemm_nvfp4.restype = i32
    L.vq_gemm_nvfp4_noalloc.argtypes = [vp, vp, sz, f32, vp, i32, i32, i32, i32, i32, vp]
    L.vq_gemm_nvfp4_noalloc.restype = i32
    L.vq_pack_affine_q4.argtypes = [vp, vp, vp, i32, i32, i32, vp, sz, vp]
    L.vq_pack_affine_q4.restype = i32
    L.vq_gemm_affine_q4.argtypes = [vp, vp, sz, vp, i32, i32, i32, i32, i32, vp, sz, vp]
    L.vq_gemm_affine_q4.restype = i32
    L.vq_gemm_fp8.argtypes = [vp, vp, sz, f32, vp, i32, i32, i32, i32, vp, sz, vp]
    L.vq_gemm_fp8.restype = i32
    L.vq_gemm_fp8_accumulate.argtypes = [vp, vp, sz, f32, vp, i32, i32, i32, vp]
    L.vq_gemm_fp8_accumulate.restype = i32
    L.vq_lmhead_argmax_accept.argtypes = [vp, vp, sz, f32, vp, i32, i32, i32, i32,
                                          vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.vq_lmhead_argmax_accept.restype = i32
    L.vq_sample_accept.argtypes = [vp, i32, i32, i32, f32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.vq_sample_accept.restype = i32
    L.vq_gdn_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    L.vq_gdn_verify.restype = i32
    L.vq_gdn_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.vq_gdn_commit.restype = i32
    L.vq_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.vq_workspace_bytes.restype = sz
    pi = ctypes.POINTER(i32)
    L.vq_schedule_info.argtypes = [i32, i32, i32, i32, pi, pi, pi]
    L.vq_schedule_info.restype = i32
    L.vq_status_str.argtypes = [i32]
    L.vq_status_str.restype = ctypes.c_char_p
    L.vq_last_error.argtypes = []
    L.vq_last_error.restype = ctypes.c_char_p
    L.vq_abi_version.argtypes = []
    L.vq_abi_version.restype = i32
    L.vq_probe_copy.argtypes = [vp, vp, sz, vp]
    L.vq_probe_copy.restype = i32
    L.vq_probe_read.argtypes = [vp, sz, vp, vp]
    L.vq_probe_read.restype = i32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().vq_status_str(int(status)).decode()


def last_error() -> str:
    return lib().vq_last_error().decode()


def _check(status: int):
    if status != VQ_OK:
        raise VerifyError(status, last_error())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _out_dtype(t) -> int:
    torch = _torch()
    return VQ_OUT_F32 if t.dtype == torch.float32 else VQ_OUT_BF16


def workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(lib().vq_workspace_bytes(op, M, N, K))


def schedule_info(op: int, N: int, K: int, M: int = 8):
    """(units, iterations per unit, workgroups) of the split a call of op with
    M rows uses (M matters only for the NVFP4 ops: M <= 8 or M > 8)."""
    u, i, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().vq_schedule_info(op, M, N, K, ctypes.byref(u), ctypes.byref(i), ctypes.byref(g)))
    return u.value, i.value, g.value


def workspace(op: int, M: int, N: int, K: int, device="cuda"):
    """A zero-filled workspace for `op` at (N, K): bound to that (op, N, K),
    reusable by any number of stream-ordered calls of it at any M."""
    torch = _torch()
    n = workspace_bytes(op, M, N, K)
    if n == 0:
        raise VerifyError(VQ_ERR_SHAPE, f"invalid shape for workspace: M={M} N={N} K={K}")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def packed_bytes(kind: int, rows: int, K: int) -> int:
    return int(lib().vq_packed_bytes(kind, rows, K))


def pack_nvfp4(codes, scales, gate_up: bool = False, stream=None):
    """Packed form (1-D uint8 device tensor) of a canonical NVFP4 matrix
    codes [rows][K/2], scales [rows][K/16]; gate_up packs a fused [gate; up]
    matrix for VQ_EPI_SILU_MUL."""
    torch = _torch()
    _need(codes, "codes", (torch.uint8,), 2)
    _need(scales, "scales", (torch.uint8,), 2)
    rows, K = codes.shape[0], 2 * codes.shape[1]
    if tuple(scales.shape) != (rows, K // 16):
        raise ValueError(f"shape mismatch: codes {tuple(codes.shape)} scales {tuple(scales.shape)}")
    n = packed_bytes(VQ_PACK_NVFP4_GATE_UP if gate_up else VQ_PACK_NVFP4, rows, K)
    if n == 0:
        raise VerifyError(VQ_ERR_SHAPE, f"invalid shape for packing: rows={rows} K={K}")
    out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _check(lib().vq_pack_nvfp4(_ptr(codes), _ptr(scales), rows, K, int(bool(gate_up)), _ptr(out), n,
                               _stream(stream)))
    return out


def pack_fp8(w, stream=None):
    """Packed form (1-D uint8 device tensor) of a canonical E4M3 matrix w [rows][K]."""
    torch = _torch()
    _need(w, "w", (torch.uint8,), 2)
    rows, K = w.shape
    n = packed_bytes(VQ_PACK_FP8, rows, K)
    if n == 0:
        raise VerifyError(VQ_ERR_SHAPE, f"invalid shape for packing: rows={rows} K={K}")
    out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check(lib().vq_pack_fp8(_ptr(w), rows, K, _ptr(out), n, _stream(stream)))
    return out


def pack_affine_q4(codes, scales, biases, gate_up: bool = False, stream=None):
    """Packed form (1-D uint8 device tensor) of an affine 4-bit matrix: codes
    uint8 [rows][K/2], scales and biases bf16 (or their int16 bit patterns)
    [rows][K/64]; gate_up packs a fused [gate; up] matrix for VQ_EPI_SILU_MUL."""
    torch = _torch()
    _need(codes, "codes", (torch.uint8,), 2)
    _need(scales, "scales", (torch.bfloat16, torch.int16), 2)
    _need(biases, "biases", (torch.bfloat16, torch.int16), 2)
    rows, K = codes.shape[0], 2 * codes.shape[1]
    if tuple(scales.shape) != (rows, K // 64) or tuple(biases.shape) != (rows, K // 64):
        raise ValueError(f"shape mismatch: codes {tuple(codes.shape)} scales {tuple(scales.shape)} "
                         f"biases {tuple(biases.shape)}")
    n = packed_bytes(VQ_PACK_AFFINE_Q4_GATE_UP if gate_up else VQ_PACK_AFFINE_Q4, rows, K)
    if n == 0:
        raise VerifyError(VQ_ERR_SHAPE, f"invalid shape for packing: rows={rows} K={K}")
    out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _check(lib().vq_pack_affine_q4(_ptr(codes), _ptr(scales), _ptr(biases), rows, K, int(bool(gate_up)), _ptr(out),
                                   n, _stream(stream)))
    return out


def vq_gemm_affine_q4(x, w, y, epilogue: int = VQ_EPI_NONE, workspace=None, stream=None):
    """y[M][N] = x . W^T (affine 4-bit W, packed by pack_affine_q4), or
    silu(gate)*up for VQ_EPI_SILU_MUL (w packed with gate_up=True)."""
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(y, "y", (torch.bfloat16, torch.float32), 2)
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} y {tuple(y.shape)}")
    ws_ptr, ws_n = _ws(workspace)
    _check(lib().vq_gemm_affine_q4(_ptr(x), _ptr(w), w.numel(), _ptr(y), _out_dtype(y), M, N, K, int(epilogue),
                                   ws_ptr, ws_n, _stream(stream)))
    return y


def _ws(workspace):
    return (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)


def vq_gemm_nvfp4(x, w, tensor_scale: float, y, epilogue: int = VQ_EPI_NONE, workspace=None, stream=None):
    """y[M][N] = x . W^T (NVFP4 W, packed by pack_nvfp4), or silu(gate)*up for
    VQ_EPI_SILU_MUL (w packed with gate_up=True)."""
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(y, "y", (torch.bfloat16, torch.float32), 2)
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} y {tuple(y.shape)}")
    ws_ptr, ws_n = _ws(workspace)
    _check(lib().vq_gemm_nvfp4(_ptr(x), _ptr(w), w.numel(), float(tensor_scale), _ptr(y),
                               _out_dtype(y), M, N, K, int(epilogue), ws_ptr, ws_n, _stream(stream)))
    return y


def vq_gemm_nvfp4_noalloc(x, w, tensor_scale: float, y, epilogue: int = VQ_EPI_NONE, stream=None):
    """vq_gemm_nvfp4 with the library's static per-device scratch instead of a
    workspace: nothing is allocated; calls that may overlap on one device race."""
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(y, "y", (torch.bfloat16, torch.float32), 2)
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} y {tuple(y.shape)}")
    _check(lib().vq_gemm_nvfp4_noalloc(_ptr(x), _ptr(w), w.numel(), float(tensor_scale), _ptr(y),
                                       _out_dtype(y), M, N, K, int(epilogue), _stream(stream)))
    return y


def vq_gemm_fp8(x, w, w_scale: float, y, workspace=None, stream=None):
    """y[M][N] = (x . E4M3(W)^T) * w_scale, W packed by pack_fp8."""
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(y, "y", (torch.bfloat16, torch.float32), 2)
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} y {tuple(y.shape)}")
    ws_ptr, ws_n = _ws(workspace)
    _check(lib().vq_gemm_fp8(_ptr(x), _ptr(w), w.numel(), float(w_scale), _ptr(y), _out_dtype(y), M, N, K,
                             ws_ptr, ws_n, _stream(stream)))
    return y


def vq_gemm_fp8_accumulate(x, w, w_scale: float, y, stream=None):
    """y[M][N] (fp32) += (x . E4M3(W)^T) * w_scale, W packed by pack_fp8; no
    workspace. Deterministic when y holds zeros on entry."""
    torch = _torch()
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(y, "y", (torch.float32,), 2)
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} y {tuple(y.shape)}")
    _check(lib().vq_gemm_fp8_accumulate(_ptr(x), _ptr(w), w.numel(), float(w_scale), _ptr(y), M, N, K,
                                        _stream(stream)))
    return y


def vq_lmhead_argmax_accept(h, w, tensor_scale: float, V: int, draft, lanes: int, R: int,
                            argmax_out, accept_len_out, maxlogit_out=None, commit_out=None,
                            logits_out=None, workspace=None, stream=None):
    """Vocabulary head (W [V][K] packed by pack_nvfp4) + per-row argmax + greedy
    accept; results stay on the device."""
    torch = _torch()
    _need(h, "h", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 1)
    _need(argmax_out, "argmax_out", (torch.int32,), 1)
    _need(accept_len_out, "accept_len_out", (torch.int32,), 1)
    if draft is not None:
        _need(draft, "draft", (torch.int32,), 2)
    if maxlogit_out is not None:
        _need(maxlogit_out, "maxlogit_out", (torch.float32,), 1)
    if commit_out is not None:
        _need(commit_out, "commit_out", (torch.int32,), 2)
    if logits_out is not None:
        _need(logits_out, "logits_out", (torch.bfloat16, torch.float32), 2)
    M, K = h.shape
    if M != lanes * R:
        raise ValueError("h must have lanes * R rows")
    if argmax_out.numel() != M or accept_len_out.numel() != lanes:
        raise ValueError("output sizes do not match lanes and R")
    if draft is not None and tuple(draft.shape) != (lanes, R - 1):
        raise ValueError("draft must be [lanes][R-1]")
    if commit_out is not None and tuple(commit_out.shape) != (lanes, R):
        raise ValueError("commit_out must be [lanes][R]")
    if logits_out is not None and tuple(logits_out.shape) != (M, V):
        raise ValueError("logits_out must be [M][V]")
    ws_ptr, ws_n = _ws(workspace)
    ld = _out_dtype(logits_out) if logits_out is not None else VQ_OUT_F32
    _check(lib().vq_lmhead_argmax_accept(
        _ptr(h), _ptr(w), w.numel(), float(tensor_scale), _ptr(draft), lanes, R, V, K,
        _ptr(argmax_out), _ptr(maxlogit_out), _ptr(accept_len_out), _ptr(commit_out),
        _ptr(logits_out), ld, ws_ptr, ws_n, _stream(stream)))


def vq_sample_accept(logits, lanes: int, R: int, temperature: float, top_k: int, top_p: float, u_draw,
                     accept_len_out, draft=None, draft_ids=None, draft_probs=None, u_accept=None,
                     token_out=None, commit_out=None, cand_out=None, prob_out=None, workspace=None, stream=None):
    """Sampled verify over fp32 logits [lanes*R][V]: truncated target
    distribution per row, a draw with u_draw, and the accept scan per lane
    (point-mass rule without draft_ids/draft_probs, speculative sampling with
    them). Results stay on the device."""
    torch = _torch()
    _need(logits, "logits", (torch.float32,), 2)
    M, V = logits.shape
    if M != lanes * R:
        raise ValueError("logits must have lanes * R rows")
    _need(u_draw, "u_draw", (torch.float32,))
    _need(accept_len_out, "accept_len_out", (torch.int32,))
    if u_draw.numel() != M or accept_len_out.numel() != lanes:
        raise ValueError("u_draw must hold lanes * R values and accept_len_out lanes")
    for name, t, dt, n in (("draft", draft, torch.int32, lanes * (R - 1)),
                           ("draft_ids", draft_ids, torch.int32, lanes * (R - 1) * 16),
                           ("draft_probs", draft_probs, torch.float32, lanes * (R - 1) * 16),
                           ("u_accept", u_accept, torch.float32, M),
                           ("token_out", token_out, torch.int32, M),
                           ("commit_out", commit_out, torch.int32, lanes * R),
                           ("cand_out", cand_out, torch.int32, M * 32),
                           ("prob_out", prob_out, torch.float32, M * 32)):
        if t is not None:
            _need(t, name, (dt,))
            if t.numel() != n:
                raise ValueError(f"{name} must hold {n} values")
    ws_ptr, ws_n = _ws(workspace)
    _check(lib().vq_sample_accept(
        _ptr(logits), lanes, R, V, float(temperature), int(top_k), float(top_p), _ptr(draft), _ptr(draft_ids),
        _ptr(draft_probs), _ptr(u_accept), _ptr(u_draw), _ptr(token_out), _ptr(accept_len_out),
        _ptr(commit_out), _ptr(cand_out), _ptr(prob_out), ws_ptr, ws_n, _stream(stream)))


def _gdn_args(state_in, state_out, q, k, v, a, b, o=None):
    torch = _torch()
    f32 = (torch.float32,)
    _need(state_in, "state_in", f32, 4)
    _need(state_out, "state_out", f32, 4)
    B, H, dk, dv = state_in.shape
    if state_out.shape != state_in.shape or (dk, dv) != (128, 128):
        raise ValueError("states must be [B][H][128][128] fp32 and of the same shape")
    _need(q, "q", f32, 4)
    _need(k, "k", f32, 4)
    T, Hk = q.shape[1], q.shape[2]
    if q.shape != (B, T, Hk, 128) or k.shape != q.shape:
        raise ValueError("q and k must be [B][T][Hk][128]")
    _need(v, "v", f32, 4)
    if v.shape != (B, T, H, 128):
        raise ValueError("v must be [B][T][H][128]")
    for name, t in (("a", a), ("b", b)):
        _need(t, name, f32, 3)
        if t.shape != (B, T, H):
            raise ValueError(f"{name} must be [B][T][H]")
    if o is not None:
        _need(o, "o", f32, 4)
        if o.shape != v.shape:
            raise ValueError("o must be [B][T][H][128]")
    return B, T, H, Hk


def vq_gdn_verify(state_in, state_out, q, k, v, a, b, o=None, stream=None):
    """Gated DeltaNet state stream of the verify pass: every entry scans its T
    rows from state_in and writes the final state to state_out (the other
    parity slot) and, if given, the row outputs to o."""
    B, T, H, Hk = _gdn_args(state_in, state_out, q, k, v, a, b, o)
    _check(lib().vq_gdn_verify(_ptr(state_in), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                               _ptr(o), B, T, H, Hk, _stream(stream)))


def vq_gdn_commit(state_in, state_out, q, k, v, a, b, accept_len, lanes: int, stream=None):
    """Commit pass: entries whose lane accepted fewer than T rows get the
    re-scan of their accepted rows from state_in; the others keep state_out."""
    torch = _torch()
    B, T, H, Hk = _gdn_args(state_in, state_out, q, k, v, a, b)
    _need(accept_len, "accept_len", (torch.int32,))
    if accept_len.numel() != lanes:
        raise ValueError("accept_len must hold one count per lane")
    _check(lib().vq_gdn_commit(_ptr(state_in), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                               _ptr(accept_len), lanes, B, T, H, Hk, _stream(stream)))


def vq_probe_copy(src, dst, stream=None):
    _check(lib().vq_probe_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(), _stream(stream)))


def vq_probe_read(src, sink, stream=None):
    _check(lib().vq_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))
