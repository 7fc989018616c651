"""Shared helpers for the GPU parity tests (imported by tests/test_gpu_*.py)."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

PARITY_TOL = 2e-3        # max|gpu - oracle| / max|oracle| on the fp32-mode output
FLIP_TOL = 1e-5          # elementwise |gpu_f32 - oracle| <= FLIP_TOL * max|oracle| (fp32 accumulation bound)
TIE_GAP = 1e-3           # argmax tie class: oracle top-2 gap <= TIE_GAP


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev_u8(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_dev_bf16(bits):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def bf16_to_bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(gpu))) if gpu.size else 0.0
    return float(np.max(np.abs(gpu - ref)) / denom)


def check_f32(gpu_f32, ref, tol=PARITY_TOL, what=""):
    e = rel_err(gpu_f32, ref)
    say(f"  parity {what}: max|gpu-oracle|/max|oracle| = {e:.3e} (gate {tol:g})")
    assert e <= tol, (what, e)
    return e


def check_bf16_store(gpu_bf16_bits, gpu_f32, ref):
    """bf16 stores: (1) equal RNE of the same kernel's fp32 result bitwise;
    (2) that fp32 result is within FLIP_TOL * max|oracle| of the oracle at
    every element (an fp32-accumulation bound, far inside the 2e-3 gate).
    Together these allow RNE(gpu) != RNE(oracle) only where a bf16 rounding
    boundary lies between the two values (the flip class); such elements are
    counted. The literal bf16-vs-oracle error is reported, not gated: bf16's
    own unit roundoff (2^-8) exceeds 2e-3."""
    import torch
    rne = torch.from_numpy(np.ascontiguousarray(gpu_f32, dtype=np.float32)).to(torch.bfloat16)
    rne_bits = rne.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gpu_bf16_bits, rne_bits), "bf16 store != RNE(fp32 store)"
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.abs(np.asarray(gpu_f32, dtype=np.float64) - ref)
    worst = float(err.max() / scale) if scale > 0 else float(err.max(initial=0.0))
    assert worst <= FLIP_TOL, f"elementwise fp32 error {worst:.3e} > {FLIP_TOL:g} * max|oracle|"
    ob = O.round_to_bf16_bits(ref)
    flips = int(np.count_nonzero(ob != gpu_bf16_bits))
    lit = rel_err(O.bf16_bits_to_f64(gpu_bf16_bits), ref)
    say(f"  bf16 store: {flips} flip-class elements of {ref.size}; fp32 elementwise err {worst:.2e}; "
        f"literal bf16 rel err {lit:.3e} (reported)")
    return lit


# ------------------------------------------------------------ packed layout
# The packed weight layout written out from its description in
# include/libverify.h, with numpy reshapes (no HIP code involved): the GPU pack
# kernels must reproduce it byte for byte.

def _row_map(rows, gate_up):
    """canonical row (or -1) of [tile][sub-tile t][row n]."""
    if gate_up:
        half = rows // 2
        T = -(-half // 32)
        r = (np.arange(T)[:, None, None] * 32 + (np.arange(4)[None, :, None] & 1) * 16
             + np.arange(16)[None, None, :])
        canon = r + (np.arange(4)[None, :, None] >> 1) * half
        return np.where(r < half, canon, -1)
    T = -(-rows // 64)
    r = np.arange(T)[:, None, None] * 64 + np.arange(4)[None, :, None] * 16 + np.arange(16)[None, None, :]
    return np.where(r < rows, r, -1)


def _gather(a, rmap):
    out = np.zeros(rmap.shape + a.shape[1:], dtype=a.dtype)
    ok = rmap >= 0
    out[ok] = a[rmap[ok]]
    return out


def pack_nvfp4_np(codes, scales, gate_up=False):
    rows, kh = codes.shape
    I = 2 * kh // 128
    rmap = _row_map(rows, gate_up)
    T = rmap.shape[0]
    c = _gather(codes, rmap).reshape(T, 4, 16, I, 4, 4, 4)       # T t n I j g b
    c = c.transpose(0, 3, 1, 5, 2, 4, 6).reshape(T, I, 4096)       # T I t g n j b
    s = _gather(scales, rmap).reshape(T, 4, 16, I, 4, 2)          # T t n I j h
    s = s.transpose(0, 3, 5, 2, 1, 4).reshape(T, I, 512)           # T I h n t j
    return np.concatenate([c, s], axis=2).reshape(-1)


def pack_fp8_np(w):
    rows, K = w.shape
    I = K // 128
    rmap = _row_map(rows, False)
    T = rmap.shape[0]
    a = _gather(w, rmap).reshape(T, 4, 16, I, 2, 2, 4, 8)         # T t n I h jj g b
    return a.transpose(0, 3, 1, 4, 6, 2, 5, 7).reshape(-1)         # T I t h g n jj b


def pack_affine_np(codes, scales_bits, biases_bits, gate_up=False):
    """Affine 4-bit packed layout from include/libverify.h: the NVFP4 code
    layout with every code dword in the affine nibble order, then per tile
    row n 32 bytes of (scale, bias) dwords for sub-tiles t = 0..3 and groups
    h = 0, 1."""
    rows, kh = codes.shape
    I = 2 * kh // 128
    rmap = _row_map(rows, gate_up)
    T = rmap.shape[0]
    c = _gather(codes, rmap).reshape(T, 4, 16, I, 4, 4, 4)       # T t n I j g b
    c = c.transpose(0, 3, 1, 5, 2, 4, 6).reshape(T, I, 1024, 4)
    # each code dword in the affine nibble order: even-k nibbles then odd-k
    lo, hi = c & 0x0F, c >> 4
    word = np.zeros(c.shape[:-1], dtype=np.uint32)
    for b in range(4):
        word |= lo[..., b].astype(np.uint32) << (4 * b)
        word |= hi[..., b].astype(np.uint32) << (16 + 4 * b)
    c = word.astype("<u4").view(np.uint8).reshape(T, I, 4096)
    pair = (scales_bits.astype(np.uint32) | (biases_bits.astype(np.uint32) << 16))  # [rows][K/64]
    pw = _gather(pair, rmap).reshape(T, 4, 16, I, 2)                 # T t n I h
    pw = pw.transpose(0, 3, 2, 1, 4).reshape(T, I, 16 * 8)           # T I n t h (dwords)
    sb = pw.astype("<u4").view(np.uint8).reshape(T, I, 512)
    return np.concatenate([c, sb], axis=2).reshape(-1)
