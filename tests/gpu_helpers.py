"""Shared helpers for the GPU parity tests (imported by tests/test_gpu_*.py)."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

PARITY_TOL = 2e-3        # max|gpu - oracle| / max|oracle| on the fp32-mode output
FLIP_TOL = 1e-5          # bf16 flip class: |oracle - midpoint| <= FLIP_TOL * max|oracle|
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
    """The bf16 store equals RNE of the same kernel's fp32 result bitwise, and
    differs from RNE(oracle) only in the flip class, by one ulp."""
    import torch
    rne = torch.from_numpy(np.ascontiguousarray(gpu_f32, dtype=np.float32)).to(torch.bfloat16)
    rne_bits = rne.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gpu_bf16_bits, rne_bits), "bf16 store != RNE(fp32 store)"
    ref = np.asarray(ref, dtype=np.float64)
    ob = O.round_to_bf16_bits(ref)
    diff = np.flatnonzero(ob.reshape(-1) != gpu_bf16_bits.reshape(-1))
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    flat_ref = ref.reshape(-1)
    for i in diff:
        a = O.bf16_bits_to_f64(ob.reshape(-1)[i:i + 1])[0]
        b = O.bf16_bits_to_f64(gpu_bf16_bits.reshape(-1)[i:i + 1])[0]
        assert abs(int(ob.reshape(-1)[i]) - int(gpu_bf16_bits.reshape(-1)[i])) == 1, (i, a, b)
        mid = (a + b) / 2
        assert abs(flat_ref[i] - mid) <= FLIP_TOL * scale, (i, flat_ref[i], a, b)
    lit = rel_err(O.bf16_bits_to_f64(gpu_bf16_bits), ref)
    say(f"  bf16 store: {diff.size} flip-class elements of {ref.size}; literal bf16 rel err {lit:.3e} (reported)")
    return lit
