"""Seeded synthetic inputs for the verify-pass weight stream.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds none of the method's arithmetic: it only draws random numbers and rounds
them to the storage formats with PyTorch's own casts (fp32 -> bf16 and
fp32 -> float8_e4m3fn, both round-to-nearest-even). Decoding, products,
argmax and accept live elsewhere.

Distributions (the synthetic stand-in for the 27B checkpoint the pages read):
  * activations: standard normal, rounded to bf16;
  * NVFP4 codes: uniform over the 16 E2M1 codes (each random byte is two
    independent uniform nibbles);
  * NVFP4 block scales: |N(0,1)| * 0.05 rounded to E4M3FN, one per 16 K;
  * FP8 projection weights: N(0, 0.02) rounded to E4M3FN;
  * drafts: draft j equals the target argmax of row j with probability 0.7,
    otherwise a uniform token id in [0, V).
  * Gated DeltaNet state stream (fp32): state N(0, 0.05); queries and keys
    unit vectors (normalised Gaussians, as after the Q/K norm); values
    N(0, 1); decays exp(-|N(0, 0.1)|) in (0, 1]; write strengths
    sigmoid(N(0, 1)) in (0, 1).

Host generation uses numpy PCG64 with one SeedSequence per (key..., chunk)
so any chunk of any tensor can be regenerated on its own. Device generation
(for the multi-gigabyte pass) uses torch's device Philox generator seeded
from the same key; the two routes give different numbers with the same
distributions.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
import zlib

import numpy as np

SEED = 0
CHUNK_ROWS = 4096

# tensor ids inside a spawn key
T_X = 0
T_CODES = 1
T_SCALES = 2
T_FP8 = 3
T_DRAFT = 4
T_LOGITS = 5
T_UNIFORM = 6
T_DRAFT_Q = 7
T_AFFINE = 8
T_GDN = 9

LOGIT_STD = 2.5

SCALE_STD = 0.05
FP8_STD = 0.02
DRAFT_P = 0.7


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=tuple(int(k) for k in key))))


def _torch():
    import torch
    return torch


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(f32: np.ndarray) -> np.ndarray:
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- host side

def x_bf16(key, m: int, k: int) -> np.ndarray:
    """Activations [m][k] as bf16 bit patterns (uint16)."""
    g = rng(*key, T_X)
    return to_bf16_bits(g.standard_normal((m, k), dtype=np.float32))


def _nvfp4_chunk(key, chunk, rows, k):
    gc = rng(*key, T_CODES, chunk)
    codes = gc.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    gs = rng(*key, T_SCALES, chunk)
    sc = np.abs(gs.standard_normal((rows, k // 16), dtype=np.float32)) * np.float32(SCALE_STD)
    return codes, to_e4m3_bits(sc)


def nvfp4_weights(key, n: int, k: int):
    """NVFP4 matrix [n][k]: codes uint8 [n][k/2], block scales uint8 [n][k/16]."""
    assert k % 32 == 0
    codes = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // 16), dtype=np.uint8)
    chunks = [(c, r0, min(n, r0 + CHUNK_ROWS)) for c, r0 in enumerate(range(0, n, CHUNK_ROWS))]

    def work(item):
        c, r0, r1 = item
        cc, ss = _nvfp4_chunk(key, c, r1 - r0, k)
        codes[r0:r1] = cc
        scales[r0:r1] = ss

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, chunks))
    return codes, scales


def fp8_weights(key, n: int, k: int, std: float = FP8_STD) -> np.ndarray:
    """FP8 E4M3FN matrix [n][k] as uint8 codes."""
    out = np.empty((n, k), dtype=np.uint8)
    chunks = [(c, r0, min(n, r0 + CHUNK_ROWS)) for c, r0 in enumerate(range(0, n, CHUNK_ROWS))]

    def work(item):
        c, r0, r1 = item
        g = rng(*key, T_FP8, c)
        out[r0:r1] = to_e4m3_bits(g.standard_normal((r1 - r0, k), dtype=np.float32) * np.float32(std))

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, chunks))
    return out


def drafts(key, argmax_rows: np.ndarray, vocab: int, p: float = DRAFT_P) -> np.ndarray:
    """Drafts [lanes][R-1] (int32): draft j is argmax_rows[l][j] with
    probability p, otherwise uniform in [0, vocab). A chance match is allowed."""
    a = np.asarray(argmax_rows, dtype=np.int64)
    lanes, r = a.shape
    g = rng(*key, T_DRAFT)
    u = g.random((lanes, r - 1))
    rand_ids = g.integers(0, vocab, size=(lanes, r - 1))
    return np.where(u < p, a[:, : r - 1], rand_ids).astype(np.int32)


def affine_weights(key, n: int, k: int):
    """Affine 4-bit matrix [n][k]: (codes uint8 [n][k/2], scales and biases as
    bf16 bit patterns uint16 [n][k/64])."""
    codes = np.empty((n, k // 2), dtype=np.uint8)
    sb = np.empty((n, k // 64), dtype=np.uint16)
    bb = np.empty((n, k // 64), dtype=np.uint16)
    chunks = [(c, r0, min(n, r0 + CHUNK_ROWS)) for c, r0 in enumerate(range(0, n, CHUNK_ROWS))]

    def work(item):
        c, r0, r1 = item
        g = rng(*key, T_AFFINE, c)
        codes[r0:r1] = g.integers(0, 256, size=(r1 - r0, k // 2), dtype=np.uint8)
        s = np.abs(g.standard_normal((r1 - r0, k // 64), dtype=np.float32)) * np.float32(0.004) + np.float32(0.001)
        b = np.float32(-7.5) * s * (np.float32(1) + g.standard_normal((r1 - r0, k // 64), dtype=np.float32) / 5)
        sb[r0:r1] = to_bf16_bits(s)
        bb[r0:r1] = to_bf16_bits(b)

    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, chunks))
    return codes, sb, bb


def logits_f32(key, m: int, v: int, std: float = LOGIT_STD) -> np.ndarray:
    """Verify logits [m][v] (float32), N(0, std^2)."""
    return (rng(*key, T_LOGITS).standard_normal((m, v), dtype=np.float32) * np.float32(std)).astype(np.float32)


def uniforms(key, *shape: int) -> np.ndarray:
    """float32 uniforms in [0, 1)."""
    return rng(*key, T_UNIFORM).random(shape, dtype=np.float32)


def draft_distributions(key, preferred, vocab: int, n: int = 16):
    """Draft distributions for a batch of verify rows: preferred [rows][P]
    token ids (P >= n // 2; -1 entries are skipped). Returns (ids [rows][n]
    int32, probs [rows][n] float32, tokens [rows] int32): per row n // 2 ids
    from its preferred list, the rest uniform over [0, vocab) (a repeat of an
    earlier id is allowed; the first occurrence counts), Dirichlet(1)
    probabilities, and one token drawn from them."""
    pref = np.atleast_2d(np.asarray(preferred, dtype=np.int64))
    rows = pref.shape[0]
    g = rng(*key, T_DRAFT_Q)
    ids = np.empty((rows, n), dtype=np.int32)
    probs = np.empty((rows, n), dtype=np.float32)
    toks = np.empty(rows, dtype=np.int32)
    for r in range(rows):
        cand = pref[r][pref[r] >= 0]
        take = g.choice(cand, size=min(n // 2, cand.size), replace=False) if cand.size else np.empty(0, np.int64)
        ids[r] = np.concatenate([take, g.integers(0, vocab, size=n - take.size)])
        probs[r] = g.dirichlet(np.ones(n)).astype(np.float32)
        toks[r] = ids[r][g.choice(n, p=probs[r].astype(np.float64) / probs[r].astype(np.float64).sum())]
    return ids, probs, toks


def gdn_inputs(key, B: int, T: int, H: int, Hk: int, dk: int = 128, dv: int = 128):
    """(state, q, k, v, a, b) as fp32 arrays: state [B][H][dk][dv],
    q, k [B][T][Hk][dk], v [B][T][H][dv], a, b [B][T][H]."""
    g = rng(*key, T_GDN)
    state = (g.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    q = g.standard_normal((B, T, Hk, dk))
    k = g.standard_normal((B, T, Hk, dk))
    q = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = g.standard_normal((B, T, H, dv)).astype(np.float32)
    a = np.exp(-np.abs(g.standard_normal((B, T, H)) * 0.1)).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-g.standard_normal((B, T, H))))).astype(np.float32)
    return state, q, k, v, a, b


# -------------------------------------------------------------- device side

def _torch_gen(device, *key):
    torch = _torch()
    seed = zlib.crc32(repr((SEED,) + tuple(int(k) for k in key)).encode()) & 0x7FFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_x_bf16(key, m: int, k: int, device):
    torch = _torch()
    g = _torch_gen(device, *key, T_X)
    return torch.randn((m, k), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def device_nvfp4_weights(key, n: int, k: int, device):
    """Same distributions as nvfp4_weights, drawn on the device."""
    torch = _torch()
    g = _torch_gen(device, *key, T_CODES)
    codes = torch.randint(0, 256, (n, k // 2), generator=g, device=device, dtype=torch.uint8)
    g2 = _torch_gen(device, *key, T_SCALES)
    sc = torch.randn((n, k // 16), generator=g2, device=device, dtype=torch.float32).abs_().mul_(SCALE_STD)
    scales = sc.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scales


def device_fp8_weights(key, n: int, k: int, device, std: float = FP8_STD):
    torch = _torch()
    g = _torch_gen(device, *key, T_FP8)
    out = torch.empty((n, k), device=device, dtype=torch.uint8)
    step = max(1, (1 << 28) // max(1, k))
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        w = torch.randn((r1 - r0, k), generator=g, device=device, dtype=torch.float32).mul_(std)
        out[r0:r1] = w.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def device_affine_weights(key, n: int, k: int, device):
    """Same distributions as affine_weights, drawn on the device."""
    torch = _torch()
    g = _torch_gen(device, *key, T_AFFINE)
    codes = torch.randint(0, 256, (n, k // 2), generator=g, device=device, dtype=torch.uint8)
    s = torch.randn((n, k // 64), generator=g, device=device, dtype=torch.float32).abs_().mul_(0.004).add_(0.001)
    b = torch.randn((n, k // 64), generator=g, device=device, dtype=torch.float32).div_(5).add_(1).mul_(s).mul_(-7.5)
    return codes, s.to(torch.bfloat16).view(torch.int16), b.to(torch.bfloat16).view(torch.int16)


def device_drafts(key, argmax_rows, vocab: int, p: float = DRAFT_P):
    """Device-side drafts from a [lanes][R] int tensor of target choices."""
    torch = _torch()
    a = argmax_rows.to(torch.int64)
    lanes, r = a.shape
    g = _torch_gen(a.device, *key, T_DRAFT)
    u = torch.rand((lanes, r - 1), generator=g, device=a.device)
    ids = torch.randint(0, vocab, (lanes, r - 1), generator=g, device=a.device)
    return torch.where(u < p, a[:, : r - 1], ids).to(torch.int32).contiguous()


def device_gdn_inputs(key, B: int, T: int, H: int, Hk: int, device, dk: int = 128, dv: int = 128):
    """Same distributions as gdn_inputs, drawn on the device (fp32 tensors)."""
    torch = _torch()
    g = _torch_gen(device, *key, T_GDN)
    f = dict(generator=g, device=device, dtype=torch.float32)
    state = torch.randn((B, H, dk, dv), **f).mul_(0.05)
    q = torch.randn((B, T, Hk, dk), **f)
    k = torch.randn((B, T, Hk, dk), **f)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((B, T, H, dv), **f)
    a = torch.exp(-torch.randn((B, T, H), **f).mul_(0.1).abs_())
    b = torch.sigmoid(torch.randn((B, T, H), **f))
    return state, q.contiguous(), k.contiguous(), v, a, b
