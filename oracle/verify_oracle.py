"""Plain, slow, obviously-correct CPU oracle of the speculative-decoding verify
pass weight stream: NVFP4 and FP8 E4M3 weight decode, the skinny GEMM, the
SiLU-times-up MLP step, the vocabulary-head argmax and the greedy accept length.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call it. It shares no code,
table or constant with the HIP library, and imports nothing from it.

All floating-point work is done in numpy float64. Every decoded weight is an
exact dyadic rational, so dequantisation is exact and the only rounding is the
fp64 summation of the matrix product.

Sources (titles of the pages the method is described on):
  [P1] "144 tok/s needs 502 GB/s, and Apple sells two M5 Max chips"
       (Splash engine analysis): sections "The engine hard-codes the model",
       "The decode step is one command buffer", "The roof", "Why Apple
       silicon, and why not the M5".
  [P2] "Beating Splash on an M5 Max: where the tokens per second actually
       were": sections "The kernels were not the gap", "What actually moved
       the needle", "The bugs a second reviewer found".
  [P3] "Speculative decoding" (mlx-dspark concepts): sections "One round",
       "Is it really lossless?".
  [P4] "lithos-metal: per-layer megakernels for Qwen3.8-27B on an M5 Max, and
       where the 200 tok/s comes from": sections "What one token costs the
       bus" (byte table, the plain-decode ceiling equation), "How DSpark is
       wired in" (the accept scan), "Formats, and what runs where".

Readings where the pages are silent (each is listed in the design doc):
  * E2M1 and E4M3 are the OCP 8-bit/4-bit formats; E4M3 is the "FN" variant
    (no infinities, NaN only at S.1111.111) because [P4] "Formats" states the
    block-scale codes top out at exactly 448.
  * Within a code byte the low nibble holds the even k, the high nibble the
    odd k. Codes are [N][K/2] bytes, scales [N][K/16] bytes, both row-major by
    output channel with K contiguous.
  * The FP32 tensor scale multiplies ([P4] "Formats").
  * Argmax takes the lowest index among exactly equal maxima, treats -0 as +0
    and never selects NaN; a row with no non-NaN value reports -1.
  * Draft j of a lane is compared with the argmax of verify row j; accept
    length = matched prefix + 1 ([P4] "How DSpark is wired in").
  * Affine 4-bit: w = scale * q + bias with q the unsigned nibble (0..15),
    low nibble = even k, scale and bias bf16 per 64 consecutive K; codes
    [N][K/2], scales and biases [N][K/64] (as bf16 bit patterns).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "e2m1_value", "e4m3fn_value", "E2M1_TABLE", "E4M3FN_TABLE",
    "bf16_bits_to_f64", "round_to_bf16_bits",
    "unpack_nibbles", "dequant_nvfp4", "dequant_fp8",
    "gemm_nvfp4", "gemm_fp8", "mlp_silu_mul", "silu",
    "AFFINE_GROUP", "dequant_affine_q4", "gemm_affine_q4", "mlp_silu_mul_affine",
    "argmax_lowest", "top2_gap", "greedy_accept",
    "bytes_nvfp4", "bytes_fp8", "pass_schedule", "pass_bytes_by_kind",
    "roof_tokens_per_s", "flops_per_byte_nvfp4",
    "exact_gemm_nvfp4_fraction",
    "HIDDEN", "INTER", "VOCAB", "LAYERS", "GDN_IN", "GDN_OUT_K", "ATTN_QG", "ATTN_KV", "ATTN_O_K",
]


# ---------------------------------------------------------------------------
# O1: value tables, written from the format definitions ([P4] "Formats").
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1),
    1 mantissa bit. Exponent field 0 is subnormal: 0.5 * mantissa."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e4m3fn_value(code: int) -> float:
    """Value of an 8-bit E4M3FN code: 1 sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN;
    there are no infinities, so the largest finite magnitude is 448."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = 2.0 ** -6 * (m / 8.0)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


# ---------------------------------------------------------------------------
# bf16 helpers (activations and outputs are bf16; [P4] "Formats").
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16/int16 array) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(y) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest-even, directly from
    fp64 (one rounding). Overflow goes to +-inf; NaN stays NaN."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    flat = y.reshape(-1)
    res = out.reshape(-1)
    for i, v in enumerate(flat):
        res[i] = _round_one_bf16(float(v))
    return out


def _round_one_bf16(v: float) -> int:
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a == 0.0:
        return sign
    # bf16: 8 exponent bits (bias 127), 7 stored mantissa bits.
    # Normal numbers have 8 significant bits; below 2^-126 the spacing is 2^-133.
    m, e = math.frexp(a)          # a = m * 2^e, 0.5 <= m < 1
    if e - 1 >= -126:
        q = 2.0 ** (e - 8)        # spacing of 8-significant-bit numbers at this binade
    else:
        q = 2.0 ** -133
    r = a / q                     # exact (power-of-two scaling)
    n = math.floor(r)
    frac = r - n
    if frac > 0.5 or (frac == 0.5 and (n % 2) == 1):
        n += 1
    val = n * q
    if val >= 2.0 ** 128:
        return sign | 0x7F80
    f32 = np.array([val], dtype=np.float32)   # exact: val has <= 8 significant bits
    return sign | int((f32.view(np.uint32)[0] >> 16) & 0x7FFF)


# ---------------------------------------------------------------------------
# O2/O3: unpack and dequantise.
# ---------------------------------------------------------------------------

def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R][K/2] code bytes -> [R][K] nibble values; byte j holds k=2j in its
    low nibble and k=2j+1 in its high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    r, half = codes.shape
    out = np.empty((r, half * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """W[n,k] = E2M1(code[n,k]) * E4M3(scale[n, k//16]) * tensor_scale, fp64.
    One E4M3 scale per 16 consecutive K elements ([P4] "What one token costs
    the bus": group_size 16; "Formats": the FP32 tensor scale is a multiplier)."""
    nib = unpack_nibbles(codes)
    r, k = nib.shape
    sc = np.asarray(scales, dtype=np.uint8)
    assert sc.shape == (r, k // 16), (sc.shape, (r, k // 16))
    w = E2M1_TABLE[nib]
    s = np.repeat(E4M3FN_TABLE[sc], 16, axis=1)
    return w * s * float(np.float32(tensor_scale))


def dequant_fp8(w: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN weight codes -> fp64 values (the per-tensor scale is applied
    after the product, which is mathematically identical)."""
    return E4M3FN_TABLE[np.asarray(w, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# O4-O7: the products.
# ---------------------------------------------------------------------------

_ROW_CHUNK = 4096


def gemm_nvfp4(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray,
               tensor_scale: float, rows: np.ndarray | None = None) -> np.ndarray:
    """Y[M,N] = X[M,K] . W^T with W dequantised from NVFP4, all in fp64.
    ``rows`` optionally restricts the output to a subset of output channels
    (used to check sampled columns of very large matrices)."""
    x = bf16_bits_to_f64(x_bits)
    if rows is not None:
        rows = np.asarray(rows)
        w = dequant_nvfp4(np.asarray(codes)[rows], np.asarray(scales)[rows], tensor_scale)
        return x @ w.T
    n = codes.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        w = dequant_nvfp4(codes[r0:r1], scales[r0:r1], tensor_scale)
        y[:, r0:r1] = x @ w.T
    return y


def gemm_fp8(x_bits: np.ndarray, w: np.ndarray, w_scale: float,
             rows: np.ndarray | None = None) -> np.ndarray:
    """Y[M,N] = (X[M,K] . E4M3(w)^T) * w_scale in fp64."""
    x = bf16_bits_to_f64(x_bits)
    s = float(np.float32(w_scale))
    if rows is not None:
        return (x @ dequant_fp8(np.asarray(w)[np.asarray(rows)]).T) * s
    n = w.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        y[:, r0:r1] = x @ dequant_fp8(w[r0:r1]).T
    return y * s


# ---------------------------------------------------------------------------
# O11: the affine 4-bit format ([P1] "The engine hard-codes the model": per
# group of 64 inputs, 32 bytes of nibbles plus a bf16 scale and a bf16 bias,
# 9 bytes per 16 weights; [P4] "Formats, and what runs where": the affine INT4
# layout of MLX/AWQ/GPTQ, kept bit-exact; [P2] "What actually moved the
# needle": the bias term needs per-group sums of the inputs).
# ---------------------------------------------------------------------------

AFFINE_GROUP = 64


def dequant_affine_q4(codes: np.ndarray, scales_bits: np.ndarray, biases_bits: np.ndarray) -> np.ndarray:
    """W[n,k] = scale[n, k//64] * q[n,k] + bias[n, k//64] in fp64, with q the
    unsigned nibble 0..15 (low nibble = even k) and scale, bias bf16. Every
    term is exact in fp64 (bf16 times a 4-bit integer plus bf16)."""
    q = unpack_nibbles(codes).astype(np.float64)
    r, k = q.shape
    sb = np.asarray(scales_bits)
    bb = np.asarray(biases_bits)
    assert sb.shape == (r, k // AFFINE_GROUP) and bb.shape == sb.shape, (sb.shape, bb.shape, (r, k))
    s = np.repeat(bf16_bits_to_f64(sb), AFFINE_GROUP, axis=1)
    b = np.repeat(bf16_bits_to_f64(bb), AFFINE_GROUP, axis=1)
    return s * q + b


def gemm_affine_q4(x_bits: np.ndarray, codes: np.ndarray, scales_bits: np.ndarray, biases_bits: np.ndarray,
                   rows: np.ndarray | None = None) -> np.ndarray:
    """Y[M,N] = X[M,K] . W^T with W dequantised from affine 4-bit, fp64."""
    x = bf16_bits_to_f64(x_bits)
    if rows is not None:
        rows = np.asarray(rows)
        w = dequant_affine_q4(np.asarray(codes)[rows], np.asarray(scales_bits)[rows], np.asarray(biases_bits)[rows])
        return x @ w.T
    n = codes.shape[0]
    y = np.empty((x.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, _ROW_CHUNK):
        r1 = min(n, r0 + _ROW_CHUNK)
        y[:, r0:r1] = x @ dequant_affine_q4(codes[r0:r1], scales_bits[r0:r1], biases_bits[r0:r1]).T
    return y


def mlp_silu_mul_affine(x_bits, codes, scales_bits, biases_bits, n_inter: int):
    """silu(gate) * up on a fused [gate; up] affine 4-bit matrix (2*n_inter
    rows), fp64, and its single bf16 rounding."""
    gu = gemm_affine_q4(x_bits, codes, scales_bits, biases_bits)
    h = silu(gu[:, :n_inter]) * gu[:, n_inter:]
    return h, round_to_bf16_bits(h)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), fp64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def mlp_silu_mul(x_bits, gu_codes, gu_scales, gu_ts, n_inter: int):
    """First half of the SwiGLU MLP on a fused [gate; up] NVFP4 matrix of
    2*n_inter rows: returns (h_f64, h_bf16_bits) with h = silu(gate) * up,
    computed in fp64 and rounded once to bf16 ([P1] "The engine hard-codes the
    model": SwiGLU gate, up, down)."""
    gu = gemm_nvfp4(x_bits, gu_codes, gu_scales, gu_ts)
    g, u = gu[:, :n_inter], gu[:, n_inter:]
    h = silu(g) * u
    return h, round_to_bf16_bits(h)


# ---------------------------------------------------------------------------
# O8: argmax and the tie class; O9: the greedy accept.
# ---------------------------------------------------------------------------

def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Per row: the lowest index among the exactly-equal maxima. -0 equals +0
    (IEEE comparison already treats them as equal); NaN is never selected; a
    row with no non-NaN value gives -1. Ties must break the same way on every
    path ([P2] "The bugs a second reviewer found")."""
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    out = np.full(lg.shape[0], -1, dtype=np.int64)
    for r in range(lg.shape[0]):
        row = lg[r]
        valid = ~np.isnan(row)
        if not valid.any():
            continue
        mx = row[valid].max()
        out[r] = int(np.flatnonzero(valid & (row == mx))[0])
    return out


def top2_gap(logits: np.ndarray) -> np.ndarray:
    """Per row: top1 - top2 over non-NaN values (0 if the maximum is shared).
    Rows with gap <= 1e-3 form the tie class, where the summation order may
    legitimately decide the argmax ([P3] "Is it really lossless?")."""
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    gaps = np.empty(lg.shape[0], dtype=np.float64)
    for r in range(lg.shape[0]):
        row = lg[r][~np.isnan(lg[r])]
        if row.size < 2:
            gaps[r] = math.inf
            continue
        top = np.partition(row, row.size - 2)[-2:]
        gaps[r] = top[1] - top[0]
    return gaps


def greedy_accept(argmax_rows: np.ndarray, drafts: np.ndarray):
    """Greedy accept per lane ([P4] "How DSpark is wired in"; [P3] "One round").

    argmax_rows: [lanes][R] target choices at the R verify rows of each lane
    (row 0 follows the anchor). drafts: [lanes][R-1] proposed tokens; draft j
    is the proposal the target's row-j choice is compared with. The matched
    prefix is accepted and the target's own token after it is the bonus, so a
    lane commits between 1 and R tokens.

    Returns (accept_len[lanes], commit[lanes][R]) with commit[l][i] the
    committed token i (the target's argmax at row i) for i < accept_len and -1
    after it. A row without a valid argmax (-1, all logits NaN) matches no
    draft, so the scan stops there.
    """
    a = np.asarray(argmax_rows, dtype=np.int64)
    d = np.asarray(drafts, dtype=np.int64)
    lanes, r = a.shape
    assert d.shape == (lanes, r - 1)
    acc_len = np.empty(lanes, dtype=np.int64)
    commit = np.full((lanes, r), -1, dtype=np.int64)
    for l in range(lanes):
        acc = 0
        while acc < r - 1 and a[l, acc] >= 0 and a[l, acc] == d[l, acc]:
            acc += 1
        acc_len[l] = acc + 1
        commit[l, : acc + 1] = a[l, : acc + 1]
    return acc_len, commit


# ---------------------------------------------------------------------------
# O10: bytes, the pass schedule and the roof.
# ---------------------------------------------------------------------------

def bytes_nvfp4(n: int, k: int) -> int:
    """Nine bytes per sixteen weights: K/2 code bytes plus K/16 scale bytes per
    row ([P4] "What one token costs the bus": codes 8.556 GB, scales 1.070 GB)."""
    assert k % 16 == 0
    return n * k // 16 * 9


def bytes_fp8(n: int, k: int) -> int:
    """One byte per FP8 E4M3 weight."""
    return n * k


HIDDEN = 5120
INTER = 17408
VOCAB = 248320
LAYERS = 64
GDN_IN = 16384
GDN_OUT_K = 6144
ATTN_QG = 12288
ATTN_KV = 1024
ATTN_O_K = 6144


def pass_schedule():
    """The GEMMs of one verify pass in model order: layer l is full attention
    iff l % 4 == 3 (three Gated DeltaNet layers, then one full-attention layer;
    [P4] "What one token costs the bus"). Each mixer has an FP8 in-projection
    and an FP8 out-projection; every layer has the NVFP4 SwiGLU MLP; the pass
    ends in the NVFP4 vocabulary head. Entries: (kind, fmt, N, K)."""
    out = []
    for layer in range(LAYERS):
        if layer % 4 == 3:
            out.append(("attn_qgkv", "fp8", ATTN_QG + 2 * ATTN_KV, HIDDEN))
            out.append(("attn_o", "fp8", HIDDEN, ATTN_O_K))
        else:
            out.append(("gdn_in", "fp8", GDN_IN, HIDDEN))
            out.append(("gdn_out", "fp8", HIDDEN, GDN_OUT_K))
        out.append(("mlp_gate_up", "nvfp4", 2 * INTER, HIDDEN))
        out.append(("mlp_down", "nvfp4", HIDDEN, INTER))
    out.append(("lm_head", "nvfp4", VOCAB, HIDDEN))
    return out


def pass_bytes_by_kind():
    """Weight bytes of one pass grouped like the pages' byte table."""
    groups = {"mlp": 0, "gdn": 0, "attn": 0, "head": 0}
    for kind, fmt, n, k in pass_schedule():
        b = bytes_nvfp4(n, k) if fmt == "nvfp4" else bytes_fp8(n, k)
        if kind.startswith("mlp"):
            groups["mlp"] += b
        elif kind.startswith("gdn"):
            groups["gdn"] += b
        elif kind.startswith("attn"):
            groups["attn"] += b
        else:
            groups["head"] += b
    return groups


def roof_tokens_per_s(bandwidth_gb_s: float, bytes_per_pass_gb: float, alpha: float) -> float:
    """tok/s <= bandwidth / bytes-per-pass * alpha ([P1] "The roof";
    [P4] "What one token costs the bus", ceiling equation with alpha = 1)."""
    return bandwidth_gb_s / bytes_per_pass_gb * alpha


def flops_per_byte_nvfp4(m: int) -> float:
    """Arithmetic intensity of an M-row NVFP4 GEMM: 2*M flops per weight over
    9/16 bytes per weight ([P1] "Why Apple silicon, and why not the M5")."""
    return 2.0 * m / (9.0 / 16.0)


# ---------------------------------------------------------------------------
# Exact rational brute force (small shapes only): a second, independent route
# used by the self-tests.
# ---------------------------------------------------------------------------

def exact_gemm_nvfp4_fraction(x_vals, w_vals):
    """Exact Y = X . W^T over Python Fractions for tiny shapes. Inputs are
    lists of lists of Fractions (already decoded by the caller)."""
    m = len(x_vals)
    n = len(w_vals)
    k = len(x_vals[0]) if m else 0
    y = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                acc += x_vals[i][t] * w_vals[j][t]
            y[i][j] = acc
    return y
