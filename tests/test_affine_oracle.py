"""Pins of the affine 4-bit oracle ("144 tok/s needs 502 GB/s ...", section
"The engine hard-codes the model": 32 bytes of nibbles plus a bf16 scale and
a bf16 bias per 64 inputs; "lithos-metal ...", section "Formats, and what
runs where": the MLX/AWQ/GPTQ affine layout) against exact rational brute
force, the per-group input-sum identity and special cases."""
from fractions import Fraction

import numpy as np
import torch

import oracle as O


def _bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _bf16_fraction(bits):
    # decode through torch, independently of the oracle's bf16 decoder
    v = torch.from_numpy(np.array([bits], dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return Fraction(float(v.item()))


def _rand_affine(seed, n, k):
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    s = np.abs(g.standard_normal((n, k // 64))).astype(np.float32) * 0.01 + 0.001
    b = (-7.5 * s * (1 + 0.2 * g.standard_normal((n, k // 64)))).astype(np.float32)
    return codes, _bf16_bits(s), _bf16_bits(b)


def _q(codes, n, k):
    byte = int(codes[n][k // 2])
    return (byte >> 4) & 15 if k % 2 else byte & 15


def test_dequant_elementwise_brute_force():
    codes, sb, bb = _rand_affine(1, 8, 256)
    w = O.dequant_affine_q4(codes, sb, bb)
    for n in range(8):
        for k in range(256):
            g = k // 64
            ex = _bf16_fraction(sb[n, g]) * _q(codes, n, k) + _bf16_fraction(bb[n, g])
            assert Fraction(w[n, k]) == ex, (n, k)


def test_gemm_exact_rational_brute_force():
    m, n, k = 3, 5, 128
    codes, sb, bb = _rand_affine(2, n, k)
    x = _bf16_bits(np.random.default_rng(3).standard_normal((m, k)).astype(np.float32))
    y = O.gemm_affine_q4(x, codes, sb, bb)
    for i in range(m):
        xf = [_bf16_fraction(x[i, t]) for t in range(k)]
        for j in range(n):
            ex = sum(xf[t] * (_bf16_fraction(sb[j, t // 64]) * _q(codes, j, t) + _bf16_fraction(bb[j, t // 64]))
                     for t in range(k))
            assert abs(Fraction(y[i, j]) - ex) <= abs(ex) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def test_input_sum_identity():
    # sum_k x (s q + b) = sum_g (s_g sum_{k in g} x q + b_g sum_{k in g} x):
    # the per-group input sums carry the whole bias term
    codes, sb, bb = _rand_affine(4, 7, 512)
    x = _bf16_bits(np.random.default_rng(5).standard_normal((4, 512)).astype(np.float32))
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    q = np.stack([[_q(codes, n, t) for t in range(512)] for n in range(7)]).astype(np.float64)
    s = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    b = torch.from_numpy(bb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    xs = xv.reshape(4, 8, 64)
    ref = np.einsum("mgk,ngk->mng", xs, q.reshape(7, 8, 64)) * s[None] + xs.sum(-1)[:, None, :] * b[None]
    np.testing.assert_allclose(O.gemm_affine_q4(x, codes, sb, bb), ref.sum(-1), rtol=1e-12, atol=1e-12)


def test_one_hot_extracts_weight_and_layout():
    codes, sb, bb = _rand_affine(6, 4, 128)
    for kk in (0, 1, 63, 64, 127):
        x = np.zeros((1, 128), dtype=np.float32)
        x[0, kk] = 1.0
        y = O.gemm_affine_q4(_bf16_bits(x), codes, sb, bb)
        for j in range(4):
            ex = _bf16_fraction(sb[j, kk // 64]) * _q(codes, j, kk) + _bf16_fraction(bb[j, kk // 64])
            assert Fraction(y[0, j]) == ex


def test_special_cases():
    k = 128
    codes = np.full((2, k // 2), 0xF0, dtype=np.uint8)  # even k: q = 0, odd k: q = 15
    sb = _bf16_bits(np.array([[0.5, 0.25], [0.0, 0.0]], dtype=np.float32))
    bb = _bf16_bits(np.array([[-1.0, 2.0], [3.0, -0.5]], dtype=np.float32))
    w = O.dequant_affine_q4(codes, sb, bb)
    assert w[0, 0] == -1.0 and w[0, 1] == 15 * 0.5 - 1.0
    assert w[0, 64] == 2.0 and w[0, 65] == 15 * 0.25 + 2.0
    assert np.all(w[1, :64] == 3.0) and np.all(w[1, 64:] == -0.5)  # zero scale: the bias only
    ones = _bf16_bits(np.ones((1, k), dtype=np.float32))
    y = O.gemm_affine_q4(ones, codes, sb, bb)
    assert y[0, 1] == 64 * 3.0 + 64 * -0.5
    assert y[0, 0] == 32 * (-1.0 + 6.5) + 32 * (2.0 + 5.75)


def test_nine_bytes_per_sixteen():
    # 32 B of nibbles + 2 B scale + 2 B bias per 64 weights
    assert (32 + 2 + 2) * 16 == 64 * 9
    assert O.AFFINE_GROUP == 64


def test_mlp_silu_mul_affine_fused_split():
    # silu(gate) * up on the fused [gate; up] matrix: rows [0, inter) are the
    # gate, rows [inter, 2 inter) the up projection of the same output column.
    # Each product is brute-forced from exact rationals (the bf16 fields decoded
    # through torch), so swapping the halves, dropping the SiLU or reading the
    # wrong row fails here, and h's single bf16 rounding is torch's cast.
    import math
    inter, k, m = 6, 128, 3
    codes, sb, bb = _rand_affine(7, 2 * inter, k)
    x = _bf16_bits(np.random.default_rng(8).standard_normal((m, k)).astype(np.float32))
    h, hb = O.mlp_silu_mul_affine(x, codes, sb, bb, inter)
    assert h.shape == (m, inter) and hb.shape == (m, inter)

    def dot(i, row):
        xf = [_bf16_fraction(x[i, t]) for t in range(k)]
        return sum(xf[t] * (_bf16_fraction(sb[row, t // 64]) * _q(codes, row, t) + _bf16_fraction(bb[row, t // 64]))
                   for t in range(k))

    asym = 0
    for i in range(m):
        for j in range(inter):
            g = float(dot(i, j))
            u = float(dot(i, inter + j))
            ref = g / (1.0 + math.exp(-g)) * u
            assert abs(h[i, j] - ref) <= 1e-12 * max(1.0, abs(ref)), (i, j)
            swapped = u / (1.0 + math.exp(-u)) * g
            asym += abs(swapped - ref) > 1e-6 * max(1.0, abs(ref))
    assert asym > 0   # the inputs tell gate and up apart
    want = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(hb, want)
