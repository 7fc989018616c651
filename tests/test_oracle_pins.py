"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/pages_numbers.json), a published format table
(tests/golden/e2m1_ocp.json), a library routine (torch's float8_e4m3fn and
bfloat16 casts, torch's SiLU), exact rational brute force, closed forms and
invariants. Nothing here needs a GPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------- independent decode

def _e2m1_from_table(code):
    return _gold("e2m1_ocp.json")["values_by_code"][code & 15]


_E4M3_TORCH = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _nib(codes_row, k):
    byte = int(codes_row[k // 2])
    return (byte >> 4) & 15 if (k % 2) else byte & 15


def _decode_fraction(codes, scales, ts, n, k):
    c = Fraction(_e2m1_from_table(_nib(codes[n], k)))
    s = Fraction(float(_E4M3_TORCH[int(scales[n][k // 16])]))
    return c * s * Fraction(float(np.float32(ts)))


def _rand_nvfp4(seed, n, k, scale_max_code=0x7E):
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = g.integers(0, scale_max_code + 1, size=(n, k // 16), dtype=np.uint8)
    return codes, scales


def _rand_x(seed, m, k):
    g = np.random.default_rng(seed)
    f = g.standard_normal((m, k)).astype(np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ O1 tables

def test_e2m1_table_matches_published_format():
    ref = _gold("e2m1_ocp.json")["values_by_code"]
    for c in range(16):
        assert O.E2M1_TABLE[c] == ref[c]
        assert math.copysign(1.0, O.E2M1_TABLE[c]) == (-1.0 if c >= 8 else 1.0)


def test_e4m3_table_matches_torch_for_all_codes():
    for c in range(256):
        a, b = O.E4M3FN_TABLE[c], _E4M3_TORCH[c]
        if math.isnan(b):
            assert math.isnan(a), c
        else:
            assert a == b and math.copysign(1, a) == math.copysign(1, b), c
    assert [c for c in range(256) if math.isnan(O.E4M3FN_TABLE[c])] == [0x7F, 0xFF]


def test_e4m3_range_matches_pages():
    facts = _gold("pages_numbers.json")["format_facts"]
    finite = O.E4M3FN_TABLE[~np.isnan(O.E4M3FN_TABLE)]
    assert finite.max() == facts["e4m3_block_scale_max"]
    assert finite[finite > 0].min() == 2.0 ** -9


def test_every_nvfp4_product_is_exact_in_bf16():
    # a consequence the kernels rely on; also exercises round_to_bf16_bits
    vals = []
    for c in range(16):
        for s in range(256):
            if s in (0x7F, 0xFF):
                continue
            vals.append(O.E2M1_TABLE[c] * O.E4M3FN_TABLE[s])
    vals = np.array(vals)
    back = O.bf16_bits_to_f64(O.round_to_bf16_bits(vals))
    assert np.array_equal(back, vals)


# ---------------------------------------------------------------- bf16 helpers

def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    f = (g.standard_normal(4000) * np.exp(g.uniform(-30, 30, 4000))).astype(np.float32)
    # exact midpoints between bf16 neighbours: low 16 bits == 0x8000
    mids = ((g.integers(0x3F00, 0x4100, 500).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, mids, np.array([0.0, -0.0, 1e-40, -3e-39, 3.3e38, -3.4e38], np.float32)])
    ours = O.round_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = O.bf16_bits_to_f64(bits)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------------- O2/O3 dequant

def test_dequant_nvfp4_elementwise_brute_force():
    codes, scales = _rand_nvfp4(2, 7, 64)
    ts = 0.37
    w = O.dequant_nvfp4(codes, scales, ts)
    for n in range(7):
        for k in range(64):
            assert Fraction(w[n, k]) == _decode_fraction(codes, scales, ts, n, k), (n, k)


def test_tensor_scale_is_a_multiplier():
    codes, scales = _rand_nvfp4(3, 4, 32)
    w1 = O.dequant_nvfp4(codes, scales, 1.0)
    w2 = O.dequant_nvfp4(codes, scales, 2.5)
    assert np.array_equal(w2, w1 * 2.5)


# ------------------------------------------------------------------ O5 GEMM

@pytest.mark.parametrize("m,n,k,ts", [(3, 5, 64, 1.0), (1, 4, 32, 0.37), (2, 3, 16, 0.125), (8, 6, 96, 3.0)])
def test_gemm_nvfp4_exact_rational_brute_force(m, n, k, ts):
    codes, scales = _rand_nvfp4(10 + m + n, n, k, scale_max_code=0x60)
    x = _rand_x(20 + k, m, k)
    y = O.gemm_nvfp4(x, codes, scales, ts)
    xf = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(x)]
    wf = [[_decode_fraction(codes, scales, ts, j, t) for t in range(k)] for j in range(n)]
    ex = O.exact_gemm_nvfp4_fraction(xf, wf)
    scale = max(abs(float(v)) for row in ex for v in row) or 1.0
    for i in range(m):
        for j in range(n):
            assert abs(y[i, j] - float(ex[i][j])) <= 1e-12 * scale


def test_gemm_rows_equal_separate_gemvs():
    codes, scales = _rand_nvfp4(4, 48, 256)
    x = _rand_x(5, 8, 256)
    y = O.gemm_nvfp4(x, codes, scales, 1.0)
    w = O.dequant_nvfp4(codes, scales, 1.0)
    xs = O.bf16_bits_to_f64(x)
    for i in range(8):
        for j in range(48):
            ref = math.fsum(xs[i, t] * w[j, t] for t in range(256))
            assert abs(y[i, j] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_one_hot_activation_extracts_weight():
    n, k = 9, 64
    codes, scales = _rand_nvfp4(6, n, k)
    for kk in (0, 1, 15, 16, 33, 63):
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, kk] = 0x3F80  # bf16 1.0
        y = O.gemm_nvfp4(x, codes, scales, 0.5)
        for j in range(n):
            assert Fraction(y[0, j]) == _decode_fraction(codes, scales, 0.5, j, kk)


def test_special_cases():
    n, k = 4, 64
    codes, scales = _rand_nvfp4(7, n, k)
    x = _rand_x(8, 2, k)
    # a zero block scale removes exactly that block's contribution
    s0 = scales.copy()
    s0[:, 1] = 0
    y0 = O.gemm_nvfp4(x, codes, s0, 1.0)
    xs = O.bf16_bits_to_f64(x)
    w = O.dequant_nvfp4(codes, scales, 1.0)
    w[:, 16:32] = 0.0
    assert np.allclose(y0, xs @ w.T, rtol=1e-13, atol=0)
    # all codes negative zero -> zero output
    yz = O.gemm_nvfp4(x, np.full((n, k // 2), 0x88, np.uint8), scales, 1.0)
    assert np.all(yz == 0.0)
    # K = 16: a single block
    c1, s1 = _rand_nvfp4(9, 3, 16)
    x1 = _rand_x(10, 1, 16)
    y1 = O.gemm_nvfp4(x1, c1, s1, 1.0)
    xs1 = O.bf16_bits_to_f64(x1)[0]
    for j in range(3):
        ref = sum(xs1[t] * float(_decode_fraction(c1, s1, 1.0, j, t)) for t in range(16))
        assert abs(y1[0, j] - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("ws", [1.0, 0.37, 0.125])
def test_gemm_fp8_brute_force(ws):
    g = np.random.default_rng(11)
    w = g.integers(0, 256, size=(5, 48), dtype=np.uint8)
    w[w == 0x7F] = 0x7E
    w[w == 0xFF] = 0xFE
    x = _rand_x(12, 3, 48)
    y = O.gemm_fp8(x, w, ws)
    xs = O.bf16_bits_to_f64(x)
    for i in range(3):
        for j in range(5):
            ex = sum(Fraction(float(xs[i, t])) * Fraction(float(_E4M3_TORCH[w[j, t]])) for t in range(48))
            ex *= Fraction(float(np.float32(ws)))
            assert abs(y[i, j] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


# -------------------------------------------------------------------- O7 MLP

def test_silu_matches_torch_and_limits():
    g = np.random.default_rng(13).standard_normal(1000) * 8
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.allclose(O.silu(g), ref, rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([60.0]))[0] == pytest.approx(60.0, rel=1e-15)
    assert abs(O.silu(np.array([-60.0]))[0]) < 1e-20


def test_mlp_fused_gate_up_split():
    inter, k = 12, 64
    codes, scales = _rand_nvfp4(14, 2 * inter, k, scale_max_code=0x58)
    x = _rand_x(15, 3, k)
    h, hb = O.mlp_silu_mul(x, codes, scales, 1.0, inter)
    xs = O.bf16_bits_to_f64(x)
    for i in range(3):
        for j in range(inter):
            g = sum(xs[i, t] * float(_decode_fraction(codes, scales, 1.0, j, t)) for t in range(k))
            u = sum(xs[i, t] * float(_decode_fraction(codes, scales, 1.0, inter + j, t)) for t in range(k))
            ref = g * u / (1.0 + math.exp(-g))
            assert abs(h[i, j] - ref) <= 1e-12 * max(1.0, abs(ref))
    ref_b = torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16)
    # bf16 of the fp64 value; agrees with torch's fp32->bf16 except where the
    # fp32 intermediate rounding crosses a bf16 midpoint (not the case here)
    assert np.array_equal(hb, ref_b.view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- O8 argmax

def test_argmax_ties_nan_and_signed_zero():
    lg = np.array([
        [1.0, 3.0, 3.0, 2.0],
        [np.nan, np.nan, np.nan, np.nan],
        [-0.0, 0.0, -1.0, np.nan],
        [np.nan, -np.inf, -np.inf, -5.0],
        [np.nan, 7.0, np.nan, 7.0],
    ])
    assert list(O.argmax_lowest(lg)) == [1, -1, 0, 3, 1]


def test_argmax_brute_force_with_many_ties():
    g = np.random.default_rng(16)
    lg = g.integers(-3, 4, size=(200, 37)).astype(np.float64)
    lg[g.random(lg.shape) < 0.05] = np.nan
    got = O.argmax_lowest(lg)
    for r in range(lg.shape[0]):
        best, bi = None, -1
        for i, v in enumerate(lg[r]):
            if not math.isnan(v) and (best is None or v > best):
                best, bi = v, i
        assert got[r] == bi


def test_top2_gap():
    lg = np.array([[1.0, 3.0, 3.0], [1.0, 2.0, 5.0], [4.0, np.nan, 1.5]])
    assert list(O.top2_gap(lg)) == [0.0, 3.0, 2.5]


# ---------------------------------------------------------------- O9 accept

def test_accept_rule_cases():
    rule = _gold("pages_numbers.json")["accept_rule"]
    r = rule["block_rows"]
    a = np.arange(100, 100 + 3 * r).reshape(3, r)
    d = np.stack([a[0, : r - 1], a[1, : r - 1], a[2, : r - 1]]).copy()
    d[1, 0] += 1          # first draft wrong -> only the bonus
    d[2, 4] += 1          # mismatch at row 4 -> 5 tokens
    ln, cm = O.greedy_accept(a, d)
    assert list(ln) == [rule["max_commit"], rule["min_commit"], 5]
    assert list(cm[0]) == list(a[0])
    assert list(cm[1]) == [a[1, 0]] + [-1] * (r - 1)
    assert list(cm[2]) == list(a[2, :5]) + [-1] * (r - 5)


def test_accept_invariants_random():
    g = np.random.default_rng(17)
    for r in (1, 2, 5, 8):
        a = g.integers(0, 4, size=(300, r))
        d = g.integers(0, 4, size=(300, r - 1))
        ln, cm = O.greedy_accept(a, d)
        assert ln.min() >= 1 and ln.max() <= r
        for l in range(300):
            acc = ln[l] - 1
            assert all(a[l, j] == d[l, j] for j in range(acc))
            if acc < r - 1:
                assert a[l, acc] != d[l, acc]
            assert list(cm[l, : ln[l]]) == list(a[l, : ln[l]])


def test_accept_length_distribution_of_synthetic_drafts():
    from bit_block_scaled_vq_amd import inputs
    lanes, r, v = 20000, 8, 248320
    a = np.random.default_rng(18).integers(0, v, size=(lanes, r))
    d = inputs.drafts((9, 9), a, v)
    ln, _ = O.greedy_accept(a, d)
    p = 0.7
    expect = [0.3 * p ** (k - 1) for k in range(1, r)] + [p ** (r - 1)]
    got = np.bincount(ln, minlength=r + 1)[1:] / lanes
    assert np.allclose(got, expect, atol=0.015)
    assert abs(ln.mean() - sum(p ** j for j in range(r))) < 0.05


# ------------------------------------------------------------ O10 bytes/roof

def test_pass_bytes_reproduce_page_table():
    t = _gold("pages_numbers.json")["lithos_byte_table"]
    mlp_codes = 64 * 3 * 17408 * 5120 // 2
    mlp_scales = 64 * 3 * 17408 * 5120 // 16
    g = O.pass_bytes_by_kind()
    assert g["mlp"] == mlp_codes + mlp_scales
    assert round(mlp_codes / 1e9, 3) == t["mlp_codes_gb"]
    assert round(mlp_scales / 1e9, 3) == t["mlp_scales_gb"]
    assert round(g["gdn"] / 1e9, 3) == t["gdn_gb"]
    assert round(g["attn"] / 1e9, 3) == t["attn_gb"]
    assert round(g["head"] / 1e9, 3) == t["head_gb"]
    total = sum(g.values())
    assert total == 17_555_292_160
    assert round(total / 1e9 + t["small_bf16_gb"], 3) == t["read_per_pass_gb"]


def test_nine_bytes_per_sixteen_and_splash_geometry():
    s = _gold("pages_numbers.json")["splash_geometry"]
    assert O.bytes_nvfp4(16, 16) == 9 * 16
    mlp = 2 * O.bytes_nvfp4(s["intermediate"], s["hidden"]) + O.bytes_nvfp4(s["hidden"], s["intermediate"])
    assert round(mlp / 1e6, 2) == s["mlp_layer_mb"]
    assert round(O.bytes_nvfp4(s["vocab"], s["hidden"]) / 1e6, 2) == s["lm_head_mb"]
    assert sum(s["attn_in_widths"]) == O.ATTN_QG + 2 * O.ATTN_KV


def test_draft_geometry_bytes():
    # the draft's layer bytes from its printed widths: qkv, two dynamic
    # projections, the attention output projection and a SwiGLU MLP
    d = _gold("pages_numbers.json")["splash_draft_geometry"]
    h = d["hidden"]
    layer = (O.bytes_nvfp4(d["qkv"], h) + 2 * O.bytes_nvfp4(d["dynamic"], h) + O.bytes_nvfp4(h, d["attn"])
             + 2 * O.bytes_nvfp4(d["swiglu"], h) + O.bytes_nvfp4(h, d["swiglu"]))
    assert round(layer / 1e6, 1) == d["layer_mb"]
    assert round(O.bytes_nvfp4(*d["context_proj_shape"]) / 1e6, 2) == d["context_proj_mb"]


def test_schedule_shape():
    sch = O.pass_schedule()
    assert len(sch) == 257
    kinds = [k for k, *_ in sch]
    assert kinds.count("attn_qgkv") == 16 and kinds.count("gdn_in") == 48
    assert kinds.count("mlp_gate_up") == 64 and kinds[-1] == "lm_head"
    assert kinds[12] == "attn_qgkv" and kinds[0] == "gdn_in"   # layer 3 is the first attention layer
    assert kinds[8] == "gdn_in" and kinds[16] == "gdn_in"


def test_roof_equations():
    c = _gold("pages_numbers.json")["lithos_ceiling"]
    t = _gold("pages_numbers.json")["lithos_byte_table"]
    assert round(O.roof_tokens_per_s(c["nominal_gbps"], t["read_per_pass_gb"] + c["state_gb"], 1.0), 1) == c["tok_s_short_context"]
    s = _gold("pages_numbers.json")["splash_roof"]
    need = s["tok_s"] * s["bytes_gb"] / s["alpha"]
    assert round(need) == s["needs_gbps"]
    assert O.roof_tokens_per_s(need, s["bytes_gb"], s["alpha"]) == pytest.approx(s["tok_s"])


def test_arithmetic_intensity():
    s = _gold("pages_numbers.json")["splash_intensity"]
    assert round(O.flops_per_byte_nvfp4(8)) == s["m8"]
    assert round(O.flops_per_byte_nvfp4(32)) == s["m32"]
