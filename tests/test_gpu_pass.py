"""GPU parity of the verify pass as one captured graph (the pass schedule).

The first four layers of the hybrid at full shapes, in model order -- layers
0, 1 and 2 are Gated DeltaNet layers and layer 3 a full-attention layer
("lithos-metal ...", section "What one token costs the bus": three GDN layers
to one full-attention layer; "144 tok/s needs 502 GB/s ...", section "The
engine hard-codes the model": every fourth layer is full attention) -- each
with its mixer in-projection and out-projection (FP8) and its SwiGLU MLP
([gate; up] + SiLU*up, then down; NVFP4), then the vocabulary head with the
per-row argmax and the greedy accept ("lithos-metal ...", section "How DSpark
is wired in"). The launches are chained through their outputs:

  in-proj(x_l) -> out-proj(first 6144 columns of the in-projection output)
  -> [gate; up](out-proj output) -> down(h) -> x_{l+1} = down output * 2^-12
  -> ... -> head(x_4)

The two steps that are not library calls stand in for the mixer core and for
the residual + norm, which are outside this stream: a column slice and a
power-of-two rescale (exact in bf16) that keeps magnitudes bounded without
norms. The out-projections run as bench.py runs them: the accumulating FP8
entry into a zeroed fp32 output (the fill is captured too), whose bf16 cast
stands in for the residual + norm in front of the MLP. Every launch of one (op, N, K) shares one workspace, as in bench.py.
The 17 library launches (plus the stand-ins) are captured once into a HIP
graph with bf16 outputs and replayed; a second graph re-runs every launch on
the first graph's bf16 inputs with fp32 outputs (the parity mode), and the
head there also writes its fp32 logits.

Checks, per launch: the fp32 output against the fp64 oracle on the same bf16
input (sampled output columns for the large matrices, every column for the
out-projections), gated at 2e-3 of max|oracle| and 1e-5 elementwise; the
bf16 store equal to RNE(fp32 store) bit for bit on the whole output; the
argmax, accept length and commit tokens exact outside the tie class; every
graph replay bitwise equal to the eager run of the same launch list, with
eager work between the replays.
"""
import zlib

import numpy as np
import pytest

import oracle as O
from bit_block_scaled_vq_amd import inputs
from tests.gpu_helpers import FLIP_TOL, PARITY_TOL, TIE_GAP, check_f32, say, torch_dev

pytestmark = pytest.mark.gpu

HIDDEN, INTER, VOCAB = 5120, 17408, 248320
GDN_IN, ATTN_QGKV, MIX_K = 16384, 12288 + 1024 + 1024, 6144
M = 8
LAYERS = 4
RESCALE = 2.0 ** -12
SAMPLE_COLS = 640


def _ops():
    from bit_block_scaled_vq_amd import ops
    return ops


def _bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _sample(n, key):
    g = np.random.default_rng(zlib.crc32(f"cols {n} {key}".encode()))
    cols = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                     g.choice(n, size=min(n, SAMPLE_COLS), replace=False)]))
    return cols


def test_pass_graph_layers_0_to_3_and_head_full_size():
    torch, dev = torch_dev()
    ops = _ops()
    bf = torch.bfloat16
    say("case: verify-pass graph, layers 0-3 (GDN, GDN, GDN, attention) + head, M=8, full shapes")

    # ------------------------------------------------------------- weights
    layers = []
    for l in range(LAYERS):
        attn = l % 4 == 3
        n_in = ATTN_QGKV if attn else GDN_IN
        key = (400, l)
        w_in = inputs.device_fp8_weights(key + (0,), n_in, HIDDEN, dev)
        w_out = inputs.device_fp8_weights(key + (1,), HIDDEN, MIX_K, dev)
        gu_c, gu_s = inputs.device_nvfp4_weights(key + (2,), 2 * INTER, HIDDEN, dev)
        dn_c, dn_s = inputs.device_nvfp4_weights(key + (3,), HIDDEN, INTER, dev)
        layers.append(dict(attn=attn, n_in=n_in, w_in=w_in, w_out=w_out, gu_c=gu_c, gu_s=gu_s, dn_c=dn_c, dn_s=dn_s,
                           p_in=ops.pack_fp8(w_in), p_out=ops.pack_fp8(w_out),
                           p_gu=ops.pack_nvfp4(gu_c, gu_s, gate_up=True), p_dn=ops.pack_nvfp4(dn_c, dn_s)))
    hd_c, hd_s = inputs.device_nvfp4_weights((400, 99), VOCAB, HIDDEN, dev)
    p_hd = ops.pack_nvfp4(hd_c, hd_s)

    # one workspace per (op, N, K), shared by every launch of that shape
    ws = {}

    def wsp(op, n, k):
        if (op, n, k) not in ws:
            ws[(op, n, k)] = ops.workspace(op, M, n, k, dev)
        return ws[(op, n, k)]

    # ------------------------------------------------------------- buffers
    x = [inputs.device_x_bf16((400, 50), M, HIDDEN, dev)] + [torch.empty((M, HIDDEN), dtype=bf, device=dev)
                                                              for _ in range(LAYERS)]
    yi = [torch.empty((M, L["n_in"]), dtype=bf, device=dev) for L in layers]
    mix = [torch.empty((M, MIX_K), dtype=bf, device=dev) for _ in range(LAYERS)]
    yo = [torch.empty((M, HIDDEN), dtype=bf, device=dev) for _ in range(LAYERS)]
    yo32 = [torch.empty((M, HIDDEN), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    h = [torch.empty((M, INTER), dtype=bf, device=dev) for _ in range(LAYERS)]
    yd = [torch.empty((M, HIDDEN), dtype=bf, device=dev) for _ in range(LAYERS)]
    f_i = [torch.empty((M, L["n_in"]), dtype=torch.float32, device=dev) for L in layers]
    f_o = [torch.empty((M, HIDDEN), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    f_h = [torch.empty((M, INTER), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    f_d = [torch.empty((M, HIDDEN), dtype=torch.float32, device=dev) for _ in range(LAYERS)]
    drafts = torch.zeros((1, M - 1), dtype=torch.int32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    mx = torch.empty(M, dtype=torch.float32, device=dev)
    al = torch.empty(1, dtype=torch.int32, device=dev)
    cm = torch.empty((1, M), dtype=torch.int32, device=dev)
    am2, al2, cm2 = torch.empty_like(am), torch.empty_like(al), torch.empty_like(cm)
    logits = torch.empty((M, VOCAB), dtype=torch.float32, device=dev)

    def run_bf16():
        """The pass in model order, bf16 outputs, chained."""
        for l, L in enumerate(layers):
            ops.vq_gemm_fp8(x[l], L["p_in"], 1.0, yi[l], workspace=wsp(ops.VQ_OP_FP8, L["n_in"], HIDDEN))
            mix[l].copy_(yi[l][:, :MIX_K])                      # stand-in for the mixer core
            yo32[l].zero_()
            ops.vq_gemm_fp8_accumulate(mix[l], L["p_out"], 1.0, yo32[l])
            yo[l].copy_(yo32[l])                                # stand-in for the residual + norm
            ops.vq_gemm_nvfp4(yo[l], L["p_gu"], 1.0, h[l], epilogue=ops.VQ_EPI_SILU_MUL,
                              workspace=wsp(ops.VQ_OP_NVFP4_SILU_MUL, INTER, HIDDEN))
            ops.vq_gemm_nvfp4(h[l], L["p_dn"], 1.0, yd[l], workspace=wsp(ops.VQ_OP_NVFP4, HIDDEN, INTER))
            x[l + 1].copy_(yd[l] * RESCALE)                     # stand-in for the residual + norm
        ops.vq_lmhead_argmax_accept(x[LAYERS], p_hd, 1.0, VOCAB, drafts, 1, M, am, al, maxlogit_out=mx,
                                    commit_out=cm, workspace=wsp(ops.VQ_OP_LMHEAD, VOCAB, HIDDEN))

    def run_f32():
        """Every launch again on the bf16 graph's inputs, fp32 outputs."""
        for l, L in enumerate(layers):
            ops.vq_gemm_fp8(x[l], L["p_in"], 1.0, f_i[l], workspace=wsp(ops.VQ_OP_FP8, L["n_in"], HIDDEN))
            f_o[l].zero_()
            ops.vq_gemm_fp8_accumulate(mix[l], L["p_out"], 1.0, f_o[l])
            ops.vq_gemm_nvfp4(yo[l], L["p_gu"], 1.0, f_h[l], epilogue=ops.VQ_EPI_SILU_MUL,
                              workspace=wsp(ops.VQ_OP_NVFP4_SILU_MUL, INTER, HIDDEN))
            ops.vq_gemm_nvfp4(h[l], L["p_dn"], 1.0, f_d[l], workspace=wsp(ops.VQ_OP_NVFP4, HIDDEN, INTER))
        ops.vq_lmhead_argmax_accept(x[LAYERS], p_hd, 1.0, VOCAB, drafts, 1, M, am2, al2, commit_out=cm2,
                                    logits_out=logits,
                                    workspace=wsp(ops.VQ_OP_LMHEAD, VOCAB, HIDDEN))

    def snapshot():
        torch.cuda.synchronize()
        s = {f"{n}{l}": _bits(t[l]) for n, t in (("x", x), ("yi", yi), ("mix", mix), ("yo", yo), ("h", h), ("yd", yd))
             for l in range(LAYERS)}
        s["x4"] = _bits(x[LAYERS])
        for l in range(LAYERS):
            s[f"yo32{l}"] = yo32[l].cpu().numpy().copy()
        for n, t in (("am", am), ("al", al), ("cm", cm), ("mx", mx)):
            s[n] = t.cpu().numpy().copy()
        return s

    # eager pass: gives the head's input, hence the oracle argmax and the drafts
    run_bf16()
    torch.cuda.synchronize()
    h_final = _bits(x[LAYERS])
    say("  oracle head logits ...")
    logits_ref = O.gemm_nvfp4(h_final, hd_c.cpu().numpy(), hd_s.cpu().numpy(), 1.0)
    am_ref = O.argmax_lowest(logits_ref)
    d_np = inputs.drafts((400, 98), am_ref.reshape(1, M), VOCAB)
    drafts.copy_(torch.from_numpy(d_np.astype(np.int32)))
    run_bf16()
    eager = snapshot()
    run_f32()
    torch.cuda.synchronize()
    eager_f32 = {f"{n}{l}": t[l].cpu().numpy().copy() for n, t in (("fi", f_i), ("fo", f_o), ("fh", f_h), ("fd", f_d))
                 for l in range(LAYERS)}
    eager_f32["lg"] = logits.cpu().numpy().copy()

    # ------------------------------------------------------------- capture
    graphs = []
    for fn in (run_bf16, run_f32):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                fn()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        graphs.append(g)
    g16, g32 = graphs
    scratch = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)
    for rep in range(3):
        say(f"  replay {rep}")
        for t in yi + yo + yo32 + h + yd + f_i + f_o + f_h + f_d + x[1:]:
            t.fill_(3.0)
        am.fill_(-7), al.fill_(-7), cm.fill_(-7)
        torch.cuda.synchronize()
        g16.replay()
        got = snapshot()
        g32.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert np.array_equal(got[k], eager[k]), (rep, k)
        for n, t in (("fi", f_i), ("fo", f_o), ("fh", f_h), ("fd", f_d)):
            for l in range(LAYERS):
                assert np.array_equal(t[l].cpu().numpy(), eager_f32[f"{n}{l}"]), (rep, n, l)
        assert np.array_equal(logits.cpu().numpy(), eager_f32["lg"]), rep
        # eager work on the same stream between replays
        scratch.normal_()
        ops.vq_gemm_fp8(x[0], layers[0]["p_in"], 1.0, f_i[0], workspace=wsp(ops.VQ_OP_FP8, layers[0]["n_in"], HIDDEN))
        torch.cuda.synchronize()
    # the fp32 buffers hold the last graph replay again
    g32.replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------------- parity
    def rne_equal(bf_bits, f32):
        r = torch.from_numpy(np.ascontiguousarray(f32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return np.array_equal(bf_bits, r)

    def check(name, x_bits, f32, bf_bits, ref_fn, n_out, full=False):
        cols = np.arange(n_out) if full else _sample(n_out, name)
        ref = ref_fn(x_bits, cols)
        got = f32[:, cols]
        check_f32(got, ref, what=name)
        err = np.max(np.abs(got.astype(np.float64) - ref)) / np.max(np.abs(ref))
        assert err <= FLIP_TOL, (name, err)
        assert rne_equal(bf_bits, f32), f"{name}: bf16 store != RNE(fp32 store)"

    for l, L in enumerate(layers):
        kind = "attention" if L["attn"] else "GDN"
        w_in = L["w_in"]
        check(f"layer {l} {kind} in-proj", eager[f"x{l}"], f_i[l].cpu().numpy(), eager[f"yi{l}"],
              lambda xb, c: O.gemm_fp8(xb, w_in[torch.from_numpy(c).to(dev)].cpu().numpy(), 1.0), L["n_in"])
        assert np.array_equal(eager[f"mix{l}"], eager[f"yi{l}"][:, :MIX_K])
        check(f"layer {l} out-proj", eager[f"mix{l}"], f_o[l].cpu().numpy(), eager[f"yo{l}"],
              lambda xb, c: O.gemm_fp8(xb, L["w_out"].cpu().numpy(), 1.0), HIDDEN, full=True)
        # the accumulating entry is deterministic: both graphs' outputs agree
        assert np.array_equal(eager[f"yo32{l}"], f_o[l].cpu().numpy())

        def gu_ref(xb, c, L=L):
            rows = torch.from_numpy(np.concatenate([c, INTER + c])).to(dev)
            y = O.gemm_nvfp4(xb, L["gu_c"][rows].cpu().numpy(), L["gu_s"][rows].cpu().numpy(), 1.0)
            return O.silu(y[:, :len(c)]) * y[:, len(c):]
        check(f"layer {l} [gate; up] + SiLU*up", eager[f"yo{l}"], f_h[l].cpu().numpy(), eager[f"h{l}"], gu_ref, INTER)

        def dn_ref(xb, c, L=L):
            rows = torch.from_numpy(c).to(dev)
            return O.gemm_nvfp4(xb, L["dn_c"][rows].cpu().numpy(), L["dn_s"][rows].cpu().numpy(), 1.0)
        check(f"layer {l} down", eager[f"h{l}"], f_d[l].cpu().numpy(), eager[f"yd{l}"], dn_ref, HIDDEN)
        # the stand-in rescale is exact: x_{l+1} = yd_l * 2^-12 in bf16
        want = (O.bf16_bits_to_f64(eager[f"yd{l}"]) * RESCALE)
        assert np.array_equal(O.bf16_bits_to_f64(eager[f"x{l + 1}"]), want)

    # head: logits, argmax (exact outside the tie class), accept and commit
    assert np.array_equal(h_final, eager["x4"])
    check_f32(logits.cpu().numpy(), logits_ref, what="head logits")
    gap = O.top2_gap(logits_ref)
    tie = gap <= TIE_GAP
    say(f"  head: tie-class rows {int(tie.sum())}, drafts {d_np.tolist()}")
    assert np.all((eager["am"] == am_ref) | tie)
    assert np.array_equal(am2.cpu().numpy(), eager["am"])
    ln_ref, cm_ref = O.greedy_accept(am_ref.reshape(1, M), d_np)
    first_tie = int(np.argmax(tie)) if tie.any() else M
    if first_tie > ln_ref[0] - 1:
        assert int(eager["al"][0]) == int(ln_ref[0])
        assert np.array_equal(eager["cm"], cm_ref)
    else:
        assert np.array_equal(eager["cm"][0][:first_tie], cm_ref[0][:first_tie])
    assert np.array_equal(al2.cpu().numpy(), eager["al"]) and np.array_equal(cm2.cpu().numpy(), eager["cm"])
    say(f"  accept_len {int(eager['al'][0])} commit {eager['cm'][0].tolist()}")
