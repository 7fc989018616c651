#!/usr/bin/env python3
"""Benchmark: one M = 8 speculative-decoding verify pass over the full weight
stream of the 27B hybrid (64 layers: 48 Gated DeltaNet + 16 full attention,
SwiGLU MLP, vocabulary head with argmax + greedy accept), 17,555,292,160
bytes of NVFP4 + FP8 weights, on one MI355X.

A step is one pass: 257 libverify launches in model order, captured once into
a HIP graph and replayed. Weights are seeded synthetic tensors already resident
in HBM. Printed: one JSON line (see the keys below): the headline pass, the
80 % target against the copy and read probes measured in the same run, a
per-kind kernel table and the roofline kernel's duration (both from graph
replays), config 1's launch latency, whole passes at 2-4 lanes (M = 16, 24,
32), the per-shape M sweep, the sampled verify, the affine 4-bit MLP, the
draft block, the GDN state stream, and the oracle timed end to end on whole
configurations on the host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HIDDEN, INTER, VOCAB, LAYERS = 5120, 17408, 248320, 64
GDN_IN, MIX_OUT_K = 16384, 6144
ATTN_QGKV = 12288 + 1024 + 1024
M_ROWS = 8
ALPHA = 4.80                      # accepted tokens per verify pass used for tok/s
HBM_PEAK_GBPS = 8000.0            # MI355X published HBM3E bandwidth

METRIC = "ms per M=8 verify pass (17.6 GB weights), effective HBM GB/s and % of peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def nvfp4_bytes(n, k):
    return n * k // 16 * 9


def schedule():
    """(kind, fmt, N_out, K) in model order; layer l is full attention iff l % 4 == 3."""
    out = []
    for layer in range(LAYERS):
        if layer % 4 == 3:
            out.append(("attn_qgkv", "fp8", ATTN_QGKV, HIDDEN))
            out.append(("attn_o", "fp8", HIDDEN, MIX_OUT_K))
        else:
            out.append(("gdn_in", "fp8", GDN_IN, HIDDEN))
            out.append(("gdn_out", "fp8", HIDDEN, MIX_OUT_K))
        out.append(("mlp_gate_up", "nvfp4_silu", INTER, HIDDEN))
        out.append(("mlp_down", "nvfp4", HIDDEN, INTER))
    out.append(("lm_head", "head", VOCAB, HIDDEN))
    return out


def weight_bytes(fmt, n, k):
    if fmt == "fp8":
        return n * k
    if fmt == "nvfp4_silu":
        return nvfp4_bytes(2 * n, k)
    return nvfp4_bytes(n, k)


def act_bytes(n, k, m=M_ROWS, accumulate=False):
    # accumulating launches write an fp32 output twice: the zero fill, then the sums
    return m * k * 2 + (2 * m * n * 4 if accumulate else m * n * 2)


# Launches that run the accumulating FP8 entry (fp32 output, zero on entry):
# the narrow out-projections, whose split-K shares are added without an
# exchange between workgroups.
ACCUMULATE_KINDS = ("gdn_out", "attn_o")


class Pass:
    """Device buffers and the launch list of one verify pass at `rows` rows
    (lanes of 8). The packed weights and the workspaces (bound to (op, N, K),
    any M) can be shared with another Pass through `share`."""

    def __init__(self, torch, ops, inputs, dev, rows=M_ROWS, share=None):
        self.torch, self.ops, self.dev = torch, ops, dev
        self.rows, self.lanes = rows, rows // M_ROWS
        self.items = schedule()
        if share is None:
            t0 = time.time()
            self.w = []
            for i, (kind, fmt, n, k) in enumerate(self.items):
                # canonical weights are generated on the device, packed once (as at
                # weight-load time) and dropped; the pass reads only packed weights
                key = (5, i)
                if fmt == "fp8":
                    self.w.append(ops.pack_fp8(inputs.device_fp8_weights(key, n, k, dev)))
                elif fmt == "nvfp4_silu":
                    c, s = inputs.device_nvfp4_weights(key, 2 * n, k, dev)
                    self.w.append(ops.pack_nvfp4(c, s, gate_up=True))
                else:
                    c, s = inputs.device_nvfp4_weights(key, n, k, dev)
                    self.w.append(ops.pack_nvfp4(c, s))
            torch.cuda.synchronize()
            log(f"weights generated and packed on device in {time.time() - t0:.1f}s")
            self.ws = {}
            for kind, fmt, n, k in self.items:
                op = {"fp8": ops.VQ_OP_FP8, "nvfp4": ops.VQ_OP_NVFP4, "nvfp4_silu": ops.VQ_OP_NVFP4_SILU_MUL,
                      "head": ops.VQ_OP_LMHEAD}[fmt]
                if (op, n, k) not in self.ws:
                    self.ws[(op, n, k)] = ops.workspace(op, M_ROWS, n, k, dev)
        else:
            self.w, self.ws = share.w, share.ws
        bf = torch.bfloat16
        key = () if rows == M_ROWS else (rows,)
        self.x_hidden = inputs.device_x_bf16((5, 1000) + key, rows, HIDDEN, dev)
        self.x_mix = inputs.device_x_bf16((5, 1001) + key, rows, MIX_OUT_K, dev)
        self.h_final = inputs.device_x_bf16((5, 1002) + key, rows, HIDDEN, dev)
        self.y_in = torch.empty((rows, max(GDN_IN, ATTN_QGKV)), dtype=bf, device=dev)
        self.y_hid = torch.empty((rows, HIDDEN), dtype=bf, device=dev)
        # one zeroed fp32 output per out-projection launch, cleared once per pass
        self.acc_slot = {}
        for i, it in enumerate(self.items):
            if it[0] in ACCUMULATE_KINDS:
                self.acc_slot[i] = len(self.acc_slot)
        self.y_acc = torch.zeros((len(self.acc_slot), rows, HIDDEN), dtype=torch.float32, device=dev)
        self.h_mlp = torch.empty((rows, INTER), dtype=bf, device=dev)
        self.argmax = torch.empty((rows,), dtype=torch.int32, device=dev)
        self.maxlogit = torch.empty((rows,), dtype=torch.float32, device=dev)
        self.accept = torch.empty((self.lanes,), dtype=torch.int32, device=dev)
        self.commit = torch.empty((self.lanes, M_ROWS), dtype=torch.int32, device=dev)
        self.drafts = torch.zeros((self.lanes, M_ROWS - 1), dtype=torch.int32, device=dev)
        self.weight_bytes = sum(weight_bytes(f, n, k) for _, f, n, k in self.items)
        self.act_bytes = sum(act_bytes(n, k, rows, kind in ACCUMULATE_KINDS) for kind, _, n, k in self.items)

    def launch(self, i):
        ops = self.ops
        kind, fmt, n, k = self.items[i]
        w = self.w[i]
        if i in self.acc_slot:
            ops.vq_gemm_fp8_accumulate(self.x_mix, w, 1.0, self.y_acc[self.acc_slot[i]])
        elif fmt == "fp8":
            x = self.x_hidden if k == HIDDEN else self.x_mix
            y = self.y_hid
            if n != HIDDEN:
                y = self.y_in.view(-1)[: self.rows * n].view(self.rows, n)
            ops.vq_gemm_fp8(x, w, 1.0, y, workspace=self.ws[(ops.VQ_OP_FP8, n, k)])
        elif fmt == "nvfp4_silu":
            ops.vq_gemm_nvfp4(self.x_hidden, w, 1.0, self.h_mlp, epilogue=ops.VQ_EPI_SILU_MUL,
                              workspace=self.ws[(ops.VQ_OP_NVFP4_SILU_MUL, n, k)])
        elif fmt == "nvfp4":
            ops.vq_gemm_nvfp4(self.h_mlp, w, 1.0, self.y_hid, workspace=self.ws[(ops.VQ_OP_NVFP4, n, k)])
        else:
            ops.vq_lmhead_argmax_accept(self.h_final, w, 1.0, n, self.drafts, self.lanes, M_ROWS, self.argmax,
                                        self.accept, maxlogit_out=self.maxlogit, commit_out=self.commit,
                                        workspace=self.ws[(ops.VQ_OP_LMHEAD, n, k)])

    def run(self):
        self.y_acc.zero_()  # a fill kernel (graph-safe), part of the timed pass
        for i in range(len(self.items)):
            self.launch(i)


def measure_probes(torch, ops, dev, gib=4, reps=10):
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    out = {}
    for name, fn, moved in (("copy", lambda: ops.vq_probe_copy(src, dst), 2 * nbytes),
                            ("read", lambda: ops.vq_probe_read(src, sink), nbytes)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def capture(torch, fn):
    """fn's launches captured into a HIP graph on a side stream (after one
    eager run), ready to replay on the current stream."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            fn()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    return g


def replay_ms(torch, g, reps):
    """Average ms per replay: HIP events around `reps` replays on the stream
    the graph is launched on."""
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def replay_stats(torch, g, reps=50):
    """ms of `reps` single replays, each between HIP events on the stream the
    graph is launched on and followed by a synchronize (median, min, max)."""
    import numpy as np
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return {"replays": reps, "median": round(float(np.median(ts)), 4), "min": round(float(np.min(ts)), 4),
            "max": round(float(np.max(ts)), 4)}


def per_kind_durations(torch, p, reps=3):
    """Average duration of each launch kind of the pass: every launch of that
    kind (rotating over the layers' weights, so nothing is cached) captured in
    one graph and replayed; the head, which occurs once, four times in a row."""
    res = {}
    for kind in ("gdn_in", "gdn_out", "mlp_gate_up", "mlp_down", "attn_qgkv", "attn_o", "lm_head"):
        idx = [i for i, it in enumerate(p.items) if it[0] == kind]
        seq = idx if len(idx) > 1 else idx * 4
        g = capture(torch, lambda seq=seq: [p.launch(i) for i in seq])
        us = replay_ms(torch, g, reps) * 1e3 / len(seq)
        _, fmt, n, k = p.items[idx[0]]
        wb = weight_bytes(fmt, n, k)
        res[kind] = {"avg_us": round(us, 2), "launches_per_pass": len(idx), "weight_bytes": wb,
                     "gbps": round(wb / (us * 1e-6) / 1e9, 1)}
        del g
    return res


def small_gemm_latency(torch, ops, inputs_mod, dev, chain=200, single=50):
    """Config 1 (M = 8, K = 512, N = 1024 NVFP4; 0.3 MB, it fits in L2): the
    latency of one launch alone (HIP events around each of `single` launches,
    median) and back to back (`chain` launches in one graph)."""
    import numpy as np
    x = inputs_mod.device_x_bf16((1,), 8, 512, dev)
    c, s = inputs_mod.device_nvfp4_weights((1,), 1024, 512, dev)
    w = ops.pack_nvfp4(c, s)
    y = torch.empty((8, 1024), dtype=torch.bfloat16, device=dev)
    ws = ops.workspace(ops.VQ_OP_NVFP4, 8, 1024, 512, dev)

    def run():
        ops.vq_gemm_nvfp4(x, w, 1.0, y, workspace=ws)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    t = []
    for _ in range(single):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    g = capture(torch, lambda: [run() for _ in range(chain)])
    chained = replay_ms(torch, g, 3) * 1e3 / chain
    return {"shape": "M=8 K=512 N=1024 NVFP4, bf16 out", "single_launch_us_median": round(float(np.median(t)), 2),
            "single_launch_us_min": round(float(np.min(t)), 2), "chained_us_per_launch": round(chained, 2)}


def lane_passes(torch, ops, inputs_mod, p, rows=(16, 24, 32), steps=10):
    """The whole pass (257 launches, one graph) at 2, 3 and 4 lanes of 8
    verify rows, on the same packed weights and workspaces."""
    out = {}
    for m in rows:
        q = Pass(torch, ops, inputs_mod, p.dev, rows=m, share=p)
        g = capture(torch, q.run)
        ms = replay_ms(torch, g, steps)
        out[str(m)] = {"lanes": m // M_ROWS, "ms_per_pass": round(ms, 4),
                       "weight_gbps": round(q.weight_bytes / (ms * 1e-3) / 1e9, 1),
                       "tok_s_at_alpha_4_80": round(ALPHA * (m // M_ROWS) / (ms * 1e-3), 1)}
        del g, q
        torch.cuda.empty_cache()
    return out


def m_sweep(torch, ops, inputs_mod, p, rows=(1, 8, 16, 24, 32), reps=2):
    """Weight GB/s per launch of the four repeated projection shapes at each
    row count (1-4 lanes of 8 verify rows), rotating over the pass's layers so
    no launch finds its weights in a cache."""
    dev = p.dev
    kinds = {"mlp_gate_up": "nvfp4_silu", "mlp_down": "nvfp4", "gdn_in": "fp8", "gdn_out": "fp8"}
    out = {}
    for m in rows:
        res = {}
        for kind, fmt in kinds.items():
            idx = [i for i, it in enumerate(p.items) if it[0] == kind]
            _, _, n, k = p.items[idx[0]]
            x = inputs_mod.device_x_bf16((5, 4000, m, k), m, k, dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            op = {"fp8": ops.VQ_OP_FP8, "nvfp4": ops.VQ_OP_NVFP4, "nvfp4_silu": ops.VQ_OP_NVFP4_SILU_MUL}[fmt]
            ws = p.ws[(op, n, k)]

            y32 = torch.zeros((m, n), dtype=torch.float32, device=dev)

            def run(i):
                if kind in ACCUMULATE_KINDS:
                    ops.vq_gemm_fp8_accumulate(x, p.w[i], 1.0, y32)  # timing only: y32 is not cleared
                elif fmt == "fp8":
                    ops.vq_gemm_fp8(x, p.w[i], 1.0, y, workspace=ws)
                else:
                    ops.vq_gemm_nvfp4(x, p.w[i], 1.0, y, epilogue=ops.VQ_EPI_SILU_MUL if fmt == "nvfp4_silu"
                                      else ops.VQ_EPI_NONE, workspace=ws)
            for i in idx[:2]:
                run(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                for i in idx:
                    run(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(idx))
            res[kind] = round(weight_bytes(fmt, n, k) / (us * 1e-6) / 1e9, 1)
        out[str(m)] = res
    return out


def affine_q4(torch, ops, inputs_mod, dev, layers=4, rows=(8, 32), reps=3):
    """The MLP in the affine 4-bit format (scale and bias per 64, the same 9
    bytes per 16 weights as NVFP4): weight GB/s per launch of [gate; up] +
    SiLU*up and of down, rotating over `layers` layers' seeded weights (more
    than the 256 MB MALL holds)."""
    gu, dn = [], []
    for l in range(layers):
        c, s, b = inputs_mod.device_affine_weights((5, 5000, l, 0), 2 * INTER, HIDDEN, dev)
        gu.append(ops.pack_affine_q4(c, s, b, gate_up=True))
        c, s, b = inputs_mod.device_affine_weights((5, 5000, l, 1), HIDDEN, INTER, dev)
        dn.append(ops.pack_affine_q4(c, s, b))
        del c, s, b
    out = {}
    for m in rows:
        x = inputs_mod.device_x_bf16((5, 5001, m), m, HIDDEN, dev)
        h = inputs_mod.device_x_bf16((5, 5002, m), m, INTER, dev)
        hy = torch.empty((m, INTER), dtype=torch.bfloat16, device=dev)
        yy = torch.empty((m, HIDDEN), dtype=torch.bfloat16, device=dev)
        ws_gu = ops.workspace(ops.VQ_OP_AFFINE_Q4_SILU_MUL, m, INTER, HIDDEN, dev)
        ws_dn = ops.workspace(ops.VQ_OP_AFFINE_Q4, m, HIDDEN, INTER, dev)
        res = {}
        for kind, run, nbytes in (
                ("mlp_gate_up", lambda w: ops.vq_gemm_affine_q4(x, w, hy, epilogue=ops.VQ_EPI_SILU_MUL,
                                                                 workspace=ws_gu), nvfp4_bytes(2 * INTER, HIDDEN)),
                ("mlp_down", lambda w: ops.vq_gemm_affine_q4(h, w, yy, workspace=ws_dn), nvfp4_bytes(HIDDEN, INTER))):
            ws_list = gu if kind == "mlp_gate_up" else dn
            for w in ws_list[:2]:
                run(w)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                for w in ws_list:
                    run(w)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(ws_list))
            res[kind] = {"avg_us": round(us, 2), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        out[str(m)] = res
    del gu, dn
    torch.cuda.empty_cache()
    return out


# The draft side of a step: the 5-layer draft (hidden 5,120; per layer a
# 6,144-row qkv projection and two 1,280-row dynamic projections, which read
# the same input and run as one 8,704-row matrix, a 5,120 x 4,096 attention
# output projection and a SwiGLU MLP of 17,408) after the context projection
# that reads five target layers at once (5,120 x 25,600), then the target's
# vocabulary head, which the draft shares. NVFP4 weights, 8 query rows.
DRAFT_LAYERS = 5
DRAFT_SHAPES = [("draft_qkv_dyn", "nvfp4", 6144 + 2 * 1280, HIDDEN), ("draft_attn_o", "nvfp4", HIDDEN, 4096),
                ("draft_gate_up", "nvfp4_silu", INTER, HIDDEN), ("draft_down", "nvfp4", HIDDEN, INTER)]
DRAFT_CTX = ("draft_context", "nvfp4", HIDDEN, 5 * HIDDEN)


def draft_stream(torch, ops, inputs_mod, p, steps=10):
    """One draft block's weight stream, captured in a graph and replayed: the
    context projection, the 5 draft layers and the shared vocabulary head
    (with argmax: the draft's proposals), at M = 8."""
    dev = p.dev
    items = [DRAFT_CTX] + [s for _ in range(DRAFT_LAYERS) for s in DRAFT_SHAPES]
    w = []
    for i, (kind, fmt, n, k) in enumerate(items):
        key = (5, 6000, i)
        if fmt == "nvfp4_silu":
            c, sc = inputs_mod.device_nvfp4_weights(key, 2 * n, k, dev)
            w.append(ops.pack_nvfp4(c, sc, gate_up=True))
        else:
            c, sc = inputs_mod.device_nvfp4_weights(key, n, k, dev)
            w.append(ops.pack_nvfp4(c, sc))
        del c, sc
    m = M_ROWS
    bf = torch.bfloat16
    xs = {k: inputs_mod.device_x_bf16((5, 6100, k), m, k, dev) for k in (HIDDEN, 4096, INTER, 5 * HIDDEN)}
    ys = {n: torch.empty((m, n), dtype=bf, device=dev) for n in (6144 + 2 * 1280, HIDDEN, INTER)}
    ws = {}
    for kind, fmt, n, k in items:
        op = ops.VQ_OP_NVFP4_SILU_MUL if fmt == "nvfp4_silu" else ops.VQ_OP_NVFP4
        if (op, n, k) not in ws:
            ws[(op, n, k)] = ops.workspace(op, m, n, k, dev)
    head = len(p.items) - 1

    def run():
        for (kind, fmt, n, k), wi in zip(items, w):
            if fmt == "nvfp4_silu":
                ops.vq_gemm_nvfp4(xs[k], wi, 1.0, ys[n], epilogue=ops.VQ_EPI_SILU_MUL,
                                  workspace=ws[(ops.VQ_OP_NVFP4_SILU_MUL, n, k)])
            else:
                ops.vq_gemm_nvfp4(xs[k], wi, 1.0, ys[n], workspace=ws[(ops.VQ_OP_NVFP4, n, k)])
        p.launch(head)

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        run()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    nbytes = sum(weight_bytes(f, n, k) for _, f, n, k in items) + weight_bytes("nvfp4", VOCAB, HIDDEN)
    del w
    torch.cuda.empty_cache()
    return {"rows": m, "launches": len(items) + 1, "weight_bytes": nbytes, "ms_per_block": round(dt * 1e3, 4),
            "gbps": round(nbytes / dt / 1e9, 1)}


GDN_LAYERS = 48
GDN_V_HEADS = 48
GDN_K_HEADS = 16
GDN_D = 128


def gdn_bytes(layers, lanes, rows, read_q=True, write_o=True):
    """Algorithmic bytes of the state stream: the fp32 state read from one
    slot and written to the other, plus the rows' keys (and queries), values,
    outputs and the two gates."""
    n = layers * lanes
    state = 2 * n * GDN_V_HEADS * GDN_D * GDN_D * 4
    qk = n * rows * GDN_K_HEADS * GDN_D * 4 * (2 if read_q else 1)
    vo = n * rows * GDN_V_HEADS * GDN_D * 4 * (2 if write_o else 1)
    gates = n * rows * GDN_V_HEADS * 4 * 2
    return state + qk + vo + gates


def gdn_state_stream(torch, ops, inputs_mod, dev, steps=10, commit_rows=4):
    """The Gated DeltaNet state stream of one verify pass: per GDN layer one
    verify launch (the state of every lane read from one parity slot, scanned
    over the lane's rows and written to the other slot, with the rows'
    outputs), and after the accept scan one commit launch over all 48 layers
    that re-scans the accepted rows from the slot the verify read (accept
    length 4 < 8 rows, so every layer is re-scanned). Graph replays."""
    out = {}
    for lanes in (1, 4):
        L, T, H, Hk = GDN_LAYERS, M_ROWS, GDN_V_HEADS, GDN_K_HEADS
        B = L * lanes
        state, q, k, v, a, b = inputs_mod.device_gdn_inputs((5, 7000, lanes), B, T, H, Hk, dev)
        slot = torch.empty_like(state)
        o = torch.empty_like(v)
        acc = torch.full((lanes,), commit_rows, dtype=torch.int32, device=dev)
        per_layer = [tuple(x[l * lanes:(l + 1) * lanes] for x in (state, slot, q, k, v, a, b, o)) for l in range(L)]

        def verify():
            for si, so, qq, kk, vv, aa, bb, oo in per_layer:
                ops.vq_gdn_verify(si, so, qq, kk, vv, aa, bb, oo)

        def commit():
            ops.vq_gdn_commit(state, slot, q, k, v, a, b, acc, lanes=lanes)

        res = {}
        for name, fn in (("verify", verify), ("commit", commit)):
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                fn()
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=st):
                    fn()
            torch.cuda.current_stream().wait_stream(st)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            res[name] = (time.perf_counter() - t0) / steps
        vb = gdn_bytes(L, lanes, T)
        cb = gdn_bytes(L, lanes, commit_rows, read_q=False, write_o=False)
        out[str(lanes * M_ROWS)] = {
            "lanes": lanes, "rows_per_lane": T, "state_bytes_per_slot": B * H * GDN_D * GDN_D * 4,
            "verify_launches": L, "verify_us_per_pass": round(res["verify"] * 1e6, 1),
            "verify_us_per_layer": round(res["verify"] * 1e6 / L, 2), "verify_bytes": vb,
            "verify_gbps": round(vb / res["verify"] / 1e9, 1),
            "commit_rows": commit_rows, "commit_us": round(res["commit"] * 1e6, 1), "commit_bytes": cb,
            "commit_gbps": round(cb / res["commit"] / 1e9, 1),
        }
        del state, q, k, v, a, b, slot, o, per_layer
        torch.cuda.empty_cache()
    return out


def pass_with_state(torch, ops, inputs_mod, p, steps=10):
    """The verify pass with its Gated DeltaNet state stream in model order:
    each GDN layer's state step runs between its in- and out-projection, and
    after the head the commit re-scans the accepted rows of every GDN layer,
    its count read on the device from the head's accept length (no host
    round trip). One graph, replayed."""
    dev = p.dev
    L, T, H, Hk = GDN_LAYERS, M_ROWS, GDN_V_HEADS, GDN_K_HEADS
    state, q, k, v, a, b = inputs_mod.device_gdn_inputs((5, 7100), L, T, H, Hk, dev)
    slot = torch.empty_like(state)
    o = torch.empty_like(v)
    per_layer = [tuple(x[l:l + 1] for x in (state, slot, q, k, v, a, b, o)) for l in range(L)]

    def run():
        p.y_acc.zero_()
        layer = 0
        for i, item in enumerate(p.items):
            p.launch(i)
            if item[0] == "gdn_in":
                ops.vq_gdn_verify(*per_layer[layer])
                layer += 1
        ops.vq_gdn_commit(state, slot, q, k, v, a, b, p.accept, lanes=1)

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        run()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    acc = int(p.accept.item())
    state_b = gdn_bytes(L, 1, T) + (gdn_bytes(L, 1, acc, read_q=False, write_o=False) if acc < T else 0)
    del state, q, k, v, a, b, slot, o, per_layer
    torch.cuda.empty_cache()
    return {"ms_per_pass": round(dt * 1e3, 4), "launches": len(p.items) + L + 1, "accept_len": acc,
            "weight_bytes": p.weight_bytes, "state_stream_bytes": state_b,
            "gbps": round((p.weight_bytes + state_b) / dt / 1e9, 1)}


def sampled_verify(torch, ops, inputs_mod, p, g_steps=10, reps=20):
    """The end of the pass at nonzero temperature (temperature 1, top_k 32,
    top_p 0.95): the head also writes fp32 logits and vq_sample_accept reads
    them (point-mass rule; the speculative-sampling rule timed beside it).
    Returns kernel times from HIP events on the launch stream and the graph
    time of the whole sampled pass."""
    import numpy as np
    dev = p.dev
    M, V = M_ROWS, VOCAB
    head = len(p.items) - 1
    logits = torch.empty((M, V), dtype=torch.float32, device=dev)
    ws_s = ops.workspace(ops.VQ_OP_SAMPLE, M, V, 0, dev)
    ws_h = p.ws[(ops.VQ_OP_LMHEAD, V, HIDDEN)]
    u = torch.from_numpy(inputs_mod.uniforms((5, 3000), M)).to(dev)
    ua = torch.from_numpy(inputs_mod.uniforms((5, 3001), M)).to(dev)
    tok = torch.empty(M, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    commit = torch.empty((1, M), dtype=torch.int32, device=dev)
    # draft distributions: 16 candidates per row around the target's argmax
    q_ids = torch.from_numpy(inputs_mod.rng(5, 3002).integers(0, V, (1, M - 1, 16), dtype=np.int32)).to(dev)
    q_ids[:, :, 0] = p.argmax[: M - 1].view(1, M - 1)
    q_p = torch.full((1, M - 1, 16), 1.0 / 16, dtype=torch.float32, device=dev)

    def head_logits():
        ops.vq_lmhead_argmax_accept(p.h_final, p.w[head], 1.0, V, p.drafts, 1, M, p.argmax, p.accept,
                                    maxlogit_out=p.maxlogit, commit_out=p.commit, logits_out=logits, workspace=ws_h)

    def sample():
        ops.vq_sample_accept(logits, 1, M, 1.0, 32, 0.95, u, acc, draft=p.drafts, token_out=tok,
                             commit_out=commit, workspace=ws_s)

    def sample_spec():
        ops.vq_sample_accept(logits, 1, M, 1.0, 32, 0.95, u, acc, draft=p.drafts, draft_ids=q_ids,
                             draft_probs=q_p, u_accept=ua, token_out=tok, commit_out=commit, workspace=ws_s)

    def timed(fn):
        # `reps` calls captured in one graph, so the host's launch cost (tens
        # of microseconds per call from Python) does not hide the kernels
        fn()
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(gr, stream=st):
                for _ in range(reps):
                    fn()
        torch.cuda.current_stream().wait_stream(st)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    head_greedy_us = timed(lambda: p.launch(head))
    head_logits_us = timed(head_logits)
    sample_us = timed(sample)
    spec_us = timed(sample_spec)

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            p.y_acc.zero_()
            for i in range(head):
                p.launch(i)
            head_logits()
            sample()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(g_steps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / g_steps
    lb = M * V * 4
    return {
        "temperature": 1.0, "top_k": 32, "top_p": 0.95, "rule": "point-mass (graph); speculative timed alone",
        "ms_per_pass_sampled": round(dt * 1e3, 4),
        "weight_gbps_sampled": round(p.weight_bytes / dt / 1e9, 1),
        "head_greedy_us": round(head_greedy_us, 2),
        "head_with_fp32_logits_us": round(head_logits_us, 2),
        "sampler_us": round(sample_us, 2),
        "sampler_spec_us": round(spec_us, 2),
        "sampler_logit_bytes": lb,
        "sampler_logit_gbps": round(lb / (sample_us * 1e-6) / 1e9, 1),
        "accept_len_last": int(acc.item()),
    }


def cpu_baseline(inputs_mod):
    """The oracle, as it stands, timed end to end on whole configurations of
    the workload (seeded host inputs; generation not timed): config 2, one
    full MLP layer at M = 8 ([gate; up] 34,816 x 5,120 + SiLU*up, then down
    5,120 x 17,408, NVFP4); config 4, the vocabulary head 248,320 x 5,120
    (NVFP4) with the per-row argmax and the greedy accept; and one FP8 GDN
    in-projection 16,384 x 5,120 (config 3's FP8 shape). `value` is their
    weight bytes over their time; the whole pass is extrapolated from the
    NVFP4 and FP8 rates (labelled as such), and the GDN state stream from one
    layer's verify scan."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    res = {}
    # config 2: one MLP layer
    x = inputs_mod.x_bf16((6, 0), M_ROWS, HIDDEN)
    gu_c, gu_s = inputs_mod.nvfp4_weights((6, 1), 2 * INTER, HIDDEN)
    dn_c, dn_s = inputs_mod.nvfp4_weights((6, 2), HIDDEN, INTER)
    t0 = time.perf_counter()
    _, hb = O.mlp_silu_mul(x, gu_c, gu_s, 1.0, INTER)
    O.gemm_nvfp4(hb, dn_c, dn_s, 1.0)
    t_mlp = time.perf_counter() - t0
    b_mlp = weight_bytes("nvfp4_silu", INTER, HIDDEN) + weight_bytes("nvfp4", HIDDEN, INTER)
    res["config2_mlp_layer"] = {"seconds": round(t_mlp, 3), "weight_bytes": b_mlp, "gbps": round(b_mlp / t_mlp / 1e9, 4)}
    del gu_c, gu_s, dn_c, dn_s
    # config 4: head + argmax + accept
    hc, hs = inputs_mod.nvfp4_weights((6, 3), VOCAB, HIDDEN)
    h = inputs_mod.x_bf16((6, 4), M_ROWS, HIDDEN)
    drafts = inputs_mod.drafts((6, 5), inputs_mod.rng(6, 6).integers(0, VOCAB, (1, M_ROWS)), VOCAB)
    t0 = time.perf_counter()
    lg = O.gemm_nvfp4(h, hc, hs, 1.0)
    am = O.argmax_lowest(lg)
    O.greedy_accept(am.reshape(1, M_ROWS), drafts)
    t_head = time.perf_counter() - t0
    b_head = weight_bytes("head", VOCAB, HIDDEN)
    res["config4_head_argmax_accept"] = {"seconds": round(t_head, 3), "weight_bytes": b_head,
                                         "gbps": round(b_head / t_head / 1e9, 4)}
    del hc, hs, lg
    # one FP8 matrix of config 3
    w8 = inputs_mod.fp8_weights((6, 7), GDN_IN, HIDDEN)
    t0 = time.perf_counter()
    O.gemm_fp8(x, w8, 1.0)
    t_f8 = time.perf_counter() - t0
    b_f8m = GDN_IN * HIDDEN
    res["config3_gdn_in_fp8"] = {"seconds": round(t_f8, 3), "weight_bytes": b_f8m, "gbps": round(b_f8m / t_f8 / 1e9, 4)}
    del w8
    items = schedule()
    b_f4 = sum(weight_bytes(f, n, k) for _, f, n, k in items if f != "fp8")
    b_f8 = sum(weight_bytes(f, n, k) for _, f, n, k in items if f == "fp8")
    gbps_f4 = (b_mlp + b_head) / (t_mlp + t_head) / 1e9
    gbps_f8 = b_f8m / t_f8 / 1e9
    s_pass = b_f4 / (gbps_f4 * 1e9) + b_f8 / (gbps_f8 * 1e9)
    # the GDN state stream's oracle: one layer's verify scan (48 value heads,
    # 16 key heads, 8 rows), scaled to the 48 GDN layers of a pass
    gin = inputs_mod.gdn_inputs((6, 8), 1, M_ROWS, GDN_V_HEADS, GDN_K_HEADS)
    t0 = time.perf_counter()
    O.gdn_scan(*gin)
    t_gdn = time.perf_counter() - t0
    gdn = {"ms_per_pass_extrapolated": round(t_gdn * GDN_LAYERS * 1e3, 1),
           "gbps": round(gdn_bytes(1, 1, M_ROWS) / t_gdn / 1e9, 4),
           "sample": "fp64 numpy oracle, one layer's verify scan (48 heads x 8 rows), x48 layers"}
    t_all = t_mlp + t_head + t_f8
    return {
        "value": round((b_mlp + b_head + b_f8m) / t_all / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle end to end on config 2 (one MLP layer, {t_mlp:.2f} s), config 4 (head + "
                   f"argmax + accept, {t_head:.2f} s) and one FP8 16384x5120 matrix ({t_f8:.2f} s): "
                   f"{b_mlp + b_head + b_f8m} weight bytes in {t_all:.2f} s"),
        "configs": res,
        "ms_per_pass_extrapolated": round(s_pass * 1e3, 1),
        "extrapolation": (f"the pass's {b_f4} NVFP4 bytes at the NVFP4 rate of configs 2 and 4 ({gbps_f4:.3f} GB/s) "
                          f"plus its {b_f8} FP8 bytes at the FP8 rate ({gbps_f8:.3f} GB/s)"),
        "gdn_state_stream": gdn,
    }


def kernel_source_digest():
    """sha256 of the kernel sources and the code generation flags: stored
    HBM-traffic figures apply only to the kernels they were counted on."""
    import hashlib
    from bit_block_scaled_vq_amd.build import CODEGEN_FLAGS
    h = hashlib.sha256()
    for f in ("vq_kernels.hip", "vq_internal.h", "vq_keys.h"):
        with open(os.path.join(ROOT, "bit_block_scaled_vq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(CODEGEN_FLAGS).encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel factor),
    or None when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "gate_up_silu_m8_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return int(t["traffic_bytes_per_launch"])


def pmc_workload(m_rows=M_ROWS, copies=4, reps=2):
    """Small fixed workload for hardware-counter runs: the copy probe on
    1 GiB (the calibration kernel of known traffic) and the dominant kernel
    ([gate; up] + SiLU*up, M = m_rows) on rotating weight copies."""
    import torch
    from bit_block_scaled_vq_amd import inputs, ops
    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    for _ in range(reps):
        ops.vq_probe_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    ws = []
    for c in range(copies):
        cc, ss = inputs.device_nvfp4_weights((5, 3000 + c), 2 * INTER, HIDDEN, dev)
        ws.append(ops.pack_nvfp4(cc, ss, gate_up=True))
        del cc, ss
    x = inputs.device_x_bf16((5, 1000), m_rows, HIDDEN, dev)
    h = torch.empty((m_rows, INTER), dtype=torch.bfloat16, device=dev)
    work = ops.workspace(ops.VQ_OP_NVFP4_SILU_MUL, m_rows, INTER, HIDDEN, dev)
    for r in range(reps):
        for w in ws:
            ops.vq_gemm_nvfp4(x, w, 1.0, h, epilogue=ops.VQ_EPI_SILU_MUL, workspace=work)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_workload": {"rows": m_rows, "copy_probe_bytes_each": nbytes, "copy_probe_launches": reps,
                                       "gate_up_launches": reps * copies,
                                       "gate_up_weight_bytes": weight_bytes("nvfp4_silu", INTER, HIDDEN),
                                       "gate_up_activation_bytes": act_bytes(INTER, HIDDEN, m_rows)}}), flush=True)


def pmc_gdn_workload(reps=2, commit_rows=4):
    """Hardware-counter workload of the GDN state stream: the copy probe on
    1 GiB (calibration), then the commit over 48 layers x 1 lane (accept
    length 4 of 8 rows, so every layer is re-scanned: the state read from one
    slot and written to the other) and one per-layer verify launch."""
    import torch
    from bit_block_scaled_vq_amd import inputs, ops
    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    for _ in range(reps):
        ops.vq_probe_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    L, T, H, Hk = GDN_LAYERS, M_ROWS, GDN_V_HEADS, GDN_K_HEADS
    state, q, k, v, a, b = inputs.device_gdn_inputs((5, 7200), L, T, H, Hk, dev)
    slot = torch.empty_like(state)
    o = torch.empty_like(v)
    acc = torch.full((1,), commit_rows, dtype=torch.int32, device=dev)
    for _ in range(reps):
        ops.vq_gdn_commit(state, slot, q, k, v, a, b, acc, lanes=1)
    ops.vq_gdn_verify(state[:1], slot[:1], q[:1], k[:1], v[:1], a[:1], b[:1], o[:1])
    torch.cuda.synchronize()
    print(json.dumps({"pmc_gdn_workload": {"copy_probe_bytes_each": nbytes, "copy_probe_launches": reps,
                                           "commit_launches": reps, "commit_rows": commit_rows,
                                           "commit_bytes": gdn_bytes(L, 1, commit_rows, read_q=False, write_o=False),
                                           "verify_launches": 1, "verify_bytes": gdn_bytes(1, 1, T)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 passes take under a second; enough that the first graph launch's
    # host-side enqueue and the closing synchronize (about 0.4 ms together)
    # add only ~2 us to a pass
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run only the small hardware-counter workload (copy probe + dominant kernel)")
    ap.add_argument("--pmc-rows", type=int, default=M_ROWS, help="activation rows M of the counter workload")
    ap.add_argument("--pmc-gdn-workload", action="store_true",
                    help="run only the hardware-counter workload of the GDN state stream (copy probe + commit)")
    args = ap.parse_args()
    if args.pmc_workload:
        pmc_workload(args.pmc_rows)
        return
    if args.pmc_gdn_workload:
        pmc_gdn_workload()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the verify-pass weight stream is built and timed on a single "
              f"MI355X (asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_block_scaled_vq_amd import inputs, ops
    ops.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    probes = measure_probes(torch, ops, dev)
    log(f"probes: copy {probes['copy']:.0f} GB/s, read {probes['read']:.0f} GB/s")

    p = Pass(torch, ops, inputs, dev)
    # a realistic draft block: the target's own argmax with p = 0.7 per draft
    p.run()
    torch.cuda.synchronize()
    p.drafts.copy_(inputs.device_drafts((5, 2000), p.argmax.view(1, M_ROWS), VOCAB))

    # capture the pass once, replay it
    g = capture(torch, p.run)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    gbps = p.weight_bytes / dt / 1e9
    log(f"pass: {dt * 1e3:.3f} ms, {gbps:.0f} GB/s effective")

    # single replays (outside the timed region): spread of the pass time
    replays = replay_stats(torch, g)
    log(f"single replays: {replays}")

    # eager (ungraphed) pass: what the graph saves
    t0 = time.perf_counter()
    p.run()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3
    kinds = per_kind_durations(torch, p)
    log("kernels (graph replays): " + ", ".join(f"{k} {v['avg_us']} us" for k, v in kinds.items()))
    dom_s = kinds["mlp_gate_up"]["avg_us"] * 1e-6
    latency = small_gemm_latency(torch, ops, inputs, dev)
    log(f"config 1 latency: {latency}")
    lanes = lane_passes(torch, ops, inputs, p)
    log(f"passes at 2-4 lanes: {lanes}")
    sweep = m_sweep(torch, ops, inputs, p)
    sampled = sampled_verify(torch, ops, inputs, p)
    affine = affine_q4(torch, ops, inputs, dev)
    draft = draft_stream(torch, ops, inputs, p)
    log(f"draft block: {draft['ms_per_block']:.3f} ms, {draft['gbps']:.0f} GB/s")
    gdn = gdn_state_stream(torch, ops, inputs, dev)
    log(f"GDN state stream at M=8: {gdn['8']}")
    with_state = pass_with_state(torch, ops, inputs, p)
    log(f"pass with the GDN state stream: {with_state}")
    log(f"affine 4-bit MLP at M=8: {affine['8']}")
    log(f"sampled verify: pass {sampled['ms_per_pass_sampled']:.3f} ms, sampler {sampled['sampler_us']:.1f} us")
    gu_w = weight_bytes("nvfp4_silu", INTER, HIDDEN)
    gu_a = act_bytes(INTER, HIDDEN)
    achieved = (gu_w + gu_a) / dom_s / 1e9
    accept = int(p.accept.item())
    target = {}
    for probe in ("copy", "read"):
        need_ms = p.weight_bytes / (0.8 * probes[probe] * 1e9) * 1e3
        target[probe] = {"probe_gbps": round(probes[probe], 1), "pct_achieved": round(100 * gbps / probes[probe], 1),
                         "ms_per_pass_for_80pct": round(need_ms, 4), "met": bool(dt * 1e3 <= need_ms)}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(inputs)

    res = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded NVFP4/FP8 weights of the 27B hybrid's shapes, generated on the device)",
        "config": {
            "workload": "full M=8 verify-pass weight stream: 64 layers (48 GDN FP8 in/out, 16 attention FP8 "
                        "q+gate+k+v/o), 64 NVFP4 SwiGLU MLPs, NVFP4 vocab head + argmax + accept",
            "rows": M_ROWS, "launches": len(p.items), "weight_bytes": p.weight_bytes,
            "activation_bytes": p.act_bytes, "graph": True,
        },
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "pct_of_measured_copy_bw": round(100 * gbps / probes["copy"], 1),
        "pct_of_measured_read_bw": round(100 * gbps / probes["read"], 1),
        "measured_copy_gbps": round(probes["copy"], 1),
        "measured_read_gbps": round(probes["read"], 1),
        "target_80pct_of_measured_bw": target,
        "tok_s_at_alpha_4_80": round(ALPHA / dt, 1),
        "pass_replay_ms": replays,
        "sum_of_kernel_times_ms": round(sum(v["avg_us"] * v["launches_per_pass"] for v in kinds.values()) / 1e3, 4),
        "eager_ms_per_pass": round(eager_ms, 3),
        "accept_len_last_pass": accept,
        "kernels": kinds,
        "config1_latency": latency,
        "lane_passes": lanes,
        "m_sweep_weight_gbps": sweep,
        "sampled_verify": sampled,
        "affine_q4_mlp": affine,
        "draft_block": draft,
        "gdn_state_stream": gdn,
        "pass_with_gdn_state": with_state,
        "roofline": {
            "kernel": "vq_gemm_kernel<NVFP4, SILU_MUL, M<=8> ([gate;up] 34816x5120 + SiLU*up)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(),
            "avg_launch_us": round(dom_s * 1e6, 2),
            "bytes_per_launch": gu_w + gu_a,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
