#!/usr/bin/env python3
"""Throughput of the PTQ1_0 ternary linear layer on one MI355X.

Step (the headline): one batch-1 decode token through one 27B-shaped
feed-forward block, i.e. the whole decode hot path:
    embedding row 248320 x 5120 -> unrotate (hadamard_unrotate_rows)
    x[5120] -> rotate -> fused gate+up 5120 -> 2 x 17408  (ptq1_ffn_block, m = 1)
            -> SwiGLU -> rotate -> down 17408 -> 5120 + residual
Weights rotate over WEIGHT_SETS independent sets (936 MB, beyond the 256 MB
Infinity Cache) so every step streams its 58.5 MB of PTQ1_0 blocks from HBM.
value = algorithmic bytes per step / step time (decode matvec GB/s).

The timed steps replay HIP graphs of the step (the step is five dependent
kernels, about 30 us in all, so eager launches leave the GPU waiting on
the host).

roofline: the dominant kernel, the table-lookup matvec over gate and up
(one launch per step), timed in a second pass of the same K steps run
eagerly, with HIP events attached to that kernel's dispatch by the library
(ptq1_profile_arm -> hipExtLaunchKernel: the kernel's own start and end)
and a spin kernel ahead of each step, so that the GPU is as busy between
steps as in the graph replays (busy()); algorithmic bytes per launch = its
PTQ1_0 blocks + x.  `traffic` is the
counter-measured HBM bytes per launch from the committed rocprofv3 summary
profiles/lut_matvec_gate_up_decode_27b_traffic.md, or null when that
kernel's source changed after the counters were taken.

Also reported (breakdown; a call's time is one HIP-graph replay of many
calls, a kernel's time its dispatch events as above): the down-projection
lookup kernel inside the same steps, cold gate+up and down calls alone, the pages' float-peel decode
on the same matrices, the hot 1024 x 1024 matvec, the prefill GEMM at
M = 128 / 256 / 512 (TFLOP/s, fraction of the bf16 MFMA peak), and the
64-layer FFN stack at batch 1 and 8 (layers/s, and the relative L2 of its
output against the oracle).  cpu_baseline: the fp64 oracle timed on the
host's cores on bounded samples of every configuration, in the GPU's units.
receipt: GPU, ROCm, clocks, host CPU and load average.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
                    [--copy-calibration]
    python bench.py --gemm-only M [--format ptq1|pq2|w2a8]   (one GEMM kind, for profilers)
    python bench.py --ffn-only M [--format ptq1|pq2]         (one FFN block, HIP graph)
    python bench.py --decode-only lut|peel|w2a8              (one decode matvec kind)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
D, F, VOCAB, LAYERS = 5120, 17408, 248320, 64
WEIGHT_SETS = 16
BYTES_PER_WEIGHT = 28 / 128    # one PTQ1_0 block = 28 B per 128 weights


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def packed(n, k):
    return n * (k // 128) * 28


# algorithmic bytes (what the method must move; fp32 activations)
GATE_UP_BYTES = 2 * packed(F, D) + 4 * D + 2 * 4 * F          # weights, x in, g & u out
DOWN_BYTES = packed(D, F) + 4 * F + 4 * D + 4 * D             # weights, h in, residual in, out
SWIGLU_BYTES = 3 * 4 * F                                      # g, u in, h out
EMBED_BYTES = 2 * 4 * D                                       # one row in, one row out
STEP_BYTES = GATE_UP_BYTES + SWIGLU_BYTES + DOWN_BYTES + EMBED_BYTES
LAYER_WEIGHT_BYTES = 3 * packed(F, D)
# the dominant kernel: the lookup-table matvec over gate and up reads both
# matrices' blocks and x once per launch (its split-K partials are scratch)
LUT_GATE_UP_BYTES = 2 * packed(F, D) + 4 * D
LUT_DOWN_BYTES = packed(D, F) + 4 * F
COPY_CAL_BYTES = 256 << 20     # plain device copy used to scale the byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lut_matvec_gate_up_decode_27b_traffic.md")
LUT_SOURCE = os.path.join(ROOT, "ternary_weight_ptq1_amd", "csrc", "matvec_lut.hip")


def lut_source_hash() -> str:
    with open(LUT_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the gate+up lookup kernel from the committed
    counter summary, if it was taken on the current kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_src = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    m_val = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    if not m_src or not m_val or m_src.group(1) != lut_source_hash():
        return None
    return int(m_val.group(1))


INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA

# Event-timed dispatches are launched eagerly from Python, which is slower
# than the GPU: between calls the GPU would idle, and a kernel that follows
# an idle gap runs longer than the same kernel inside a graph replay (the
# gate+up lookup kernel: mean 13.0 against 11.9 us, 90th percentile 15.1
# against 12.1).  A spin kernel (torch.cuda._sleep: a clock loop, no memory
# traffic) ahead of each such call keeps the GPU busy while the host
# launches, as in the timed graph replays.
SPIN_CYCLES = 200000


def busy(torch):
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is None:
        raise RuntimeError("torch.cuda._sleep is missing: the event-timed passes need a spin kernel")
    spin(SPIN_CYCLES)


def gemm_only(args, torch, synth, sdev, P, dev) -> int:
    """The prefill GEMM alone (for counter runs): M x 5120 activations against
    one 17408 x 5120 PTQ1_0 matrix, --steps calls after --warmup; --format
    w2a8 runs the 8-bit-activation GEMM (int8 MFMA) instead, --format pq2 the
    same matrix in PQ2_0."""
    m, n, k = args.gemm_only, F, D
    w8 = args.format == "w2a8"
    q2 = args.format == "pq2"
    pack, tile = (P.pq2_pack, P.pq2_tile) if q2 else (P.ptq1_pack, P.ptq1_tile)
    w = tile(pack(sdev.trits(1, 1, n, k), sdev.scales(1, 2, n, k // 128)), n, k)
    x = torch.from_numpy(synth.activations(1, m, k)).to(dev)
    sg = torch.from_numpy(synth.signs(1)).to(dev)
    y = torch.empty(m, n, device=dev)
    nws = (P.lib().ptq1_gemm_w2a8_workspace_bytes(m, n, k) if w8 else
           P.workspace_bytes("pq2_gemm", m, n, k) if q2 else P.workspace_bytes("gemm", m, n, k))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def call():
        if w8:
            P.ptq1_gemm_w2a8(w, n, k, x, out=y, ws=ws)
        elif q2:
            P.pq2_gemm(w, n, k, x, sg, out=y, ws=ws)
        else:
            P.ptq1_gemm(w, n, k, x, sg, out=y, ws=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    kt = P.KernelTimer("gemm", args.steps)
    with kt:
        for _ in range(args.steps):
            busy(torch)
            call()
    torch.cuda.synchronize()
    ms = sorted(kt.durations_ms())
    kt.close()
    us = ms[len(ms) // 2] * 1e3
    fl = 2.0 * m * n * k
    peak = INT8_PEAK_TOPS if w8 else BF16_PEAK_TFLOPS
    print(json.dumps({"workload": f"prefill GEMM {m}x{k} -> {n} ({'int8 W2A8' if w8 else 'bf16, PQ2_0' if q2 else 'bf16'})",
                      "us_kernel_median": us, "TFLOP/s": fl / (us * 1e-6) / 1e12,
                      "mfma_frac": fl / (us * 1e-6) / 1e12 / peak}))
    return 0


def decode_only(args, torch, synth, sdev, P, dev) -> int:
    """One decode matvec kind alone (for counter runs): the down projection's
    17408 -> 5120 PTQ1_0 matrix over WEIGHT_SETS cold copies, --steps calls
    after --warmup: 'lut' (table lookups, fp32), 'peel' (the pages' float
    peel, eight lanes per block), 'w2a8' (8-bit activations, int32 sums)."""
    kind = args.decode_only
    mats = [P.ptq1_tile(P.ptq1_pack(sdev.trits(1, synth.layer_stream(synth.S_DOWN_TRITS, j), D, F),
                                    sdev.scales(1, synth.layer_stream(synth.S_DOWN_SCALES, j), D, F // 128)), D, F)
            for j in range(WEIGHT_SETS)]
    h = torch.from_numpy(synth.activations(2, 1, F)[0]).to(dev)
    sg = torch.from_numpy(synth.signs(1)).to(dev)
    y = torch.empty(D, device=dev)
    ws = torch.zeros(P.workspace_bytes("matvec", D, F), dtype=torch.uint8, device=dev)
    fam = {"lut": "lut_matvec_1", "peel": "peel_matvec", "w2a8": "lut_matvec_1"}[kind]

    def call(i):
        W = mats[i % WEIGHT_SETS]
        if kind == "lut":
            P.ptq1_matvec(W, D, F, h, sg, out=y, ws=ws)
        elif kind == "peel":
            P.ptq1_matvec_float_peel(W, D, F, h, sg, out=y, ws=ws)
        else:
            P.ptq1_matvec_w2a8(W, D, F, h, out=y, ws=ws)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    kt = P.KernelTimer(fam, args.steps)
    with kt:
        for i in range(args.steps):
            busy(torch)
            call(i)
    torch.cuda.synchronize()
    d = kt.durations_ms()
    kt.close()
    us = 1e3 * sum(d) / len(d)
    b = packed(D, F) + 4 * F
    print(json.dumps({"workload": f"decode matvec {F} -> {D} ({kind}), {WEIGHT_SETS} cold weight sets",
                      "us_kernel_mean": us, "GB/s": b / (us * 1e-6) / 1e9, "frac_hbm": b / (us * 1e-6) / 8e12}))
    return 0


def ffn_only(args, torch, synth, sdev, P, dev) -> int:
    """One 27B-shaped FFN block at batch M alone (for kernel traces): --steps
    calls (one weight set) replayed from a HIP graph of 16 calls after
    --warmup eager ones."""
    m = args.ffn_only
    q2 = args.format == "pq2"
    pack, tile = (P.pq2_pack, P.pq2_tile) if q2 else (P.ptq1_pack, P.ptq1_tile)
    w = [tile(pack(sdev.trits(4, tr, n, k), sdev.scales(4, sc, n, k // 128)), n, k)
         for tr, sc, n, k in ((synth.S_GATE_TRITS, synth.S_GATE_SCALES, F, D),
                              (synth.S_UP_TRITS, synth.S_UP_SCALES, F, D),
                              (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, D, F))]
    x = torch.from_numpy(synth.activations(4, m, D)).to(dev)
    sg = torch.from_numpy(synth.signs(4)).to(dev)
    out = torch.empty_like(x)
    nws = P.lib().pq2_ffn_workspace_bytes(m, D, F) if q2 else P.workspace_bytes("ffn", m, D, F)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    block = P.pq2_ffn_block if q2 else P.ptq1_ffn_block
    wbytes = 2 * P.pq2_tiled_bytes(F, D) + P.pq2_tiled_bytes(D, F) if q2 else LAYER_WEIGHT_BYTES

    def call():
        block(x, w[0], w[1], w[2], sg, D, F, rms_eps=1e-6, out=out, ws=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # one graph of `per` calls (a graph launch per call would add its own
    # launch cost to every call), replayed until --steps calls have run
    per = min(16, max(1, args.steps))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // per)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * per)
    fmt = "PQ2_0" if q2 else "PTQ1_0"
    print(json.dumps({"workload": f"FFN block {m} x {D} -> {F} -> {D} ({fmt}), HIP graph", "us_per_layer": us,
                      "weight_GB/s": wbytes / (us * 1e-6) / 1e9}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--quick", action="store_true", help="headline only (no breakdown)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (scale for the byte counters)")
    ap.add_argument("--gemm-only", type=int, default=0, metavar="M",
                    help="profiling aid: run the prefill GEMM (M x 5120 -> 17408) --steps times, print its "
                         "kernel time, and exit")
    ap.add_argument("--format", choices=("ptq1", "pq2", "w2a8"), default="ptq1",
                    help="weight format of --gemm-only and --ffn-only (PTQ1_0 or PQ2_0); w2a8 makes "
                         "--gemm-only run the 8-bit-activation GEMM (there is no W2A8 FFN block)")
    ap.add_argument("--decode-only", choices=("lut", "peel", "w2a8"), default=None,
                    help="profiling aid: run one decode matvec kind (17408 -> 5120, cold weights) --steps "
                         "times, print its kernel time, and exit")
    ap.add_argument("--ffn-only", type=int, default=0, metavar="M",
                    help="profiling aid: replay one FFN block at batch M --steps times from a HIP graph, print "
                         "its time per layer, and exit")
    args = ap.parse_args()
    if args.ffn_only > 0 and args.format == "w2a8":
        print("--ffn-only takes --format ptq1 or pq2 (there is no W2A8 FFN block)", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the sharded path is a "
              "design note, not built", file=sys.stderr)
        return 2

    import torch

    import synth
    import synth.device as sdev
    import ternary_weight_ptq1_amd as P

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    P.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    rec = receipt(torch, dev)
    stream = torch.cuda.current_stream()
    if args.decode_only is not None:
        return decode_only(args, torch, synth, sdev, P, dev)
    if args.gemm_only > 0:
        return gemm_only(args, torch, synth, sdev, P, dev)
    if args.ffn_only > 0:
        return ffn_only(args, torch, synth, sdev, P, dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, warm, mode="graph"):
        """ms per call of fn(0) .. fn(reps - 1) after `warm` eager calls.  mode
        "graph": the calls replayed from one HIP graph (GPU time, launches back
        to back); "events": launched eagerly with a spin kernel ahead of each
        (busy()), for passes whose kernel dispatches carry HIP events (which a
        graph does not) -- the returned time then includes the spins and is not
        used; "eager": plain eager calls."""
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        if mode == "graph":
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    fn(i)
            g.replay()  # the first replay uploads the graph
            torch.cuda.synchronize()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            del g
        else:
            a.record(stream)
            for i in range(reps):
                if mode == "events":
                    busy(torch)
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) / reps  # ms per call

    def weight_set(seed, layer):
        ls = synth.layer_stream
        out = []
        for tr, sc, n, k in ((synth.S_GATE_TRITS, synth.S_GATE_SCALES, F, D),
                             (synth.S_UP_TRITS, synth.S_UP_SCALES, F, D),
                             (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, D, F)):
            t = sdev.trits(seed, ls(tr, layer), n, k, device=dev)
            s = sdev.scales(seed, ls(sc, layer), n, k // 128, device=dev)
            out.append(P.ptq1_tile(P.ptq1_pack(t, s), n, k))
            del t, s
        return out

    log("bench: generating inputs")
    seed = 1
    signs = torch.from_numpy(synth.signs(seed)).to(dev)
    sets = [weight_set(seed, L) for L in range(WEIGHT_SETS)]
    table = sdev.gauss(2, synth.S_TABLE, VOCAB * D, device=dev).view(VOCAB, D)
    ids = torch.from_numpy(synth.token_ids(2, 4096, VOCAB)).to(dev)
    emb = torch.empty((1, D), dtype=torch.float32, device=dev)
    x_out = torch.empty(D, dtype=torch.float32, device=dev)
    ws = torch.zeros(P.workspace_bytes("ffn", 1, D, F), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        W = sets[i % WEIGHT_SETS]
        P.hadamard_unrotate_rows(table, signs, ids=ids[i % 4096:i % 4096 + 1], out=emb)
        P.ptq1_ffn_block(emb, W[0], W[1], W[2], signs, D, F, rms_eps=1e-6, out=x_out, ws=ws)

    log("bench: headline step")
    for i in range(args.warmup):  # eager warm-up (also settles per-kernel launch attributes)
        step(i)
    torch.cuda.synchronize()
    # The step is launch-bound (five dependent kernels, about 30 us), so the
    # timed steps replay HIP graphs: one of WEIGHT_SETS steps (a pass over
    # every weight set) and one of the remainder, so that exactly K steps run.
    graphs = []
    for count in (WEIGHT_SETS, args.steps % WEIGHT_SETS):
        if count == 0:
            graphs.append(None)
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    if graphs[0] is not None:
        graphs[0].replay()  # first replay uploads the graph
    if graphs[1] is not None:
        graphs[1].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(args.steps // WEIGHT_SETS):
        graphs[0].replay()
    if graphs[1] is not None:
        graphs[1].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk_end = clocks()
    ms_step = e0.elapsed_time(e1) / args.steps
    gbs = STEP_BYTES / (ms_step * 1e-3) / 1e9
    del graphs

    # roofline pass: the same K steps run eagerly with HIP events attached to
    # the dispatches of the gate+up and down lookup kernels (ptq1_profile_arm),
    # a spin kernel ahead of each step keeping the GPU as busy as in the
    # graph replays (busy())
    log("bench: roofline pass")
    t_gu = P.KernelTimer("lut_matvec_2", args.steps)
    t_dn = P.KernelTimer("lut_matvec_1", args.steps)
    with t_gu, t_dn:
        for i in range(args.steps):
            busy(torch)
            step(i)
    torch.cuda.synchronize()
    d_gu, d_dn = t_gu.durations_ms(), t_dn.durations_ms()
    t_gu.close()
    t_dn.close()
    assert len(d_gu) == args.steps and len(d_dn) == args.steps, "one gate+up and one down launch per step"
    us_gu = 1e3 * sum(d_gu) / len(d_gu)
    us_dn = 1e3 * sum(d_dn) / len(d_dn)

    def spread(d):  # median, min and max of the per-launch event durations (us)
        v = sorted(1e3 * t for t in d)
        return {"median": round(v[len(v) // 2], 3), "min": round(v[0], 3), "max": round(v[-1], 3)}
    lut_gu_gbs = LUT_GATE_UP_BYTES / (us_gu * 1e-6) / 1e9
    lut_dn_gbs = LUT_DOWN_BYTES / (us_dn * 1e-6) / 1e9

    # dominant kernel: the fused gate+up decode matvec (cold), timed alone on the same stream
    ws_gu = torch.zeros(P.workspace_bytes("gate_up", F, D), dtype=torch.uint8, device=dev)
    xg = torch.from_numpy(synth.activations(seed, 1, D)[0]).to(dev)
    g_buf = torch.empty(F, dtype=torch.float32, device=dev)
    u_buf = torch.empty(F, dtype=torch.float32, device=dev)

    def gate_up(i):
        W = sets[i % WEIGHT_SETS]
        P.ptq1_gate_up(W[0], W[1], F, D, xg, signs, g=g_buf, u=u_buf, ws=ws_gu)

    ms_gu = timed(gate_up, max(args.steps, 100), args.warmup)
    gu_gbs = GATE_UP_BYTES / (ms_gu * 1e-3) / 1e9

    breakdown = {"lut_kernel_gate_up_in_step": dict({"us": us_gu, "GB/s": lut_gu_gbs, "bytes": LUT_GATE_UP_BYTES},
                                                    **spread(d_gu)),
                 "lut_kernel_down_in_step": dict({"us": us_dn, "GB/s": lut_dn_gbs, "bytes": LUT_DOWN_BYTES},
                                                 **spread(d_dn)),
                 "gate_up_call_cold": {"us": ms_gu * 1e3, "GB/s": gu_gbs, "bytes": GATE_UP_BYTES}}
    if not args.quick:
        log("bench: breakdown")
        ws_dn = torch.zeros(P.workspace_bytes("matvec", D, F), dtype=torch.uint8, device=dev)
        h = torch.from_numpy(synth.gauss(seed, 99, F)).to(dev)
        y = torch.empty(D, dtype=torch.float32, device=dev)

        def down(i):
            W = sets[i % WEIGHT_SETS]
            P.ptq1_matvec(W[2], D, F, h, signs, residual=xg, out=y, ws=ws_dn)

        ms_dn = timed(down, 200, 20)
        breakdown["down_call_cold"] = {"us": ms_dn * 1e3, "GB/s": DOWN_BYTES / (ms_dn * 1e-3) / 1e9,
                                       "bytes": DOWN_BYTES}

        # the pages' own decode (float peel, eight lanes per block, tiled layout) on the same
        # cold matrices: the down projection and one 17408 x 5120 (gate-shaped) matrix
        peel = {}
        for tag, (wi, n_, k_, xin, yb) in {"down_17408_to_5120": (2, D, F, h, y),
                                           "gate_5120_to_17408": (0, F, D, xg, g_buf)}.items():
            wsp = torch.zeros(P.workspace_bytes("matvec", n_, k_), dtype=torch.uint8, device=dev)
            timed(lambda i: P.ptq1_matvec_float_peel(sets[i % WEIGHT_SETS][wi], n_, k_, xin, signs, out=yb, ws=wsp),
                  5, 0, "eager")
            tp = P.KernelTimer("peel_matvec", 64)
            with tp:
                timed(lambda i: P.ptq1_matvec_float_peel(sets[i % WEIGHT_SETS][wi], n_, k_, xin, signs, out=yb,
                                                         ws=wsp), 64, 0, "events")
            dp = tp.durations_ms()
            tp.close()
            us_p = 1e3 * sum(dp) / len(dp)
            pb = packed(n_, k_) + 4 * k_
            peel[tag] = {"us_kernel": us_p, "GB/s": pb / (us_p * 1e-6) / 1e9, "frac_hbm": pb / (us_p * 1e-6) / 8e12}
            del wsp
        peel["lookup_kernel_down_us_in_step"] = us_dn
        breakdown["float_peel_decode"] = peel

        def unrot(i):
            P.hadamard_unrotate_rows(table, signs, ids=ids[i % 4096:i % 4096 + 1], out=emb)

        breakdown["embed_unrotate_row"] = {"us": timed(unrot, 200, 20) * 1e3}

        # prefill embedding gather: 256 rows of the table un-rotated in one call
        emb256 = torch.empty((256, D), dtype=torch.float32, device=dev)
        breakdown["embed_unrotate_256_rows"] = {
            "us": timed(lambda i: P.hadamard_unrotate_rows(table, signs, ids=ids[(i % 16) * 256:(i % 16 + 1) * 256],
                                                           out=emb256), 100, 10) * 1e3}
        del emb256

        # other folded projections at synthetic shapes (the pages give no
        # attention shapes): the same kernels, a wide and a narrow matrix,
        # decode (32 weight sets, beyond the Infinity Cache) and M = 256 prefill
        proj = {}
        for n_p, k_p in ((8192, D), (D, 8192)):
            psets = [P.ptq1_tile(P.ptq1_pack(sdev.trits(5, synth.layer_stream(synth.S_W_TRITS, j), n_p, k_p, device=dev),
                                             sdev.scales(5, synth.layer_stream(synth.S_W_SCALES, j), n_p, k_p // 128,
                                                         device=dev)), n_p, k_p) for j in range(32)]
            xp = torch.from_numpy(synth.activations(5, 256, k_p)).to(dev)
            yp = torch.empty(n_p, dtype=torch.float32, device=dev)
            wsp = torch.zeros(P.workspace_bytes("matvec", n_p, k_p), dtype=torch.uint8, device=dev)
            ms_p = timed(lambda i: P.ptq1_matvec(psets[i % 32], n_p, k_p, xp[0], signs, out=yp, ws=wsp), 200, 20)
            yg = torch.empty((256, n_p), dtype=torch.float32, device=dev)
            wsg = torch.zeros(P.workspace_bytes("gemm", 256, n_p, k_p), dtype=torch.uint8, device=dev)
            timed(lambda i: P.ptq1_gemm(psets[i % 32], n_p, k_p, xp, signs, out=yg, ws=wsg), 3, 0, "eager")  # warm-up
            tg = P.KernelTimer("gemm", 30)
            with tg:
                timed(lambda i: P.ptq1_gemm(psets[i % 32], n_p, k_p, xp, signs, out=yg, ws=wsg), 30, 0, "events")
            dg = tg.durations_ms()
            tg.close()
            us_gk = 1e3 * sum(dg) / len(dg)
            mv_bytes = packed(n_p, k_p) + 4 * (n_p + k_p)
            proj[f"{n_p}x{k_p}"] = {"matvec_us": ms_p * 1e3, "matvec_GB/s": mv_bytes / (ms_p * 1e-3) / 1e9,
                                    "gemm_M256_us_kernel": us_gk,
                                    "gemm_M256_TFLOP/s": 2.0 * 256 * n_p * k_p / (us_gk * 1e-6) / 1e12}
            del psets, xp, yp, wsp, yg, wsg
        breakdown["projections_synthetic_shapes"] = proj
        torch.cuda.empty_cache()

        # the same gate+up decode in the PQ2_0 format (2.125 bits per weight):
        # the two matrices stacked as one [2F, D] matrix, 32 weight sets, the
        # lookup kernel timed alone, against the PTQ1_0 kernel's figure above
        n2 = 2 * F
        q2sets = [P.pq2_tile(P.pq2_pack(sdev.trits(seed, synth.layer_stream(synth.S_W_TRITS, j), n2, D, device=dev),
                                        sdev.scales(seed, synth.layer_stream(synth.S_W_SCALES, j), n2, D // 128,
                                                    device=dev)), n2, D) for j in range(32)]
        y2 = torch.empty(n2, dtype=torch.float32, device=dev)
        ws2 = torch.zeros(P.workspace_bytes("pq2_matvec", n2, D), dtype=torch.uint8, device=dev)
        ms_q2 = timed(lambda i: P.pq2_matvec(q2sets[i % 32], n2, D, xg, signs, out=y2, ws=ws2), 200, 20)
        t2 = P.KernelTimer("pq2_matvec", 200)
        with t2:
            timed(lambda i: P.pq2_matvec(q2sets[i % 32], n2, D, xg, signs, out=y2, ws=ws2), 200, 0, "events")
        d2 = t2.durations_ms()
        t2.close()
        us_q2 = 1e3 * sum(d2) / len(d2)
        q2_bytes = P.pq2_tiled_bytes(n2, D) + 4 * D
        breakdown["pq2_gate_up_decode"] = {"us_kernel": us_q2, "GB/s": q2_bytes / (us_q2 * 1e-6) / 1e9,
                                           "bytes": q2_bytes, "call_us": ms_q2 * 1e3,
                                           "ptq1_kernel_us": us_gu}
        # and its M = 256 prefill GEMM (register-decode kernel at every M)
        xq = torch.from_numpy(synth.activations(seed, 256, D)).to(dev)
        yq = torch.empty((256, n2), dtype=torch.float32, device=dev)
        wsq = torch.zeros(P.workspace_bytes("pq2_gemm", 256, n2, D), dtype=torch.uint8, device=dev)
        timed(lambda i: P.pq2_gemm(q2sets[i % 32], n2, D, xq, signs, out=yq, ws=wsq), 3, 0, "eager")  # warm-up
        tq = P.KernelTimer("gemm", 30)
        with tq:
            timed(lambda i: P.pq2_gemm(q2sets[i % 32], n2, D, xq, signs, out=yq, ws=wsq), 30, 0, "events")
        dq = tq.durations_ms()
        tq.close()
        us_gq = 1e3 * sum(dq) / len(dq)
        breakdown["pq2_gate_up_prefill_M256"] = {"us_kernel": us_gq,
                                                 "TFLOP/s": 2.0 * 256 * n2 * D / (us_gq * 1e-6) / 1e12}
        del q2sets, y2, ws2, xq, yq, wsq
        torch.cuda.empty_cache()

        # the whole batch-1 block in PQ2_0 (16 rotating layers, replayed from a graph)
        def pq2_mat(role_t, role_s, j, n_, k_):
            return P.pq2_tile(P.pq2_pack(sdev.trits(seed, synth.layer_stream(role_t, j), n_, k_, device=dev),
                                         sdev.scales(seed, synth.layer_stream(role_s, j), n_, k_ // 128,
                                                     device=dev)), n_, k_)

        l2 = [(pq2_mat(synth.S_GATE_TRITS, synth.S_GATE_SCALES, j, F, D),
               pq2_mat(synth.S_UP_TRITS, synth.S_UP_SCALES, j, F, D),
               pq2_mat(synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, j, D, F)) for j in range(16)]
        xb2 = torch.from_numpy(synth.activations(seed, 1, D)).to(dev)
        ob2 = torch.empty_like(xb2)
        wsb2 = torch.zeros(P.lib().pq2_ffn_workspace_bytes(1, D, F), dtype=torch.uint8, device=dev)
        ms_b2 = timed(lambda i: P.pq2_ffn_block(xb2, *l2[i % 16], signs, D, F, 1e-6, out=ob2, ws=wsb2), 200, 20)
        b2_bytes = 2 * P.pq2_tiled_bytes(F, D) + P.pq2_tiled_bytes(D, F) + 4 * D
        breakdown["pq2_ffn_block_decode"] = {"us": ms_b2 * 1e3, "GB/s": b2_bytes / (ms_b2 * 1e-3) / 1e9,
                                                   "bytes": b2_bytes}
        del l2, xb2, ob2, wsb2

        # W2A8: the down projection's matvec with 8-bit activations (quantise,
        # lookups over integer-valued q, scaled sum), 16 weight sets as above
        ws8 = torch.zeros(P.lib().ptq1_matvec_w2a8_workspace_bytes(D, F), dtype=torch.uint8, device=dev)
        y8 = torch.empty(D, dtype=torch.float32, device=dev)
        ms8 = timed(lambda i: P.ptq1_matvec_w2a8(sets[i % WEIGHT_SETS][2], D, F, h, residual=xg, out=y8, ws=ws8),
                    200, 20)
        breakdown["w2a8_down_call_cold"] = {"us": ms8 * 1e3, "GB/s": DOWN_BYTES / (ms8 * 1e-3) / 1e9,
                                            "bytes": DOWN_BYTES, "float_call_us": ms_dn * 1e3}
        del ws8, y8
        # and the W2A8 prefill GEMM (per-token int8 rows on the bf16 MFMA path), M = 256, gate-sized matrix
        x8 = torch.from_numpy(synth.activations(seed, 256, D)).to(dev)
        yg8 = torch.empty((256, F), dtype=torch.float32, device=dev)
        wsg8 = torch.zeros(P.lib().ptq1_gemm_w2a8_workspace_bytes(256, F, D), dtype=torch.uint8, device=dev)
        ms_g8 = timed(lambda i: P.ptq1_gemm_w2a8(sets[i % WEIGHT_SETS][0], F, D, x8, out=yg8, ws=wsg8), 30, 3)
        breakdown["w2a8_gemm_M256_call"] = {"us": ms_g8 * 1e3, "TFLOP/s": 2.0 * 256 * F * D / (ms_g8 * 1e-3) / 1e12}
        del x8, yg8, wsg8
        torch.cuda.empty_cache()

        # hot 1024 x 1024 matvec (configuration 0; L2-resident, latency-bound)
        w0 = P.ptq1_tile(P.ptq1_pack(sdev.trits(0, synth.S_W_TRITS, 1024, 1024),
                                     sdev.scales(0, synth.S_W_SCALES, 1024, 8)), 1024, 1024)
        x0 = torch.from_numpy(synth.activations(0, 1, 1024)[0]).to(dev)
        s0 = torch.from_numpy(synth.signs(0)).to(dev)
        ws0 = torch.zeros(P.workspace_bytes("matvec", 1024, 1024), dtype=torch.uint8, device=dev)
        y0 = torch.empty(1024, dtype=torch.float32, device=dev)
        ms0 = timed(lambda i: P.ptq1_matvec(w0, 1024, 1024, x0, s0, out=y0, ws=ws0), 500, 50)
        breakdown["matvec_1024_hot"] = {"us": ms0 * 1e3}

        # measured streaming-read rate of this GPU, for context beside the
        # 8 TB/s published peak: torch row sums over 2 GiB of fp32 (8x the
        # Infinity Cache) viewed as [2^19, 1024], a read-only kernel with one
        # output per 4 KB row (the fastest of the plain torch reductions and
        # copies tried: a full sum reads at about 4 TB/s, a copy at 4.9)
        big = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        ms_rd = timed(lambda i: big.view(-1, 1024).sum(dim=1), 20, 3, "eager")
        rd_gbs = big.numel() * 4 / (ms_rd * 1e-3) / 1e9
        breakdown["hbm_read_measured"] = {"GB/s": rd_gbs, "how": "torch row sums over [2^19, 1024] fp32 (2 GiB), 20 calls",
                                          "lut_gate_up_frac_of_it": lut_gu_gbs / rd_gbs}
        del big
        torch.cuda.empty_cache()

        # prefill GEMM (configuration 3)
        wq = P.ptq1_tile(P.ptq1_pack(sdev.trits(3, synth.S_W_TRITS, F, D),
                                     sdev.scales(3, synth.S_W_SCALES, F, D // 128)), F, D)
        gemm = {}
        for m in (128, 256, 512):
            xm = torch.from_numpy(synth.activations(3, m, D)).to(dev)
            ym = torch.empty((m, F), dtype=torch.float32, device=dev)
            wsm = torch.zeros(P.workspace_bytes("gemm", m, F, D), dtype=torch.uint8, device=dev)
            ms = timed(lambda i: P.ptq1_gemm(wq, F, D, xm, signs, out=ym, ws=wsm), 50, 3)
            tg = P.KernelTimer("gemm", 50)
            with tg:
                timed(lambda i: P.ptq1_gemm(wq, F, D, xm, signs, out=ym, ws=wsm), 50, 0, "events")
            dg = tg.durations_ms()
            tg.close()
            us_k = 1e3 * sum(dg) / len(dg)
            fl = 2.0 * m * F * D
            gemm[f"M{m}"] = {"us_call": ms * 1e3, "us_kernel": us_k, "TFLOP/s": fl / (us_k * 1e-6) / 1e12,
                             "mfma_frac": fl / (us_k * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
        breakdown["prefill_gemm"] = gemm

        # 64-layer FFN stack (configuration 4): 3.74 GB of weights, cold by construction
        del sets
        torch.cuda.empty_cache()
        stack = [weight_set(4, L) for L in range(LAYERS)]
        stk = {}
        stack_out = {}
        for m in (1, 8):
            xs = torch.from_numpy(synth.activations(4, m, D)).to(dev)
            wss = torch.zeros(P.workspace_bytes("ffn", m, D, F), dtype=torch.uint8, device=dev)
            xa = xs.clone()

            def run_stack(i):
                for L in range(LAYERS):
                    W = stack[L]
                    P.ptq1_ffn_block(xa, W[0], W[1], W[2], signs, D, F, rms_eps=1e-6, out=xa, ws=wss)

            ms_eager = timed(run_stack, 3, 1, "eager")
            # the stack replayed from one HIP graph of its 64 layers (no host
            # launch gaps between the dependent kernels), as the decode step
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_stack(0)
            torch.cuda.synchronize()
            ms = timed(lambda i: g.replay(), 5, 1, "eager")
            stk[f"M{m}"] = {"ms_per_stack": ms, "us_per_layer": ms * 1e3 / LAYERS,
                            "layers_per_s": LAYERS / (ms * 1e-3),
                            "weight_GB/s": LAYERS * LAYER_WEIGHT_BYTES / (ms * 1e-3) / 1e9,
                            "us_per_layer_eager": ms_eager * 1e3 / LAYERS,
                            "finite": bool(torch.isfinite(xa).all().item())}
            # one fresh pass of the 64 layers from the seeded input, kept for
            # the end-to-end comparison with the oracle (token 0; at M = 8 it
            # has the same input row as the M = 1 stack)
            xa.copy_(xs)
            run_stack(0)
            torch.cuda.synchronize()
            stack_out[f"M{m}"] = xa[0].cpu().numpy().copy()
            del g, wss, xa
        breakdown["ffn_stack_64"] = stk
        del stack

    if args.copy_calibration:
        log("bench: copy calibration")
        src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes COPY_CAL_BYTES
        torch.cuda.synchronize()
        del src, dst

    traffic = measured_traffic()
    cpu = None
    if not args.no_cpu:
        log("bench: oracle CPU baseline")
        cpu = cpu_baseline(torch, dev, None if args.quick else stack_out)
        if "stack_64_vs_oracle" in cpu:
            breakdown.setdefault("ffn_stack_64", {})["rel_l2_vs_oracle"] = cpu["stack_64_vs_oracle"]
        cpu["gpu_over_oracle"] = gpu_over_oracle(gbs, breakdown, cpu)
    load_end = os.getloadavg()

    line = {
        "metric": "decode matvec GB/s (27B-shaped FFN block, batch 1, cold weights)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode step: unrotate 1 row of a 248320x5120 fp32 table, then one "
                               "FFN block x[5120] -> rotate -> gate+up 5120->2x17408 (PTQ1_0) -> "
                               "SwiGLU -> rotate -> down 17408->5120 + residual, batch 1, RMS scale on, "
                               f"{WEIGHT_SETS} rotating weight sets; steps replayed from HIP graphs",
                   "d": D, "f": F, "batch": 1, "weight_sets": WEIGHT_SETS,
                   "step_bytes": STEP_BYTES, "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "hbm", "kernel": "k_matvec_lut over gate+up (17408x5120 x 2, PTQ1_0), in the step",
                     "achieved": round(lut_gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(lut_gu_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": LUT_GATE_UP_BYTES, "us_per_launch": round(us_gu, 3),
                     "launches_timed": len(d_gu), "source_sha256_16": lut_source_hash()},
        "cpu_baseline": cpu,
        "receipt": dict(rec, loadavg_end=[round(v, 2) for v in load_end], clocks_after_timed_work=clk_end),
        "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)
    return 0


def _drm_dir(props):
    """The sysfs device directory of this GPU, matched on its PCI address (None if absent)."""
    import glob

    want = None
    if props is not None and hasattr(props, "pci_bus_id"):
        want = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}."
    cards = sorted(glob.glob("/sys/class/drm/card*/device"))
    for d in cards:
        if want is None or os.path.basename(os.path.realpath(d)).startswith(want):
            if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                return d
    return None


_PROPS = None


def clocks():
    """Current GPU clock levels, read from the driver's sysfs DPM tables (the
    level marked active); read directly rather than through rocm-smi so that
    no program is started (a child started under the profiler's preload would
    replace itself with an interpreter after the GPU is initialised)."""
    d = _drm_dir(_PROPS)
    if d is None:
        return "unavailable (no pp_dpm_* files)"
    out = {}
    for name in ("sclk", "mclk", "fclk", "socclk"):
        try:
            lines = open(os.path.join(d, f"pp_dpm_{name}")).read().splitlines()
        except OSError:
            continue
        cur = [ln for ln in lines if ln.rstrip().endswith("*")]
        out[name] = cur[0].split(":", 1)[1].strip(" *") if cur else None
    return out


def receipt(torch, dev):
    """Where the numbers were taken: GPU, ROCm, clocks, host CPU and load."""
    global _PROPS
    props = _PROPS = torch.cuda.get_device_properties(dev)
    name = props.name  # the runtime's name can be generic or empty; the board's own name is preferred
    d = _drm_dir(props)
    if d is not None:
        try:
            name = open(os.path.join(d, "product_name")).read().strip() or name
        except OSError:
            pass
    r = {"gpu": name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
         "hbm_GiB": round(props.total_memory / 2 ** 30, 1), "hip_runtime": torch.version.hip,
         "torch": torch.__version__}
    try:
        r["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        r["rocm"] = None
    r["clocks_at_start"] = clocks()
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    r["host_cpu"] = model
    r["host_logical_cpus"] = os.cpu_count()
    r["host_cpus_usable"] = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    r["loadavg_start"] = [round(v, 2) for v in os.getloadavg()]
    return r


def gpu_over_oracle(step_gbs, breakdown, cpu):
    """The GPU's rate over the oracle's on each configuration both measured
    (same units: bytes, flops or layers per second)."""
    cfg = cpu.get("configs", {})
    r = {"decode_step": round(step_gbs / cpu["value"], 1)}
    if "matvec_1024_hot" in breakdown and "matvec_1024" in cfg:
        gpu = (packed(1024, 1024) + 8 * 1024) / (breakdown["matvec_1024_hot"]["us"] * 1e-6) / 1e9
        r["matvec_1024"] = round(gpu / cfg["matvec_1024"]["GB/s"], 1)
    for m in (128, 256, 512):
        g = breakdown.get("prefill_gemm", {}).get(f"M{m}")
        if g and f"gemm_M{m}" in cfg:
            r[f"gemm_M{m}"] = round(1e3 * g["TFLOP/s"] / cfg[f"gemm_M{m}"]["GFLOP/s"], 1)
    for m in (1, 8):
        g = breakdown.get("ffn_stack_64", {}).get(f"M{m}")
        if g and f"ffn_layer_M{m}" in cfg:
            r[f"ffn_layer_M{m}"] = round(g["layers_per_s"] / cfg[f"ffn_layer_M{m}"]["layers/s"], 1)
    return r


def cpu_baseline(torch, dev, stack_out=None):
    """The fp64 oracle (as it stands, never tuned for this) on this host's
    cores, timed on bounded samples of each configuration in the GPU's units:
    the decode step (the headline, GB/s), the 1024 x 1024 matvec (GB/s), the
    prefill GEMM at M = 128 / 256 / 512 on 64 sampled output columns
    (GFLOP/s of the sample, rotation included), and the 27B FFN layer at M = 1
    and M = 8 (layers/s).  With stack_out (the GPU's 64-layer outputs for
    token 0 at M = 1 and M = 8, which share their input row) the oracle also
    runs the whole 64-layer stack once and reports the end-to-end relative L2
    of each (reported, not gated).  Weights come from the seeded generator's
    device fill (bit-exact with its host version), copied to the host and
    packed by the oracle."""
    import concurrent.futures as cf

    import oracle
    import synth
    import synth.device as sdev

    pool = cf.ThreadPoolExecutor(3)

    def host_pack(seed, tr, sc, n, k, rows=None):
        t = sdev.trits(seed, tr, rows or n, k, device=dev).cpu().numpy()
        sv = sdev.scales(seed, sc, rows or n, k // 128, device=dev).cpu().numpy().view(np.uint16)
        return oracle.pack(t, sv)

    def layer_mats(seed, layer):
        ls = synth.layer_stream
        jobs = [pool.submit(host_pack, seed, ls(tr, layer), ls(sc, layer), n, k)
                for tr, sc, n, k in ((synth.S_GATE_TRITS, synth.S_GATE_SCALES, F, D),
                                     (synth.S_UP_TRITS, synth.S_UP_SCALES, F, D),
                                     (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, D, F))]
        return [j.result() for j in jobs]

    out = {"kind": "oracle", "cores": oracle.threads()}
    # ---- headline: the decode step (1 embedding row + 1 FFN block, batch 1)
    seed = 1
    mats = layer_mats(seed, 0)
    s = synth.signs(seed)
    row = synth.table_rows(2, synth.S_TABLE, np.array([7]), D)
    reps, t0 = 0, time.perf_counter()
    while True:
        e = oracle.embedding_unrotate(row, s)
        oracle.ffn_block(e, mats[0], mats[1], mats[2], s, D, F, 1e-6)
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 50:
            break
    out.update({"value": round(STEP_BYTES * reps / el / 1e9, 4), "unit": "GB/s",
                "sample": f"{reps} decode steps (1 embedding row + 1 full 5120/17408 FFN block, fp64) in "
                          f"{el:.1f} s"})
    cfg = {}
    # ---- 1024 x 1024 matvec with its rotation
    b0 = host_pack(0, synth.S_W_TRITS, synth.S_W_SCALES, 1024, 1024)
    x0, s0 = synth.activations(0, 1, 1024)[0], synth.signs(0)
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        oracle.matvec(b0, 1024, 1024, oracle.rotate(x0, s0))
        reps += 1
    el = time.perf_counter() - t0
    cfg["matvec_1024"] = {"GB/s": round((packed(1024, 1024) + 8 * 1024) * reps / el / 1e9, 4), "calls": reps}
    # ---- prefill GEMM on 64 sampled output columns (rows 0..63 of the 17408 x 5120 matrix)
    bq = host_pack(3, synth.S_W_TRITS, synth.S_W_SCALES, F, D, rows=64)
    s3 = synth.signs(1)
    for m in (128, 256, 512):
        xm = synth.activations(3, m, D)
        t0 = time.perf_counter()
        oracle.gemm(bq, 64, D, oracle.rotate(xm, s3))
        el = time.perf_counter() - t0
        cfg[f"gemm_M{m}"] = {"GFLOP/s": round(2.0 * m * 64 * D / el / 1e9, 4),
                             "sample": f"{m} x 5120 rotated, times 64 of the 17408 weight rows, {el:.2f} s"}
    # ---- FFN layer at M = 8 (one layer), and the 64-layer stack at M = 1
    s1 = synth.signs(1)
    m0 = layer_mats(4, 0)
    x8 = synth.activations(4, 8, D)
    t0 = time.perf_counter()
    oracle.ffn_block(x8, m0[0], m0[1], m0[2], s1, D, F, 1e-6)
    el = time.perf_counter() - t0
    cfg["ffn_layer_M8"] = {"layers/s": round(1.0 / el, 4), "sample": f"layer 0 at M = 8 in {el:.2f} s"}
    xs = synth.activations(4, 1, D)[0].astype(np.float64)
    layers = LAYERS if stack_out else 2
    t_comp = 0.0
    for L in range(layers):
        if L % 16 == 0:
            log(f"bench: oracle stack, layer {L} of {layers}")
        mL = m0 if L == 0 else layer_mats(4, L)
        t0 = time.perf_counter()
        xs = oracle.ffn_block(xs, mL[0], mL[1], mL[2], s1, D, F, 1e-6)[0]
        t_comp += time.perf_counter() - t0
    cfg["ffn_layer_M1"] = {"layers/s": round(layers / t_comp, 4),
                           "sample": f"{layers} layers at M = 1 in {t_comp:.2f} s of oracle time"}
    out["configs"] = cfg
    if stack_out:
        ref = np.linalg.norm(xs)
        out["stack_64_vs_oracle"] = {
            k: float(np.linalg.norm(np.asarray(v, dtype=np.float64) - xs) / ref) for k, v in stack_out.items()}
        out["stack_64_vs_oracle"]["note"] = ("relative L2 of token 0 after 64 layers against the fp64 oracle "
                                             "(M1: fixed-point lookup path; M8: bf16 MFMA path); reported, not gated")
    pool.shutdown()
    return out


if __name__ == "__main__":
    sys.exit(main())
