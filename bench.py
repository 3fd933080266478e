#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

A step is one pass of the whole path -- moe_topk_compact (the top-k softmax
gate and the route compaction, the compaction's count pass inside the gate
kernel) -> moe_grouped_ffn -> moe_combine -- over one batch of the prefill layer
(T=4096 tokens, E=128 experts all local, top-8 renormalised, hidden 2048,
expert FFN 768, bf16, seeded synthetic inputs already resident in HBM).
`value` is tokens/s of that layer.  One JSON line goes to stdout; progress
goes to stderr.  The GPU raises its clocks only under sustained load, so
untimed steps run for half a second (settle_steps in the line) before the W
warm-up steps and the K timed ones, and every timed graph of the secondaries
is replayed untimed for 0.1 s first.

Besides the contract fields the line carries:
  roofline      the grouped FFN call (GEMM1 + silu_and_mul kernel and GEMM2
                kernel): its algorithmic flops over its duration from HIP
                events on the launch stream, against the 2.5 PFLOP/s dense
                bf16 matrix-core peak (the bar this call is held to); the HBM
                rate on its minimum bytes (weights + x) and on the bytes with
                the act / y hand-over rides along, and both against the
                measured peaks; library_bmm_same_shapes_frac is the vendor
                library's batched GEMM on dense per-expert operands of the
                same shapes (no gather, no epilogue), for scale
  measured_peaks  what this GPU achieves in the same run: a 2 GiB streaming
                read, a 1 GiB copy and a bf16 MFMA loop (library probes), the
                loop with loop-invariant operands and with operands that
                change every round as real data does, each with the clock it
                ran at (data-dependent power lowers the clock)
  cpu_baseline  the fp64 CPU oracle on a bounded token sample of the same
                workload, on this host's cores
  breakdown     per-call milliseconds of the step
  secondary     gate throughput (65536 rows, E=128 and 160, bf16) in Mrows/s
                and %-of-HBM with rotating buffers larger than the 256 MB
                last-level cache; decode layer (M=2, top-6, 40 local
                experts) per route pattern with achieved weight-stream GB/s,
                the scheduler A/B against the generic control and the boundary
                fusion A/B; MXFP4 decode (T = 2, 16, 64) with the A/B of its
                two arithmetics; the padded layout; the library GEMM
                reference.  The short calls are timed from HIP-graph replays
                so that host launch overhead is not counted.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SETTLE_S = 0.5  # seconds of untimed steps before the warm-up (clock ramp)
SETTLE_REPLAY_S = 0.1  # the same before each secondary's timed graph replays
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--quick", action="store_true", help="short secondary runs")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB five times (the reference kernel "
                        "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--profile", default="", metavar="WHAT",
                   help="only run one secondary for a kernel trace and exit: 'peaks' (the read, copy and "
                        "MFMA probes), 'libgemm' (torch.bmm on the expert GEMM shapes), 'gate' (the five gate "
                        "configurations), 'decode:PATTERN' (one decode route pattern, every path) or "
                        "'mxfp4[:T<n>_<routes>]' (the MXFP4 weight-streaming cases)")
    return p.parse_args()


def bf16_dev(bits, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def i32_dev(a, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def f32_dev(a, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def settle_replays(graphs, seconds=SETTLE_REPLAY_S):
    """Untimed replays for `seconds` so the clocks are up before timing."""
    import torch

    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()


def graph_ms(fn, reps, dev):
    """Milliseconds per fn() call on the GPU, without host launch overhead:
    fn() (a fixed sequence of library calls on the current stream) is captured
    once in a HIP graph, and the graph is replayed `reps` times between two
    events.  The calls hold no allocation and no memset, so they capture."""
    import torch

    fn()  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    settle_replays([g])
    s = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return ms


def ab_graph_ms(fa, fb, reps, dev):
    """A/B timing: fa() and fb() captured in one graph each, replays
    alternated (A, B, A, B, ...), each replay between two events; returns
    the median milliseconds of each."""
    import statistics

    import torch

    graphs = []
    for f in (fa, fb):
        f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        g.replay()
        torch.cuda.synchronize()
        graphs.append(g)
    settle_replays(graphs)
    s = torch.cuda.current_stream(dev)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
          for _ in range(2)]
    for r in range(reps):
        for i, g in enumerate(graphs):
            ev[i][r][0].record(s)
            g.replay()
            ev[i][r][1].record(s)
    torch.cuda.synchronize()
    return [statistics.median(a.elapsed_time(b) for a, b in ev[i]) for i in range(2)]


# ---------------------------------------------------------------------------
# main workload: the prefill layer


def bench_prefill(args, dev):
    import torch

    import mixture_experts_routing_amd as moe
    import synth

    log("[bench] generating prefill layer inputs (T=4096, E=128, K=8, H=2048, F=768)")
    c = synth.prefill_layer(0)
    T, E, K, H, F = c.T, c.E_local, c.K, c.H, c.F
    logits, x = bf16_dev(c.logits, dev), bf16_dev(c.x, dev)
    w1, w2 = bf16_dev(c.w1, dev), bf16_dev(c.w2, dev)
    # weights stored once in the tile-packed layout (a load-time transform,
    # outside the timed region)
    w1, w2 = moe.moe_pack_ffn_weights(w1, w2)
    torch.cuda.synchronize()
    N = T * K
    # every output and workspace is allocated once, outside the timed region
    tw = torch.empty((T, K), dtype=torch.float32, device=dev)
    tid = torch.empty((T, K), dtype=torch.int32, device=dev)
    tei = torch.empty((T, K), dtype=torch.int32, device=dev)
    cmp_out = (torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev))
    cws_n = moe.route_compact_workspace_bytes(T, K, E)
    cws = torch.empty(max(cws_n, 16), dtype=torch.uint8, device=dev)
    fws = torch.empty(moe.grouped_ffn_workspace_bytes(T, K, H, F, E, moe.MOE_BF16_TILED), dtype=torch.uint8,
                      device=dev)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        # gate + route compaction in one call (the compaction's count pass
        # runs in the gate kernel), the grouped FFN, the combine
        if ev:
            ev[0].record(stream)
        _, (counts, offsets, s2r, r2s) = moe.moe_topk_compact(logits, K, True, "softmax", None, E,
                                                               gate_out=(tw, tid, tei), route_out=cmp_out,
                                                               workspace=cws, stream=stream)
        if ev:
            ev[1].record(stream)
        moe.moe_grouped_ffn(x, K, w1, w2, counts, offsets, r2s, y=y, workspace=fws, stream=stream, tiled=True)
        if ev:
            ev[2].record(stream)
        moe.moe_combine(y, tw, s2r, out=out, stream=stream)
        if ev:
            ev[3].record(stream)

    # The GPU raises its clocks only under sustained load (measured: the FFN
    # takes ~16% longer in the first ~0.2 s of back-to-back steps), so untimed
    # steps run for SETTLE_S seconds first -- reported as settle_steps --
    # before the W warm-up steps and the K timed ones.
    settle = 0
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(32):
            step()
        torch.cuda.synchronize()
        settle += 32
    log(f"[bench] settle {settle} steps, warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["gate_compact", "grouped_ffn", "combine"]
    per = {n: 0.0 for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: v / args.steps for n, v in per.items()}
    ms_per_step = wall * 1000.0 / args.steps
    # algorithmic work of one moe_grouped_ffn call (all routes local: R = T*K)
    flops = 2.0 * N * (2 * F * H + H * F)
    weight_bytes = E * (2 * F * H + H * F) * 2       # every expert's W1 and W2 once
    row_bytes = N * (2 * F * 2 + H * 2)              # act written + read, y written (bf16)
    x_bytes = T * H * 2                              # each token's x once
    alg_bytes = weight_bytes + row_bytes + x_bytes
    min_bytes = weight_bytes + x_bytes               # what must cross HBM at least once
    ffn_s = per["grouped_ffn"] / 1000.0
    tflops = flops / ffn_s / 1e12
    # The bar for this call is stated against the bf16 matrix-core peak, so
    # the roofline is the MFMA one; the HBM view rides along, on the minimum
    # bytes (every expert's weights and each token's x once) and on the
    # bytes including the act and y rows the two kernels hand over.
    roofline = {
        "bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic_for("grouped_ffn_prefill"),
        "kernel": "moe_grouped_ffn (ffn_tiled_kernel: GEMM1 + silu_and_mul, then GEMM2)",
        "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(per["grouped_ffn"], 4),
        "hbm": {"min_bytes_per_launch": min_bytes, "min_bytes_gbs": round(min_bytes / ffn_s / 1e9, 1),
                "min_bytes_frac": round(min_bytes / ffn_s / 1e9 / HBM_PEAK_GBS, 4),
                "with_act_y_bytes_per_launch": alg_bytes,
                "with_act_y_gbs": round(alg_bytes / ffn_s / 1e9, 1),
                "with_act_y_frac": round(alg_bytes / ffn_s / 1e9 / HBM_PEAK_GBS, 4)},
    }
    log(f"[bench] prefill layer: {ms_per_step:.3f} ms/step, {T / (ms_per_step / 1e3):.0f} tokens/s; "
        + ", ".join(f"{n} {v:.3f} ms" for n, v in per.items()))
    # the remap boundary at prefill: gate then compaction as two calls vs the
    # one call with the count pass fused into the gate (alternated replays)
    # (no stream argument: the calls go to the current stream, which is the
    # capture stream while a graph is recorded)
    def separate():
        moe.moe_topk_softmax(logits, K, True, tw, tid, tei)
        moe.moe_route_compact(tid, None, E, out=cmp_out, workspace=cws)

    def fused():
        moe.moe_topk_compact(logits, K, True, "softmax", None, E, gate_out=(tw, tid, tei), route_out=cmp_out,
                             workspace=cws)

    t_sep, t_fus = ab_graph_ms(separate, fused, 400, dev)
    gate_fusion = {"separate_ms": round(t_sep, 5), "fused_ms": round(t_fus, 5)}
    log(f"[bench] prefill gate + compaction: separate {t_sep * 1e3:.1f} us, fused {t_fus * 1e3:.1f} us")
    return c, ms_per_step, per, roofline, settle, gate_fusion


def traffic_parts_for(name):
    """(read bytes, written bytes) per launch from the same counter runs as
    traffic_for, or None under the same conditions."""
    if traffic_for(name) is None:
        return None
    d = json.load(open(os.path.join(ROOT, "profiles", f"traffic_{name}.json")))
    return (d["fetch_kib_per_launch"] * 1024 * d["fetch_scale"], d["write_kib_per_launch"] * 1024 * d["write_scale"])


def traffic_for(name):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration), if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        h = hashlib.sha256()
        for f in d["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if d.get("source_sha256") != h.hexdigest():
            return None
        return d.get("bytes_per_launch")
    except Exception:
        return None


# ---------------------------------------------------------------------------
# context: the vendor GEMM library on the prefill FFN's expert GEMMs


def library_gemm_reference(dev, reps=30):
    """torch.bmm (hipBLASLt / rocBLAS) on dense per-expert GEMMs of the
    prefill workload's shapes: 128 experts x 256 rows (the mean), H=2048,
    F=768, bf16 -- without the row gather, the silu_and_mul epilogue or the
    ragged row counts the library's own FFN handles.  A reference point for
    the FFN's matrix-core fraction, not a step of the layer."""
    import statistics

    import torch

    E, M, H, F = 128, 256, 2048, 768
    out = {}
    g = torch.Generator(device=dev).manual_seed(0)
    for name, (k, n) in {"gemm1": (H, 2 * F), "gemm2": (F, H)}.items():
        a = torch.randn((E, M, k), device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn((E, k, n), device=dev, dtype=torch.bfloat16, generator=g).contiguous()
        for _ in range(10):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        t_end = time.perf_counter() + SETTLE_REPLAY_S
        while time.perf_counter() < t_end:
            torch.bmm(a, b)
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.bmm(a, b)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = statistics.median(x.elapsed_time(y) for x, y in evs)
        flops = 2.0 * E * M * k * n
        out[name] = {"shape": [E, M, k, n], "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                     "mfma_frac": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
    tot = out["gemm1"]["ms"] + out["gemm2"]["ms"]
    fl = 2.0 * E * M * (H * 2 * F + F * H)
    out["both"] = {"ms": round(tot, 4), "mfma_frac": round(fl / tot / 1e9 / BF16_PEAK_TFLOPS, 4)}
    log("[bench] library bmm at the expert GEMM shapes: " + json.dumps(out))
    return out


# ---------------------------------------------------------------------------
# secondary: gate throughput with rotating buffers


def bench_gate(dev, E, reps, scoring="softmax"):
    import torch

    import mixture_experts_routing_amd as moe
    import synth

    T, K = 65536, 8
    nbuf = 16  # 16 x T*E*2 bytes > 256 MB last-level cache
    base = synth.gate_case(E, T=T, K=K, seed=0).logits
    bufs = []
    for i in range(nbuf):
        lb = bf16_dev(base, dev).roll(i, dims=0).contiguous()
        bufs.append((lb, torch.empty((T, K), dtype=torch.float32, device=dev),
                     torch.empty((T, K), dtype=torch.int32, device=dev), torch.empty((T, K), dtype=torch.int32, device=dev)))

    fn = moe.moe_topk_softmax if scoring == "softmax" else moe.moe_topk_sigmoid

    def calls():
        for b in bufs:
            fn(b[0], K, False, b[1], b[2], b[3])

    ms = graph_ms(calls, max(1, reps // nbuf), dev) / nbuf
    nbytes = T * E * 2 + T * K * 12
    gbs = nbytes / (ms / 1e3) / 1e9
    res = {"scoring": scoring, "E": E, "T": T, "K": K, "ms": round(ms, 5), "mrows_per_s": round(T / (ms / 1e3) / 1e6, 1),
           "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes}
    if scoring == "softmax":
        # the same loads and stores without the selection: this access
        # pattern's ceiling, timed the same way
        def loads_only():
            for b in bufs:
                moe.moe_probe_gate_loads(b[0], K, b[1], b[2], b[3])

        ms0 = graph_ms(loads_only, max(1, reps // nbuf), dev) / nbuf
        res["load_only_ms"] = round(ms0, 5)
        res["load_only_hbm_frac"] = round(nbytes / (ms0 / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
    return res


def measured_peaks(dev):
    """What this GPU achieves, next to the spec peaks: a streaming read of
    2 GiB and a 1 GiB -> 1 GiB copy (both larger than the 256 MB last-level
    cache; HIP events around each call, median of 10), and a bf16 MFMA loop
    (4 independent 32x32x16 MFMAs per round on register operands, 8192 waves;
    median of 10 calls of ~4 ms) twice: with loop-invariant operands, and with
    operands that change every round as real data does (half their bits
    flip), which draws more power, so the chip runs it at a lower clock.  The
    loop's own shader-clock and reference-clock counters give that clock."""
    import statistics

    import torch

    import mixture_experts_routing_amd as moe

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream(dev)
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    rd = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    rd.fill_(1)
    out = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    t_read = timed(lambda: moe.moe_probe_read(rd, out))
    del rd
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: moe.moe_probe_copy(src, dst))
    del src, dst
    blocks, iters = 2048, 8000
    mo = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 4 * 2, dtype=torch.int64, device=dev)
    flops = blocks * 4 * iters * 4 * 32768
    mfma = {}
    for name, toggle in (("constant", False), ("toggling", True)):
        t = timed(lambda: moe.moe_probe_mfma_clock(iters, blocks, toggle, mo, clk))
        c = clk.view(-1, 2).double().sum(0).tolist()
        mfma[name] = {"tflops": round(flops / (t / 1e3) / 1e12, 1), "clock_ghz": round(c[0] / c[1] * 0.1, 3)}
    return {"read_gbs": round((2 << 30) / (t_read / 1e3) / 1e9, 1),
            "copy_gbs": round(2 * (1 << 30) / (t_copy / 1e3) / 1e9, 1),
            "mfma_bf16_tflops": mfma["constant"]["tflops"],
            "mfma_bf16_tflops_toggling": mfma["toggling"]["tflops"],
            "mfma_clock_ghz": {k: v["clock_ghz"] for k, v in mfma.items()},
            "spec": {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": BF16_PEAK_TFLOPS},
            "probes": "moe_probe_read (2 GiB), moe_probe_copy (1 GiB -> 1 GiB, bytes read + written), "
                      "moe_probe_mfma_clock (2048 x 256 threads, 8000 rounds of 4 MFMAs; loop-invariant and "
                      "toggling operands; clock = s_memtime cycles / s_memrealtime ticks x 100 MHz)"}


# ---------------------------------------------------------------------------
# secondary: decode layer per route pattern


def bench_decode(dev, reps, only=None):
    import numpy as np
    import torch

    import mixture_experts_routing_amd as moe
    import synth

    log("[bench] decode: generating 40 bf16 experts (2.0 GB)")
    w1h, w2h = synth.decode_weights(0)
    w1, w2 = bf16_dev(w1h, dev), bf16_dev(w2h, dev)
    del w1h, w2h
    T, K, Eg, El, H, F = 2, 6, 256, 40, 4096, 2048
    emap = synth.contiguous_expert_map(Eg, El)
    emap_d = i32_dev(emap, dev)
    inv = np.flatnonzero(emap >= 0)  # local -> global under the contiguous map
    res = {}
    nvar = 8  # rotated copies of each pattern: consecutive calls touch different experts
    for pat in synth.decode_patterns():
        if only is not None and pat != only:
            continue
        base = synth.decode_case(pat, "contiguous", seed=0, with_weights=False)
        x = bf16_dev(base.x, dev)
        tw = f32_dev(base.topk_weights, dev)
        variants = []
        for v in range(nvar):
            rows = [[None if l is None else (l + 5 * v) % El for l in r] for r in synth.DECODE_PATTERNS[pat]]
            ids = np.array([[int(inv[l]) if l is not None else int(base.topk_ids[t, k])
                             for k, l in enumerate(r)] for t, r in enumerate(rows)], dtype=np.int32)
            variants.append(i32_dev(ids, dev))
        # one set of compaction outputs per variant, so each phase can be
        # captured and timed on its own
        outs = [(torch.empty(El, dtype=torch.int32, device=dev), torch.empty(El + 1, dtype=torch.int32, device=dev),
                 torch.empty(T * K, dtype=torch.int32, device=dev), torch.empty(T * K, dtype=torch.int32, device=dev))
                for _ in range(nvar)]
        fws = torch.empty(moe.grouped_ffn_workspace_bytes(T, K, H, F, El, moe.MOE_BF16), dtype=torch.uint8,
                          device=dev)
        y = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

        def compact(v):
            moe.moe_route_compact(variants[v], emap_d, El, E_global=Eg, out=outs[v])

        def ffn(v):
            counts, offsets, _, r2s = outs[v]
            moe.moe_grouped_ffn(x, K, w1, w2, counts, offsets, r2s, y=y, workspace=fws)

        def combine(v):
            moe.moe_combine(y, tw, outs[v][2], out=out)

        def each(*fns):
            def run():
                for v in range(nvar):
                    for f in fns:
                        f(v)
            return run

        t_cmp = graph_ms(each(compact), reps, dev) / nvar
        t_ffn = graph_ms(each(ffn), reps, dev) / nvar
        t_cmb = graph_ms(each(combine), reps, dev) / nvar
        t_layer = graph_ms(each(compact, ffn, combine), reps, dev) / nvar
        # A/B against the generic persistent scheduler (atomic work counter
        # over every local expert, 64-column N tiles), alternated replays
        cws = torch.empty(moe.grouped_ffn_control_workspace_bytes(T, K, H, F, El, moe.MOE_BF16), dtype=torch.uint8,
                          device=dev)

        def ffn_control(v):
            counts, offsets, _, r2s = outs[v]
            moe.moe_grouped_ffn_control(x, K, w1, w2, counts, offsets, r2s, y=y, workspace=cws)

        t_a, t_b = ab_graph_ms(each(compact, ffn, combine), each(compact, ffn_control, combine), reps, dev)
        t_a, t_b = t_a / nvar, t_b / nvar
        t_fa, t_fb = ab_graph_ms(each(ffn), each(ffn_control), reps, dev)
        t_fa, t_fb = t_fa / nvar, t_fb / nvar
        # boundary fusion: compaction and combine inside the two FFN kernels,
        # A/B against the three separate calls (alternated replays)
        xws = torch.empty(moe.fused_experts_workspace_bytes(T, K, H, F, El, moe.MOE_BF16), dtype=torch.uint8,
                          device=dev)

        def fused(v):
            moe.moe_fused_experts(x, variants[v], tw, w1, w2, emap_d, Eg, out=out, routes=outs[v], workspace=xws)

        t_sep, t_fus = ab_graph_ms(each(compact, ffn, combine), each(fused), reps, dev)
        t_sep, t_fus = t_sep / nvar, t_fus / nvar
        n_exp = len({l for r in synth.DECODE_PATTERNS[pat] for l in r if l is not None})
        wbytes = n_exp * (2 * F * H + H * F) * 2
        d = {"layer_ms": round(t_layer, 4), "compact_ms": round(t_cmp, 4), "ffn_ms": round(t_ffn, 4),
             "combine_ms": round(t_cmb, 4), "tokens_per_s": round(T / (t_layer / 1e3), 1),
             "local_experts": n_exp, "weight_bytes": wbytes,
             "ab_layer_ms": {"compact": round(t_a, 4), "generic_control": round(t_b, 4)},
             "projected_saved_ms_43_layers": round((t_b - t_a) * 43, 4),
             "boundary_fusion": {"upper_bound_saved_ms_43_layers": round((t_layer - t_ffn) * 43, 4),
                                 "ab_layer_ms": {"separate": round(t_sep, 4), "fused": round(t_fus, 4)},
                                 "saved_ms_43_layers": round((t_sep - t_fus) * 43, 4)}}
        d["ab_ffn_ms"] = {"compact": round(t_fa, 4), "generic_control": round(t_fb, 4)}
        if wbytes:
            gbs = wbytes / (t_ffn / 1e3) / 1e9
            d.update({"ffn_weight_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "ab_ffn_hbm_frac": {"compact": round(wbytes / (t_fa / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                          "generic_control": round(wbytes / (t_fb / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}})
        res[pat] = d
        log(f"[bench] decode {pat}: " + json.dumps(d))
    if only is not None:
        return {"patterns": res}
    nonempty = [p for p in res if res[p]["local_experts"] > 0]
    worst = min(nonempty, key=lambda p: res[p]["hbm_frac"])
    saved = {p: res[p]["projected_saved_ms_43_layers"] for p in res}
    fsaved = {p: res[p]["boundary_fusion"]["saved_ms_43_layers"] for p in res}
    return {"patterns": res, "min_hbm_frac_pattern": worst, "min_hbm_frac": res[worst]["hbm_frac"],
            "min_tokens_per_s": min(res[p]["tokens_per_s"] for p in res),
            "scheduler_ab": {"min_projected_saved_ms_43_layers": min(saved.values()),
                             "min_pattern": min(saved, key=saved.get)},
            "boundary_fusion": {"min_saved_ms_43_layers": min(fsaved.values()), "min_pattern": min(fsaved, key=fsaved.get),
                                "min_upper_bound_ms_43_layers": min(
                                    res[p]["boundary_fusion"]["upper_bound_saved_ms_43_layers"] for p in res)}}


# ---------------------------------------------------------------------------
# secondary: MXFP4 experts (weight streaming at T = 2, 16, 64)


def bench_mxfp4(dev, reps, only=None):
    import numpy as np
    import torch

    import mixture_experts_routing_amd as moe
    import synth

    T_LIST, K, Eg, El, H, F = (2, 16, 64), 8, 256, 32, 4096, 2048
    log("[bench] mxfp4: generating 32 experts (e2m1 codes + e8m0 scales, 0.43 GB)")
    w1h, w1sh, w2h, w2sh = synth.mxfp4_weights(0, El, H, F)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    w1, w1s, w2, w2s = u8(w1h), u8(w1sh), u8(w2h), u8(w2sh)
    del w1h, w1sh, w2h, w2sh
    # bytes one expert's weights occupy: codes (2 per byte) + one scale byte per 32
    per_expert = (2 * F * H + H * F) // 2 + (2 * F * H + H * F) // 32
    emap = synth.contiguous_expert_map(Eg, El)
    emap_d = i32_dev(emap, dev)
    inv = np.flatnonzero(emap >= 0)
    nvar = 8  # rotated copies of the routes: consecutive calls touch different experts
    res = {}
    for routes in ("uniform", "all_local"):
        for T in T_LIST:
            name = f"T{T}_{routes}"
            if only is not None and name != only:
                continue
            base = synth.mxfp4_case(T, routes, seed=0, with_weights=False)
            x = bf16_dev(base.x, dev)
            tw = f32_dev(base.topk_weights, dev)
            loc = emap[base.topk_ids]
            variants, n_exp = [], []
            for v in range(nvar):
                ids = np.where(loc >= 0, inv[(np.maximum(loc, 0) + 5 * v) % El], base.topk_ids).astype(np.int32)
                variants.append(i32_dev(ids, dev))
                n_exp.append(len(set(((loc[loc >= 0] + 5 * v) % El).tolist())))
            N = T * K
            outs = [(torch.empty(El, dtype=torch.int32, device=dev), torch.empty(El + 1, dtype=torch.int32, device=dev),
                     torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev))
                    for _ in range(nvar)]
            fws = torch.empty(max(moe.grouped_ffn_workspace_bytes(T, K, H, F, El, moe.MOE_MXFP4), 16),
                              dtype=torch.uint8, device=dev)
            y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

            def compact(v):
                moe.moe_route_compact(variants[v], emap_d, El, E_global=Eg, out=outs[v])

            def ffn(v):
                counts, offsets, _, r2s = outs[v]
                moe.moe_grouped_ffn(x, K, w1, w2, counts, offsets, r2s, w1_scale=w1s, w2_scale=w2s, y=y,
                                    workspace=fws)

            def combine(v):
                moe.moe_combine(y, tw, outs[v][2], out=out)

            def each(*fns):
                def run():
                    for v in range(nvar):
                        for f in fns:
                            f(v)
                return run

            # the routes of every variant first (the FFN timing below reads
            # them), checked on the host before any FFN launch
            each(compact)()
            torch.cuda.synchronize(dev)
            for v in range(nvar):
                c_, o_, _, r_ = (t.cpu().numpy() for t in outs[v])
                R = int(o_[El])
                assert R == int((loc >= 0).sum()) == int(c_.sum()) and np.all(np.diff(o_) == c_) and o_[0] == 0
                assert np.all((r_[:R] >= 0) & (r_[:R] < N))
            t_ffn = graph_ms(each(ffn), reps, dev) / nvar
            t_layer = graph_ms(each(compact, ffn, combine), reps, dev) / nvar
            wbytes = float(np.mean(n_exp)) * per_expert
            # A/B of the two MXFP4 arithmetics (bf16 widening vs the block-scaled
            # f8f6f4 matrix cores), alternated replays of the FFN; the mode is read
            # when a call is captured
            prev = moe.moe_get_mxfp4_mma()
            ab = ab_graph_ms(lambda: (moe.moe_set_mxfp4_mma(moe.MOE_MXFP4_MMA_BF16), each(ffn)())[1],
                             lambda: (moe.moe_set_mxfp4_mma(moe.MOE_MXFP4_MMA_F8F6F4), each(ffn)())[1], reps, dev)
            moe.moe_set_mxfp4_mma(prev)
            mma_ab = {"bf16_widen_ffn_ms": round(ab[0] / nvar, 4), "f8f6f4_ffn_ms": round(ab[1] / nvar, 4)}
            d = {"T": T, "routes": routes, "local_slots": int((loc >= 0).sum()),
                 "local_experts_mean": round(float(np.mean(n_exp)), 2), "layer_ms": round(t_layer, 4),
                 "ffn_ms": round(t_ffn, 4), "tokens_per_s": round(T / (t_layer / 1e3), 1),
                 "weight_bytes_mean": int(wbytes), "mxfp4_mma_ab": mma_ab}
            if N <= 64:  # the boundary-fused layer (compaction in GEMM1, combine in GEMM2)
                xws = torch.empty(max(moe.fused_experts_workspace_bytes(T, K, H, F, El, moe.MOE_MXFP4), 16),
                                  dtype=torch.uint8, device=dev)

                def fused(v):
                    moe.moe_fused_experts(x, variants[v], tw, w1, w2, emap_d, Eg, w1_scale=w1s, w2_scale=w2s,
                                          out=out, routes=outs[v], workspace=xws)

                d["fused_layer_ms"] = round(graph_ms(each(fused), reps, dev) / nvar, 4)
            if wbytes:
                gbs = wbytes / (t_ffn / 1e3) / 1e9
                d.update({"ffn_weight_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
            res[name] = d
            log(f"[bench] mxfp4 {name}: " + json.dumps(d))
    return res


# ---------------------------------------------------------------------------
# secondary: block-aligned layout (moe_route_align)


def bench_align(dev, reps):
    import numpy as np
    import torch

    import mixture_experts_routing_amd as moe
    import synth

    out = []
    for name, T, K, Eg, El, bs in (("prefill", 4096, 8, 128, 128, 128), ("decode", 2, 6, 256, 40, 16)):
        rng = np.random.default_rng(0)
        emap = None if El == Eg else i32_dev(synth.contiguous_expert_map(Eg, El), dev)
        ids = [i32_dev(rng.integers(0, Eg, size=(T, K)), dev) for _ in range(8)]
        N = T * K
        res = (torch.empty(El + 1, dtype=torch.int32, device=dev),
               torch.empty(N + El * (bs - 1), dtype=torch.int32, device=dev),
               torch.empty(-(-N // bs) + El, dtype=torch.int32, device=dev),
               torch.empty(N, dtype=torch.int32, device=dev))
        ws = torch.empty(moe.route_align_workspace_bytes(T, K, El), dtype=torch.uint8, device=dev)

        def calls():
            for i in ids:
                moe.moe_route_align(i, emap, El, bs, E_global=Eg, out=res, workspace=ws)

        ms = graph_ms(calls, reps, dev) / len(ids)
        out.append({"workload": name, "T": T, "K": K, "E_local": El, "block": bs, "ms": round(ms, 5)})
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the prefill workload


def cpu_baseline(c, n_tokens, min_seconds=10.0, max_reps=20):
    """The oracle, as it stands, on the first n_tokens tokens of the workload,
    repeated until at least min_seconds of CPU work have run."""
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    sub = synth.MoECase(**{**c.__dict__})
    sub.T = n_tokens
    sub.logits = c.logits[:n_tokens]
    sub.x = c.x[:n_tokens]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_layer(sub)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(reps * n_tokens / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tokens} of the {c.T} prefill tokens (gate, compaction, fp64 FFN of all "
                      f"{n_tokens * c.K} routes over the {c.E_local} experts, combine), run {reps} times; "
                      f"{dt:.1f} s wall",
            "host_cores_available": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 (the path would shard "
                                   "by experts across GPUs; that is not implemented)"}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return
    if args.profile:
        if args.profile == "peaks":
            res = measured_peaks(dev)
        elif args.profile == "libgemm":
            res = library_gemm_reference(dev)
        elif args.profile == "gate":
            res = [bench_gate(dev, E, 64) for E in (128, 160)]
            res += [bench_gate(dev, E, 64, "sigmoid") for E in (128, 160, 256)]
        elif args.profile.startswith("decode:"):
            res = bench_decode(dev, 5, only=args.profile.split(":", 1)[1])
        elif args.profile == "mxfp4" or args.profile.startswith("mxfp4:"):
            res = bench_mxfp4(dev, 5, only=args.profile.split(":", 1)[1] if ":" in args.profile else None)
        else:
            raise SystemExit(f"unknown --profile {args.profile!r}")
        print(json.dumps({"profile": args.profile, "result": res}), flush=True)
        return
    c, ms, per, roofline, settle, gate_fusion = bench_prefill(args, dev)
    secondary = {"prefill_gate_compaction": gate_fusion}
    peaks = measured_peaks(dev)
    log(f"[bench] measured peaks: read {peaks['read_gbs']} GB/s, copy {peaks['copy_gbs']} GB/s, "
        f"bf16 MFMA loop {peaks['mfma_bf16_tflops']} TFLOP/s (constant operands, "
        f"{peaks['mfma_clock_ghz']['constant']} GHz), {peaks['mfma_bf16_tflops_toggling']} TFLOP/s (toggling "
        f"operands, {peaks['mfma_clock_ghz']['toggling']} GHz)")
    roofline["measured_peak"] = peaks["mfma_bf16_tflops"]
    roofline["frac_of_measured_peak"] = round(roofline["achieved"] / peaks["mfma_bf16_tflops"], 4)
    roofline["measured_peak_toggling"] = peaks["mfma_bf16_tflops_toggling"]
    roofline["frac_of_measured_peak_toggling"] = round(roofline["achieved"] / peaks["mfma_bf16_tflops_toggling"], 4)
    roofline["hbm"]["min_bytes_frac_of_measured_read"] = round(roofline["hbm"]["min_bytes_gbs"] / peaks["read_gbs"], 4)
    if roofline["traffic"]:
        # the bytes the counters saw (reads and writes) at the call's duration,
        # against the measured streaming-read and copy rates of the same run
        tg = roofline["traffic"] / (roofline["avg_launch_ms"] / 1e3) / 1e9
        roofline["hbm"]["traffic_gbs"] = round(tg, 1)
        roofline["hbm"]["traffic_frac_of_measured_read"] = round(tg / peaks["read_gbs"], 4)
        roofline["hbm"]["traffic_frac_of_measured_copy"] = round(tg / peaks["copy_gbs"], 4)
        parts = traffic_parts_for("grouped_ffn_prefill")
        if parts:
            # reads at the streaming-read rate, writes at the rate the copy
            # (half reads, half writes) leaves for them: the time this traffic
            # needs at the rates this GPU reaches
            rd, wr = parts
            read_s = 1.0 / (peaks["read_gbs"] * 1e9)
            write_s = max(2.0 / (peaks["copy_gbs"] * 1e9) - read_s, read_s)
            floor_ms = (rd * read_s + wr * write_s) * 1e3
            roofline["hbm"]["traffic_floor_ms"] = round(floor_ms, 4)
            roofline["hbm"]["traffic_floor_frac"] = round(floor_ms / roofline["avg_launch_ms"], 4)
    if not args.no_secondary:
        # context for the FFN's matrix-core fraction: the vendor library on
        # dense per-expert GEMMs of the same shapes (no gather, no epilogue)
        secondary["library_gemm_reference"] = library_gemm_reference(dev)
        roofline["library_bmm_same_shapes_frac"] = secondary["library_gemm_reference"]["both"]["mfma_frac"]
        reps = 50 if args.quick else 400
        secondary["gate"] = [bench_gate(dev, E, reps) for E in (128, 160)]
        secondary["gate"] += [bench_gate(dev, E, reps, "sigmoid") for E in (128, 160, 256)]
        for g in secondary["gate"]:
            g["hbm_frac_of_measured_read"] = round(g["gbs"] / peaks["read_gbs"], 4)
            log(f"[bench] gate {g['scoring']} E={g['E']}: {g['ms'] * 1e3:.2f} us, {g['mrows_per_s']} Mrows/s, "
                f"{g['gbs']} GB/s ({100 * g['hbm_frac']:.1f}% of HBM)"
                + (f"; loads only {g['load_only_ms'] * 1e3:.2f} us ({100 * g['load_only_hbm_frac']:.1f}%)"
                   if "load_only_ms" in g else ""))
        secondary["decode"] = bench_decode(dev, 5 if args.quick else 20)
        secondary["mxfp4"] = bench_mxfp4(dev, 5 if args.quick else 20)
        secondary["route_align"] = bench_align(dev, 5 if args.quick else 20)
        for a in secondary["route_align"]:
            log(f"[bench] route_align {a['workload']} (T={a['T']}, K={a['K']}, E_local={a['E_local']}, "
                f"block {a['block']}): {a['ms'] * 1e3:.2f} us")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(c, 1024 if args.quick else c.T, min_seconds=2.0 if args.quick else 10.0)
        log(f"[bench] cpu: {cpu}")
    line = {
        "metric": "MoE-layer tokens/s + gate Mrows/s; % of HBM BW / MFMA peak, 1 MI355X",
        "value": round(c.T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": settle, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_moe_layer", "tokens": c.T, "experts": c.E_local, "top_k": c.K,
                   "renormalize": True, "hidden": c.H, "expert_ffn": c.F, "weights": "bf16 (tile-packed layout)",
                   "parallelism": "single-gpu"},
        "roofline": roofline, "cpu_baseline": cpu, "measured_peaks": peaks,
        "breakdown_ms": {k: round(v, 4) for k, v in per.items()},
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
