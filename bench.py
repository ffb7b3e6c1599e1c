"""Benchmark of the BitNet b1.58 BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 80]
                    [--no-cpu-baseline] [--no-prefill] [--no-m16]

Headline (``value``): decode throughput of the 70B-shaped sweep at M = 1
token -- 80 layers x 7 BitLinear projections, 17.1 GB of packed ternary
weights resident in HBM -- in GB/s of algorithmic bytes (packed weights +
float32 activations in + float32 outputs out + per-token scales) per second.
One step = one grouped forward: quantize all 560 activation rows, then one
contraction kernel over every projection with the dequant fused.

Also reported:
  roofline      the contraction kernel alone (its own launch, the
                quantize stage precomputed), timed with HIP events on the
                stream it runs on, against 8 TB/s HBM3E.
  prefill       the 3B-shaped prefill GEMMs (M = 2048: 3200->8640 and
                8640->3200) on pre-quantized activations with the row sums
                the quantizer writes (as the fused forward runs them), int8
                TOP/s against the 5.0 POP/s dense int8 MFMA peak; also the
                same contraction summing the rows itself and the quantizer.
  decode_m16    the same sweep at M = 16 tokens.
  cpu_baseline  the CPU oracle (plain C, all host threads) on a bounded
                sample of the same sweep (the first layers at M = 1).
  ceilings      what this part sustains, measured by the library's probes:
                a 4 GiB streaming read and an int8 MFMA loop on the prefill
                operands; roofline and prefill lines also give their
                fraction of these (frac_of_measured).
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

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
METRIC = "BitLinear decode GEMV GB/s (% HBM peak) at M=1; prefill int8 TOPS (% MFMA)"


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def system_info(torch) -> dict:
    """The part, its runtime and the host CPU the numbers were taken on."""
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", ""),
            "cus": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "cpu": cpu, "host_threads": len(os.sched_getaffinity(0))}


def time_events(torch, fn, reps: int) -> float:
    """Mean milliseconds per call of fn() over reps calls, HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def time_graph(torch, call, count: int, replays: int = 10) -> float:
    """Mean milliseconds per call of call(i, stream) for i = 0 .. count - 1,
    captured once into a HIP graph (on a side stream of default priority)
    and replayed: the device time of the sequence without the host's
    per-call issue cost (Python and ctypes take several microseconds per
    call, more than a single-layer decode kernel runs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(count):          # eager pass: first-touch work outside the capture
            call(i, side.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(count):
            call(i, side.cuda_stream)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(cur)
    for _ in range(replays):
        graph.replay()
    end.record(cur)
    end.synchronize()
    ms = start.elapsed_time(end) / (replays * count)
    del graph
    return ms


def contraction_only_plan(sw, M, fmt="2bit"):
    """A plan over the same problems whose activations are already quantized
    (x = NULL): forward then launches the contraction kernel alone."""
    L, torch = sw.L, sw.torch
    specs = []
    for layer in range(sw.layers):
        for p in sw.projs:
            key = (layer, p.name, M)
            specs.append(dict(x=None, xq=sw.xq[key], eta=sw.eta[key],
                              packed=sw.packed[(fmt, layer, p.name)], y=sw.y[key],
                              gamma=sw.gamma[(layer, p.name)], N=p.N, K=p.K,
                              format=L.BITLINEAR_FORMAT_2BIT if fmt == "2bit" else L.BITLINEAR_FORMAT_BASE3))
    probs = L.make_problems(specs)
    tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
    table = torch.empty(tb, dtype=torch.uint8, device="cuda")
    plan = L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb)
    return plan, table


def bench_decode_base3(torch, sw, steps: int):
    """The 70B-shaped decode step (one grouped forward over all 560
    projections) with the weights in the base-3 layout (13.7 GB, 1.6 bits per
    weight) next to the same step in the 2-bit layout (17.1 GB), at each
    token count both are planned for; the contraction kernel alone too."""
    out = []
    for M in sw.Ms["base3"]:
        row = {"M": M}
        for fmt in ("2bit", "base3"):
            if (fmt, M) not in sw.plans:
                continue
            for _ in range(2):
                sw.step(M, fmt=fmt)
            ms = time_events(torch, lambda: sw.step(M, fmt=fmt), max(5, steps // 2))
            plan_c, _table = contraction_only_plan(sw, M, fmt)
            sw.L.bitlinear_forward_grouped(plan_c)
            kern = time_events(torch, lambda: sw.L.bitlinear_forward_grouped(plan_c), max(5, steps // 2))
            del plan_c, _table
            gbs = sw.algorithmic_bytes(M, fmt) / (ms * 1e-3) / 1e9
            kgbs = sw.contraction_bytes(M, fmt) / (kern * 1e-3) / 1e9
            row[fmt] = {"ms_per_step": round(ms, 4), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "contraction_ms": round(kern, 4), "contraction_gbs": round(kgbs, 1),
                        "contraction_frac": round(kgbs / HBM_PEAK_GBS, 4),
                        "weight_bytes": sw.weight_bytes(fmt)}
        if "2bit" in row and "base3" in row:
            row["base3_over_2bit"] = round(row["base3"]["ms_per_step"] / row["2bit"]["ms_per_step"], 3)
        out.append(row)
    return out


def bench_prefill(torch, L, S, reps: int):
    import numpy as np
    out = []
    for which in (0, 1):
        K, N = S.C3_SHAPES[which]
        W, x = S.c3_inputs(which)
        M = x.shape[0]
        Wd = torch.from_numpy(W).cuda()
        xd = torch.from_numpy(x).cuda()
        packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        ws_bytes = L.bitlinear_workspace_bytes(M, N, K)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        import ctypes
        g = ctypes.c_float()
        L.bitlinear_pack_weights(Wd, N, K, packed, None, g, ws, ws_bytes)
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        eta = torch.empty(M, dtype=torch.float32, device="cuda")
        xsum = torch.empty(M, dtype=torch.int32, device="cuda")
        L.bitlinear_quantize_act(xd, M, K, xq, eta, xsum)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        # Device addresses and the stream resolved once, outside the timed
        # loop, so that host-side argument handling does not open gaps
        # between launches of a ~50 us kernel.
        st = torch.cuda.current_stream().cuda_stream
        a = [t.data_ptr() for t in (xq, eta, packed, y, ws, xd, xsum)]
        # The contraction as the fused forward runs it: row sums from the
        # quantizer (timed with them below).
        fwd = lambda: L.bitlinear_forward_xsum(a[0], a[1], a[6], a[2], g.value, M, N, K, a[3], None, a[4],
                                               ws_bytes, st)
        fwd_own = lambda: L.bitlinear_forward(a[0], a[1], a[2], g.value, M, N, K, a[3], None, a[4], ws_bytes, st)
        # Warm-up by time: the first few hundred launches of a process run at
        # lower clocks than the steady state.
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(20):
                fwd()
            torch.cuda.synchronize()
        ms = time_events(torch, fwd, reps)
        own_ms = time_events(torch, fwd_own, reps)
        if which == 0:
            mfma_ceiling = bench_mfma_ceiling(torch, L, xq, packed)
        quant_ms = time_events(torch, lambda: L.bitlinear_quantize_act(a[5], M, K, a[0], a[1], a[6], st), reps)
        ops = 2 * M * N * K
        tops = ops / (ms * 1e-3) / 1e12
        out.append({"gemm": f"M={M} K={K} N={N}", "us": round(ms * 1e3, 2),
                    "tops": round(tops, 1), "frac": round(tops / INT8_PEAK_TOPS, 4),
                    "quantize_us": round(quant_ms * 1e3, 2),
                    "us_own_row_sums": round(own_ms * 1e3, 2)})
        del Wd, xd, packed, ws, xq, eta, y, xsum
    for r in out:
        r["frac_of_measured"] = round(r["tops"] / mfma_ceiling["tops"], 4)
    return out, mfma_ceiling


COLD_BYTES = 1_200_000_000   # distinct data cycled through for cold timings (> 4x the 256 MB MALL)


def bench_block(torch, L, S, reps: int, which: int):
    """One transformer block's seven projections from float32 activations to
    float32 outputs, (a) as one grouped forward (quantize + contraction, and
    the split-K epilogue where the plan splits) and (b) as seven fused
    bitlinear_forward_f32 calls.  which = 5: batched decode with skewed
    sparsity (hidden 4096, FFN 11008; ternary weights drawn directly,
    P(0) = 0.6; 1% outlier channels), M = 32, 64, 128.  which = 2: the
    3B-shaped block (hidden 3200, FFN 8640; latent N(0, 0.02) weights), M = 1, 8.

    Cold: the block is copied (packed weights, activations, outputs, plan)
    until the copies hold COLD_BYTES, and consecutive calls cycle through the
    copies, so every call reads its weights from HBM.  Hot: one copy, called
    repeatedly, stays in the caches (the block is smaller than the MALL)."""
    import ctypes
    st = torch.cuda.current_stream().cuda_stream
    projs = S.C5_PROJS if which == 5 else S.C2_PROJS
    packed, gammas = [], []
    for p in projs:
        buf = torch.empty(L.bitlinear_packed_bytes(p.N, p.K), dtype=torch.uint8, device="cuda")
        if which == 5:
            Wt, g = S.c5_ternary(p)
            L.bitlinear_pack_ternary(torch.from_numpy(Wt).cuda(), p.N, p.K, buf)
        else:
            W = torch.from_numpy(S.c2_weight(p)).cuda()
            wsb = L.bitlinear_workspace_bytes(0, p.N, p.K)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            gh = ctypes.c_float()
            L.bitlinear_pack_weights(W, p.N, p.K, buf, None, gh, ws, wsb)
            g = gh.value
            del W, ws
        packed.append(buf)
        gammas.append(float(g))
    wbytes = sum(int(L.bitlinear_packed_bytes(p.N, p.K)) for p in projs)
    ncopies = -(-COLD_BYTES // wbytes)
    copies = [packed] + [[b.clone() for b in packed] for _ in range(ncopies - 1)]
    out = []
    for M in ((32, 64, 128) if which == 5 else (1, 8)):
        xs0 = [torch.from_numpy(S.c5_x(p, M) if which == 5 else S.c2_x(p, M)).cuda() for p in projs]
        plans, keep, singles_calls = [], [], []
        for c, wts in enumerate(copies):
            xs = xs0 if c == 0 else [x.clone() for x in xs0]
            ys = [torch.empty((M, p.N), dtype=torch.float32, device="cuda") for p in projs]
            xqs = [torch.empty((M, p.K), dtype=torch.int8, device="cuda") for p in projs]
            etas = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in projs]
            specs = [dict(x=x, xq=xq, eta=eta, packed=w, y=y, y_int=None, gamma=g, N=p.N, K=p.K)
                     for p, x, xq, eta, w, y, g in zip(projs, xs, xqs, etas, wts, ys, gammas)]
            probs = L.make_problems(specs)
            tb = L.bitlinear_grouped_table_bytes(probs, len(specs), M)
            table = torch.empty(tb, dtype=torch.uint8, device="cuda")
            plans.append(L.bitlinear_grouped_plan_init(probs, len(specs), M, table, tb))
            keep.append((xs, ys, xqs, etas, table))
            # Raw addresses resolved once, outside the timed loops.
            singles_calls.append([(x.data_ptr(), w.data_ptr(), g, p.N, p.K, y.data_ptr())
                                  for p, x, w, y, g in zip(projs, xs, wts, ys, gammas)])
        wsb = max(L.bitlinear_workspace_bytes(M, p.N, p.K) for p in projs)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        wsp = ws.data_ptr()
        fwd = L._lib.bitlinear_forward_grouped
        plan_refs = [ctypes.byref(pl) for pl in plans]
        f32 = L._lib.bitlinear_forward_f32

        def singles(calls):
            for xa, wa, g, N, K, ya in calls:
                f32(xa, wa, g, M, N, K, ya, wsp, wsb, st)
        rot = {"i": 0}

        def grouped_cold():
            i = rot["i"]
            fwd(plan_refs[i], st)
            rot["i"] = (i + 1) % len(plans)

        def singles_cold():
            i = rot["i"]
            singles(singles_calls[i])
            rot["i"] = (i + 1) % len(plans)
        grouped_hot = lambda: fwd(plan_refs[0], st)
        singles_hot = lambda: singles(singles_calls[0])
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            grouped_hot()
            singles_hot()
            torch.cuda.synchronize()
        # Issued call by call from Python (host issue cost included) ...
        g_hot_eager = time_events(torch, grouped_hot, reps)
        s_hot = time_events(torch, singles_hot, reps)
        cold_reps = max(reps, 2 * len(plans))
        for _ in range(len(plans)):
            grouped_cold()
        g_cold_eager = time_events(torch, grouped_cold, cold_reps)
        s_cold = time_events(torch, singles_cold, cold_reps)
        # ... and as the device runs them, replayed from a HIP graph: hot = one
        # copy 50 times, cold = each copy once in turn.
        g_hot = time_graph(torch, lambda i, s: fwd(plan_refs[0], s), 50)
        g_cold = time_graph(torch, lambda i, s: fwd(plan_refs[i], s), len(plans))
        ops = 2 * M * sum(p.N * p.K for p in projs)
        fbytes = wbytes + sum(4 * M * p.K + 4 * M * p.N for p in projs)
        floor_us = max(fbytes / HBM_PEAK_GBS / 1e3, ops / INT8_PEAK_TOPS / 1e6)
        out.append({"M": M, "grouped_us_cold": round(g_cold * 1e3, 2), "grouped_us_hot": round(g_hot * 1e3, 2),
                    "grouped_us_cold_eager": round(g_cold_eager * 1e3, 2),
                    "grouped_us_hot_eager": round(g_hot_eager * 1e3, 2),
                    "single_calls_us_cold_eager": round(s_cold * 1e3, 2),
                    "single_calls_us_hot_eager": round(s_hot * 1e3, 2),
                    "algorithmic_bytes": fbytes, "roofline_floor_us": round(floor_us, 2),
                    "frac_of_roofline_cold": round(floor_us / (g_cold * 1e3), 4),
                    "weight_gbs_cold": round(wbytes / (g_cold * 1e-3) / 1e9, 1),
                    "tops_cold": round(ops / (g_cold * 1e-3) / 1e12, 1)})
        del keep, plans, ws
    workload = ("hidden 4096, FFN 11008 block (q,k,v,o 4096->4096; gate,up 4096->11008; down 11008->4096), "
                "ternary P(0)=0.6, 1% outlier channels x20, float32 in/out") if which == 5 else \
               ("hidden 3200, FFN 8640 block (q,k,v,o 3200->3200; gate,up 3200->8640; down 8640->3200), "
                "latent N(0,0.02) weights, x ~ N(0,1), float32 in/out")
    return {"workload": workload, "packed_weight_bytes": wbytes, "cold_copies": ncopies,
            "cold": f"{ncopies} copies of the block ({ncopies * wbytes / 1e9:.2f} GB of weights) cycled, "
                    "one copy per call; hot: one copy called repeatedly",
            "timing": "grouped_us_*: device time per call, the calls replayed from one HIP graph; *_eager: "
                      "issued call by call from Python (host issue cost included)", "per_M": out}


def bench_c1(torch, L, S, reps: int):
    """The single 2048 x 2048 layer at M = 1 (seed 0): the contraction with
    its dequant (bitlinear_forward on x~), the quantizer, and the fused
    forward from float32, each hot (one weight copy) and cold (COLD_BYTES of
    weight copies cycled).  Algorithmic bytes: packed weights + x~ + eta + y
    (the fused forward reads float32 x instead of x~)."""
    import ctypes
    W, x = S.c1_inputs()
    M, K = x.shape
    N = W.shape[0]
    st = torch.cuda.current_stream().cuda_stream
    wsb = L.bitlinear_workspace_bytes(M, N, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    packed = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gh = ctypes.c_float()
    L.bitlinear_pack_weights(torch.from_numpy(W).cuda(), N, K, packed, None, gh, ws, wsb)
    g = gh.value
    xd = torch.from_numpy(x).cuda()
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    eta = torch.empty(M, dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    L.bitlinear_quantize_act(xd, M, K, xq, eta)
    ncopies = -(-COLD_BYTES // packed.numel())
    copies = [packed] + [packed.clone() for _ in range(ncopies - 1)]
    wp = [c.data_ptr() for c in copies]
    a = [t.data_ptr() for t in (xd, xq, eta, y, ws)]
    fwd, q, f32 = L._lib.bitlinear_forward, L._lib.bitlinear_quantize_act, L._lib.bitlinear_forward_f32
    rot = {"i": 0}

    def nxt():
        i = rot["i"]
        rot["i"] = (i + 1) % ncopies
        return wp[i]
    runs = {
        "forward": (lambda w, s: fwd(a[1], a[2], w, g, M, N, K, a[3], None, a[4], wsb, s),
                    N * K // 4 + M * K + 4 * M + 4 * M * N),
        "fused_f32": (lambda w, s: f32(a[0], w, g, M, N, K, a[3], a[4], wsb, s),
                      N * K // 4 + 4 * M * K + 4 * M + 4 * M * N),
    }
    out = {"layer": f"M={M} K={K} N={N}", "cold": f"{ncopies} weight copies "
           f"({ncopies * packed.numel() / 1e9:.2f} GB) cycled, one per call"}
    for name, (fn, nbytes) in runs.items():
        for _ in range(200):
            fn(wp[0], st)
        hot_eager = time_events(torch, lambda: fn(wp[0], st), max(reps, 200))
        for _ in range(ncopies):
            fn(nxt(), st)
        cold_eager = time_events(torch, lambda: fn(nxt(), st), max(reps, 2 * ncopies))
        hot = time_graph(torch, lambda i, s: fn(wp[0], s), 200)
        cold = time_graph(torch, lambda i, s: fn(wp[i], s), ncopies, replays=3)
        out[name] = {"us_hot": round(hot * 1e3, 2), "us_cold": round(cold * 1e3, 2),
                     "gbs_hot": round(nbytes / (hot * 1e-3) / 1e9, 1),
                     "gbs_cold": round(nbytes / (cold * 1e-3) / 1e9, 1), "algorithmic_bytes": nbytes,
                     "us_hot_eager": round(hot_eager * 1e3, 2), "us_cold_eager": round(cold_eager * 1e3, 2)}
    qt = time_graph(torch, lambda i, s: q(a[0], M, K, a[1], a[2], None, s), 200)
    out["quantize_us_hot"] = round(qt * 1e3, 2)
    out["timing"] = ("us_*: device time per call, the calls replayed from one HIP graph; *_eager: issued call "
                     "by call from Python (host issue cost included)")
    del copies, ws
    return out


def bench_mfma_ceiling(torch, L, xq, packed) -> dict:
    """The int8 matrix-core loop (bitlinear_measure_mfma_i8) fed with the first
    8 KB of these activations and 2 KB of these packed weights: what the
    MFMAs alone sustain on this part, on this data, with every CU busy."""
    sink = torch.empty(L.bitlinear_measure_sink_bytes(), dtype=torch.uint8, device="cuda")
    iters = 40000
    run = lambda: L.bitlinear_measure_mfma_i8(xq, packed, iters, sink)
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        run()
        torch.cuda.synchronize()
    ms = time_events(torch, run, 5)
    tops = L.bitlinear_measure_mfma_ops(iters) / (ms * 1e-3) / 1e12
    return {"tops": round(tops, 1), "frac_of_peak": round(tops / INT8_PEAK_TOPS, 4),
            "kernel": "mfma_loop_kernel: 2 workgroups per CU, 8 independent v_mfma_i32_32x32x32_i8 "
                      "per round, operands from the M=2048 K=3200 activations and packed weights"}


def bench_stream_ceiling(torch, L) -> dict:
    """The streaming-read probe (bitlinear_measure_stream_read) over 4 GiB."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(L.bitlinear_measure_sink_bytes(), dtype=torch.uint8, device="cuda")
    run = lambda: L.bitlinear_measure_stream_read(buf, nbytes, sink)
    for _ in range(3):
        run()
    ms = time_events(torch, run, 10)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del buf
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "stream_read_kernel: 4 GiB read once, one contiguous run per wavefront, 16-byte "
                      "non-temporal loads, a ring of 24 in flight per lane, 4 wavefronts per SIMD"}


def bench_rmsnorm(torch, L, S, reps: int):
    """The fused RMSNorm + absmax quantizer next to the plain quantizer on the
    prefill activations (M = 2048) and decode rows; HBM bytes = 4MK read +
    MK written + 4M scales."""
    out = []
    cases = [(f"prefill x K={S.C3_SHAPES[w][0]}", S.c3_inputs(w)[1]) for w in (0, 1)]
    cases += [(f"decode x M={M} K={K}", S.random_x(9000 + M + K, M, K)) for M, K in ((16, 8192), (16, 28672))]
    # Heavy-tailed rows (a few of them land next to a float32 rounding boundary
    # of the mean of squares and take the exact path) against normal rows.
    cases += [(f"student-t x K=11008", S.random_x(9100, 1024, 11008, "t3")),
              (f"normal x K=11008", S.random_x(9101, 1024, 11008))]
    for name, x in cases:
        M, K = x.shape
        xd = torch.from_numpy(x).cuda()
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        eta = torch.empty(M, dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        a = [t.data_ptr() for t in (xd, xq, eta)]
        rms = lambda: L.bitlinear_rmsnorm_quantize_act(a[0], M, K, a[1], a[2], None, None, st)
        plain = lambda: L.bitlinear_quantize_act(a[0], M, K, a[1], a[2], None, st)
        for _ in range(3):
            rms()
            plain()
        ms_r = time_events(torch, rms, reps)
        ms_q = time_events(torch, plain, reps)
        nbytes = 5 * M * K + 4 * M
        out.append({"rows": f"{name} (M={M})", "rmsnorm_quant_us": round(ms_r * 1e3, 2),
                    "rmsnorm_quant_gbs": round(nbytes / (ms_r * 1e-3) / 1e9, 1),
                    "quant_us": round(ms_q * 1e3, 2),
                    "quant_gbs": round(nbytes / (ms_q * 1e-3) / 1e9, 1)})
        del xd, xq, eta
    return out


def bench_lut(torch, L, reps: int):
    """Decode (M = 1) on the largest 70B-shaped projections, one call each way:
    dot4 on the 2-bit layout (the decode path of bitlinear_forward), the
    matrix-core path on the base-3 layout (bitlinear_forward3) and the
    lookup-table path on both layouts.  Device time per call from HIP-graph
    replays, hot (one weight copy, called repeatedly: it stays in the 256 MB
    MALL) and cold (copies of more than 1.2 GB in all cycled, one per call).
    Weight GB/s counts each layout's own bytes; weights/s is the
    format-independent rate."""
    out = []
    for K, N in ((8192, 28672), (28672, 8192)):
        gen = torch.Generator(device="cuda").manual_seed(K + N)
        Wt = (torch.randint(0, 3, (N, K), generator=gen, device="cuda", dtype=torch.int32) - 1).to(torch.int8)
        p2 = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        p3 = torch.empty(L.bitlinear_packed3_bytes(N, K), dtype=torch.uint8, device="cuda")
        L.bitlinear_pack_ternary(Wt, N, K, p2)
        L.bitlinear_pack_ternary3(Wt, N, K, p3)
        del Wt
        xq = torch.randint(-127, 128, (1, K), generator=gen, device="cuda", dtype=torch.int32).to(torch.int8)
        eta = torch.ones(1, dtype=torch.float32, device="cuda")
        y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        ws_bytes = max(L.bitlinear_workspace_bytes(1, N, K), L.bitlinear_forward3_workspace_bytes(1, N, K),
                       L.bitlinear_lut_workspace_bytes(1, N, K, L.BITLINEAR_FORMAT_2BIT),
                       L.bitlinear_lut_workspace_bytes(1, N, K, L.BITLINEAR_FORMAT_BASE3))
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        copies = {}
        for name, src in (("2bit", p2), ("base3", p3)):
            n = max(2, -(-COLD_BYTES // src.numel()))
            copies[name] = [src] + [src.clone() for _ in range(n - 1)]
        a = [t.data_ptr() for t in (xq, eta, y, ws)]
        runs = {
            "dot4_2bit": ("2bit", lambda pk, st: L.bitlinear_forward(a[0], a[1], pk, 0.02, 1, N, K, a[2], None,
                                                                     a[3], ws_bytes, st)),
            "base3_mfma": ("base3", lambda pk, st: L.bitlinear_forward3(a[0], a[1], pk, 0.02, 1, N, K, a[2], None,
                                                                        a[3], ws_bytes, st)),
            "lut_2bit": ("2bit", lambda pk, st: L.bitlinear_forward_lut(a[0], a[1], pk, L.BITLINEAR_FORMAT_2BIT,
                                                                        0.02, 1, N, K, a[2], None, a[3],
                                                                        ws_bytes, st)),
            "lut_base3": ("base3", lambda pk, st: L.bitlinear_forward_lut(a[0], a[1], pk, L.BITLINEAR_FORMAT_BASE3,
                                                                          0.02, 1, N, K, a[2], None, a[3],
                                                                          ws_bytes, st)),
        }
        row = {"gemv": f"M=1 K={K} N={N}",
               "cold": f"{len(copies['2bit'])} 2-bit / {len(copies['base3'])} base-3 weight copies cycled"}
        for name, (fmt, fn) in runs.items():
            cs = copies[fmt]
            ptrs = [c.data_ptr() for c in cs]
            hot = time_graph(torch, lambda i, st: fn(ptrs[0], st), 20, max(5, reps // 2))
            cold = time_graph(torch, lambda i, st: fn(ptrs[i], st), len(ptrs), max(3, reps // 5))
            nbytes = cs[0].numel()
            row[name] = {"us_hot": round(hot * 1e3, 2), "us_cold": round(cold * 1e3, 2),
                         "weight_gbs_cold": round(nbytes / (cold * 1e-3) / 1e9, 1),
                         "gweights_per_s_cold": round(N * K / (cold * 1e-3) / 1e9, 1)}
        row["base3_over_dot4"] = {k: round(row["base3_mfma"][k] / row["dot4_2bit"][k], 3)
                                  for k in ("us_cold", "us_hot")}
        # the floor of one launch that only reads that many bytes (the stream
        # probe, cold, same copies)
        sink = torch.empty(L.bitlinear_measure_sink_bytes() // 4, dtype=torch.int32, device="cuda")
        for fmt in ("2bit", "base3"):
            cs = copies[fmt]
            ms = time_graph(torch, lambda i, st: L.bitlinear_measure_stream_read(cs[i], cs[i].numel(), sink, st),
                            len(cs), max(3, reps // 5))
            row[f"read_only_{fmt}_us_cold"] = round(ms * 1e3, 2)
        out.append(row)
        del p2, p3, xq, eta, y, ws, copies
        torch.cuda.empty_cache()
    return out


def lut_line(r) -> str:
    return f"decode {r['gemv']}: " + "; ".join(
        f"{k} {v['us_cold']} us cold / {v['us_hot']} hot ({v['weight_gbs_cold']} GB/s, "
        f"{v['gweights_per_s_cold']} Gw/s cold)"
        for k, v in r.items() if isinstance(v, dict) and "weight_gbs_cold" in v) + \
        f"; base-3 / dot4 {r['base3_over_dot4']['us_cold']} cold, {r['base3_over_dot4']['us_hot']} hot" + \
        f"; read-only launch {r['read_only_2bit_us_cold']} us (2-bit bytes), {r['read_only_base3_us_cold']} us (base-3)"


def bench_pack(torch, L, reps: int):
    """Offline weight preparation of the largest 70B projection (28672 x 8192
    latent float32): absmean and absmedian scales into the 2-bit layout, and
    absmean into the base-3 layout; GB/s of latent weights."""
    import ctypes
    N, K = 28672, 8192
    gen = torch.Generator(device="cuda").manual_seed(5)
    W = torch.randn((N, K), generator=gen, device="cuda") * 0.02
    p2 = torch.empty(L.bitlinear_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    p3 = torch.empty(L.bitlinear_packed3_bytes(N, K), dtype=torch.uint8, device="cuda")
    ws_bytes = L.bitlinear_workspace_bytes(0, N, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    calls = {
        "absmean_2bit": lambda: L.bitlinear_pack_weights(W, N, K, p2, None, None, ws, ws_bytes),
        "absmedian_2bit": lambda: L.bitlinear_pack_weights_absmedian(W, N, K, p2, None, None, ws,
                                                                     ws_bytes),
        "absmean_base3": lambda: L.bitlinear_pack_weights3(W, N, K, p3, None, None, ws, ws_bytes),
    }
    out = {"matrix": f"{N}x{K} float32 latent"}
    for name, fn in calls.items():
        fn()
        ms = time_events(torch, fn, reps)
        out[name] = {"ms": round(ms, 3), "latent_gbs": round(4 * N * K / (ms * 1e-3) / 1e9, 1)}
    del W, p2, p3, ws
    return out


def cpu_baseline(sw, S, budget_s: float = 8.0):
    """The oracle (unchanged) on bounded samples of the workloads, timed on
    this host's cores: (a) layer 0's seven projections of the 70B-shaped
    sweep at M = 1 (quantize + contract + dequant) on all host threads, run
    repeatedly for about budget_s seconds -- the reported value; (b) the same
    on one thread over layer 0's q and k projections; (c) the 3B prefill GEMM
    3200 -> 8640 on a sample of its 2048 Student-t token rows (quantize +
    contract + dequant), on all threads and on one."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    O = oracle.default()
    prepared = []
    for p in sw.projs:
        W = S.c4_weight_device(0, p).cpu().numpy()
        Wt, g = O.quantize_weights(W)
        del W
        prepared.append((sw.x[(0, p.name, 1)].cpu().numpy(), Wt, g, p))
        log(f"cpu oracle: prepared layer 0 {p.name}")

    def timed(items, nthreads, budget, what):
        nbytes = sum(p.N * p.K // 4 + 4 * p.K + 4 * p.N + 4 for *_, p in items)
        t_total, passes = 0.0, 0
        while t_total < budget and passes < 200:
            t0 = time.perf_counter()
            for x, Wt, g, p in items:
                O.forward(x, Wt, g, threads=nthreads)
            t_total += time.perf_counter() - t0
            passes += 1
        log(f"cpu oracle ({what}, {nthreads} threads): {passes} passes, {t_total:.1f} s")
        return nbytes, passes, t_total

    nb, passes, t_all = timed(prepared, threads, budget_s, "layer 0")
    value = nb * passes / t_all / 1e9
    qk = [it for it in prepared if it[3].name in ("q", "k")]
    nb1, passes1, t_one = timed(qk, 1, budget_s / 2, "layer 0 q, k")
    single = {"value": round(nb1 * passes1 / t_one / 1e9, 4), "unit": "GB/s", "cores": 1,
              "sample": f"layer 0 q and k projections ({nb1 / 1e6:.1f} MB of packed weights) at M=1, "
                        f"{passes1} passes, {t_one:.1f} s timed"}

    W, x = S.c3_inputs(0)
    Wt, g = O.quantize_weights(W)
    del W
    prefill = {}
    for nthreads, rows in ((threads, 64), (1, 4)):
        t0 = time.perf_counter()
        O.forward(x[:rows], Wt, g, threads=nthreads)
        t = time.perf_counter() - t0
        ops = 2 * rows * Wt.shape[0] * Wt.shape[1]
        key = "all_threads" if nthreads == threads else "single_thread"
        prefill[key] = {"value": round(ops / t / 1e12, 6), "unit": "TOP/s", "cores": nthreads,
                        "sample": f"{rows} of the 2048 token rows of the 3200->8640 prefill GEMM, {t:.2f} s"}
        log(f"cpu oracle prefill ({nthreads} threads, {rows} rows): {t:.2f} s")
    return {"value": round(value, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of the 70B-shaped sweep (7 projections, {nb / 1e6:.1f} MB "
                      f"of packed weights) at M=1, quantize+contract+dequant, {passes} passes, "
                      f"{t_all:.1f} s timed",
            "single_thread": single, "prefill_c3": prefill}


COPY_BYTES = 1 << 30


def profile_run(torch, L, sw, args) -> int:
    """Kernels for rocprofv3: full steps, contraction-only launches, a calibration copy."""
    M, fmt = args.profile_m, args.profile_fmt
    for _ in range(max(1, args.steps)):
        sw.step(M, fmt=fmt)
    plan_c, _table = contraction_only_plan(sw, M, fmt)
    for _ in range(max(1, args.steps)):
        L.bitlinear_forward_grouped(plan_c)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)   # reads and writes exactly COPY_BYTES each
    torch.cuda.synchronize()
    log(f"profile run done: {fmt} M={M}, contraction bytes per launch {sw.contraction_bytes(M, fmt)}")
    return 0


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profile(root: str) -> str:
    """Markdown summary of rocprofv3 output under root: kernel stats (from a
    --kernel-trace --stats run in root/trace) and per-dispatch FETCH_SIZE /
    WRITE_SIZE (from --pmc runs in root/fetch and root/write), the latter
    scaled by the counters of the 1 GiB calibration copy."""
    import glob
    out = []
    stats = glob.glob(os.path.join(root, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        rows = _csv_rows(stats[0])
        out.append("| kernel | calls | avg us | min us | max us | total % |")
        out.append("|---|---|---|---|---|---|")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
            name = r["Name"][:90].replace("|", "/")
            out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                       f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                       f"{float(r['Percentage']):.2f} |")
    for kind in ("fetch", "write"):
        files = glob.glob(os.path.join(root, kind, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            continue
        rows = _csv_rows(files[0])
        per = {}
        for r in rows:
            key = "copy" if "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower() \
                else ("contraction" if any(k in r["Kernel_Name"] for k in
                                           ("gemv_dot4_kernel", "skinny_mfma_kernel", "gemm_prefill_kernel",
                                            "base3_mfma_kernel"))
                      else None)
            if key:
                per.setdefault(key, []).append(float(r["Counter_Value"]))
        if "copy" in per and "contraction" in per:
            copy_kib = max(per["copy"])
            factor = (COPY_BYTES / 1024) / copy_kib
            vals = sorted(per["contraction"])
            med = vals[len(vals) // 2]
            out.append(f"\n{kind.upper()}_SIZE: calibration copy reads {copy_kib:.0f} KiB for "
                       f"{COPY_BYTES / 1024:.0f} KiB moved (factor {factor:.4f}); contraction kernel "
                       f"median {med:.0f} KiB per dispatch -> {med * factor * 1024 / 1e9:.4f} GB scaled "
                       f"({len(vals)} dispatches)")
    return "\n".join(out)


def summarize_pmc(root: str) -> str:
    """Markdown table of the counters of every rocprofv3 --pmc run under
    root/pmc*/: per contraction kernel of this library (and the int8 MFMA-loop probe), the
    median of each counter over its dispatches, with the matrix-core busy
    fraction SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs) where
    both were collected (GRBM_GUI_ACTIVE sums the XCDs' active cycles)."""
    import glob
    import statistics
    per = {}
    for path in sorted(glob.glob(os.path.join(root, "pmc*", "**", "*counter_collection.csv"), recursive=True)):
        for r in _csv_rows(path):
            name = r["Kernel_Name"]
            if not any(k in name for k in ("gemm_prefill", "mfma_loop", "skinny_mfma", "gemv_dot4", "gemv_fused")):
                continue
            per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        return ""
    out = ["| kernel | counter | median per dispatch | dispatches |", "|---|---|---|---|"]
    for name, cs in per.items():
        short = name[:70].replace("|", "/")
        for c in sorted(cs):
            out.append(f"| {short} | {c} | {statistics.median(cs[c]):,.0f} | {len(cs[c])} |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and "GRBM_GUI_ACTIVE" in cs:
            busy = statistics.median(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
            active = statistics.median(cs["GRBM_GUI_ACTIVE"]) / 8.0
            out.append(f"| {short} | matrix cores busy | {busy / (active * 1024):.1%} "
                       f"(of {active:,.0f} cycles per XCD, 1024 SIMDs) | |")
    return "\n".join(out)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_dot4_grouped_decode70b_m1_traffic.json")


def measured_traffic():
    """HBM bytes per launch of the decode contraction kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None once the kernel's sources have
    changed since those counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["kernel_source_sha256"]:
            return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-m16", action="store_true")
    ap.add_argument("--no-base3", action="store_true", help="skip the base-3 layout of the 70B sweep")
    ap.add_argument("--profile-m", type=int, default=1, choices=(1, 16),
                    help="token count of the --profile-run sweep")
    ap.add_argument("--profile-fmt", default="2bit", choices=("2bit", "base3"),
                    help="weight layout of the --profile-run sweep (base-3: M=1 only)")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run for rocprofv3: the M=1 sweep, the contraction kernel alone and a "
                         "1 GiB copy whose counters calibrate FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="short run for rocprofv3: the two 3B prefill GEMMs and a calibration copy")
    ap.add_argument("--profile-blocks", action="store_true",
                    help="time only the single-block grouped forwards (3B block at M=1, 8; "
                         "hidden-4096 block at M=32, 64, 128), for a rocprofv3 run")
    ap.add_argument("--profile-decode3", action="store_true",
                    help="time only the M=1 decode of the two largest 70B projections in both weight "
                         "formats (dot4, base-3 matrix cores, lookup tables), for a rocprofv3 run")
    ap.add_argument("--summarize", metavar="DIR", help="summarize rocprofv3 output under DIR")
    args = ap.parse_args()
    if args.summarize:
        print(summarize_profile(args.summarize))
        print(summarize_pmc(args.summarize))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    import torch
    from ternary_weight_linear_fwd_amd import bitlinear as L
    from ternary_weight_linear_fwd_amd import synthetic as S
    from ternary_weight_linear_fwd_amd.sweep import DecodeSweep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device {torch.cuda.get_device_name(0)}; building the sweep ({args.layers} layers)")
    Ms = (1,) if args.no_m16 else (1, 16)
    if args.profile_run:
        Ms = (args.profile_m,)
    if args.profile_blocks:
        for which in (2, 5):
            for r in bench_block(torch, L, S, max(1, args.steps), which)["per_M"]:
                log(f"C{which} block M={r['M']}: grouped {r['grouped_us_cold']} us cold / "
                    f"{r['grouped_us_hot']} us hot")
        return 0
    if args.profile_decode3:
        for r in bench_lut(torch, L, max(5, args.steps)):
            log(lut_line(r))
        return 0
    if args.profile_prefill:
        for r in bench_prefill(torch, L, S, max(1, args.steps))[0]:
            log(f"prefill {r['gemm']}: {r['us']} us; own row sums {r['us_own_row_sums']} us; "
                f"quantize {r['quantize_us']} us")
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        return 0
    # The prefill GEMMs are timed first, on a GPU that has not just spent
    # seconds streaming the 17 GB sweep (their own warm-up settles the clocks).
    prefill = mfma_ceiling = None
    if not args.no_prefill and not args.profile_run:
        prefill, mfma_ceiling = bench_prefill(torch, L, S, max(10, args.steps))
        for r in prefill:
            log(f"prefill {r['gemm']}: {r['us']} us, {r['tops']} TOP/s ({r['frac']:.1%}); "
                f"own row sums {r['us_own_row_sums']} us; quantize {r['quantize_us']} us")
    if args.profile_run:
        formats = (args.profile_fmt,)
        base3_Ms = Ms
    else:
        formats = ("2bit",) if args.no_base3 else ("2bit", "base3")
        base3_Ms = (1,)
    sw = DecodeSweep(layers=args.layers, Ms=Ms, progress=log, formats=formats, base3_Ms=base3_Ms)
    log(f"packed weights resident: {sum(sw.weight_bytes(f) for f in formats) / 1e9:.3f} GB ({', '.join(formats)})")
    if args.profile_run:
        return profile_run(torch, L, sw, args)

    # ---- headline: full step at M = 1
    for _ in range(args.warmup):
        sw.step(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(torch, lambda: sw.step(1), args.steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_bytes = sw.algorithmic_bytes(1)
    value = step_bytes / (ms * 1e-3) / 1e9
    log(f"M=1 step: {ms:.3f} ms (wall {wall_ms:.3f} ms), {value:.1f} GB/s")

    # ---- dominant kernel: the contraction alone, events on its stream
    plan_c, _table_c = contraction_only_plan(sw, 1)
    L.bitlinear_forward_grouped(plan_c)
    kern_ms = time_events(torch, lambda: L.bitlinear_forward_grouped(plan_c), args.steps)
    kern_bytes = sw.contraction_bytes(1)
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    log(f"contraction kernel: {kern_ms:.3f} ms, {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBS:.1%})")

    stream_ceiling = bench_stream_ceiling(torch, L)
    log(f"measured ceilings: stream read {stream_ceiling['gbs']} GB/s"
        + (f", int8 MFMA loop {mfma_ceiling['tops']} TOP/s" if mfma_ceiling else ""))
    extra = {"ceilings": {"stream_read": stream_ceiling}}
    if mfma_ceiling:
        extra["ceilings"]["mfma_i8"] = mfma_ceiling
    if not args.no_m16:
        for _ in range(2):
            sw.step(16)
        ms16 = time_events(torch, lambda: sw.step(16), max(5, args.steps // 2))
        gbs16 = sw.algorithmic_bytes(16) / (ms16 * 1e-3) / 1e9
        extra["decode_m16"] = {"ms_per_step": round(ms16, 4), "value": round(gbs16, 1),
                               "unit": "GB/s", "frac": round(gbs16 / HBM_PEAK_GBS, 4),
                               "tops": round(sw.ops(16) / (ms16 * 1e-3) / 1e12, 1)}
        log(f"M=16 step: {ms16:.3f} ms, {gbs16:.1f} GB/s")

    if "base3" in sw.formats:
        extra["decode_base3"] = bench_decode_base3(torch, sw, args.steps)
        for r in extra["decode_base3"]:
            log(f"70B decode step M={r['M']}: " + "; ".join(
                f"{f} {r[f]['ms_per_step']} ms ({r[f]['gbs']} GB/s, {r[f]['frac']:.1%}; contraction "
                f"{r[f]['contraction_ms']} ms, {r[f]['contraction_frac']:.1%})" for f in ("2bit", "base3") if f in r)
                + (f"; base-3 / 2-bit {r['base3_over_2bit']}" if "base3_over_2bit" in r else ""))

    if prefill is not None:
        extra["prefill"] = prefill

    if not args.no_prefill:
        extra["single_layer_c1"] = bench_c1(torch, L, S, max(10, args.steps))
        c1 = extra["single_layer_c1"]
        log(f"C1 forward: {c1['forward']['us_cold']} us cold, {c1['forward']['us_hot']} us hot; fused "
            f"{c1['fused_f32']['us_cold']} / {c1['fused_f32']['us_hot']} us; quantize {c1['quantize_us_hot']} us")
        for which, key in ((2, "block_decode_c2"), (5, "batched_decode_c5")):
            extra[key] = bench_block(torch, L, S, max(10, args.steps), which)
            for r in extra[key]["per_M"]:
                log(f"C{which} block M={r['M']}: grouped {r['grouped_us_cold']} us cold / {r['grouped_us_hot']} "
                    f"hot (graph replay; eager {r['grouped_us_cold_eager']} / {r['grouped_us_hot_eager']}), seven "
                    f"single calls {r['single_calls_us_cold_eager']} / {r['single_calls_us_hot_eager']} us eager "
                    f"(floor {r['roofline_floor_us']} us, {r['frac_of_roofline_cold']:.1%} cold)")

    if not args.no_prefill:
        extra["rmsnorm_quant"] = bench_rmsnorm(torch, L, S, max(10, args.steps))
        for r in extra["rmsnorm_quant"]:
            log(f"rmsnorm+quant {r['rows']}: {r['rmsnorm_quant_us']} us "
                f"({r['rmsnorm_quant_gbs']} GB/s); quant alone {r['quant_us']} us")

    if not args.no_prefill:
        extra["lut_decode"] = bench_lut(torch, L, max(10, args.steps))
        for r in extra["lut_decode"]:
            log(lut_line(r))

    if not args.no_prefill:
        extra["pack"] = bench_pack(torch, L, 3)
        log("pack " + "; ".join(f"{k} {v['ms']} ms ({v['latent_gbs']} GB/s)"
                                for k, v in extra["pack"].items() if k != "matrix"))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the sweep")
        cpu = cpu_baseline(sw, S)
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads, "
            f"{cpu['single_thread']['value']} GB/s on one")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"70B-shaped decode sweep: {args.layers} layers x 7 BitLinear "
                               "projections (q,o 8192->8192; k,v 8192->1024; gate,up "
                               "8192->28672; down 28672->8192), M=1, one grouped forward per step",
                   "tokens_per_step": 1, "packed_weight_bytes": sw.weight_bytes(),
                   "algorithmic_bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "gemv_dot4_kernel<1, grouped> (contraction + fused dequant)",
                     "kernel_ms": round(kern_ms, 4), "algorithmic_bytes": kern_bytes,
                     "frac_of_measured": round(achieved / stream_ceiling["gbs"], 4)},
        "cpu_baseline": cpu,
        "system": system_info(torch),
    }
    line.update(extra)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
