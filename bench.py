#!/usr/bin/env python3
"""Benchmark of the ternary linear layer on one MI355X (gfx950).

Headline workload: decode GEMV at M = 1 with 2-bit packed ternary weights, the
three projections of a LLaMA-style block at hidden 4096 / MLP 11008
(4096x4096, 4096->11008, 11008->4096).  One step = the three tri_linear launches
on cold weights: every matrix rotates over 64 distinct copies (1.7 GB in all),
so the 256 MB Infinity Cache cannot serve a step's weights.  The value is
effective HBM bandwidth: (packed weights as stored + fp16 X read) per step /
wall time per step, inputs resident in HBM.

Timing.  The timed region replays a HIP graph of the steps (captured once from
the same tri_linear calls), so the host's per-launch cost stays out of it.
Per-kernel durations come from HIP events on the launch stream around a batch
of back-to-back launches of one kernel, queued while a sleep kernel holds the
GPU, so no host time enters them (they agree with rocprofv3's per-dispatch
durations).

The same JSON line carries the roofline fraction of the decode kernel, the
size-matched streaming-read floor, the CPU oracle timed on this host, and the
batched-decode, block-step and prefill workloads.

  python bench.py [--gpus 1] [--steps 1000] [--warmup 20] [--skip-extra] [--skip-cpu]
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6   # MI355X dense fp16 MFMA peak (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "effective HBM GB/s (% of peak) for M=1 ternary GEMV; prefill GEMM TFLOP/s (% MFMA)"
COPIES = 64                     # distinct copies of every decode weight matrix
COUNTERS = os.path.join(ROOT, "profiles", "decode_mv1_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def effective_bytes(M, N, K, fmt):
    """Effective bytes of one layer launch: the packed weights as stored plus the fp16 activations
    read (the output's 2*M*N bytes are not counted)."""
    import bit_mixed_precision_tri_amd as tri
    return N * tri.tri_row_bytes(K, fmt) + 2 * M * K


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and its logical CPU count."""
    name = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return name, os.cpu_count()


class Layer:
    """One ternary linear on the GPU with a pool of distinct packed-weight copies."""

    def __init__(self, workload_id, layer_id, M, N, K, fmt, scale=None, copies=COPIES, X=None):
        import torch
        import bit_mixed_precision_tri_amd as tri
        from bit_mixed_precision_tri_amd import synth
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        W, Xh, self.scale = synth.layer_inputs(workload_id, layer_id, M, N, K, scale)
        Wp = tri.pack(torch.from_numpy(W).cuda(), fmt)
        self.pool = torch.empty((copies,) + tuple(Wp.shape), dtype=torch.uint8, device="cuda")
        self.pool[:] = Wp                       # distinct addresses, same content
        self.X = X if X is not None else torch.from_numpy(Xh).cuda()
        self.Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        self.bytes = effective_bytes(M, N, K, fmt)
        self.flops = 2 * M * N * K
        self.i = 0

    def launch(self, algo=0):
        import bit_mixed_precision_tri_amd as tri
        Wp = self.pool[self.i % self.pool.shape[0]]
        self.i += 1
        if algo:
            tri.tri_linear_algo(self.X, Wp, self.scale, self.M, self.N, self.K, self.fmt, self.Y, algo)
        else:
            tri.tri_linear(self.X, Wp, self.scale, self.M, self.N, self.K, self.fmt, self.Y)


class Clock:
    """Back-to-back kernel timing with HIP events on the current (launch) stream."""

    def __init__(self):
        import torch
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)                  # first call compiles/loads the sleep kernel
        a.record()
        torch.cuda._sleep(5_000_000)
        b.record()
        torch.cuda.synchronize()
        self.cycles_per_us = 5_000_000 / (a.elapsed_time(b) * 1e3)

    def hold(self, us):
        """Queue a sleep kernel that keeps the GPU busy for about `us` microseconds."""
        import torch
        torch.cuda._sleep(int(us * self.cycles_per_us))

    def run(self, calls, warmup=5):
        """Run the callables back to back on the GPU; mean time per call (s).

        A sleep kernel holds the GPU until every call is queued, and one pair of events
        brackets the batch, so the figure is kernel duration plus the launch gap of an
        in-order stream, with no host time in it.  Also returns whether the queue stayed
        ahead of the GPU."""
        import torch
        for c in calls[:warmup]:
            c()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_us = 40.0 * len(calls) + 5000.0      # generous host cost per queued call
        self.hold(hold_us)
        t0 = time.perf_counter()
        a.record()
        for c in calls:
            c()
        b.record()
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / len(calls), host_us < 0.8 * hold_us


def read_floor(nbytes, clock, reps=200):
    """Size-matched streaming read (tri_probe_read) over a rotating >= 1 GiB pool: mean duration (s)."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    nb = (nbytes + 15) // 16 * 16
    ncopies = max(1, -(-(1 << 30) // nb))
    pool = torch.empty((ncopies, nb), dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    calls = [(lambda i=i: tri.tri_probe_read(pool[i % ncopies], nb, sink)) for i in range(reps)]
    t, _ = clock.run(calls)
    del pool
    torch.cuda.empty_cache()
    return t


def counters():
    """HBM traffic of the decode kernel per decode step from the committed rocprofv3 summary,
    or None when the kernel source changed after the counters were taken."""
    import hashlib
    if not os.path.exists(COUNTERS):
        return None
    m = re.search(r"^traffic-json: (\{.*\})\s*$", open(COUNTERS).read(), re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    src = open(os.path.join(ROOT, "bit_mixed_precision_tri_amd", "csrc", rec["source"]), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec


def cpu_baseline(shapes, budget_s=10.0):
    """The CPU oracle (unpack + float64 layer, OpenMP over output rows) on the full decode step."""
    import numpy as np
    import oracle
    from bit_mixed_precision_tri_amd import configs, synth
    threads = oracle.max_threads()
    work = []
    for li, (name, K, N) in enumerate(shapes):
        W, X, s = synth.layer_inputs(configs.DECODE["workload_id"], li, 1, N, K)
        work.append((X, oracle.pack2(W), K, s))
    total_bytes = sum(effective_bytes(1, Wp.shape[0], K, 0) for (X, Wp, K, s) in work)
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        for (X, Wp, K, s) in work:
            oracle.linear_packed_f64(X, Wp, K, 0, s, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if len(times) >= 200:
            break
    t = float(np.median(times))
    model, ncpu = cpu_model()
    return {"value": round(total_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_logical_cpus": ncpu,
            "sample": "the full decode step (3 shapes, M=1, 2-bit: unpack + float64 layer) run %d times in ~%d s, "
                      "median %.3f s per step" % (len(times), budget_s, t)}


def cpu_oracle_detail(shapes):
    """The oracle beside the GPU in more detail (bounded, a few seconds): the decode step on one
    thread, and the prefill layer (8192 -> 28672, 2-bit) on a fixed 16-row subset of its 2048
    rows on every thread, extrapolated to all rows."""
    import numpy as np
    import oracle
    from bit_mixed_precision_tri_amd import configs, synth
    threads = oracle.max_threads()              # (before the one-thread runs, which set the OpenMP count)
    work = []
    for li, (name, K, N) in enumerate(shapes):
        W, X, s = synth.layer_inputs(configs.DECODE["workload_id"], li, 1, N, K)
        work.append((X, oracle.pack2(W), K, s))
    one = []
    for _ in range(2):
        t0 = time.perf_counter()
        for (X, Wp, K, s) in work:
            oracle.linear_packed_f64(X, Wp, K, 0, s, nthreads=1)
        one.append(time.perf_counter() - t0)
    pc = configs.PREFILL
    name, K, N = pc["shapes"][0]
    W = synth.trits(synth.rng_for(pc["workload_id"], 0, synth.STREAM_W), N, K)
    X = synth.activations(synth.rng_for(pc["workload_id"], 0, synth.STREAM_X), 16, K)
    Wp = oracle.pack2(W)
    del W
    t0 = time.perf_counter()
    oracle.linear_packed_f64(X, Wp, K, 0, pc["scale"], nthreads=threads)
    tp = (time.perf_counter() - t0) * pc["M"] / 16
    return {"decode_step_1_thread_s": round(float(np.median(one)), 4),
            "prefill_%s_2bit" % name: {"rows_timed": 16, "threads": threads, "extrapolated_s": round(tp, 2),
                                        "TFLOPs": round(2 * pc["M"] * N * K / tp / 1e12, 5)}}


def capture(layers, steps):
    """A HIP graph of `steps` decode steps (each: every layer once, next weight copy)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L in layers:
            L.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(steps):
            for L in layers:
                L.launch()
    torch.cuda.synchronize()
    return g


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-extra", action="store_true", help="skip the batched, block and prefill workloads")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--floor", action="store_true",
                    help="only the decode floor: empty and loads-only probes on the decode grid, streaming reads")
    ap.add_argument("--profile", choices=["decode", "copy", "prefill", "batched", "floor", "block"],
                    help="only launch one workload a few times (for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the ternary linear layer runs on one GPU here; --gpus %d is not supported "
              "(multi-GPU sharding is a design note only)" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tri.lib()
    torch.cuda.set_device(0)
    F2 = tri.TRI_FMT_2BIT

    if args.profile:
        return profile_mode(args.profile)
    if args.floor:
        print(json.dumps({"floor": bench_floor(Clock())}), flush=True)
        return

    # ---- headline: decode GEMV, M = 1, 2-bit, three shapes, cold weights
    dcfg = configs.DECODE
    layers = [Layer(dcfg["workload_id"], li, 1, N, K, F2) for li, (name, K, N) in enumerate(dcfg["shapes"])]
    step_bytes = sum(L.bytes for L in layers)
    chunk = min(args.steps, COPIES)
    g_main = capture(layers, chunk)
    g_rest = capture(layers, args.steps % chunk) if args.steps % chunk else None
    for _ in range(max(1, args.warmup // chunk)):
        g_main.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps // chunk):
        g_main.replay()
    if g_rest is not None:
        g_rest.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    value = step_bytes * args.steps / elapsed / 1e9
    del g_main, g_rest

    # per-kernel durations: 200 back-to-back launches of each shape (rotating weight copies)
    clock = Clock()
    per_launch, ahead = [], True
    for L in layers:
        t, ok = clock.run([L.launch] * 200)
        per_launch.append(t)
        ahead = ahead and ok
    achieved = step_bytes / sum(per_launch) / 1e9
    shapes_out = []
    for (name, K, N), L, t in zip(dcfg["shapes"], layers, per_launch):
        shapes_out.append({"shape": name, "K": K, "N": N, "bytes": L.bytes, "kernel_us": round(t * 1e6, 3),
                           "GBps": round(L.bytes / t / 1e9, 1),
                           "algo": tri.ALGO_NAMES[tri.tri_select_algo(1, N, K, F2)]})
    # the VALU GEMV kernel at M = 1, same shapes (the alternative the MFMA kernel is chosen over)
    for so, L in zip(shapes_out, layers):
        t, _ = clock.run([lambda L=L: L.launch(tri.TRI_ALGO_GEMV)] * 100)
        so["gemv_kernel_us"] = round(t * 1e6, 3)
        so["gemv_GBps"] = round(L.bytes / t / 1e9, 1)
    del layers
    torch.cuda.empty_cache()
    floors = []
    for (name, K, N) in dcfg["shapes"]:
        nb = N * tri.tri_row_bytes(K, F2)
        t = read_floor(nb, clock)
        floors.append({"shape": name, "bytes": nb, "read_us": round(t * 1e6, 3), "GBps": round(nb / t / 1e9, 1)})
    for so, fl in zip(shapes_out, floors):      # the read floor's time over the kernel's: 1.0 = at the floor
        so["read_floor_over_kernel"] = round(fl["read_us"] / so["kernel_us"], 3)
    small = bench_small(clock)
    ctr = counters()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1, 2-bit packed ternary weights, shapes 4096x4096 + 4096->11008 + "
                               "11008->4096 per step, each matrix rotating over 64 copies (cold)",
                   "M": 1, "shapes": [[K, N] for (_, K, N) in dcfg["shapes"]], "format": "2bit",
                   "accumulate": "f32", "bytes_per_step": step_bytes, "timing": "HIP graph replay"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        # per launch, averaged over the three decode shapes (one launch each per step)
        "roofline": {"bound": "hbm", "kernel": "k_mv1 (tri_mv1.hip)", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(ctr["traffic_bytes_per_step"] / len(per_launch)) if ctr else None),
                     "algorithmic_bytes": round(step_bytes / len(per_launch)),
                     "per": "launch, mean over the three decode shapes",
                     "launches_per_step": len(per_launch),
                     "mean_launch_us": round(sum(per_launch) / len(per_launch) * 1e6, 3), "queue_ahead": ahead},
        "context": "the pages report relative speed-ups only, on NVIDIA GPUs: TriRun up to 5x end-to-end generation "
                   "vs PyTorch FP16 on an L40S (64+64 tokens), about 8x per ternary layer; no absolute GB/s or "
                   "TFLOP/s to compare with (vs_baseline is null)",
        "per_shape": shapes_out,
        "read_floor": floors,
        "small": small,
    }
    if not args.skip_extra:
        out["decode_1p6bit"] = bench_decode_1p6(clock)
        out["decode_large"] = bench_decode_large(clock)
        out["batched"] = bench_batched(clock)
        out["mid_m"] = bench_mid_m(clock)
        out["block"] = bench_block(clock)
        out["prefill"] = bench_prefill(clock)
        out["quantize"] = bench_quantize(clock)
    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline(dcfg["shapes"])
        out["cpu_oracle_detail"] = cpu_oracle_detail(dcfg["shapes"])
    print(json.dumps(out), flush=True)


def bench_small(clock):
    """The small layer (M = 1, K = 512, N = 256, scale 0.02) in both formats: latency per launch
    (32 KB of 2-bit weights are far below any bandwidth regime), timed as 200 back-to-back launches
    with events around a sleep-held queue and as a replayed HIP graph of them."""
    import torch
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.SMALL
    res = []
    for fmt in cfg["fmts"]:
        L = Layer(cfg["workload_id"], 0, cfg["M"], cfg["N"], cfg["K"], fmt, cfg["scale"])
        t_ev, _ = clock.run([L.launch] * 200)
        t_gr = graph_time(L.launch, 200, replays=3)
        res.append({"M": cfg["M"], "K": cfg["K"], "N": cfg["N"], "format": configs.FMT_NAMES[fmt],
                    "bytes": L.bytes, "kernel_us_events": round(t_ev * 1e6, 3),
                    "kernel_us_graph": round(t_gr * 1e6, 3)})
        del L
        torch.cuda.empty_cache()
    return res


def bench_batched(clock):
    import torch
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.BATCHED
    res = []
    for fmt in cfg["fmts"]:
        for li, (name, K, N) in enumerate(cfg["shapes"]):
            for M in cfg["Ms"]:
                L = Layer(cfg["workload_id"], 10 * li + M, M, N, K, fmt, copies=32)
                t, _ = clock.run([L.launch] * 100)
                res.append({"shape": name, "M": M, "format": configs.FMT_NAMES[fmt], "kernel_us": round(t * 1e6, 3),
                            "GBps": round(L.bytes / t / 1e9, 1), "frac_hbm": round(L.bytes / t / 1e9 / HBM_PEAK_GBS, 4)})
                del L
                torch.cuda.empty_cache()
    return res


def bench_mid_m(clock):
    """16 < M <= 256 with cold weights, on the kernel family tri_linear picks for the shape."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.MID_M
    res = []
    for li, (name, K, N) in enumerate(cfg["shapes"]):
        for M in cfg["Ms"]:
            L = Layer(cfg["workload_id"], 10 * li + M, M, N, K, cfg["fmt"], copies=16)
            t, _ = clock.run([L.launch] * 50)
            res.append({"shape": name, "M": M, "format": configs.FMT_NAMES[cfg["fmt"]],
                        "algo": tri.ALGO_NAMES[tri.tri_select_algo(M, N, K, cfg["fmt"])],
                        "kernel_us": round(t * 1e6, 3), "GBps": round(L.bytes / t / 1e9, 1),
                        "TFLOPs": round(L.flops / t / 1e12, 2)})
            del L
            torch.cuda.empty_cache()
    return res


def bench_decode_large(clock):
    """Decode (M = 1, 2) on the 58.7 MB (2-bit) prefill matrices, cold weights (eight copies,
    beyond the last-level cache), with the size-matched read floor of the packed bytes."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.DECODE_LARGE
    res = []
    for fmt in cfg["fmts"]:
        for li, (name, K, N) in enumerate(cfg["shapes"]):
            nb = N * tri.tri_row_bytes(K, fmt)
            tf = read_floor(nb, clock)
            for M in cfg["Ms"]:
                L = Layer(cfg["workload_id"], 10 * li + M, M, N, K, fmt, copies=8)
                t, _ = clock.run([L.launch] * 100)
                res.append({"shape": name, "M": M, "format": configs.FMT_NAMES[fmt], "kernel_us": round(t * 1e6, 3),
                            "GBps": round(L.bytes / t / 1e9, 1), "frac_hbm": round(L.bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                            "read_floor_us": round(tf * 1e6, 3), "read_floor_over_kernel": round(tf / t, 3)})
                del L
                torch.cuda.empty_cache()
    return res


def bench_decode_1p6(clock):
    """The decode shapes at M = 1 with 1.6-bit packed weights (k_mv1, base-3 quotients by
    multiply-shift), cold weights; with the size-matched read floor of the 1.6-bit bytes."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    dcfg = configs.DECODE
    F16 = tri.TRI_FMT_1P6BIT
    res = []
    for li, (name, K, N) in enumerate(dcfg["shapes"]):
        L = Layer(dcfg["workload_id"], 20 + li, 1, N, K, F16)
        t, _ = clock.run([L.launch] * 200)
        nb = N * tri.tri_row_bytes(K, F16)
        del L
        torch.cuda.empty_cache()
        tf = read_floor(nb, clock)
        res.append({"shape": name, "K": K, "N": N, "bytes": effective_bytes(1, N, K, F16),
                    "kernel_us": round(t * 1e6, 3), "GBps": round(effective_bytes(1, N, K, F16) / t / 1e9, 1),
                    "read_floor_us": round(tf * 1e6, 3)})
    return res


def graph_time(step, nsteps, replays=10):
    """Mean GPU time (s) of one call of `step`: `nsteps` calls captured in a HIP graph, replayed."""
    import torch
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(nsteps):
                step()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / 1e3 / (replays * nsteps)


def bench_block(clock):
    """One block decode step: Q, K, V, O (4096x4096), gate, up (4096->11008), down (11008->4096),
    inputs pre-staged, weights rotating over copies.  Timed as seven launches, as four (Q/K/V
    and gate/up each one grouped launch: they read the same activations), and as the whole
    block with its glue (RMSNorm, residuals, silu gate) folded into four fused launches.  The
    bytes are those of the seven linears (the glue reads a few KB more).  Each variant is timed
    as a replayed HIP graph, so no host time enters it."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs, synth
    cfg = configs.BLOCK
    res = []
    copies = 16
    for M in cfg["Ms"]:
        pools, scales, Ns, Ks = [], [], [], []
        for li, (name, K, N) in enumerate(cfg["layers"]):
            W, _, s = synth.layer_inputs(cfg["workload_id"], 100 * M + li, M, N, K)
            Wp = tri.pack(torch.from_numpy(W).cuda(), cfg["fmt"])
            pool = torch.empty((copies,) + tuple(Wp.shape), dtype=torch.uint8, device="cuda")
            pool[:] = Wp
            pools.append(pool)
            scales.append(s)
            Ns.append(N)
            Ks.append(K)
        _, Xh, _ = synth.layer_inputs(cfg["workload_id"], 100 * M + 50, M, 1, cfg["hidden"])
        _, Xm, _ = synth.layer_inputs(cfg["workload_id"], 100 * M + 51, M, 1, cfg["mlp"])
        Xh, Xm = torch.from_numpy(Xh).cuda(), torch.from_numpy(Xm).cuda()
        Ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N in Ns]
        nbytes = sum(effective_bytes(M, N, K, cfg["fmt"]) for N, K in zip(Ns, Ks))
        F = cfg["fmt"]
        ctr = [0]

        def one(i, Xi):
            c = ctr[0] % copies
            tri.tri_linear(Xi, pools[i][c], scales[i], M, Ns[i], Ks[i], F, Ys[i])

        def step7():
            for i in range(7):
                one(i, Xm if i == 6 else Xh)
            ctr[0] += 1

        def group(ids, Xi):
            c = ctr[0] % copies
            tri.tri_linear_grouped(Xi, [pools[i][c] for i in ids], [scales[i] for i in ids], M, [Ns[i] for i in ids],
                                   Ks[ids[0]], F, [Ys[i] for i in ids])

        def step4():
            group([0, 1, 2], Xh)
            one(3, Xh)
            group([4, 5], Xh)
            one(6, Xm)
            ctr[0] += 1

        # the whole block with its glue on the GPU, folded into four fused launches: RMSNorm into
        # Q/K/V and into gate/up, the residual into O and down, the silu gate into the gate/up
        # launch (one workgroup serves the same rows of both and writes silu(gate) * up)
        Yq = [Ys[0], Ys[1], Ys[2]]
        Yh = torch.empty((M, cfg["hidden"]), dtype=torch.float16, device="cuda")
        Ya = torch.empty((M, cfg["mlp"]), dtype=torch.float16, device="cuda")
        Yout = torch.empty_like(Yh)

        def fused(ids, Xi, Ys_, norm=False, pair=False, res=None):
            c = ctr[0] % copies
            tri.tri_linear_fused(Xi, [pools[i][c] for i in ids], [scales[i] for i in ids], M, [Ns[i] for i in ids],
                                 Ks[ids[0]], F, Ys_, norm=norm, eps=1e-5, pair=pair, residuals=res)

        def step_glue():
            fused([0, 1, 2], Xh, Yq, norm=True)
            fused([3], Ys[2], [Yh], res=[Xh])
            fused([4, 5], Yh, [Ya, None], norm=True, pair=True)
            fused([6], Ya, [Yout], res=[Yh])
            ctr[0] += 1

        # each variant: a HIP graph of `copies` steps (every step on other weight copies), replayed
        t7 = graph_time(step7, copies)
        t4 = graph_time(step4, copies)
        tg = graph_time(step_glue, copies)
        res.append({"M": M, "bytes": nbytes,
                    "separate": {"launches": 7, "step_us": round(t7 * 1e6, 3), "GBps": round(nbytes / t7 / 1e9, 1),
                                 "frac_hbm": round(nbytes / t7 / 1e9 / HBM_PEAK_GBS, 4)},
                    "grouped": {"launches": 4, "step_us": round(t4 * 1e6, 3), "GBps": round(nbytes / t4 / 1e9, 1),
                                "frac_hbm": round(nbytes / t4 / 1e9 / HBM_PEAK_GBS, 4)},
                    "fused_with_glue": {"launches": 4, "step_us": round(tg * 1e6, 3),
                                        "GBps": round(nbytes / tg / 1e9, 1),
                                        "frac_hbm": round(nbytes / tg / 1e9 / HBM_PEAK_GBS, 4)}})
        del pools
        torch.cuda.empty_cache()
    return res


def bench_prefill(clock):
    import torch
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.PREFILL
    res = []
    for fmt in cfg["fmts"]:
        for li, (name, K, N) in enumerate(cfg["shapes"]):
            L = Layer(cfg["workload_id"], li, cfg["M"], N, K, fmt, cfg["scale"], copies=1)
            # the GEMM is compute-bound: after idle time the GPU runs it at a lower clock for tens of
            # milliseconds, so it runs back to back for half a second before it is timed (the
            # sustained rate of a long prefill)
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.5:
                for _ in range(8):
                    L.launch()
                torch.cuda.synchronize()
            # (timed with plain events: a launch takes ~1 ms, far longer than the host needs to queue
            # it, and an idle sleep kernel in front would let the clock drop again)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(20):
                L.launch()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / 20
            tf = L.flops / t / 1e12
            res.append({"shape": name, "M": cfg["M"], "format": configs.FMT_NAMES[fmt], "kernel_us": round(t * 1e6, 2),
                        "TFLOPs": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                        "timing": "events around 20 back-to-back launches, after 0.5 s of the same GEMM"})
            del L
            torch.cuda.empty_cache()
    return res


def bench_quantize(clock):
    """tri_quantize on the prefill matrices (235M latent float32 weights each): the weights are read
    twice (mean |w|, then the trits), the packed bytes written once."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs, synth
    cfg = configs.PREFILL
    res = []
    for fmt in cfg["fmts"]:
        K, N = cfg["shapes"][0][1], cfg["shapes"][0][2]
        W = torch.from_numpy(synth.latent_weights(synth.rng_for(cfg["workload_id"], 90 + fmt, synth.STREAM_LATENT),
                                                  N, K)).cuda()
        Wp = torch.empty((N, tri.tri_row_bytes(K, fmt)), dtype=torch.uint8, device="cuda")
        scale = torch.empty(1, dtype=torch.float32, device="cuda")
        nws = tri.tri_quantize_workspace_bytes(N, K)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        t, _ = clock.run([lambda: tri.tri_quantize(W, N, K, fmt, Wp, scale, ws, nws)] * 10, warmup=2)
        nbytes = 2 * 4 * N * K + Wp.numel()
        res.append({"shape": "%dx%d" % (N, K), "format": configs.FMT_NAMES[fmt], "us": round(t * 1e6, 1),
                    "bytes": nbytes, "GBps": round(nbytes / t / 1e9, 1),
                    "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
        del W, Wp, ws
        torch.cuda.empty_cache()
    return res


def bench_floor(clock):
    """Where a decode launch's time goes (M = 1, 2-bit, the three decode shapes, cold weights):
    the decode kernel against (a) an empty kernel on the decode kernel's grid (the fixed cost of a
    launch of that many workgroups), (b) the decode kernel's loads alone on the same grid
    (tri_probe_rows: the same weight chunks per lane and the same activation loads, no decode,
    contraction, reduction or epilogue), (c) streaming reads of the same bytes: the one-load-per-
    thread grid (tri_probe_read) and resident grids of 256..2048 workgroups keeping 1..8 loads in
    flight per lane (tri_probe_stream; the best of them is the read floor).  Every figure is the
    mean per launch of 200 back-to-back launches, timed two ways: HIP events around a sleep-held
    queue (launch gaps of an in-order stream included) and a replayed HIP graph of the 200."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    F2 = tri.TRI_FMT_2BIT
    cfg = configs.DECODE
    reps = 200

    def both(calls):
        t_ev, _ = clock.run(calls)
        k = [0]

        def step():
            calls[k[0] % len(calls)]()
            k[0] += 1
        t_gr = graph_time(step, len(calls), replays=3)
        return round(t_ev * 1e6, 3), round(t_gr * 1e6, 3)

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = []
    for li, (name, K, N) in enumerate(cfg["shapes"]):
        L = Layer(cfg["workload_id"], li, 1, N, K, F2)
        wg = (N + 15) // 16
        nb = N * tri.tri_row_bytes(K, F2)
        Yp = torch.empty(N, dtype=torch.float16, device="cuda")
        rec = {"shape": name, "K": K, "N": N, "weight_bytes": nb, "workgroups": wg, "threads": 512}
        rec["decode_us"] = both([L.launch] * reps)
        rec["empty_same_grid_us"] = both([lambda: tri.tri_probe_empty(wg, 512, sink)] * reps)
        rec["empty_one_wave_us"] = both([lambda: tri.tri_probe_empty(1, 64, sink)] * reps)
        ctr = [0]

        def rows():
            Wp = L.pool[ctr[0] % L.pool.shape[0]]
            ctr[0] += 1
            tri.tri_probe_rows(L.X, Wp, N, K, F2, 8, Yp)
        rec["loads_only_us"] = both([rows] * reps)
        del L
        torch.cuda.empty_cache()
        ncopies = max(1, -(-(1 << 30) // nb))
        pool = torch.empty((ncopies, nb), dtype=torch.uint8, device="cuda")
        pool.fill_(1)
        c2 = [0]

        def rd():
            tri.tri_probe_read(pool[c2[0] % ncopies], nb, sink)
            c2[0] += 1
        rec["read_grid_stride_us"] = both([rd] * reps)
        best = None
        sweep = []
        for wgs in (256, 512, 1024, 2048):
            for u in (1, 2, 4, 8):
                if wgs * 256 * u * 16 > 4 * nb:
                    continue

                def st(wgs=wgs, u=u):
                    tri.tri_probe_stream(pool[c2[0] % ncopies], nb, wgs, u, sink)
                    c2[0] += 1
                t = both([st] * reps)
                sweep.append({"workgroups": wgs, "unroll": u, "us": t})
                if best is None or t[0] < best["us"][0]:
                    best = sweep[-1]
        rec["stream_sweep"] = sweep
        rec["stream_best"] = best
        del pool
        torch.cuda.empty_cache()
        out.append(rec)
        log("floor", json.dumps(rec))
    return out


def profile_mode(which):
    """Launch one workload a few times and exit (for rocprofv3 counter passes)."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    if which == "decode":
        cfg = configs.DECODE
        for fmt in (tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT):
            layers = [Layer(cfg["workload_id"], li + (0 if fmt == tri.TRI_FMT_2BIT else 20), 1, N, K, fmt)
                      for li, (name, K, N) in enumerate(cfg["shapes"])]
            for _ in range(20):
                for L in layers:
                    L.launch()
            torch.cuda.synchronize()
            del layers
            torch.cuda.empty_cache()
    elif which == "block":
        bench_block(Clock())
    elif which == "prefill":
        cfg = configs.PREFILL
        name, K, N = cfg["shapes"][0]
        for fmt in cfg["fmts"]:
            L = Layer(cfg["workload_id"], 0, cfg["M"], N, K, fmt, scale=cfg["scale"], copies=1)
            for _ in range(3):
                L.launch()
            torch.cuda.synchronize()
            del L
            torch.cuda.empty_cache()
    elif which == "batched":
        cfg = configs.BATCHED
        for fmt in cfg["fmts"]:
            for li, (name, K, N) in enumerate(cfg["shapes"]):
                for M in (8, 16):
                    L = Layer(cfg["workload_id"], 10 * li + M, M, N, K, fmt, copies=8)
                    for _ in range(10):
                        L.launch()
                    torch.cuda.synchronize()
                    del L
                    torch.cuda.empty_cache()
    elif which == "floor":
        bench_floor(Clock())
    elif which == "copy":
        nb = 64 << 20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            tri.tri_probe_copy(src, dst, nb)
    torch.cuda.synchronize()
    log("profile run done:", which)


if __name__ == "__main__":
    main()
