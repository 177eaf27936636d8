#!/usr/bin/env python3
"""Benchmark of the ternary linear layer on one MI355X (gfx950).

Headline workload: decode GEMV at M = 1 with 2-bit packed ternary weights, the
three projections of a LLaMA-style block at hidden 4096 / MLP 11008
(4096x4096, 4096->11008, 11008->4096).  One step = the three tri_linear launches
on fresh (cold) weights: each step reads a different copy of every packed
matrix from a pool of >= 1 GiB, so the 256 MB Infinity Cache cannot serve them.
The value is effective HBM bandwidth: (packed weights as stored + fp16 X read +
fp16 Y written) per step / wall time per step, inputs resident in HBM.

The same JSON line also carries the roofline fraction of the GEMV kernel
(HIP-event-timed launch durations), the size-matched streaming-read floor, the
CPU oracle timed on this host, and the batched-decode and prefill workloads.

  python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--skip-extra] [--skip-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6   # MI355X dense fp16 MFMA peak (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "effective HBM GB/s (% of peak) for M=1 ternary GEMV; prefill GEMM TFLOP/s (% MFMA)"
POOL_BYTES = 1 << 30            # rotate every weight matrix over >= 1 GiB of copies


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def effective_bytes(M, N, K, fmt):
    import bit_mixed_precision_tri_amd as tri
    return N * tri.tri_row_bytes(K, fmt) + 2 * M * K + 2 * M * N


class Layer:
    """One ternary linear on the GPU with a rotating pool of packed-weight copies."""

    def __init__(self, workload_id, layer_id, M, N, K, fmt, scale=None, pool_bytes=POOL_BYTES, max_copies=64):
        import torch
        import bit_mixed_precision_tri_amd as tri
        from bit_mixed_precision_tri_amd import synth
        self.M, self.N, self.K, self.fmt = M, N, K, fmt
        W, X, self.scale = synth.layer_inputs(workload_id, layer_id, M, N, K, scale)
        Wp = tri.pack(torch.from_numpy(W).cuda(), fmt)
        self.S = Wp.shape[1]
        ncopies = max(1, min(max_copies, -(-pool_bytes // Wp.numel())))
        self.pool = torch.empty((ncopies,) + tuple(Wp.shape), dtype=torch.uint8, device="cuda")
        self.pool[:] = Wp                       # distinct addresses, same content
        self.X = torch.from_numpy(X).cuda()
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


def time_launches(layer, reps, warmup, algo=0):
    """Average kernel duration (s) from HIP events around each launch, cold weights."""
    import torch
    for _ in range(warmup):
        layer.launch(algo)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        layer.launch(algo)
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps / 1e3


def read_floor(nbytes, reps=200):
    """Size-matched streaming read (tri_probe_read) over a rotating >= 1 GiB pool: average duration (s)."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    nb = (nbytes + 15) // 16 * 16
    ncopies = max(1, -(-POOL_BYTES // nb))
    pool = torch.empty((ncopies, nb), dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for i in range(20):
        tri.tri_probe_read(pool[i % ncopies], nb, sink)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        tri.tri_probe_read(pool[i % ncopies], nb, sink)
        b.record()
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in evs) / reps / 1e3
    del pool
    torch.cuda.empty_cache()
    return t


def counters_for(kernel_file):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", "decode_gemv2_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "bit_mixed_precision_tri_amd", "csrc", kernel_file), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None                     # the kernel changed since the counters were taken
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
    return {"value": round(total_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "full decode step (3 shapes, M=1, 2-bit: unpack + float64 layer), median of %d runs, "
                      "%.3f s per step" % (len(times), t)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-extra", action="store_true", help="skip the batched-decode and prefill workloads")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", choices=["decode", "batched", "prefill", "copy"],
                    help="only launch one workload a few times (for rocprofv3 runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the ternary linear layer on one GPU only; --gpus %d is not supported"
              % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tri.lib()
    torch.cuda.set_device(0)
    F2, F16 = tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT

    if args.profile:
        return profile_mode(args.profile)

    # ---- headline: decode GEMV, M = 1, 2-bit, three shapes, cold weights
    dcfg = configs.DECODE
    layers = [Layer(dcfg["workload_id"], li, 1, N, K, F2) for li, (name, K, N) in enumerate(dcfg["shapes"])]
    step_bytes = sum(L.bytes for L in layers)
    for _ in range(args.warmup):
        for L in layers:
            L.launch()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in layers]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for step in range(args.steps):
        for L, (a, b) in zip(layers, evs[step]):
            a.record()
            L.launch()
            b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_launch = [sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)) / args.steps / 1e3
                  for i in range(len(layers))]
    value = step_bytes * args.steps / elapsed / 1e9
    achieved = step_bytes / sum(per_launch) / 1e9
    shapes_out = []
    for (name, K, N), L, t in zip(dcfg["shapes"], layers, per_launch):
        shapes_out.append({"shape": name, "K": K, "N": N, "bytes": L.bytes, "kernel_us": round(t * 1e6, 3),
                           "GBps": round(L.bytes / t / 1e9, 1),
                           "algo": tri.ALGO_NAMES[tri.tri_select_algo(1, N, K, F2)]})
    # the smallm MFMA kernel at M = 1, same shapes (kernel choice evidence)
    for so, L in zip(shapes_out, layers):
        t = time_launches(L, 100, 10, algo=tri.TRI_ALGO_SMALLM)
        so["smallm_kernel_us"] = round(t * 1e6, 3)
        so["smallm_GBps"] = round(L.bytes / t / 1e9, 1)
    del layers
    torch.cuda.empty_cache()
    floors = []
    for (name, K, N) in dcfg["shapes"]:
        nb = N * tri.tri_row_bytes(K, F2)
        t = read_floor(nb)
        floors.append({"shape": name, "bytes": nb, "read_us": round(t * 1e6, 3), "GBps": round(nb / t / 1e9, 1)})
    ctr = counters_for("tri_gemv.hip")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "accumulate": "f32", "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1, 2-bit packed ternary weights, shapes 4096x4096 + 4096->11008 + "
                               "11008->4096 per step, weights cold (rotating >= 1 GiB pool)",
                   "M": 1, "shapes": [[K, N] for (_, K, N) in dcfg["shapes"]], "format": "2bit",
                   "bytes_per_step": step_bytes},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gemv2 (tri_gemv.hip)", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (ctr or {}).get("traffic_bytes_per_step")},
        "per_shape": shapes_out,
        "read_floor": floors,
    }
    if not args.skip_extra:
        out["batched"] = bench_batched()
        out["prefill"] = bench_prefill()
    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline(dcfg["shapes"])
    print(json.dumps(out), flush=True)


def bench_batched():
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.BATCHED
    res = []
    for fmt in cfg["fmts"]:
        for li, (name, K, N) in enumerate(cfg["shapes"]):
            for M in cfg["Ms"]:
                L = Layer(cfg["workload_id"], 10 * li + M, M, N, K, fmt)
                t = time_launches(L, 100, 10)
                res.append({"shape": name, "M": M, "format": configs.FMT_NAMES[fmt], "kernel_us": round(t * 1e6, 3),
                            "GBps": round(L.bytes / t / 1e9, 1), "frac_hbm": round(L.bytes / t / 1e9 / HBM_PEAK_GBS, 4)})
                del L
                torch.cuda.empty_cache()
    return res


def bench_prefill():
    import torch
    from bit_mixed_precision_tri_amd import configs
    cfg = configs.PREFILL
    res = []
    for fmt in cfg["fmts"]:
        for li, (name, K, N) in enumerate(cfg["shapes"]):
            L = Layer(cfg["workload_id"], li, cfg["M"], N, K, fmt, cfg["scale"], pool_bytes=0, max_copies=1)
            t = time_launches(L, 10, 2)
            tf = L.flops / t / 1e12
            res.append({"shape": name, "M": cfg["M"], "format": configs.FMT_NAMES[fmt], "kernel_us": round(t * 1e6, 2),
                        "TFLOPs": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
            del L
            torch.cuda.empty_cache()
    return res


def profile_mode(which):
    """Launch one workload a few times and exit (for rocprofv3 --kernel-trace / --pmc)."""
    import torch
    import bit_mixed_precision_tri_amd as tri
    from bit_mixed_precision_tri_amd import configs
    F2 = tri.TRI_FMT_2BIT
    if which == "decode":
        cfg = configs.DECODE
        layers = [Layer(cfg["workload_id"], li, 1, N, K, F2) for li, (name, K, N) in enumerate(cfg["shapes"])]
        for _ in range(20):
            for L in layers:
                L.launch()
    elif which == "batched":
        return bench_batched()
    elif which == "prefill":
        return bench_prefill()
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
