"""Benchmark of the BATQuant W4A4 hot path on one MI355X.

One step = the whole online path for one batch: the fused activation block
transform + clip + MXFP4 quantisation kernel followed by the W4A4 MXFP4 GEMM
(bf16 output).  The weight side (P^-1 W^T, clip, quantise) is offline and runs
once before timing.  Default workload: the up/gate projection prefill layer,
X 2048 x 4096 bf16 and W 12288 x 4096 bf16, shared factor 8x8 / private 4x4.

Inputs are resident in HBM when timing starts.  Steps rotate through several
copies of every buffer (more bytes than the 256 MB Infinity Cache) so a step
cannot be served from the cache a previous step filled.

Prints ONE JSON line.  ``value`` is the step throughput in TFLOP/s of W4A4 GEMM
work (2 M N K per step) including the activation kernel's time.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MXFP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix, published
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 matrix, published: the FP8 x FP4 MFMA's rate
METRIC = "transform+MXFP4-quant GB/s (% HBM peak); MXFP4 GEMM TFLOPS (% MFMA peak)"
METRIC_W4A8 = "transform+MXFP8-quant GB/s (% HBM peak); MXFP8 x MXFP4 GEMM TFLOP/s (% MFMA peak)"
METRIC_KV = "KV-cache write (per-head transform + MX quant into cache slots) GB/s (% HBM peak)"
METRIC_DECODE = "fused decode step (transform+MXFP4 quant in the GEMM prologue) GB/s (% HBM peak)"
CACHE_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--a", type=int, default=8, help="shared factor size (config 5 sweep)")
    ap.add_argument("--factors", choices=["gpk", "hadamard"], default="gpk",
                    help="transform factors: seeded near-identity GPK, or the block-Hadamard rotation (BRQ)")
    ap.add_argument("--no-clip", action="store_true", help="no block-wise clipping (activations and weights)")
    ap.add_argument("--gemm", choices=["packed", "unpacked"], default="packed",
                    help="weight operand layout of the GEMM (packed: lane-ordered, prepared offline)")
    ap.add_argument("--act-format", choices=["mxfp4", "mxfp8"], default="mxfp4",
                    help="activation format: mxfp4 (W4A4) or mxfp8 (W4A8, E4M3; packed GEMM only)")
    ap.add_argument("--decode", action="store_true",
                    help="fused decode step (w4a4_decode: activation path inside the GEMM), M <= 32 (config 4)")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: replay the steps from a captured HIP graph (no host launch overhead)")
    ap.add_argument("--kv-cache", type=int, choices=[4, 8], default=None,
                    help="KV-cache write of the config's tokens, 8 heads x 128 channels, MXFP4 (4) or MXFP8 (8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB -> 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="minimum oracle time for the CPU baseline")
    return ap.parse_args()


def kernel_source_digest(name: str, text_of=None, headers=None) -> str:
    """sha256[:16] of a kernel source plus the shared headers (every .h in
    csrc/), with comments and blank space removed: a comment edit keeps a
    counter summary valid, any code change invalidates it."""
    def read(rel):
        if text_of is not None:
            return text_of(rel)
        with open(os.path.join(ROOT, "w4a4_bit_gemm_amd", "csrc", rel)) as f:
            return f.read()

    if headers is None:
        headers = sorted(os.path.basename(h) for h in
                         __import__("glob").glob(os.path.join(ROOT, "w4a4_bit_gemm_amd", "csrc", "*.h")))
    parts = []
    for rel in [name] + list(headers):
        t = re.sub(r"/\*.*?\*/", "", read(rel), flags=re.S)
        t = re.sub(r"//[^\n]*", "", t)
        parts.append("\n".join(ln.strip() for ln in t.splitlines() if ln.strip()))
    return hashlib.sha256("\n\0\n".join(parts).encode()).hexdigest()[:16]


def load_traffic(kernel_file: str, kernel: str, workload: str):
    """HBM bytes per launch (fetched + written, calibrated) from the committed
    rocprofv3 counter summary, only if it was taken on the current kernel
    source, for this kernel instance and workload."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_digest(kernel_file)
    with open(path) as f:
        for ln in f:
            parts = ln.split()
            if ln.startswith("#") or len(parts) != 6:
                continue
            if parts[0] == kernel_file and parts[1] == kernel and parts[2] == want and parts[5] == workload:
                return float(parts[3]) + float(parts[4])
    return None


def cpu_baseline(wl, min_seconds: float, fmt: str = "e2m1"):
    """The oracle, as it stands, on the same workload: the whole step (every
    token row through the activation path, then the full GEMM against every
    prepared weight row), repeated until ``min_seconds`` have passed."""
    import threadpoolctl

    from oracle import batquant as ob

    wprep = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)  # offline, untimed
    reps, t_act, t_gemm = 0, 0.0, 0.0
    while reps == 0 or (t_act + t_gemm < min_seconds and reps < 8):
        t0 = time.perf_counter()
        x = ob.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta, fmt=fmt)
        t1 = time.perf_counter()
        ob.gemm(x.codes, x.scales, wprep.codes, wprep.scales, x_fmt=fmt)
        t2 = time.perf_counter()
        t_act += t1 - t0
        t_gemm += t2 - t1
        reps += 1
    flops = 2.0 * wl.M * wl.N * wl.K
    info = threadpoolctl.threadpool_info()
    blas_threads = max([d.get("num_threads", 1) for d in info] or [1])
    return {
        "value": flops * reps / (t_act + t_gemm) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"the full step ({wl.M} token rows through the fp64 oracle activation path, then the "
                   f"{wl.M}x{wl.N}x{wl.K} dequantised fp64 GEMM), {reps} repetition(s): activation "
                   f"{t_act / reps:.2f} s, GEMM {t_gemm / reps:.2f} s per step; weight preparation offline "
                   f"and untimed; BLAS threads {blas_threads}, host cores visible "
                   f"{len(os.sched_getaffinity(0))}"),
        "seconds_measured": t_act + t_gemm,
        "steps_per_second": reps / (t_act + t_gemm),
    }


def run_decode(args, torch, w, wl, dev):
    """The fused decode step: one w4a4_decode call (the activation transform,
    clip and MXFP4 quantisation run inside the GEMM kernel; a second small
    launch sums its K splits).  Bound: HBM (the packed weights are read once
    per step).  Buffers rotate over enough sets that every step reads its
    weights from HBM."""
    M, K, N = wl.M, wl.K, wl.N
    if M > w.DECODE_MAX_M:
        print(f"--decode needs M <= {w.DECODE_MAX_M} (config 4); config {args.config} has M = {M}", file=sys.stderr)
        sys.exit(2)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if args.factors == "hadamard":
        wl.A, wl.B = gen.hadamard_factors(K, wl.a)
    if args.no_clip:
        wl.alpha = wl.beta = wl.walpha = wl.wbeta = None
    A, B = f32(wl.A), f32(wl.B)
    rh = None if args.no_clip else f32(w.clip_ratios(wl.alpha))
    rl = None if args.no_clip else f32(w.clip_ratios(wl.beta))
    Wq0, Ws0 = w.prepare_weight(bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)  # offline
    Wp0 = w.weight_pack(Wq0, Ws0)
    X0 = bf16(wl.X_bits)
    ws = w.decode_workspace(M, N, K, dev)
    wp_bytes = Wp0.data.numel()
    set_bytes = M * K * 2 + wp_bytes + M * N * 2
    nsets = min(64, max(2, int(np.ceil(2.2 * CACHE_BYTES / set_bytes))))
    sets = [dict(X=X0.clone(), Wp=w.PackedWeight(Wp0.data.clone(), N, K),
                 Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    torch.cuda.synchronize()

    def step(i):
        st = sets[i % nsets]
        w.w4a4_decode(st["X"], A, B, rh, rl, st["Wp"], ws, out=st["Y"])

    steps = args.steps
    if args.graph:
        # one captured graph holds one step per buffer set; the timed steps are
        # a whole number of replays
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            for i in range(nsets):
                step(i)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cs):
                for i in range(nsets):
                    step(i)
        torch.cuda.synchronize()
        reps = -(-steps // nsets)
        steps = reps * nsets
        run = lambda: [g.replay() for _ in range(reps)]
        for _ in range(max(1, -(-args.warmup // nsets))):
            g.replay()
    else:
        run = lambda: [step(i) for i in range(steps)]
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = e0.elapsed_time(e1) * 1e-3 / steps  # GPU time per step, events on the launch stream
    alg_bytes = M * K * 2 + wp_bytes + M * N * 2  # X read, packed weights read, Y written
    gbs = alg_bytes / t_step / 1e9
    out = {
        "metric": METRIC_DECODE,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: X {M}x{K} bf16 ({wl.meta['x_kind']}, {wl.meta['outliers']}), W {N}x{K} bf16 "
                        f"N(0,0.02) prepared and packed offline; step = one fused decode launch pair "
                        f"({'graph replay' if args.graph else 'eager launches'})",
            "M": M, "K": K, "N": N, "a": wl.a, "b": wl.b, "buffer_sets": nsets, "graph": args.graph,
            "factors": args.factors, "clip": not args.no_clip,
        },
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_partial_kernel + decode_reduce_kernel (one step)"},
        "kernels": {"decode_step": {"us": t_step * 1e6, "GB/s": gbs, "algorithmic_bytes": alg_bytes,
                                    "TFLOP/s": 2.0 * M * N * K / t_step / 1e12}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_min_seconds)
        cb["value"] = alg_bytes * cb["steps_per_second"] / 1e9
        cb["unit"] = "GB/s"
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


def run_kv(args, torch, w, wl, dev):
    """KV-cache write: the config's tokens, 8 KV heads x 128 channels (the
    key/value width of the pages' 8B model layers), through the per-head block
    transform, clipping and MXFP4 / MXFP8 quantisation into permuted slots of a
    cache four times as long.  Bound: HBM."""
    from workloads import gen

    T, HD = wl.M, 8 * 128
    kv = gen.make_custom(T, HD, 8, seed=1000 * args.config + 77)
    fmt = args.kv_cache
    rows = 4 * T

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    X0 = torch.from_numpy(np.ascontiguousarray(kv.X_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    A, B = f32(kv.A), f32(kv.B)
    rh = None if args.no_clip else f32(w.clip_ratios(kv.alpha))
    rl = None if args.no_clip else f32(w.clip_ratios(kv.beta))
    qcols = HD // 2 if fmt == 4 else HD
    set_bytes = T * HD * 2 + rows * (qcols + HD // 32)
    nsets = min(64, max(2, int(np.ceil(2.2 * CACHE_BYTES / set_bytes))))
    rng = np.random.default_rng(5)
    sets = [dict(X=X0.clone(), slots=torch.from_numpy(rng.permutation(rows)[:T].astype(np.int64)).to(dev),
                 q=torch.zeros((rows, qcols), dtype=torch.uint8, device=dev),
                 s=torch.zeros((rows, HD // 32), dtype=torch.uint8, device=dev)) for _ in range(nsets)]

    def step(i):
        st = sets[i % nsets]
        w.kv_cache_quant(st["X"], A, B, rh, rl, st["slots"], st["q"], st["s"], fmt=fmt)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = e0.elapsed_time(e1) * 1e-3 / args.steps
    alg_bytes = T * HD * 2 + T * (qcols + HD // 32) + T * 8  # rows read, codes + scales written, slots read
    gbs = alg_bytes / t_step / 1e9
    kv_kernel = f"kv_cache_quant_kernel<{'true' if fmt == 8 else 'false'}>"
    out = {
        "metric": METRIC_KV, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4" if fmt == 4 else "mxfp8", "data": "synthetic",
        "config": {"workload": f"KV-cache write: {T} tokens x {HD} channels (8 heads x 128) bf16 (t3), GPK a=8 b=4, "
                               f"{'MXFP4' if fmt == 4 else 'MXFP8 E4M3'} into permuted slots of a {rows}-row cache",
                   "T": T, "HD": HD, "cache_rows": rows, "fmt": fmt, "buffer_sets": nsets, "clip": not args.no_clip},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic("transform_quant.hip", kv_kernel, f"kv{fmt}_{T}x{HD}"),
                     "kernel": kv_kernel},
        "kernels": {"kv_cache_quant": {"us": t_step * 1e6, "GB/s": gbs, "algorithmic_bytes": alg_bytes}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import batquant as ob

        t_start, reps = time.perf_counter(), 0
        while reps == 0 or (time.perf_counter() - t_start < args.cpu_min_seconds and reps < 8):
            ob.kv_cache_quant(kv.X_bits, kv.A, kv.B, None if args.no_clip else kv.alpha,
                              None if args.no_clip else kv.beta, fmt="e2m1" if fmt == 4 else "e4m3")
            reps += 1
        dt = (time.perf_counter() - t_start) / reps
        import threadpoolctl

        cores = max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": alg_bytes / dt / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
                               "sample": f"the full write ({T} rows through the fp64 oracle path), {reps} repetition(s), "
                                         f"{dt:.2f} s each"}
    print(json.dumps(out), flush=True)


def calibrate_copy(torch, dev, steps):
    """A plain elementwise copy of known size (fp32 negation: reads 1 GiB, writes
    1 GiB per launch), profiled with the same HBM counters as the kernels so
    that their readings can be scaled to bytes."""
    n = 2 ** 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"calibration": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": 2 * steps, "GB/s": 8 * n / dt / 1e9}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    fp8 = args.act_format == "mxfp8"
    if fp8 and args.gemm != "packed":
        print("--act-format mxfp8 runs on the packed GEMM only", file=sys.stderr)
        sys.exit(2)
    import torch

    import w4a4_bit_gemm_amd as w
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.steps)
        return
    wl = gen.make_workload(args.config, a=args.a)
    M, K, N = wl.M, wl.K, wl.N
    if args.decode:
        run_decode(args, torch, w, wl, dev)
        return
    if args.kv_cache:
        run_kv(args, torch, w, wl, dev)
        return

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if args.factors == "hadamard":
        wl.A, wl.B = gen.hadamard_factors(K, wl.a)
    if args.no_clip:
        wl.alpha = wl.beta = wl.walpha = wl.wbeta = None
    X0 = bf16(wl.X_bits)
    A = f32(wl.A)
    B = f32(wl.B)
    rh = None if args.no_clip else f32(w.clip_ratios(wl.alpha))
    rl = None if args.no_clip else f32(w.clip_ratios(wl.beta))
    Wq0, Ws0 = w.prepare_weight(bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)  # offline
    packed = args.gemm == "packed"
    Wp0 = w.weight_pack(Wq0, Ws0) if packed else None  # offline
    torch.cuda.synchronize()

    xq_row = K if fp8 else K // 2  # activation code bytes per row
    set_bytes = M * K * 2 + M * xq_row + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2
    nsets = max(2, int(np.ceil(2.2 * CACHE_BYTES / set_bytes)))
    nsets = min(nsets, 64)
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            X=X0.clone(),
            Wq=None if packed else Wq0.clone(), Ws=None if packed else Ws0.clone(),
            Wp=w.PackedWeight(Wp0.data.clone(), N, K) if packed else None,
            Xq=torch.empty((M, xq_row), dtype=torch.uint8, device=dev),
            Xs=torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
            Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()

    def act(i):
        s = sets[i % nsets]
        (w.act_transform_quant_mxfp8 if fp8 else w.act_transform_quant)(s["X"], A, B, rh, rl, out=(s["Xq"], s["Xs"]))

    def gemm(i):
        s = sets[i % nsets]
        if fp8:
            w.mxfp8_gemm_packed(s["Xq"], s["Xs"], s["Wp"], out=s["Y"])
        elif packed:
            w.mxfp4_gemm_packed(s["Xq"], s["Xs"], s["Wp"], out=s["Y"])
        else:
            w.mxfp4_gemm(s["Xq"], s["Xs"], s["Wq"], s["Ws"], out=s["Y"])

    def step(i):
        act(i)
        gemm(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps between two synchronisations
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-kernel launch durations inside the step: a second pass over the same
    # `steps` steps with a HIP event before the transform, one between the two
    # kernels and one after the GEMM, all recorded on the stream the kernels
    # are launched on (torch's current stream).  The events stay out of the
    # timed region above.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[3 * i].record()
        act(i)
        evs[3 * i + 1].record()
        gemm(i)
        evs[3 * i + 2].record()
    torch.cuda.synchronize()
    t_act = np.array([evs[3 * i].elapsed_time(evs[3 * i + 1]) for i in range(args.steps)]) * 1e-3
    t_gemm = np.array([evs[3 * i + 1].elapsed_time(evs[3 * i + 2]) for i in range(args.steps)]) * 1e-3

    flops = 2.0 * M * N * K
    act_bytes = M * K * 2 + M * xq_row + M * K // 32  # algorithmic: read bf16, write codes + scales
    gemm_bytes = M * xq_row + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2
    mma_peak = FP8_PEAK_TFLOPS if fp8 else MXFP4_PEAK_TFLOPS
    act_gbs = act_bytes / t_act.mean() / 1e9
    gemm_tflops = flops / t_gemm.mean() / 1e12
    ai = flops / gemm_bytes
    gemm_hbm_bound = ai < mma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gemm_hbm_bound:
        gemm_roof = {"bound": "hbm", "achieved": gemm_bytes / t_gemm.mean() / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s"}
    else:
        gemm_roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": mma_peak, "unit": "TFLOP/s"}
    gemm_roof["frac"] = gemm_roof["achieved"] / gemm_roof["peak"]
    act_roof = {"bound": "hbm", "achieved": act_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": act_gbs / HBM_PEAK_GBS}
    dominant_is_gemm = t_gemm.mean() >= t_act.mean()
    roof = dict(gemm_roof if dominant_is_gemm else act_roof)
    nst = K // 256
    gs = "true" if nst % 4 == 0 else "false"
    a8 = "true" if fp8 else "false"
    if not packed:
        gemm_src, gemm_kernel = "mxfp4_gemm.hip", "mxfp4_gemm_dma_kernel"
    elif w.packed_gemm_kernel(M, N, K, fp8) == 1:  # the library's own choice for this shape
        gemm_src = "mxfp4_gemm_packed_dma.hip"
        gemm_kernel = f"{'w4a8' if fp8 else 'mxfp4'}_gemm_packed_dma_kernel<{nst}>"
    else:
        gemm_src = "mxfp4_gemm_packed.hip"
        gemm_kernel = f"mxfp4_gemm_packed_kernel<{nst if nst in (1, 2, 4, 8, 16, 48) else 0},{gs},{a8}>"
    act_kernel = f"transform_quant_kernel<false,{a8}>"
    act_roof["traffic"] = load_traffic("transform_quant.hip", act_kernel, wl.name)
    gemm_roof["traffic"] = load_traffic(gemm_src, gemm_kernel, wl.name)
    roof["traffic"] = gemm_roof["traffic"] if dominant_is_gemm else act_roof["traffic"]
    roof["kernel"] = gemm_kernel if dominant_is_gemm else act_kernel

    out = {
        "metric": METRIC_W4A8 if fp8 else METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8xmxfp4" if fp8 else "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: X {M}x{K} bf16 ({wl.meta['x_kind']}, {wl.meta['outliers']}), "
                        f"W {N}x{K} bf16 N(0,0.02) prepared offline ({args.gemm} MXFP4); "
                        f"{'MXFP8 (E4M3) activations; ' if fp8 else ''}"
                        f"{'block-Hadamard (BRQ) factors' if args.factors == 'hadamard' else 'GPK'} a={wl.a} b={wl.b}"
                        f"{', no clipping' if args.no_clip else ''}; "
                        f"step = act transform+clip+{args.act_format.upper()} quant + GEMM (bf16 out)",
            "M": M, "K": K, "N": N, "a": wl.a, "b": wl.b, "buffer_sets": nsets, "gemm": args.gemm,
            "factors": args.factors, "clip": not args.no_clip, "act_format": args.act_format,
        },
        "roofline": roof,
        "kernels": {
            "transform_quant": {"us": float(t_act.mean() * 1e6), "GB/s": act_gbs,
                                "frac_hbm": act_gbs / HBM_PEAK_GBS, "algorithmic_bytes": act_bytes,
                                "roofline": act_roof},
            "gemm": {"kernel": gemm_kernel, "us": float(t_gemm.mean() * 1e6), "TFLOP/s": gemm_tflops,
                     "frac_mfma": gemm_tflops / mma_peak, "flops": flops,
                     "operand_output_bytes": gemm_bytes, "roofline": gemm_roof},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_min_seconds, "e4m3" if fp8 else "e2m1")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
