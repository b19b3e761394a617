"""Benchmark of the BATQuant W4A4 hot path on one MI355X.

One step = the whole online path for one batch: the fused activation block
transform + clip + MXFP4 quantisation kernel followed by the W4A4 MXFP4 GEMM
(bf16 output).  The weight side (P^-1 W^T, clip, quantise, pack) is offline
and runs once before timing.  Default workload: the large-prefill layer (batch
64 x prefill 256 = 16384 tokens), X 16384 x 4096 bf16 and W 4096 x 4096 bf16,
shared factor 8x8 / private 4x4; ``--config 2`` is the up/gate projection
(2048 x 4096 x 12288), ``--config 5 --a N`` a point of the shared-factor sweep.

Inputs are resident in HBM when timing starts.  Steps rotate through several
copies of every buffer (more bytes than the 256 MB Infinity Cache) so a step
cannot be served from the cache a previous step filled.  Before the W warm-up
steps, untimed steps run for at least 0.3 s: from a cold start the chip runs
this memory-heavy workload up to 20 % slower for its first tens of
milliseconds, so without them a short run times that ramp rather than the
steady state (the line reports how many settling steps ran).

Prints ONE JSON line.  ``value`` is the step throughput in TFLOP/s of W4A4 GEMM
work (2 M N K per step) including the activation kernel's time.  Per-kernel
durations come from loops of that kernel alone over the same buffers (direct
C-ABI calls, each loop run once untimed first), timed with HIP events on the
launch stream at the loops' ends only (an event between the two kernels of a
step adds its own gap to both), and the line checks that they add up inside
the step.  ``--ceiling`` runs only the ceiling probes (the
FP4 matrix instruction in a register loop with the shader clock it sustains,
HBM read and copy streams).
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
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
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
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only the GEMM: the packed W4A4 GEMM beside hipBLASLt's MXFP4 GEMM on the same operands "
                         "(large prefill only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB -> 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--ceiling", action="store_true",
                    help="run only the ceiling probes (FP4 MFMA loop and shader clock, HBM read and copy)")
    ap.add_argument("--no-ceiling", action="store_true", help="leave the ceiling probes out of the bench line")
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


def _blas_threads() -> int:
    import threadpoolctl

    return int(max([d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()] or [1]))


def scalar_oracle_tiny():
    """The pure-Python loop oracle, single-threaded, on the tiny config:
    activations (64 x 256), weights (256 x 256) and the exact rational GEMM of
    the first 16 token rows; seconds each."""
    from oracle import scalar as osc
    from workloads import gen

    wl = gen.make_workload(1)
    t0 = time.perf_counter()
    xc, xs = osc.act_transform_quant(wl.X_bits, wl.A, wl.B, wl.alpha, wl.beta)
    t1 = time.perf_counter()
    wc, ws = osc.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)
    t2 = time.perf_counter()
    osc.gemm_exact(xc[:16], xs[:16], wc, ws)
    t3 = time.perf_counter()
    return {"act_s": t1 - t0, "weight_prep_s": t2 - t1, "gemm_exact_16_rows_s": t3 - t2,
            "act_GBs": wl.M * wl.K * (2 + 0.5 + 1 / 32) / (t1 - t0) / 1e9,
            "gemm_exact_GFLOPs": 2.0 * 16 * wl.N * wl.K / (t3 - t2) / 1e9, "threads": 1}


def cpu_baseline(wl, min_seconds: float, fmt: str = "e2m1", max_rows: int = 1024):
    """The oracle, as it stands, on a bounded sample of the same workload: the
    first ``max_rows`` token rows (every row of a smaller config) through the
    activation path, then their GEMM against every prepared weight row,
    repeated until ``min_seconds`` have passed, scaled to the step's TFLOP/s.
    Beside it: the oracle's offline weight preparation of the whole weight
    (once) and the single-threaded loop oracle on the tiny config."""
    from oracle import batquant as ob

    rows = min(wl.M, max_rows)
    t0 = time.perf_counter()
    wprep = ob.weight_prep(wl.W_bits, wl.A, wl.B, wl.walpha, wl.wbeta)  # offline, timed once
    t_wprep = time.perf_counter() - t0
    xb = wl.X_bits[:rows]
    reps, t_act, t_gemm = 0, 0.0, 0.0
    while reps == 0 or (t_act + t_gemm < min_seconds and reps < 64):
        t0 = time.perf_counter()
        x = ob.act_transform_quant(xb, wl.A, wl.B, wl.alpha, wl.beta, fmt=fmt)
        t1 = time.perf_counter()
        ob.gemm(x.codes, x.scales, wprep.codes, wprep.scales, x_fmt=fmt)
        t2 = time.perf_counter()
        t_act += t1 - t0
        t_gemm += t2 - t1
        reps += 1
    flops = 2.0 * rows * wl.N * wl.K
    threads = _blas_threads()
    scal = scalar_oracle_tiny()
    wbytes = wl.N * wl.K * (2 + 0.5 + 1 / 32)
    return {
        "value": flops * reps / (t_act + t_gemm) / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{rows} of the {wl.M} token rows through the fp64 oracle activation path, then their "
                   f"{rows}x{wl.N}x{wl.K} dequantised fp64 GEMM, {reps} repetition(s): activation "
                   f"{t_act / reps:.2f} s, GEMM {t_gemm / reps:.2f} s each; BLAS threads {threads}, host cores "
                   f"visible {len(os.sched_getaffinity(0))}; also timed: the oracle's weight preparation of the "
                   f"whole {wl.N}x{wl.K} weight (once) and the single-threaded loop oracle on the tiny config"),
        "seconds_measured": t_act + t_gemm,
        "act_GBs": rows * wl.K * (2 + 0.5 + 1 / 32) * reps / t_act / 1e9,
        "gemm_TFLOPs": flops * reps / t_gemm / 1e12,
        "weight_prep": {"s": t_wprep, "GBs": wbytes / t_wprep / 1e9, "rows": wl.N},
        "scalar_tiny": scal,
    }


SETTLE_SECONDS = 0.3


def settle(torch, step, min_seconds: float = SETTLE_SECONDS) -> int:
    """Untimed steps until `min_seconds` of wall time have passed, before the
    W warm-up steps.  From a cold start the chip runs this workload's
    memory-bound work slowly for its first tens of milliseconds: on
    16384 x 4096 x 4096, 20-step loops started at 195 us per step and reached
    160 us only after about 40 ms of steps.  A GPU spin of 140 ms without
    memory traffic, or 250 ms idle, left the same ramp; 250 ms of steps
    removed it.  Returns the number of steps run."""
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def run_decode(args, torch, w, wl, dev):
    """The fused decode step: one w4a4_decode call, one launch (the activation
    transform, clip and MXFP4 quantisation run inside the GEMM kernel, and the
    last workgroup of each column chunk sums its K splits).  Bound: HBM (the
    packed weights are read once per step).  Buffers rotate over enough sets
    that every step reads its weights from HBM."""
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
        settled = settle(torch, lambda i: g.replay())
        for _ in range(max(1, -(-args.warmup // nsets))):
            g.replay()
    else:
        run = lambda: [step(i) for i in range(steps)]
        settled = settle(torch, step)
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
    dec_kernel = f"decode_fused_kernel<{int(wl.a).bit_length() - 1}>"  # log2 a
    gbs = alg_bytes / t_step / 1e9
    out = {
        "metric": METRIC_DECODE,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "settle": {"steps": settled, "min_seconds": SETTLE_SECONDS},
        "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: X {M}x{K} bf16 ({wl.meta['x_kind']}, {wl.meta['outliers']}), W {N}x{K} bf16 "
                        f"N(0,0.02) prepared and packed offline; step = one "
                        f"fused decode launch ({'graph replay' if args.graph else 'eager launches'})",
            "M": M, "K": K, "N": N, "a": wl.a, "b": wl.b, "buffer_sets": nsets, "graph": args.graph,
            "factors": args.factors, "clip": not args.no_clip,
        },
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic("decode_fused.hip", dec_kernel, wl.name),
                     "kernel": dec_kernel},
        "kernels": {"decode_step": {"us": t_step * 1e6, "GB/s": gbs, "algorithmic_bytes": alg_bytes,
                                    "TFLOP/s": 2.0 * M * N * K / t_step / 1e12}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_min_seconds)
        # the oracle's rate over the same bytes per step (its sample covers every token row here)
        step_s = 2.0 * wl.M * wl.N * wl.K / (cb["value"] * 1e12)
        cb["value"] = alg_bytes / step_s / 1e9
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

    settled = settle(torch, step)
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
    # The kernel alone: direct C-ABI calls with the arguments the binding
    # passes (a kernel shorter than the binding's host time per call would
    # otherwise time the host).
    lib = w.native_library()
    stream = torch.cuda.current_stream().cuda_stream
    rp = (0 if rh is None else rh.data_ptr(), 0 if rl is None else rl.data_ptr())
    kargs = [(st["X"].data_ptr(), T, HD, HD, A.shape[0], B.shape[1], A.data_ptr(), B.data_ptr(), rp[0], rp[1],
              st["slots"].data_ptr(), rows, fmt, st["q"].data_ptr(), st["s"].data_ptr(), stream) for st in sets]
    torch.cuda.synchronize()
    e0.record()
    bad = 0
    for i in range(args.steps):
        bad |= lib.batq_kv_cache_quant(*kargs[i % nsets])
    e1.record()
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError(f"bench: a direct call returned an error status ({bad})")
    t_kernel = e0.elapsed_time(e1) * 1e-3 / args.steps
    alg_bytes = T * HD * 2 + T * (qcols + HD // 32) + T * 8  # rows read, codes + scales written, slots read
    gbs = alg_bytes / t_step / 1e9
    kgbs = alg_bytes / t_kernel / 1e9
    kvk = "kv_cache_quant_kernel" if w.transform_kernel(T, HD) == 0 else "kv_cache_quant_dl_kernel"
    kv_kernel = f"{kvk}<{'true' if fmt == 8 else 'false'}>"
    out = {
        "metric": METRIC_KV, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"steps": settled, "min_seconds": SETTLE_SECONDS},
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4" if fmt == 4 else "mxfp8", "data": "synthetic",
        "config": {"workload": f"KV-cache write: {T} tokens x {HD} channels (8 heads x 128) bf16 (t3), GPK a=8 b=4, "
                               f"{'MXFP4' if fmt == 4 else 'MXFP8 E4M3'} into permuted slots of a {rows}-row cache",
                   "T": T, "HD": HD, "cache_rows": rows, "fmt": fmt, "buffer_sets": nsets, "clip": not args.no_clip},
        "roofline": {"bound": "hbm", "achieved": kgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kgbs / HBM_PEAK_GBS,
                     "traffic": load_traffic("transform_quant.hip", kv_kernel, f"kv{fmt}_{T}x{HD}"),
                     "kernel": kv_kernel},
        "kernels": {"kv_cache_quant": {"us": t_kernel * 1e6, "GB/s": kgbs, "algorithmic_bytes": alg_bytes,
                                       "eager_step_us": t_step * 1e6,
                                       "timing": "us: a loop of direct C-ABI calls; value: the steps through "
                                                 "the binding"}},
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
        out["cpu_baseline"] = {"value": alg_bytes / dt / 1e9, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
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


def measure_ceilings(torch, w, dev, act_read_bytes=None, act_write_ratio=4):
    """The ceilings the kernels are set against, measured on this GPU: the
    block-scaled FP4 MFMA in a register-only loop (random and constant operand
    bits, 2 and 1 waves per SIMD) with the shader clock it ran at, HBM read
    and copy streams over buffers eight times the Infinity Cache, and a
    stream shaped like the activation transform's traffic (its bf16 bytes
    read, a quarter as many written) over buffers rotated past the cache."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    mf = {}
    iters = 20000
    for name, data, per_cu in (("random_2w", 1, 2), ("const_2w", 0, 2), ("random_1w", 1, 1)):
        wgs = cus * per_cu
        sink = torch.empty(4 * wgs, dtype=torch.float32, device=dev)
        clocks = torch.zeros(8 * wgs, dtype=torch.int64, device=dev)
        for _ in range(2):
            w.probe_mfma_fp4(wgs, iters, data, 7, sink, clocks)
        reps = 4
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            w.probe_mfma_fp4(wgs, iters, data, 7, sink, clocks)
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) * 1e-3 / reps
        flops = 4.0 * wgs * iters * 8 * 2 * 32 * 32 * 64
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        mf[f"{name}_TFLOPs"] = flops / dt / 1e12
        # shader-clock cycles per 100 MHz real-time tick, over every wave of the last launch
        mf[f"{name}_clock_MHz"] = float(c[:, 0].sum() / c[:, 1].sum() * 100.0)
    gran = w.probe_stream_granule()
    nbytes = (2 << 30) // gran * gran  # 2 GiB
    assert nbytes == 2 << 30, gran
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    rsink = torch.empty(4096, dtype=torch.int32, device=dev)
    csrc = src[: nbytes // 8]
    cdst = torch.empty(nbytes // 8, dtype=torch.int32, device=dev)

    def stream(fn, nb, reps=5):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return nb * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    read = stream(lambda: w.probe_hbm_read(src, rsink), nbytes)
    copy = stream(lambda: w.probe_hbm_copy(csrc, cdst), 2 * (nbytes // 2))
    del src, cdst
    shaped = None
    if act_read_bytes:
        rb = -(-act_read_bytes // gran) * gran
        nbuf = max(2, -(-int(2.2 * CACHE_BYTES) // (rb + rb // act_write_ratio)))
        bufs = [(torch.empty(rb // 4, dtype=torch.int32, device=dev),
                 torch.empty(rb // act_write_ratio // 4, dtype=torch.int32, device=dev)) for _ in range(nbuf)]
        k = [0]

        def one():
            s_, d_ = bufs[k[0] % nbuf]
            k[0] += 1
            w.probe_hbm_stream(s_, d_, act_write_ratio)

        gbs = stream(one, rb + rb // act_write_ratio, reps=4 * nbuf)
        shaped = {"read_bytes": rb, "write_bytes": rb // act_write_ratio, "GBs": gbs,
                  "us": (rb + rb // act_write_ratio) / gbs / 1e3}
        del bufs
    return {"mfma_fp4_loop": mf, "hbm_read_GBs": read, "hbm_copy_GBs": copy, "act_shaped_stream": shaped,
            "note": "FP4 32x32x64 block-scaled MFMA, 8 independent chains per wave, no memory traffic; clock = "
                    "s_memtime cycles per s_memrealtime tick x 100 MHz; HBM read of 2 GiB, copy of 1 GiB -> 1 GiB"}


def run_ceilings(args, torch, w, dev):
    ceil = measure_ceilings(torch, w, dev)
    print(json.dumps({"ceilings": ceil, "published": {"mfma_fp4_TFLOPs": MXFP4_PEAK_TFLOPS,
                                                     "hbm_GBs": HBM_PEAK_GBS}}), flush=True)


def run_vendor_gemm(args, torch, w, wl, dev):
    """The packed W4A4 GEMM beside hipBLASLt's block-scaled MXFP4 GEMM
    (include/batq_vendor.h) on the same operands: this workload's activations
    through the transform kernel and its prepared weights, quantised once.
    Both GEMMs run `steps` launches over the same rotating buffer sets (more
    bytes than the Infinity Cache), with events at the loop's two ends.  Every
    algorithm hipBLASLt's heuristic offers (up to 8) is timed, and each one's output is
    compared with the packed GEMM's: how many bf16 outputs differ from its fp32
    result rounded to nearest even (its own bf16 output) and rounded toward
    zero, and the largest difference from the fp32 result relative to max |Y|.
    The packed GEMM is timed before and after the library's loops; the faster
    loop counts.  Large prefill only: at 2048 x 12288 x 4096 the library's first
    calls did not return within three minutes."""
    from w4a4_bit_gemm_amd import vendor_gemm as vg

    M, K, N = wl.M, wl.K, wl.N

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    rh, rl = f32(w.clip_ratios(wl.alpha)), f32(w.clip_ratios(wl.beta))
    Xq0, Xs0 = w.act_transform_quant(bf16(wl.X_bits), f32(wl.A), f32(wl.B), rh, rl)
    Wq0, Ws0 = w.prepare_weight(bf16(wl.W_bits), wl.A, wl.B, wl.walpha, wl.wbeta)
    torch.cuda.synchronize()
    set_bytes = M * K // 2 + M * K // 32 + 2 * (N * K // 2 + N * K // 32) + M * N * 2
    nsets = min(64, max(2, int(np.ceil(2.2 * CACHE_BYTES / set_bytes))))
    sets = [dict(Xq=Xq0.clone(), Xs=Xs0.clone(), Wq=Wq0.clone(), Ws=Ws0.clone(), Wp=w.weight_pack(Wq0, Ws0),
                 Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    plan = vg.VendorGemm(M, N, K, dev, max_algos=8)
    torch.cuda.synchronize()
    print(f"vendor: hipBLASLt offers {plan.algos} algorithms", file=sys.stderr, flush=True)

    def loop_us(fn):
        for i in range(min(args.warmup, 10)):
            fn(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    def ours(i):
        s = sets[i % nsets]
        w.mxfp4_gemm_packed(s["Xq"], s["Xs"], s["Wp"], out=s["Y"])

    ours(0)
    y32 = w.mxfp4_gemm_packed(sets[0]["Xq"], sets[0]["Xs"], sets[0]["Wp"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref = sets[0]["Y"].clone()  # bf16: the fp32 result rounded to nearest even
    ref_max = float(y32.abs().max())
    # the fp32 result rounded toward zero to bf16 (low 16 bits dropped)
    y_rz = (y32.view(torch.int32) >> 16).to(torch.int16)
    t_ours_first = loop_us(ours)
    print(f"vendor: packed GEMM {t_ours_first:.1f} us", file=sys.stderr, flush=True)
    per_algo = []
    y_v = torch.empty_like(y_ref)
    for a in range(plan.algos):
        s0 = sets[0]
        try:
            plan.run(a, s0["Xq"], s0["Xs"], s0["Wq"], s0["Ws"], y_v)
        except RuntimeError as e:  # an algorithm the library offers but then refuses to run
            per_algo.append({"algo": a, "error": str(e)})
            continue
        torch.cuda.synchronize()
        differ = int((y_v.view(torch.int16) != y_ref.view(torch.int16)).sum())
        differ_rz = int((y_v.view(torch.int16) != y_rz).sum())
        max_rel = float((y_v.float() - y32).abs().max()) / ref_max

        def theirs(i, a=a):
            s = sets[i % nsets]
            plan.run(a, s["Xq"], s["Xs"], s["Wq"], s["Ws"], s["Y"])

        per_algo.append({"algo": a, "us": loop_us(theirs), "outputs": M * N, "differ_from_batq_bf16": differ,
                         "differ_from_batq_fp32_rounded_to_zero": differ_rz,
                         "max_diff_to_batq_fp32_over_max_abs": max_rel})
        # each algorithm's first launch takes seconds inside the library
        print(f"vendor: algorithm {a}: {per_algo[-1]['us']:.1f} us", file=sys.stderr, flush=True)
    plan.close()
    t_ours_after = loop_us(ours)  # again, after the library's loops, on a GPU as warm as theirs
    print(f"vendor: packed GEMM {t_ours_after:.1f} us", file=sys.stderr, flush=True)
    t_ours = min(t_ours_first, t_ours_after)
    flops = 2.0 * M * N * K
    best = min((r for r in per_algo if "us" in r), key=lambda r: r["us"])
    kernel = ("mxfp4_gemm_packed_dma_kernel" if w.packed_gemm_kernel(M, N, K) == 1 else "mxfp4_gemm_packed_kernel")
    print(json.dumps({
        "comparison": "packed W4A4 GEMM against hipBLASLt's MXFP4 GEMM (VEC32_UE8M0 scales), same operands, bf16 out",
        "config": {"workload": f"{wl.name}: {M}x{K} activations (transform kernel, a={wl.a}) x {N}x{K} prepared "
                               f"weights", "M": M, "N": N, "K": K, "buffer_sets": nsets, "steps": args.steps},
        "batq": {"kernel": kernel, "us": t_ours, "us_before_after": [t_ours_first, t_ours_after],
                 "TFLOP/s": flops / t_ours / 1e6, "frac_mfma": flops / t_ours / 1e6 / MXFP4_PEAK_TFLOPS},
        "hipblaslt": {"version": vg.version(), "algos": len(per_algo), "best": best,
                      "TFLOP/s": flops / best["us"] / 1e6, "per_algo": per_algo},
        "batq_speedup_over_best": best["us"] / t_ours,
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
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
    if args.ceiling:
        run_ceilings(args, torch, w, dev)
        return
    wl = gen.make_workload(args.config, a=args.a)
    M, K, N = wl.M, wl.K, wl.N
    if args.decode:
        run_decode(args, torch, w, wl, dev)
        return
    if args.kv_cache:
        run_kv(args, torch, w, wl, dev)
        return
    if args.vendor_gemm:
        if args.config != 5:
            print("--vendor-gemm runs on the large prefill (--config 5) only", file=sys.stderr)
            sys.exit(2)
        run_vendor_gemm(args, torch, w, wl, dev)
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

    settled = settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps between two synchronisations; HIP
    # events on the launch stream (torch's current stream) at its two ends
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    t_step = ev0.elapsed_time(ev1) * 1e-3 / args.steps

    # Per-kernel launch durations: each kernel alone, `steps` launches over the
    # same rotating buffers, events at the loop's two ends only (an event
    # between the two kernels of a step would add its own gap to both).  The
    # loops call the C ABI directly with the arguments the binding passes,
    # built once per buffer set: a kernel shorter than the binding's host time
    # per call (its shape and dtype checks) would otherwise time the host.
    lib = w.native_library()
    stream = torch.cuda.current_stream().cuda_stream
    rp = (0 if rh is None else rh.data_ptr(), 0 if rl is None else rl.data_ptr())
    act_fn = lib.batq_act_transform_quant_mxfp8 if fp8 else lib.batq_act_transform_quant
    act_args = [(s["X"].data_ptr(), M, K, K, A.shape[0], B.shape[1], A.data_ptr(), B.data_ptr(), rp[0], rp[1],
                 s["Xq"].data_ptr(), s["Xs"].data_ptr(), stream) for s in sets]
    if fp8 or packed:
        gemm_fn = lib.batq_mxfp8_gemm_packed if fp8 else lib.batq_mxfp4_gemm_packed
        gemm_args = [(s["Xq"].data_ptr(), s["Xs"].data_ptr(), s["Wp"].data.data_ptr(), M, N, K, s["Y"].data_ptr(), 0,
                      stream) for s in sets]
    else:
        gemm_fn = lib.batq_mxfp4_gemm
        gemm_args = [(s["Xq"].data_ptr(), s["Xs"].data_ptr(), s["Wq"].data_ptr(), s["Ws"].data_ptr(), M, N, K,
                      s["Y"].data_ptr(), 0, stream) for s in sets]

    # Each loop first runs once untimed: the chip's clock follows its power
    # draw over milliseconds, and a GEMM loop that starts straight after the
    # low-power transform loop ran its first launches faster than its own
    # steady state (126.9 against 133.7 us on 16384 x 4096 x 4096).
    def loop_seconds(fn, fargs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bad = 0
        for i in range(args.steps):
            bad |= fn(*fargs[i % nsets])
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            bad |= fn(*fargs[i % nsets])
        e1.record()
        torch.cuda.synchronize()
        if bad:
            raise RuntimeError(f"bench: a direct call returned an error status ({bad})")
        return e0.elapsed_time(e1) * 1e-3 / args.steps

    t_act = loop_seconds(act_fn, act_args)
    t_gemm = loop_seconds(gemm_fn, gemm_args)

    # The two kernels' own times must fit inside the step they make up (5 %
    # for box noise).
    consistent = bool((t_act + t_gemm) <= 1.05 * t_step)
    if not consistent:
        print(f"bench: per-kernel times {1e6 * t_act:.2f} + {1e6 * t_gemm:.2f} us exceed the step's "
              f"{1e6 * t_step:.2f} us", file=sys.stderr)
    flops = 2.0 * M * N * K
    act_bytes = M * K * 2 + M * xq_row + M * K // 32  # algorithmic: read bf16, write codes + scales
    gemm_bytes = M * xq_row + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2
    mma_peak = FP8_PEAK_TFLOPS if fp8 else MXFP4_PEAK_TFLOPS
    act_gbs = act_bytes / t_act / 1e9
    gemm_tflops = flops / t_gemm / 1e12
    ai = flops / gemm_bytes
    gemm_hbm_bound = ai < mma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gemm_hbm_bound:
        gemm_roof = {"bound": "hbm", "achieved": gemm_bytes / t_gemm / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s"}
    else:
        gemm_roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": mma_peak, "unit": "TFLOP/s"}
    gemm_roof["frac"] = gemm_roof["achieved"] / gemm_roof["peak"]
    act_roof = {"bound": "hbm", "achieved": act_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": act_gbs / HBM_PEAK_GBS}
    dominant_is_gemm = t_gemm >= t_act
    roof = dict(gemm_roof if dominant_is_gemm else act_roof)
    nst = K // 256
    gs = "true" if nst % 4 == 0 else "false"
    a8 = "true" if fp8 else "false"
    if not packed:
        gemm_src, gemm_kernel = "mxfp4_gemm.hip", "mxfp4_gemm_dma_kernel"
    elif w.packed_gemm_kernel(M, N, K, fp8) == 1:  # the library's own choice for this shape
        gemm_src = "mxfp4_gemm_packed_dma.hip"
        # bf16 output: the instance with the per-wave bf16 epilogue
        gemm_kernel = f"{'w4a8' if fp8 else 'mxfp4'}_gemm_packed_dma_kernel<{nst},false>"
    else:
        gemm_src = "mxfp4_gemm_packed.hip"
        gemm_kernel = f"mxfp4_gemm_packed_kernel<{nst if nst in (1, 2, 4, 8, 16, 48) else 0},{gs},{a8}>"
    tq = "transform_quant_kernel" if w.transform_kernel(M, K) == 0 else "transform_quant_dl_kernel"
    act_kernel = f"{tq}<false,{a8}>"
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
        "settle": {"steps": settled, "min_seconds": SETTLE_SECONDS},
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
            "transform_quant": {"us": t_act * 1e6, "GB/s": act_gbs,
                                "frac_hbm": act_gbs / HBM_PEAK_GBS, "algorithmic_bytes": act_bytes,
                                "roofline": act_roof},
            "gemm": {"kernel": gemm_kernel, "us": t_gemm * 1e6, "TFLOP/s": gemm_tflops,
                     "frac_mfma": gemm_tflops / mma_peak, "flops": flops,
                     "operand_output_bytes": gemm_bytes, "roofline": gemm_roof},
        },
        "step": {"gpu_us": t_step * 1e6, "kernels_sum_us": (t_act + t_gemm) * 1e6,
                 "kernels_sum_over_step": (t_act + t_gemm) / t_step,
                 "consistent": consistent,
                 "timing": "step: events around the timed steps; kernels: events around a loop of each kernel alone "
                           "(direct C-ABI calls)"},
        "cpu_baseline": None,
    }
    if not args.no_ceiling:
        ceil = measure_ceilings(torch, w, dev, act_read_bytes=M * K * 2, act_write_ratio=2 if fp8 else 4)
        out["ceilings"] = ceil
        out["kernels"]["gemm"]["frac_of_mfma_loop"] = gemm_tflops / ceil["mfma_fp4_loop"]["random_2w_TFLOPs"]
        out["kernels"]["transform_quant"]["frac_of_hbm_read"] = act_gbs / ceil["hbm_read_GBs"]
        out["kernels"]["transform_quant"]["frac_of_shaped_stream"] = ceil["act_shaped_stream"]["us"] / (t_act * 1e6)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_min_seconds, "e4m3" if fp8 else "e2m1")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
