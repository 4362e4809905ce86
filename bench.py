"""Benchmark: seconds per exact Lloyd iteration on one MI355X, with assign
TFLOP/s and update GB/s, on the skewed large-K workload (16,777,216 x 128,
K = 32,768, Zipf(1.2) mixture).

One step = one full Lloyd iteration (FlashAssign + fp64 near-tie recheck +
Sort-Inverse Update) through the C ABI, with X and C resident in HBM.  Prints
one JSON line.  Phase times come from HIP events the library records on the
stream it launches on; the FlashAssign kernel's average duration gives the
roofline line.  The CPU baseline times the fp64 oracle on a bounded sample of
the same workload on this host's cores and scales it to the full N.

The headline line uses split-bf16 scoring (three bf16 MFMAs per product on
hi/lo halves of the fp32 operands; the near-tie recheck makes the result the
same exact assignment as fp32 scoring).  Its roofline is priced against the
bf16 dense MFMA peak with the algorithmic 2NKd FLOPs; the FLOPs the matrix
cores actually execute (3 x 2NKd) are reported beside it.  The fp32-scoring
path is timed after it on the same inputs and reported under "other_scores".

usage: python bench.py [--gpus 1] [--steps 5] [--warmup 1] [--workload NAME]
                       [--score split_bf16|fp32] [--no-compare] [--no-cpu-baseline]
                       [--ivf-build | --knn [WORKLOAD] | --ooc [--ooc-rows N]]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, TFLOP/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, TFLOP/s
# per scoring mode: MFMA input type, its dense peak, matrix products issued per
# algorithmic product, and the main FlashAssign kernel's template arguments
SCORES = {
    "fp32": {"mfma_dtype": "fp32", "peak": FP32_MFMA_PEAK_TFLOPS, "products": 1, "dtype": "f32"},
    "split_bf16": {"mfma_dtype": "bf16", "peak": BF16_MFMA_PEAK_TFLOPS, "products": 3, "dtype": "bf16"},
}
ASSIGN_SRC = os.path.join(ROOT, "exact_lloyd_means_flashassign_amd", "csrc", "fk_assign.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def run_env(torch, np):
    """Versions and hardware the numbers were taken with (the seeded streams
    and the timings both depend on them)."""
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "numpy": np.__version__,
            "gpu": torch.cuda.get_device_name(0), "cpu": cpu, "host_cores_available": cores}


def traffic_file(workload, score):
    return os.path.join(ROOT, "profiles", f"flash_assign_{score}_{workload}_traffic.json")


def traffic_per_launch(workload, score):
    """HBM bytes per FlashAssign launch from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    try:
        with open(traffic_file(workload, score)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_sha(ASSIGN_SRC):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, X, C, budget_s=15.0):
    """Time the fp64 oracle on a bounded sample (the first n rows, all K
    centroids) and scale seconds per iteration linearly to the full N."""
    import oracle
    probe = 512
    t0 = time.perf_counter()
    oracle.lloyd_iter(X[:probe], C)
    dt = time.perf_counter() - t0
    n = int(min(w.N, max(probe, budget_s / max(dt, 1e-9) * probe)))
    t0 = time.perf_counter()
    oracle.lloyd_iter(X[:n], C)
    dt = time.perf_counter() - t0
    return {"value": dt * w.N / n, "unit": "s/iter", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {n} of {w.N} points against all K={w.K} centroids, one iteration in {dt:.1f} s; "
                      f"seconds per iteration scaled linearly by N/{n}"}


def _micro_lib():
    import ctypes
    path = os.path.join(ROOT, "exact_lloyd_means_flashassign_amd", "libfk_micro.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.fkm_stream_copy.argtypes = [P, P, I64, I32, P]
    lib.fkm_stream_read.argtypes = [P, I64, P, I32, P]
    lib.fkm_gather_rows.argtypes = [P, P, I64, I32, I32, P, P]
    lib.fkm_mfma.argtypes = [I32, I32, I32, P, P, P]
    return lib


def micro_peaks(torch, gather_rows=1 << 24, d=128, reps=3):
    """Measured on this machine (fk_micro.hip): HBM copy and read rates over 4 GiB,
    the segmented reduction's row gather (rows of d floats in a random
    order), back-to-back bf16 and fp32 matrix products on every SIMD with the
    clock they ran at, and the pinned host-to-device copy rate.  Each is the
    best of `reps` event-timed runs."""
    import ctypes
    import statistics
    lib = _micro_lib()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(st.cuda_stream)

    def timed(fn):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = fn()
            e1.record(st)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"microbenchmark launch failed ({rc})")
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best / 1e3

    out = {}
    n4 = 1 << 28  # float4s: 4 GiB
    src = torch.ones(4 * n4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    red = torch.empty(8192, dtype=torch.float32, device=dev)
    t = timed(lambda: lib.fkm_stream_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n4,
                                          4096, sp))
    out["hbm_copy_gbps"] = 2 * 16 * n4 / t / 1e9
    t = timed(lambda: lib.fkm_stream_read(ctypes.c_void_p(src.data_ptr()), n4, ctypes.c_void_p(red.data_ptr()),
                                          4096, sp))
    out["hbm_read_gbps"] = 16 * n4 / t / 1e9
    del src, dst
    X = torch.ones((gather_rows, d), dtype=torch.float32, device=dev)
    perm = torch.randperm(gather_rows, device=dev, dtype=torch.int64).to(torch.int32)
    rpw = 1024
    waves = (gather_rows + rpw - 1) // rpw
    gout = torch.empty(waves * 64, dtype=torch.float64, device=dev)
    t = timed(lambda: lib.fkm_gather_rows(ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(perm.data_ptr()),
                                          gather_rows, d, rpw, ctypes.c_void_p(gout.data_ptr()), sp))
    out["row_gather_gbps"] = (gather_rows * d * 4 + gather_rows * 4) / t / 1e9
    out["row_gather_shape"] = f"{gather_rows} rows x {d} floats in a random order, {rpw} rows per wave"
    del X, perm, gout
    blocks, iters = 2048, 4096
    clocks = torch.empty(blocks * 4 * 2, dtype=torch.int64, device=dev)
    sink = torch.empty(blocks * 4 * 64, dtype=torch.float32, device=dev)
    for name, bf16, flop in (("bf16", 1, 32 * 32 * 16 * 2), ("fp32", 0, 32 * 32 * 2 * 2)):
        t = timed(lambda: lib.fkm_mfma(bf16, blocks, iters, ctypes.c_void_p(clocks.data_ptr()),
                                       ctypes.c_void_p(sink.data_ptr()), sp))
        c = clocks.view(-1, 2).cpu().numpy()
        ghz = statistics.median((c[:, 0] / (c[:, 1] / 100e6)).tolist()) / 1e9
        out[f"mfma_{name}_tflops"] = blocks * 4 * iters * 4 * flop / t / 1e12
        out[f"mfma_{name}_clock_ghz"] = ghz
    h = torch.empty(1 << 30, dtype=torch.float32, pin_memory=True)
    g = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    t = timed(lambda: (g.copy_(h, non_blocking=True), 0)[1])
    out["h2d_pinned_gbps"] = 4 * (1 << 30) / t / 1e9
    del h, g
    torch.cuda.empty_cache()
    return out


def micro_bench(args, torch):
    m = micro_peaks(torch)
    out = {"metric": "on-box peaks (HBM copy GB/s, row gather GB/s, bf16/fp32 MFMA TFLOP/s, pinned H2D GB/s)",
           "value": m["hbm_copy_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": 3, "warmup": 0,
           "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic", "config": {"workload": "microbenchmarks"},
           "spec": {"hbm_gbps": HBM_PEAK_GBS, "mfma_bf16_tflops": BF16_MFMA_PEAK_TFLOPS,
                    "mfma_fp32_tflops": FP32_MFMA_PEAK_TFLOPS},
           "measured": m, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


IVF_BUILD_H200_S = 10.6  # the LEANN FlashLib guide's build time at this shape (NVIDIA H200), context only


def ivf_build_bench(args, fk, synth, np, torch):
    """Seconds per IVF-Flat build (quantizer: niter = 20 Lloyd iterations from
    seeded initial rows, then the cell-contiguous lists) at the shape of the
    FlashLib guide's build measurement: 1M x 768 unit rows, nlist = 4096."""
    w = synth.WORKLOADS["ivf_1m_d768_k4096"]
    n_iter = 20
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    X = synth.rows(w)
    init = synth.init_indices(w).astype(np.int32)
    log(f"generated {w.name}: N={w.N} d={w.d} nlist={w.K} in {time.perf_counter() - t0:.1f} s")
    Xd = torch.from_numpy(X).to(dev)
    ws = torch.empty(fk.fk_ivf_workspace_size(w.N, w.d, w.K, w.metric) + 256, dtype=torch.uint8, device=dev)

    def run(score):
        for i in range(args.warmup):
            fk.fk_ivf_build(Xd, w.K, init, n_iter=n_iter, metric=w.metric, workspace=ws, score=score)
        torch.cuda.synchronize()
        fk.fk_profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            out = fk.fk_ivf_build(Xd, w.K, init, n_iter=n_iter, metric=w.metric, workspace=ws, score=score)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        prof = fk.fk_profile_read()
        fk.fk_profile_enable(False)
        assert int(out["offsets"][-1].item()) == w.N
        log(f"{score}: {el:.3f} s per build")
        return {"s_per_build": el,
                "phase_ms_per_build": {k: round(v / args.steps, 3) for k, v in prof["ms"].items()},
                "s_per_iteration": el / (n_iter + 1)}

    r = run(args.score)
    out = {"metric": "s per IVF-Flat build (1M x 768, nlist 4096, niter 20)", "value": r["s_per_build"], "unit": "s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * r["s_per_build"],
           "higher_is_better": False, "scaling": "weak", "vs_baseline": r["s_per_build"] / IVF_BUILD_H200_S,
           "dtype": SCORES[args.score]["dtype"], "data": "synthetic",
           "config": {"workload": w.name, "N": w.N, "d": w.d, "nlist": w.K, "niter": n_iter, "metric": w.metric,
                      "seed": w.seed, "score": args.score},
           "phase_ms_per_build": r["phase_ms_per_build"],
           "baseline_context": f"{IVF_BUILD_H200_S} s on an NVIDIA H200 (FlashLib), 140.7 s FAISS CPU, as the "
                               "LEANN FlashLib guide reports; other hardware"}
    if not args.no_compare:
        out["other_scores"] = {o: run(o) for o in SCORES if o != args.score}
    if not args.no_cpu_baseline:
        import oracle
        C0 = X[init]
        probe = 256
        t0 = time.perf_counter()
        oracle.lloyd_iter(X[:probe], C0)
        dt = time.perf_counter() - t0
        n = int(min(w.N, max(probe, 15.0 / max(dt, 1e-9) * probe)))
        t0 = time.perf_counter()
        oracle.lloyd_iter(X[:n], C0)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": dt * w.N / n * (n_iter + 1), "unit": "s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"one oracle iteration on the first {n} of {w.N} rows against the {w.K} "
                                         f"initial centroids in {dt:.1f} s, scaled by N/{n} and by {n_iter + 1} "
                                         "(the iterations plus the final assignment)"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def knn_bench(args, fk, synth, np, torch):
    """Queries per second of exact k-NN (fk_knn) at the FlashLib guide's
    example shape: 10,000 queries against a 1,000,000 x 128 database, 10
    neighbours (or the workload named by --knn).  One step = one fk_knn call
    over all queries, inputs resident in HBM."""
    w = synth.WORKLOADS[args.knn]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    DB = synth.rows(w)
    Q = synth.queries(w)
    log(f"generated {w.name}: Ndb={w.N} d={w.d} M={w.queries} k={w.k} in {time.perf_counter() - t0:.1f} s")
    DBd = torch.from_numpy(DB).to(dev)
    Qd = torch.from_numpy(Q).to(dev)
    M = Q.shape[0]
    ws = torch.empty(fk.fk_knn_workspace_size(M, w.d, w.N, w.k, w.metric) + 256, dtype=torch.uint8, device=dev)
    flops = 2.0 * M * w.N * w.d

    def run(score):
        for i in range(args.warmup):
            fk.fk_knn(Qd, DBd, w.k, metric=w.metric, workspace=ws, score=score)
        torch.cuda.synchronize()
        fk.fk_profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            idx, dist = fk.fk_knn(Qd, DBd, w.k, metric=w.metric, workspace=ws, score=score)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        prof = fk.fk_profile_read()
        fk.fk_profile_enable(False)
        ms = {k: v / args.steps for k, v in prof["ms"].items()}
        sweep_s = ms.get("assign", 0.0) / 1e3
        log(f"{score}: {1e3 * el:.2f} ms per call, sweep {1e3 * sweep_s:.2f} ms")
        peak = SCORES[score]["peak"]
        ach = flops / sweep_s / 1e12 if sweep_s > 0 else None
        return {"queries_per_s": M / el, "ms_per_call": 1e3 * el,
                "phase_ms_per_call": {k: round(v, 3) for k, v in ms.items()},
                "roofline": {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                             "frac": (ach / peak) if ach else None, "traffic": None,
                             "kernel": "FlashAssign sweep with per-query top-L lists",
                             "mfma_dtype": SCORES[score]["mfma_dtype"],
                             "executed_frac": (ach * SCORES[score]["products"] / peak) if ach else None}}

    r = run(args.score)
    out = {"metric": f"queries/s (exact {w.k}-NN against {w.N} x {w.d})", "value": r["queries_per_s"],
           "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": r["ms_per_call"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": SCORES[args.score]["dtype"], "data": "synthetic",
           "config": {"workload": w.name, "Ndb": w.N, "d": w.d, "queries": M, "k": w.k, "metric": w.metric,
                      "seed": w.seed, "score": args.score},
           "phase_ms_per_call": r["phase_ms_per_call"], "roofline": r["roofline"]}
    if not args.no_compare:
        out["other_scores"] = {o: run(o) for o in SCORES if o != args.score}
    if not args.no_cpu_baseline:
        import oracle
        # every call promotes the whole database to fp64 first: time that
        # fixed part with one query, the per-query part with 128 more
        t0 = time.perf_counter()
        oracle.knn(Q[:1], DB, w.k, w.metric)
        fixed = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.knn(Q[:129], DB, w.k, w.metric)
        per_q = max(time.perf_counter() - t0 - fixed, 1e-6) / 128
        n = int(min(M, max(129, (15.0 - fixed) / per_q)))
        t0 = time.perf_counter()
        oracle.knn(Q[:n], DB, w.k, w.metric)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / dt, "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"the first {n} of {M} queries against the whole database in {dt:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


OOC_H200_S = 41.4  # the Flash-KMeans article's time per iteration at 1e9 x 128, K = 32768 (H200), context only


def ooc_bench(args, fk, synth, np, torch):
    """Seconds per out-of-core Lloyd iteration (fk_lloyd_iter_stream: X in
    pinned host memory, streamed in 2^26-row chunks, PCIe included) on the
    article's headline mixture (1e9 x 128, K = 32768) cut to --ooc-rows rows,
    the most a box's host memory comfortably holds; also given per 1e9 rows
    (the time is linear in N)."""
    w0 = synth.WORKLOADS["ooc_1b_d128_k32768"]
    N = int(args.ooc_rows)
    w = w0.scaled(N)
    t0 = time.perf_counter()
    Xh = torch.empty((N, w.d), dtype=torch.float32, pin_memory=True)
    X = Xh.numpy()
    piece = 1 << 25
    for lo in range(0, N, piece):
        hi = min(N, lo + piece)
        synth.rows(w, lo, hi, out=X[lo:hi])
        log(f"generated rows [{lo}, {hi}) of {N}")
    C = X[synth.init_indices(w)].copy()
    ah = torch.empty(N, dtype=torch.int32, pin_memory=True)
    Cd = torch.from_numpy(C).to("cuda:0")
    log(f"generated {w.name} cut to N={N} (pinned) in {time.perf_counter() - t0:.1f} s")
    ws = torch.empty(fk.fk_workspace_size(N, w.d, w.K, w.metric, chunk_rows=w.chunk_rows) + 256,
                     dtype=torch.uint8, device="cuda:0")

    def run(score):
        for i in range(args.warmup):
            fk.fk_lloyd_iter_stream(Xh, Cd, w.chunk_rows, assign_host=ah, workspace=ws, score=score)
        torch.cuda.synchronize()
        fk.fk_profile_enable(True)
        t0 = time.perf_counter()
        for i in range(args.steps):
            C1, cnt = fk.fk_lloyd_iter_stream(Xh, Cd, w.chunk_rows, assign_host=ah, workspace=ws, score=score)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        prof = fk.fk_profile_read()
        fk.fk_profile_enable(False)
        assert int(cnt.sum().item()) == N
        log(f"{score}: {el:.3f} s per iteration")
        return {"s_per_iter": el, "s_per_1e9_rows": el * 1e9 / N, "x_gbps_incl_pcie": N * w.d * 4 / el / 1e9,
                "phase_ms_per_step": {k: round(v / args.steps, 3) for k, v in prof["ms"].items()}}

    r = run(args.score)
    out = {"metric": f"s per out-of-core Lloyd iteration (X pinned on the host, {N} x {w.d}, K={w.K}, "
                     "PCIe included)", "value": r["s_per_iter"], "unit": "s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": 1e3 * r["s_per_iter"], "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": SCORES[args.score]["dtype"], "data": "synthetic",
           "config": {"workload": w.name, "N": N, "d": w.d, "K": w.K, "chunk_rows": w.chunk_rows, "seed": w.seed,
                      "score": args.score},
           "s_per_1e9_rows": r["s_per_1e9_rows"], "x_gbps_incl_pcie": r["x_gbps_incl_pcie"],
           "phase_ms_per_step": r["phase_ms_per_step"],
           "baseline_context": f"{OOC_H200_S} s per iteration at 1e9 x 128, K = 32768 on an NVIDIA H200, as the "
                               "Flash-KMeans article reports; other hardware"}
    if not args.no_compare:
        out["other_scores"] = {o: run(o) for o in SCORES if o != args.score}
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w, X, C)
    print(json.dumps(out), flush=True)


def _rows_label(n):
    """16777216 -> '16M' (a multiple of 2^20), else the plain count."""
    return f"{n >> 20}M" if n % (1 << 20) == 0 else str(n)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="zipf_16m_d128_k32768")
    ap.add_argument("--score", default="split_bf16", choices=["split_bf16", "fp32"],
                    help="FlashAssign scoring: bf16 MFMA on split operands, or fp32 MFMA (same exact result)")
    ap.add_argument("--no-compare", action="store_true", help="do not also time the other scoring mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ivf-build", action="store_true",
                    help="instead: time the IVF-Flat build (1,000,000 x 768, nlist 4096, niter 20, seed 0)")
    ap.add_argument("--knn", nargs="?", const="knn_1m_d128_q10k", default=None,
                    help="time exact k-NN (fk_knn) on a k-NN workload instead of the Lloyd iteration")
    ap.add_argument("--ooc", action="store_true",
                    help="time the out-of-core iteration (pinned host X, PCIe included) on --ooc-rows rows of the "
                         "1e9 x 128, K = 32768 mixture")
    ap.add_argument("--ooc-rows", type=int, default=1 << 27)
    ap.add_argument("--micro", action="store_true",
                    help="only run the on-box microbenchmarks (HBM copy/read, row gather, MFMA loops, pinned H2D)")
    ap.add_argument("--no-micro", action="store_true", help="do not measure the on-box peaks beside the spec")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference kernel that scales the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path; "
              "a GPU's shard of the points is what one GPU measures.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_lloyd_means_flashassign_amd as fk
    import synth

    if args.copy_calibration:
        n = 1 << 28  # 2^28 floats = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 3}))
        return

    if args.micro:
        return micro_bench(args, torch)
    fk.load()
    if args.knn:
        return knn_bench(args, fk, synth, np, torch)
    if args.ooc:
        return ooc_bench(args, fk, synth, np, torch)
    if args.ivf_build:
        return ivf_build_bench(args, fk, synth, np, torch)
    w = synth.WORKLOADS[args.workload]
    if w.chunk_rows:
        raise SystemExit("the out-of-core workload is not a bench line; use the in-core workloads")
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    X = synth.rows(w)
    C0 = synth.initial_centroids(w, X)
    log(f"generated {w.name}: N={w.N} d={w.d} K={w.K} in {time.perf_counter() - t0:.1f} s")
    Xd = torch.from_numpy(X).to(dev)
    Cs = [torch.from_numpy(C0).to(dev), torch.empty((w.K, w.d), dtype=torch.float32, device=dev)]
    a = torch.empty(w.N, dtype=torch.int32, device=dev)
    counts = torch.empty(w.K, dtype=torch.int32, device=dev)
    ws = torch.empty(fk.fk_workspace_size(w.N, w.d, w.K, w.metric) + 256, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run(score, steps, warmup):
        def step(i):
            fk.fk_lloyd_iter(Xd, Cs[i % 2], metric=w.metric, assign=a, C_out=Cs[(i + 1) % 2], counts=counts,
                             workspace=ws, score=score)

        # every run starts from the same initial centroids
        Cs[0].copy_(C0d)
        for i in range(warmup):
            step(i)
            log(f"{score}: warmup step {i} done")
        torch.cuda.synchronize()
        # the timed steps: no phase events inside
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        log(f"{score}: timed {steps} steps in {elapsed:.3f} s")
        assert int(counts.sum().item()) == w.N
        # the same steps again with the library's phase events (the per-phase
        # times and the FlashAssign kernel's duration for the roofline line)
        fk.fk_profile_enable(True)
        for i in range(steps):
            step(warmup + steps + i)
        torch.cuda.synchronize()
        prof = fk.fk_profile_read()
        fk.fk_profile_enable(False)
        # the update on its own (fk_update: sort, reduce, finish) on the last
        # assignment, event-timed with nothing between its kernels
        Cu = torch.empty_like(Cs[0])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fk.fk_update(Xd, a, Cs[0], metric=w.metric, C_out=Cu, counts=counts, workspace=ws)
        e0.record()
        for i in range(steps):
            fk.fk_update(Xd, a, Cs[0], metric=w.metric, C_out=Cu, counts=counts, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        t_upd = e0.elapsed_time(e1) / 1e3 / steps
        return summarize(score, steps, elapsed, prof, t_upd)

    def summarize(score, steps, elapsed, prof, t_update):
        N, d, K = w.N, w.d, w.K
        sc = SCORES[score]
        ms, calls = prof["ms"], prof["calls"]
        per = {k: ms[k] / max(steps, 1) for k in ms}
        t_assign = (per["prep"] + per["assign"] + per["recheck"]) / 1e3
        flops = 2.0 * N * K * d
        upd_bytes = 4.0 * (N * d + N + K * d + K)
        fa_ms = ms["assign"] / max(calls["assign"], 1)
        fa_tflops = flops / (fa_ms / 1e3) / 1e12
        return {
            "s_per_iter": elapsed / steps,
            "assign_tflops": flops / t_assign / 1e12,
            "update_gbps": upd_bytes / t_update / 1e9,
            "assign_frac_fp32_mfma": flops / t_assign / 1e12 / FP32_MFMA_PEAK_TFLOPS,
            "assign_frac_own_mfma": flops / t_assign / 1e12 / sc["peak"],
            "update_frac_hbm": upd_bytes / t_update / 1e9 / HBM_PEAK_GBS,
            "phase_ms_per_step": {k: round(v, 4) for k, v in per.items()},
            "near_tie_fraction": {"pair": prof["paired"] / max(prof["assigned"], 1),
                                  "window": prof["windowed"] / max(prof["assigned"], 1),
                                  "all_k": prof["rechecked"] / max(prof["assigned"], 1)},
            "roofline": {"kernel": "k_flash_assign", "bound": "mfma", "mfma_dtype": sc["mfma_dtype"],
                         "achieved": fa_tflops, "peak": sc["peak"], "unit": "TFLOP/s",
                         "frac": fa_tflops / sc["peak"], "avg_ms": fa_ms,
                         "executed": fa_tflops * sc["products"],
                         "executed_frac": fa_tflops * sc["products"] / sc["peak"],
                         # split scoring issues three bf16 products per
                         # algorithmic one: frac can never exceed 1/3 there
                         "algorithmic_frac_ceiling": 1.0 / sc["products"],
                         "traffic": traffic_per_launch(w.name, score)},
        }

    C0d = torch.from_numpy(C0).to(dev)
    r = run(args.score, args.steps, args.warmup)
    out = {
        "metric": f"s per Lloyd iter; assign TFLOP/s & update GB/s at N={_rows_label(w.N)},d={w.d},K={w.K}",
        "value": r["s_per_iter"],
        "unit": "s/iter",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * r["s_per_iter"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": SCORES[args.score]["dtype"],
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "d": w.d, "K": w.K, "metric": w.metric, "sigma": w.sigma,
                   "weights": w.weights if w.weights == "equal" else f"zipf({w.zipf_s})", "seed": w.seed,
                   "score": args.score},
    }
    out.update({k: v for k, v in r.items() if k != "s_per_iter"})
    if not args.no_compare:
        out["other_scores"] = {}
        for other in SCORES:
            if other != args.score:
                out["other_scores"][other] = run(other, args.steps, args.warmup)
    if not args.no_micro:
        log("measuring the on-box peaks")
        m = micro_peaks(torch)
        out["measured_peaks"] = m
        key = "mfma_bf16_tflops" if SCORES[args.score]["mfma_dtype"] == "bf16" else "mfma_fp32_tflops"
        rf = out["roofline"]
        rf["peak_measured"] = m[key]
        rf["frac_of_measured"] = rf["achieved"] / m[key]
        rf["executed_frac_of_measured"] = rf["executed"] / m[key]
        # the update's bytes are reads (the gathered rows) with little
        # written, so it is set against the faster of the two read patterns
        read_peak = max(m["hbm_read_gbps"], m["row_gather_gbps"])
        out["update_peak_measured_gbps"] = read_peak
        out["update_frac_hbm_measured"] = out["update_gbps"] / read_peak
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, X, C0)
    else:
        out["cpu_baseline"] = None
    out["env"] = run_env(torch, np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
