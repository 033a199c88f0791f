#!/usr/bin/env python3
"""Throughput of lscd_spmm (Load-as-Sparse, Compute-as-Dense skinny SpMM) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--shape 0] [--n N] [--sparsity S]

A step is one lscd_spmm call, C[N][M] = A_sparse[M][K] . B[N][K]^T, over inputs already
resident in HBM; the format is encoded once before timing (ahead of time, as the method
prescribes).  To keep the 256 MB Infinity Cache from serving A, the timed loop rotates over
several device copies of the encoded matrix whose total exceeds three times that cache.

Printed (one JSON line on stdout):
  value         effective GB/s = (4*nnz + 4*(tiles+1) + 2*K*N + 2*M*N) / wall time per step
  tflops        dense-equivalent 2*M*N*K / wall time per step
  roofline      the product kernel's algorithmic bytes / its average duration from a HIP
                event pair around the timed steps (one graph replay), against 8 TB/s HBM
  dense_hipblaslt  the same product as a dense fp16 GEMM: hipBLASLt with the fastest of its
                heuristic's candidates (lscd_tune_dense, through lscd_linear), timed the same way;
                torch.mm's default choice beside it
  cpu_baseline  the CPU oracle on a bounded row sample (reported baseline only)
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MALL_BYTES = 256 << 20
HBM_PEAK_GBS = 8000.0
METRIC = "dense-equiv TFLOPS & effective HBM GB/s (% of roofline) per skinny SpMM, 1 GPU"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="1..5: tiny, OPT-30B MLP1, OPT-66B QKV, "
                                                           "OPT-175B MLP2, OPT-175B layer at 50%%")
    ap.add_argument("--shape", type=int, default=0, help="config 5 only: 0 QKV, 1 OutProj, 2 MLP1, 3 MLP2")
    ap.add_argument("--n", type=int, default=None, help="batch width N (default: the config's)")
    ap.add_argument("--sparsity", type=float, default=None, help="override the config's sparsity")
    ap.add_argument("--format", choices=("tiled-csl", "bitmap", "three-level"), default="tiled-csl",
                    help="sparse format of A: Tiled-CSL (the method's, default), the bitmap-tile variant or "
                         "the three-level (4:2 + slot filling + residual) variant")
    ap.add_argument("--copies", type=int, default=0, help="encoded copies rotated in the timed loop (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense hipBLASLt baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU baseline sample budget")
    ap.add_argument("--eager", action="store_true",
                    help="time eager calls with an event pair around each (default: one HIP graph replay)")
    ap.add_argument("--sweep-n", default=None, metavar="N1,N2,...",
                    help="instead of the benchmark line: time the sparse product, the dense GEMM and "
                         "lscd_linear (cost-model choice) for each N on the config's matrix, one JSON line each")
    ap.add_argument("--encode", action="store_true",
                    help="instead of the benchmark line: time the device encoder (lscd_encode_device) and "
                         "the host encoder (lscd_pack) on the config's matrix, one JSON line")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (scale for the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Short hash of the device source: committed counter figures are valid only for it."""
    with open(os.path.join(ROOT, "unstructured_sparse_skinny_amd/csrc/lscd_kernels.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def calibrate():
    """A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE give the counters' scale."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy (torch copy_ of a 1 GiB uint8 tensor)",
                      "bytes_read_per_dispatch": n, "bytes_written_per_dispatch": n, "dispatches": 5}))


def time_calls(fn_args, steps, warmup, torch, graph=True):
    """Time `steps` calls rotating over fn_args, after `warmup` eager calls.

    graph=True: the steps are captured once into a HIP graph on a side stream and the timed
    region is one replay (how a serving loop would launch them; no Python in between).  A
    HIP event pair on that stream around the replay gives the average device time per
    step.  graph=False: eager calls with an event pair around each one.
    Returns (wall ms per step, mean device ms per step, median, p10, p90).
    """
    k = len(fn_args)
    for i in range(warmup):
        f, a = fn_args[i % k]
        f(*a)
    torch.cuda.synchronize()
    if graph:
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    f, a = fn_args[i % k]
                    f(*a)
        g.replay()                                    # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        t_s, t_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        with torch.cuda.stream(side):
            t_s.record(side)
            g.replay()
            t_e.record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dev = t_s.elapsed_time(t_e) / steps
        return wall / steps * 1e3, dev, dev, dev, dev
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        f, a = fn_args[i % k]
        starts[i].record(stream)
        f(*a)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = sorted(s_.elapsed_time(e) for s_, e in zip(starts, ends))
    return wall / steps * 1e3, sum(ev) / len(ev), ev[len(ev) // 2], ev[len(ev) // 10], ev[(len(ev) * 9) // 10]


def cpu_baseline(case, alg_bytes, flops, budget_s):
    """The oracle's fp64 product on a bounded sample of rows, scaled to the same units as `value`."""
    import numpy as np
    from oracle import spmm as osp
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(case.M, size=min(case.M, 256), replace=False))
    t0 = time.perf_counter()
    osp.spmm_f64(case.A16, case.mask, case.B16, rows=probe)
    t_probe = time.perf_counter() - t0
    rows_n = int(min(case.M, max(len(probe), len(probe) * budget_s / max(t_probe, 1e-6))))
    rows = np.sort(rng.choice(case.M, size=rows_n, replace=False))
    passes, dt = 0, 0.0
    while passes == 0 or dt < budget_s:       # repeat a fast sample until the budget is used
        t0 = time.perf_counter()
        osp.spmm_f64(case.A16, case.mask, case.B16, rows=rows)
        dt += time.perf_counter() - t0
        passes += 1
    frac = rows_n * passes / case.M
    return {"value": round(alg_bytes * frac / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "tflops": round(flops * frac / dt / 1e12, 5), "seconds": round(dt, 2),
            "sample": f"{passes} pass(es) over {rows_n} of {case.M} rows (random, seed 0) of the same matrices; "
                      f"fp64 numpy/BLAS product of the masked rows; bytes and flops scaled by rows computed / M"}


def sweep_n(args, case, L, torch, np):
    """N sweep to the dense crossover: sparse (lscd_spmm), dense (torch.mm -> hipBLASLt's default
    choice, and the library's dense path with hipBLASLt tuned for N) and lscd_linear's own
    choice on the attached dense copy, for every N of --sweep-n."""
    M, K = case.M, case.K
    if args.format == "tiled-csl":
        tm = L.lscd_default_tile_m(M, K)
        words, offs = L.lscd_pack(case.A16, case.mask, tm, 64)
        h0 = L.lscd_import(words, offs, M, K, tm, 64)
        info = h0.info
        copies = max(1, min(8, math.ceil(3 * MALL_BYTES / info["format_bytes"])))
        hs = [h0] + [L.lscd_import(words, offs, M, K, tm, 64) for _ in range(copies - 1)]
        del words, offs
    else:
        enc = L.lscd_encode_bitmap if args.format == "bitmap" else L.lscd_encode_three_level
        h0 = enc(case.A16, case.mask)
        info = h0.info
        copies = max(1, min(8, math.ceil(3 * MALL_BYTES / info["format_bytes"])))
        hs = [h0] + [enc(case.A16, case.mask) for _ in range(copies - 1)]
    Ad = torch.from_numpy(np.where(case.mask.astype(bool), case.A16, 0).astype(np.uint16).view(np.float16))
    dcopies = max(1, min(4, math.ceil(3 * MALL_BYTES / (2 * M * K))))
    Ads = [Ad.to("cuda") for _ in range(dcopies)]
    del Ad
    L.lscd_attach_dense(h0)
    gen = torch.Generator().manual_seed(1234)
    last_sparse_win = None
    for N in [int(x) for x in args.sweep_n.split(",")]:
        B = torch.randn(N, K, generator=gen).half().to("cuda")
        C = torch.empty(N, M, dtype=torch.float16, device="cuda")
        _, ts, *_ = time_calls([(L.lscd_spmm, (h, B, C)) for h in hs], args.steps, args.warmup, torch)
        _, td, *_ = time_calls([(torch.mm, (B, a.t())) for a in Ads], args.steps, args.warmup, torch)
        # the library's dense path with hipBLASLt tuned for this N, then lscd_linear's own choice
        tune_us, _ = L.lscd_tune_dense(h0, B, C)
        L.lscd_set_linear_crossover(h0, 0)
        _, tt, *_ = time_calls([(L.lscd_linear, (h0, B, C))], args.steps, args.warmup, torch, graph=False)
        L.lscd_set_linear_crossover(h0, -1)
        _, tl, *_ = time_calls([(L.lscd_linear, (h0, B, C))], args.steps, args.warmup, torch, graph=False)
        ms, md = L.lscd_linear_model(M, K, info["nnz_padded"], info["num_tiles"], N)
        if args.format != "tiled-csl":
            ms = None  # the variant formats are costed per tile, not by this model
        if ts < min(td, tt):
            last_sparse_win = N
        print(json.dumps({"sweep": "n", "workload": case.name, "format": args.format, "M": M, "K": K, "N": N,
                          "sparsity": round(case.sparsity, 4), "sparse_us": round(ts * 1e3, 1),
                          "dense_hipblaslt_us": round(td * 1e3, 1), "dense_tuned_us": round(tt * 1e3, 1),
                          "tune_us": round(tune_us, 1), "linear_us": round(tl * 1e3, 1),
                          "linear_path": ["sparse", "dense"][L.lscd_linear_path(h0, N)],
                          "model_sparse_us": None if ms is None else round(ms, 1), "model_dense_us": round(md, 1),
                          "sparse_tflops": round(2 * M * N * K / (ts * 1e-3) / 1e12, 1)}), flush=True)
    print(json.dumps({"sweep": "n", "workload": case.name, "largest_n_sparse_wins": last_sparse_win}), flush=True)


def bench_encode(args, case, L, torch, np):
    """Device encoder vs host encoder on the same matrix (dense fp16 + mask in, format out)."""
    M, K = case.M, case.K
    Ad = torch.from_numpy(case.A16.view(np.float16)).to("cuda")
    md = torch.from_numpy(case.mask.astype(np.uint8)).to("cuda")
    in_bytes = 3 * M * K                                   # fp16 values + mask bytes
    L.lscd_encode_device(Ad, md).close()                   # warm-up (module load, first allocations)
    torch.cuda.synchronize()
    reps = max(3, args.steps // 20)
    t0 = time.perf_counter()
    for _ in range(reps):
        h = L.lscd_encode_device(Ad, md)
        h.close()
    t_dev = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    words, offs = L.lscd_pack(case.A16, case.mask, L.lscd_default_tile_m(M, K), 64)
    t_host = time.perf_counter() - t0
    print(json.dumps({"encode": "tiled-csl 64x64", "workload": case.name, "M": M, "K": K,
                      "nnz_padded": int(words.size), "device_ms": round(t_dev * 1e3, 3),
                      "device_input_gbs": round(in_bytes / t_dev / 1e9, 1), "device_reps": reps,
                      "host_ms": round(t_host * 1e3, 1), "host_threads": os.cpu_count(),
                      "speedup": round(t_host / t_dev, 1),
                      "note": "wall time per synchronous call, allocations included"}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part of this "
              "build: the product shards by rows or by K with no kernel change (see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calibrate:
        calibrate()
        return
    import lscd_synth as syn
    import unstructured_sparse_skinny_amd as L

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    t_gen = time.perf_counter()
    case = syn.make_config(args.config, args.shape, N=args.n, sparsity=args.sparsity)
    M, K, N = case.M, case.K, case.N
    log(f"[bench] {case.name}: M={M} K={K} N={N} sparsity={case.sparsity:.4f} "
        f"(generated in {time.perf_counter() - t_gen:.1f}s)")
    if args.sweep_n:
        sweep_n(args, case, L, torch, np)
        return
    if args.encode:
        bench_encode(args, case, L, torch, np)
        return

    t_enc = time.perf_counter()
    if args.format == "bitmap":
        words, offs = L.lscd_pack_bitmap(case.A16, case.mask)
        h0 = L.lscd_encode_bitmap(case.A16, case.mask)
    elif args.format == "three-level":
        words, offs = L.lscd_pack_three_level(case.A16, case.mask)
        h0 = L.lscd_encode_three_level(case.A16, case.mask)
    else:
        tm = L.lscd_default_tile_m(M, K)       # the tile height lscd_encode would use
        words, offs = L.lscd_pack(case.A16, case.mask, tm, 64)
        h0 = L.lscd_import(words, offs, M, K, tm, 64)
    info = h0.info
    fmt_bytes = info["format_bytes"]
    copies = args.copies or max(2, min(32, math.ceil(3 * MALL_BYTES / fmt_bytes) + 1))
    if args.format == "bitmap":
        handles = [h0] + [L.lscd_encode_bitmap(case.A16, case.mask) for _ in range(copies - 1)]
    elif args.format == "three-level":
        handles = [h0] + [L.lscd_encode_three_level(case.A16, case.mask) for _ in range(copies - 1)]
    else:
        handles = [h0] + [L.lscd_import(words, offs, M, K, tm, 64) for _ in range(copies - 1)]
    del words, offs
    log(f"[bench] encoded {copies} copies of {fmt_bytes / 1e6:.1f} MB in {time.perf_counter() - t_enc:.1f}s; "
        f"splits={info['splits']} variants={info['variant']} reg_vectors={info['reg_vectors']} "
        f"max_tile_words={info['max_tile_words']}")

    nnz, tiles = info["nnz"], info["num_tiles"]
    if N <= 64:
        split, variant_id = info["splits"][L.npad_index(N)], info["variant"][L.npad_index(N)]
    else:  # the N > 64 kernel; the first launch's plan when N > 256 takes several
        npw = 128 if N <= 128 else (192 if N <= 192 else 256)
        split, variant_id = info["splits_wide"][(npw - 128) // 64], 3
    # Tiled-CSL: one 4-byte word per nonzero; bitmap and three-level tiles: the blob as stored
    stored = 4 * info["nnz_padded"] if args.format != "tiled-csl" else 4 * nnz
    alg_bytes = stored + 4 * (tiles + 1) + 2 * K * N + 2 * M * N
    flops = 2 * M * N * K

    B = torch.from_numpy(case.B16.view(np.float16)).to("cuda")
    C = torch.empty((N, M), dtype=torch.float16, device="cuda")
    fn = L._lib.lscd_spmm

    def checked(*a):
        st = fn(*a)
        if st != 0:
            raise L.LSCDError(st, "lscd_spmm")

    # the stream argument is read at call time, so captured calls land on the capture stream
    class _Cur:
        @property
        def _as_parameter_(self):
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    calls = [(checked, (ctypes.c_void_p(h.ptr), ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(C.data_ptr()),
                        N, _Cur())) for h in handles]
    log("[bench] timing lscd_spmm (HIP graph of the timed steps)")
    ms_step, ev_mean, ev_med, ev_p10, ev_p90 = time_calls(calls, args.steps, args.warmup, torch, graph=not args.eager)
    if not torch.isfinite(C.float()).all():
        raise RuntimeError("non-finite output")
    value = alg_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (ev_mean * 1e-3) / 1e9
    log(f"[bench] lscd: {ms_step * 1e3:.1f} us/step wall, device events {ev_mean * 1e3:.1f} us/step "
        f"(p10 {ev_p10 * 1e3:.1f}, p50 {ev_med * 1e3:.1f}, p90 {ev_p90 * 1e3:.1f}) -> {achieved:.0f} GB/s")

    dense = None
    if not args.no_dense:
        dense_bytes = 2 * M * K + 2 * K * N + 2 * M * N
        ncopy = min(len(handles), max(2, min(16, math.ceil(3 * MALL_BYTES / (2 * M * K)) + 1)))
        Cd = torch.empty((N, M), dtype=torch.float16, device="cuda")
        # hipBLASLt with the fastest of its heuristic's candidates for this N (lscd_tune_dense),
        # run through lscd_linear's dense path on dense copies decoded from the encoding and
        # timed like the sparse product: rotating copies, one graph replay
        log("[bench] timing dense fp16 GEMM: hipBLASLt, fastest of its heuristic's candidates")
        tuned = []
        for h in handles[:ncopy]:
            L.lscd_attach_dense(h)
            tuned.append(L.lscd_tune_dense(h, B, Cd))
            L.lscd_set_linear_crossover(h, 0)
        lin = L._lib.lscd_linear

        def lin_checked(*a):
            st = lin(*a)
            if st != 0:
                raise L.LSCDError(st, "lscd_linear")

        dcalls = [(lin_checked, (ctypes.c_void_p(h.ptr), ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(Cd.data_ptr()),
                                 N, _Cur())) for h in handles[:ncopy]]
        d_graph = not args.eager
        try:
            d_ms, d_mean, _, _, _ = time_calls(dcalls, args.steps, args.warmup, torch, graph=d_graph)
        except RuntimeError:
            d_graph = False
            d_ms, d_mean, _, _, _ = time_calls(dcalls, args.steps, args.warmup, torch, graph=False)
        # torch.mm on the masked matrix (hipBLASLt through PyTorch, its default choice), eager
        log("[bench] timing dense fp16 GEMM: torch.mm (default algorithm)")
        Ad = torch.from_numpy(np.where(case.mask.astype(bool), case.A16, 0).astype(np.uint16).view(np.float16))
        Ads = [Ad.to("cuda") for _ in range(ncopy)]
        del Ad
        tcalls = [(lambda x, y: torch.mm(x, y, out=Cd), (B, a.t())) for a in Ads]
        t_ms, _, _, _, _ = time_calls(tcalls, args.steps, args.warmup, torch, graph=False)
        del Ads
        dense = {"ms_per_step": round(d_ms, 5), "kernel_ms_mean": round(d_mean, 5),
                 "effective_gbs": round(dense_bytes / (d_ms * 1e-3) / 1e9, 1),
                 "tflops": round(flops / (d_ms * 1e-3) / 1e12, 2), "copies": ncopy,
                 "lscd_speedup": round(d_ms / ms_step, 3),
                 "library": "hipBLASLt, fastest of %d heuristic candidates (lscd_tune_dense)" % tuned[0][1],
                 "timing": "one HIP graph replay" if d_graph else "eager, event pair per call",
                 "tune_us_back_to_back": [round(t[0], 2) for t in tuned],
                 "torch_mm_ms_per_step": round(t_ms, 5), "lscd_speedup_vs_torch_mm": round(t_ms / ms_step, 3),
                 "blas": str(torch.backends.cuda.preferred_blas_library())}
        log(f"[bench] dense (tuned hipBLASLt): {d_ms * 1e3:.1f} us/step -> speedup of lscd {d_ms / ms_step:.2f}x; "
            f"torch.mm {t_ms * 1e3:.1f} us/step ({t_ms / ms_step:.2f}x)")

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(case, alg_bytes, flops, args.cpu_seconds)

    # HBM bytes per launch from the committed counter summary of this workload, valid only
    # while the kernel sources are the ones the counters were taken with.
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{case.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        launch = t.get("launch", {})
        if (args.format == "tiled-csl" and t.get("kernel_source_hash") == kernel_source_hash() and launch.get("splits") == split
                and launch.get("reg_vectors") == info["reg_vectors"]):
            traffic = t.get("hbm_bytes_per_launch")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": case.name, "format": args.format, "M": M, "K": K, "N": N,
                   "sparsity": round(case.sparsity, 4),
                   "nnz": nnz, "tile": f"{info['tile_m']}x{info['tile_k']}", "splits": split,
                   "variant": ["shared-B", "independent-4", "independent-8", "wide", "bitmap", "three-level"][variant_id],
                   "copies_rotated": copies, "gpu": props.name, "cus": props.multi_processor_count},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "pct_roofline": round(100 * value / HBM_PEAK_GBS, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "lscd_spmm" + (" (product kernel + split-K pass)" if split > 1 else " (product kernel)"),
                     "bytes_per_launch": alg_bytes, "kernel_source_hash": kernel_source_hash(),
                     "kernel_us_mean": round(ev_mean * 1e3, 2), "kernel_us_p50": round(ev_med * 1e3, 2),
                     "timing": "eager, event pair per call" if args.eager else
                               "one HIP graph replay of the timed steps, event pair around it"},
        "dense_hipblaslt": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
