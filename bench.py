#!/usr/bin/env python3
"""Throughput of lscd_spmm (Load-as-Sparse, Compute-as-Dense skinny SpMM) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 4] [--shape 0] [--n N] [--sparsity S]

A step is one lscd_spmm call, C[N][M] = A_sparse[M][K] . B[N][K]^T, over inputs already
resident in HBM; the format is encoded once before timing (ahead of time, as the method
prescribes).  The default workload is the largest configuration, the OPT-175B-shaped MLP2
(12288 x 49152, 60 % unstructured sparsity, N = 64).  To keep the 256 MB Infinity Cache from
serving A, the timed loop rotates over several device copies of the encoded matrix whose
total exceeds three times that cache.

Printed (one JSON line on stdout):
  value         effective GB/s = (4*nnz + 4*(tiles+1) + 2*K*N + 2*M*N) / wall time per step
  tflops        dense-equivalent 2*M*N*K / wall time per step
  roofline      the product's algorithmic bytes / its average device time per step, from a HIP
                event pair on the launch stream around the timed steps (one graph replay),
                against 8 TB/s HBM; stream_frac = the same against the streaming-read reference
  stream_ref    a plain streaming read of the same byte count with the product's own loads
                (lscd_stream_read), rotated over as many buffers and timed the same way: how
                fast this GPU streams that many bytes, the ceiling of a memory-bound kernel
  dense_hipblaslt  the same product as a dense fp16 GEMM: hipBLASLt with the fastest of its
                heuristic's candidates (lscd_tune_dense, through lscd_linear), timed the same way;
                torch.mm's default choice beside it
  cpu_baseline  the plain C oracle (decode + fp64 triple loop, OpenMP over rows) on a bounded
                row sample, and single-threaded on the tiny configuration (reported baseline only)
"""
import argparse
import ctypes
import hashlib
import importlib.util
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MALL_BYTES = 256 << 20
HBM_PEAK_GBS = 8000.0
METRIC = "dense-equiv TFLOPS & effective HBM GB/s (% of roofline) per skinny SpMM, 1 GPU"
DEFAULT_CONFIG = 4          # the largest configuration: OPT-175B MLP2, 12288 x 49152, 60 %, N = 64
WARM_S = 0.3                # untimed graph replays before the timed one, seconds


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG,
                    help="1..5: tiny, OPT-30B MLP1, OPT-66B QKV, OPT-175B MLP2 (default), OPT-175B layer at 50%%")
    ap.add_argument("--shape", type=int, default=0, help="config 5 only: 0 QKV, 1 OutProj, 2 MLP1, 3 MLP2")
    ap.add_argument("--n", type=int, default=None, help="batch width N (default: the config's)")
    ap.add_argument("--sparsity", type=float, default=None, help="override the config's sparsity")
    ap.add_argument("--format", choices=("tiled-csl", "bitmap", "three-level"), default="tiled-csl",
                    help="sparse format of A: Tiled-CSL (the method's, default), the bitmap-tile variant or "
                         "the three-level (4:2 + slot filling + residual) variant")
    ap.add_argument("--copies", type=int, default=0, help="encoded copies rotated in the timed loop (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense hipBLASLt baseline")
    ap.add_argument("--no-stream-ref", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU baseline sample budget")
    ap.add_argument("--eager", action="store_true",
                    help="time eager calls with an event pair around each (default: one HIP graph replay)")
    ap.add_argument("--sweep-n", default=None, metavar="N1,N2,...",
                    help="instead of the benchmark line: time the sparse product, the tuned dense GEMM and "
                         "lscd_linear's choice for each N on the config's matrix, one JSON line each")
    ap.add_argument("--encode", action="store_true",
                    help="instead of the benchmark line: time the device encoder (lscd_encode_device) and "
                         "the host encoder (lscd_pack) on the config's matrix, one JSON line")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (scale for the HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(fmt="tiled-csl"):
    """Short hash of the device sources behind one format's product: committed counter figures
    are valid only for them."""
    spec = importlib.util.spec_from_file_location("_lscd_build", os.path.join(ROOT, "unstructured_sparse_skinny_amd",
                                                                               "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    h = hashlib.sha256()
    for rel in mod.DEVICE_SOURCES_BY_FORMAT[fmt]:
        with open(os.path.join(ROOT, "unstructured_sparse_skinny_amd", rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


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


class Timing:
    """Result of time_calls (all times in ms per step)."""

    def __init__(self, wall, dev_mean, spread=None, pct=None):
        self.wall, self.dev_mean, self.spread, self.pct = wall, dev_mean, spread, pct


def time_calls(fn_args, steps, warmup, torch, graph=True, spread_replays=5):
    """Time `steps` calls rotating over fn_args, after `warmup` eager calls.

    graph=True: the steps are captured once into a HIP graph on a side stream and, after
    untimed replays for WARM_S seconds, the timed region is one replay (how a serving loop
    would launch them; no Python in between).  A
    HIP event pair on that stream around the replay gives the average device time per step.
    Then `spread_replays` further replays, each between its own event pair, give the spread
    of that average from replay to replay (a graph replay has no per-step events, so no
    per-step percentiles are claimed).  graph=False: eager calls with an event pair around
    each one; p10 / p50 / p90 over the calls.
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
        # untimed replays: the first uploads the graph; the rest, for at least WARM_S seconds,
        # bring the GPU to its steady clocks (a first replay right after a cold start measured
        # up to 8 % slower than the ones after it)
        t_w = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t_w >= WARM_S:
                break
        t_s, t_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):            # one more untimed replay, with the timing events
            t_s.record(side)                       # themselves already in use
            g.replay()
            t_e.record(side)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(side):
            t_s.record(side)
            g.replay()
            t_e.record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dev = t_s.elapsed_time(t_e) / steps
        spread = []
        for _ in range(spread_replays):
            with torch.cuda.stream(side):
                t_s.record(side)
                g.replay()
                t_e.record(side)
            torch.cuda.synchronize()
            spread.append(t_s.elapsed_time(t_e) / steps)
        del g
        return Timing(wall / steps * 1e3, dev, spread=spread)
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
    return Timing(wall / steps * 1e3, sum(ev) / len(ev),
                  pct=(ev[len(ev) // 10], ev[len(ev) // 2], ev[(len(ev) * 9) // 10]))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(case, tile_m, alg_bytes, flops, budget_s):
    """The plain C oracle on a bounded sample of the same matrices, scaled to the whole product:
    the Tiled-CSL decode of a few whole row blocks (encoded by the oracle's own encoder, untimed,
    ahead of time as the method prescribes) and the fp64 triple loop over a random sample of rows
    sized to the budget, both with every OpenMP thread of the host.  Also the tiny configuration,
    whole and single-threaded."""
    import numpy as np
    import lscd_synth as syn
    from oracle import loop, tiled_csl
    threads = loop.max_threads()
    rng = np.random.default_rng(0)
    MB = -(-case.M // tile_m)
    # decode leg: 8 random row blocks
    blocks = np.sort(rng.choice(MB, size=min(MB, 8), replace=False))
    rows_d = np.concatenate([np.arange(b * tile_m, min(case.M, (b + 1) * tile_m)) for b in blocks])
    w, o = tiled_csl.encode_canonical(case.A16[rows_d], case.mask[rows_d], tile_m, 64)
    t0 = time.perf_counter()
    loop.decode(w, o, rows_d.size, case.K, tile_m, 64)
    t_dec = (time.perf_counter() - t0) * MB / blocks.size
    # loop leg: rows of the decoded matrix (the masked weights), sized from a probe to the budget
    probe = np.sort(rng.choice(case.M, size=min(case.M, 4 * threads), replace=False))
    dp = tiled_csl.masked(case.A16[probe], case.mask[probe])
    t0 = time.perf_counter()
    loop.spmm(dp, case.B16)
    t_probe = time.perf_counter() - t0
    rows_n = int(min(case.M, max(probe.size, probe.size * budget_s / max(t_probe, 1e-6))))
    rows = np.sort(rng.choice(case.M, size=rows_n, replace=False))
    dense = tiled_csl.masked(case.A16[rows], case.mask[rows])
    t0 = time.perf_counter()
    loop.spmm(dense, case.B16)
    t_loop = time.perf_counter() - t0
    del dense
    t_full = t_dec + t_loop * case.M / rows_n
    # the tiny configuration (1024 x 1024, 80 %, N = 8), whole, on one thread
    tiny = syn.make_config(1)
    tw, to = tiled_csl.encode_canonical(tiny.A16, tiny.mask, 64, 64)
    t0 = time.perf_counter()
    d1 = loop.decode(tw, to, tiny.M, tiny.K, 64, 64)
    loop.spmm(d1, tiny.B16, threads=1)
    t1 = time.perf_counter() - t0
    nnz1 = int(np.count_nonzero(tiny.mask))
    b1 = 4 * nnz1 + 4 * to.size + 2 * tiny.K * tiny.N + 2 * tiny.M * tiny.N
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"value": round(alg_bytes / t_full / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "tflops": round(flops / t_full / 1e12, 6), "seconds_full_matrix": round(t_full, 2),
            "nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu": cpu_model(),
            "sample": f"C oracle (oracle/spmm_loop.c) with {threads} OpenMP threads: Tiled-CSL decode of {blocks.size} "
                      f"random row blocks of {tile_m} rows (scaled by {MB} / {blocks.size}) plus the fp64 triple loop "
                      f"over {rows_n} random rows of the decoded weights ({t_loop:.2f} s, scaled by M / {rows_n}); "
                      f"seed 0",
            "tiny_single_thread": {"workload": tiny.name, "value": round(b1 / t1 / 1e9, 4), "unit": "GB/s",
                                   "seconds": round(t1, 4), "cores": 1,
                                   "what": "decode + triple loop of the whole tiny product on one thread"}}


def stream_reference(L, torch, nbytes, copies, steps, warmup, eager):
    """lscd_stream_read over `nbytes` rotated over `copies` buffers, timed like the product; the
    best of 1, 2, 4 and 8 workgroups per CU."""
    nb = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    for b in bufs:
        b.random_(0, 255)
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    fn = L._lib.lscd_stream_read

    def checked(*a):
        st = fn(*a)
        if st != 0:
            raise L.LSCDError(st, "lscd_stream_read")

    res = {}
    for bpc in (1, 2, 4, 8):
        calls = [(checked, (ctypes.c_void_p(b.data_ptr()), nb, bpc, ctypes.c_void_p(sink.data_ptr()), _Cur(torch)))
                 for b in bufs]
        t = time_calls(calls, steps, warmup, torch, graph=not eager, spread_replays=0)
        res[bpc] = t.dev_mean
    del bufs
    best = min(res, key=res.get)
    return {"gbs": round(nbytes / (res[best] * 1e-3) / 1e9, 1), "us": round(res[best] * 1e3, 2),
            "bytes": int(nbytes), "workgroups_per_cu": best, "copies": copies,
            "us_by_workgroups_per_cu": {str(k): round(v * 1e3, 2) for k, v in res.items()},
            "frac_of_peak": round(nbytes / (res[best] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "lscd_stream_read (128-bit non-temporal buffer loads, one contiguous range per workgroup)"}


class _Cur:
    """ctypes stream argument read at call time, so captured calls land on the capture stream."""

    def __init__(self, torch):
        self.torch = torch

    @property
    def _as_parameter_(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)


def dense_copies(M, K):
    return max(2, min(16, math.ceil(3 * MALL_BYTES / (2 * M * K)) + 1))


def sweep_n(args, case, L, torch, np):
    """N sweep to the dense crossover: the sparse product (lscd_spmm), the dense GEMM (torch.mm, i.e.
    hipBLASLt's default choice, and the library's dense path with hipBLASLt tuned for N) and
    lscd_linear's own choice, for every N of --sweep-n.  Every leg rotates over copies of its
    matrix (sparse: encoded copies; dense: decoded copies) whose total exceeds three times the
    Infinity Cache, and runs as one graph replay (lscd_linear eagerly when its dense path cannot
    be captured)."""
    M, K = case.M, case.K
    if args.format == "tiled-csl":
        tm = L.lscd_default_tile_m(M, K)
        words, offs = L.lscd_pack(case.A16, case.mask, tm, 64)
        h0 = L.lscd_import(words, offs, M, K, tm, 64)
        info = h0.info
        copies = max(2, min(8, math.ceil(3 * MALL_BYTES / info["format_bytes"]) + 1))
        hs = [h0] + [L.lscd_import(words, offs, M, K, tm, 64) for _ in range(copies - 1)]
        del words, offs
    else:
        enc = L.lscd_encode_bitmap if args.format == "bitmap" else L.lscd_encode_three_level
        h0 = enc(case.A16, case.mask)
        info = h0.info
        copies = max(2, min(8, math.ceil(3 * MALL_BYTES / info["format_bytes"]) + 1))
        hs = [h0] + [enc(case.A16, case.mask) for _ in range(copies - 1)]
    nd = min(len(hs), dense_copies(M, K))
    for h in hs[:nd]:
        L.lscd_attach_dense(h)
    Ad = torch.from_numpy(np.where(case.mask.astype(bool), case.A16, 0).astype(np.uint16).view(np.float16))
    Ads = [Ad.to("cuda") for _ in range(nd)]
    del Ad
    gen = torch.Generator().manual_seed(1234)
    last_sparse_win = None
    for N in [int(x) for x in args.sweep_n.split(",")]:
        B = torch.randn(N, K, generator=gen).half().to("cuda")
        C = torch.empty(N, M, dtype=torch.float16, device="cuda")
        ts = time_calls([(L.lscd_spmm, (h, B, C)) for h in hs], args.steps, args.warmup, torch).dev_mean
        td = time_calls([(torch.mm, (B, a.t())) for a in Ads], args.steps, args.warmup, torch).dev_mean
        tune = [L.lscd_tune_dense(h, B, C)[0] for h in hs[:nd]]
        for h in hs[:nd]:
            L.lscd_set_linear_crossover(h, 0)
        try:
            tt = time_calls([(L.lscd_linear, (h, B, C)) for h in hs[:nd]], args.steps, args.warmup, torch).dev_mean
        except RuntimeError:
            tt = time_calls([(L.lscd_linear, (h, B, C)) for h in hs[:nd]], args.steps, args.warmup, torch,
                            graph=False).dev_mean
        for h in hs[:nd]:
            L.lscd_set_linear_crossover(h, -1)
        path = L.lscd_linear_path(hs[0], N)
        lt_s, lt_d, lt_measured = L.lscd_linear_times(hs[0], N)
        tl = ts if path == 0 else tt
        ms, md = L.lscd_linear_model(M, K, info["nnz_padded"], info["num_tiles"], N)
        if args.format != "tiled-csl":
            ms = None  # the variant formats are costed per tile, not by this model
        if ts < min(td, tt):
            last_sparse_win = N
        print(json.dumps({"sweep": "n", "workload": case.name, "format": args.format, "M": M, "K": K, "N": N,
                          "sparsity": round(case.sparsity, 4), "sparse_us": round(ts * 1e3, 1),
                          "dense_torch_mm_us": round(td * 1e3, 1), "dense_tuned_us": round(tt * 1e3, 1),
                          "tune_us": [round(t, 1) for t in tune], "linear_us": round(tl * 1e3, 1),
                          "linear_path": ["sparse", "dense"][path],
                          "linear_picks_faster": (path == 0) == (ts <= tt),
                          "linear_compared_us": [round(lt_s, 1), round(lt_d, 1)], "linear_measured": lt_measured,
                          "model_sparse_us": None if ms is None else round(ms, 1), "model_dense_us": round(md, 1),
                          "sparse_pct_roofline": round(100 * (4 * info["nnz"] + 4 * (info["num_tiles"] + 1) +
                                                              2 * K * N + 2 * M * N) / (ts * 1e-3) / 1e9 /
                                                       HBM_PEAK_GBS, 1) if args.format == "tiled-csl" else None,
                          "speedup_vs_tuned_dense": round(tt / ts, 3),
                          "speedup_vs_fastest_dense": round(min(tt, td) / ts, 3),
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


VARIANTS = ["shared-B", "independent-4", "independent-8", "wide", "bitmap", "three-level", "shared-B-3"]


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
    tm = L.lscd_default_tile_m(M, K)           # the tile height lscd_encode would use
    if args.format == "bitmap":
        h0 = L.lscd_encode_bitmap(case.A16, case.mask)
    elif args.format == "three-level":
        h0 = L.lscd_encode_three_level(case.A16, case.mask)
    else:
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

    calls = [(checked, (ctypes.c_void_p(h.ptr), ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(C.data_ptr()),
                        N, _Cur(torch))) for h in handles]
    log("[bench] timing lscd_spmm (HIP graph of the timed steps)" if not args.eager else "[bench] timing lscd_spmm")
    ts = time_calls(calls, args.steps, args.warmup, torch, graph=not args.eager)
    if not torch.isfinite(C.float()).all():
        raise RuntimeError("non-finite output")
    value = alg_bytes / (ts.wall * 1e-3) / 1e9
    achieved = alg_bytes / (ts.dev_mean * 1e-3) / 1e9
    if ts.pct:
        log(f"[bench] lscd: {ts.wall * 1e3:.1f} us/step wall, device events {ts.dev_mean * 1e3:.1f} us/step "
            f"(p10 {ts.pct[0] * 1e3:.1f}, p50 {ts.pct[1] * 1e3:.1f}, p90 {ts.pct[2] * 1e3:.1f}) -> {achieved:.0f} GB/s")
    else:
        log(f"[bench] lscd: {ts.wall * 1e3:.1f} us/step wall, device events {ts.dev_mean * 1e3:.1f} us/step "
            f"(mean of {args.steps} steps in one replay; further replays "
            f"{', '.join(f'{x * 1e3:.1f}' for x in ts.spread)}) -> {achieved:.0f} GB/s")

    stream = None
    if not args.no_stream_ref:
        log("[bench] streaming-read reference of the same byte count")
        stream = stream_reference(L, torch, alg_bytes, copies, args.steps, args.warmup, args.eager)
        log(f"[bench] stream read: {stream['us']:.1f} us -> {stream['gbs']:.0f} GB/s "
            f"({stream['workgroups_per_cu']} workgroups per CU); product at "
            f"{100 * achieved / stream['gbs']:.1f} % of it")

    dense = None
    if not args.no_dense:
        dense_bytes = 2 * M * K + 2 * K * N + 2 * M * N
        ncopy = min(len(handles), dense_copies(M, K))
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
                                 N, _Cur(torch))) for h in handles[:ncopy]]
        d_graph = not args.eager
        try:
            td = time_calls(dcalls, args.steps, args.warmup, torch, graph=d_graph, spread_replays=0)
        except RuntimeError:
            d_graph = False
            td = time_calls(dcalls, args.steps, args.warmup, torch, graph=False)
        # torch.mm on the masked matrix (hipBLASLt through PyTorch, its default choice), eager
        log("[bench] timing dense fp16 GEMM: torch.mm (default algorithm)")
        Ad = torch.from_numpy(np.where(case.mask.astype(bool), case.A16, 0).astype(np.uint16).view(np.float16))
        Ads = [Ad.to("cuda") for _ in range(ncopy)]
        del Ad
        tcalls = [(lambda x, y: torch.mm(x, y, out=Cd), (B, a.t())) for a in Ads]
        tt = time_calls(tcalls, args.steps, args.warmup, torch, graph=False)
        del Ads
        dense = {"ms_per_step": round(td.wall, 5), "kernel_ms_mean": round(td.dev_mean, 5),
                 "effective_gbs": round(dense_bytes / (td.wall * 1e-3) / 1e9, 1),
                 "tflops": round(flops / (td.wall * 1e-3) / 1e12, 2), "copies": ncopy,
                 "lscd_speedup": round(td.wall / ts.wall, 3),
                 "lscd_speedup_device": round(td.dev_mean / ts.dev_mean, 3),
                 "lscd_speedup_vs_fastest_dense": round(min(td.wall, tt.wall) / ts.wall, 3),
                 "library": "hipBLASLt, fastest of %d heuristic candidates (lscd_tune_dense)" % tuned[0][1],
                 "timing": "one HIP graph replay" if d_graph else "eager, event pair per call",
                 "tune_us_rotating": [round(t[0], 2) for t in tuned],
                 "torch_mm_ms_per_step": round(tt.wall, 5), "lscd_speedup_vs_torch_mm": round(tt.wall / ts.wall, 3),
                 "blas": str(torch.backends.cuda.preferred_blas_library())}
        log(f"[bench] dense (tuned hipBLASLt): {td.wall * 1e3:.1f} us/step -> speedup of lscd "
            f"{td.wall / ts.wall:.2f}x; torch.mm {tt.wall * 1e3:.1f} us/step ({tt.wall / ts.wall:.2f}x)")

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(case, info["tile_m"], alg_bytes, flops, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['cpu']})")

    # HBM bytes per launch from the committed counter summary of this workload, valid only
    # while the kernel sources and launch plan are the ones the counters were taken with.
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{case.name}.json")
    src_hash = kernel_source_hash(args.format)
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        launch = t.get("launch", {})
        if (args.format == "tiled-csl" and t.get("kernel_source_hash") == src_hash and launch.get("splits") == split
                and launch.get("reg_vectors") == info["reg_vectors"]):
            traffic = t.get("hbm_bytes_per_launch")

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "stream_frac": round(achieved / stream["gbs"], 4) if stream else None,
                "kernel": "lscd_spmm" + (" (product kernel + split-K pass)" if split > 1 else " (product kernel)"),
                "bytes_per_launch": alg_bytes, "kernel_source_hash": src_hash,
                "kernel_us_mean": round(ts.dev_mean * 1e3, 2),
                "timing": "eager, event pair per call" if args.eager else
                          "one HIP graph replay of the timed steps, event pair on its stream around it"}
    if ts.pct:
        roofline.update({"kernel_us_p10": round(ts.pct[0] * 1e3, 2), "kernel_us_p50": round(ts.pct[1] * 1e3, 2),
                         "kernel_us_p90": round(ts.pct[2] * 1e3, 2)})
    else:
        roofline["replay_means_us"] = [round(x * 1e3, 2) for x in ts.spread]
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ts.wall, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": case.name, "format": args.format, "M": M, "K": K, "N": N,
                   "sparsity": round(case.sparsity, 4),
                   "nnz": nnz, "tile": f"{info['tile_m']}x{info['tile_k']}", "splits": split,
                   "variant": VARIANTS[variant_id],
                   "copies_rotated": copies, "gpu": props.name, "cus": props.multi_processor_count},
        "tflops": round(flops / (ts.wall * 1e-3) / 1e12, 2),
        "pct_roofline": round(100 * value / HBM_PEAK_GBS, 1),
        "roofline": roofline,
        "stream_ref": stream,
        "dense_hipblaslt": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
