"""IVF-PQ search benchmark on one MI355X.

One step = one IVF-PQ search of the whole query batch (coarse top-nprobe,
per-(query, list) tables, code scan, top-k merged across the lists) with the
index, queries and outputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--lut f32|f16]

The default workload is the largest single-GPU configuration, the 1B-entry
index with Zipf(1.1) list sizes (nlist 262,144, d 96, m 8, nprobe 128, k 100,
10,000 queries; 8 GB of codes and 8 GB of ids in HBM).  Other workloads:
the 1M and 10M Gaussian-mixture indexes, the exact bf16 flat search, index
building, k-means and the k-NN graph.  Synthetic data only (seeded).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "queries/sec at fixed nprobe,k; PQ-code scan GB/s as % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


ZIPF_WORKLOAD = "ivfpq_zipf_n1000000000_d96_m8_nlist262144"
# the Infinity Cache (MALL) of an MI355X: a code array this small stays cache
# resident across searches, so its code-byte rate is an effective rate, not
# an HBM one
MALL_BYTES = 256 << 20
# lists this long make a query's scan many times the mean (1B Zipf index)
GIANT_LIST = 1_000_000


def workload(name: str):
    from approximate_nearest_neighbour_amd import datagen as G
    makers = {"ivfpq_n1m_d128_m16_nlist1024": lambda: G.gmm1m(keep_vectors=True),
              "ivfpq_tiny_n10k_d32_m4": G.tiny,
              "ivfpq_n10m_d96_m32_nlist4096": lambda: G.gmm10m(keep_vectors=True),
              ZIPF_WORKLOAD: G.zipf_workload}
    if name not in makers:
        raise SystemExit(f"unknown workload {name}; choose from "
                         f"{sorted(makers) + EXTRA_WORKLOADS}")
    return makers[name]()


# The sources that define the scan kernel and how a search launches it (work
# items, workspace): a change to any of them retires stored counter readings.
SCAN_SOURCES = ("api.hip", "common.hpp", "internal.hpp", "kernels_search.hip", "network.hpp",
                "plan.hpp", "wave_ops.hpp", "wave_select.hpp")


def source_digest() -> str:
    """SHA-256 over the scan path's HIP sources: ties stored counter readings
    to a kernel version."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "approximate_nearest_neighbour_amd", "csrc")
    for f in SCAN_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def stored_traffic(workload: str, lut: str):
    """HBM bytes per scan launch from profiles/traffic.json (FETCH_SIZE and
    WRITE_SIZE of rocprofv3 --pmc runs scaled by a copy-kernel calibration),
    only while the kernels are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        import json as _json
        rec = _json.load(open(path)).get(f"{workload}:{lut}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest():
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def summarize_counters(paths):
    """Print per-kernel averages of rocprofv3 counter CSVs (one per pass)."""
    import collections
    import csv
    for path in paths:
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(path)):
            k = r["Kernel_Name"].split("(")[0].replace("void ", "")
            agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
        print(f"## {os.path.basename(path)}")
        for k in sorted(agg):
            n = len(disp[k])
            vals = ", ".join(f"{c}={v / n:.6g}" for c, v in sorted(agg[k].items()))
            print(f"- `{k}` ({n} dispatches, per dispatch): {vals}")


def summarize_stats(paths):
    """Print rocprofv3 --stats kernel tables (CSV) as markdown."""
    import csv
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        print(f"## {os.path.basename(path)}")
        print("| kernel | calls | total ms | average us |")
        print("|---|---:|---:|---:|")
        for r in rows:
            print(f"| `{r['Name'].split('(')[0].replace('void ', '')}` | {r['Calls']} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e3:.1f} |")


def measured_read_gbs(torch, A, gib: int = 4, reps: int = 5) -> float:
    """Streaming-read rate of this GPU: the library's reference read kernel
    over `gib` GiB (every byte read once, 16-byte loads), timed with events on
    the current stream; the best of `reps`."""
    x = torch.ones((gib << 28,), dtype=torch.float32, device="cuda:0")
    sink = torch.zeros((8192,), dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    A.ivfpq_stream_read(x, sink, stream=st)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        A.ivfpq_stream_read(x, sink, stream=st)
        b.record(st)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x, sink
    torch.cuda.empty_cache()
    return (gib << 30) / (best * 1e-3) / 1e9


def host_pointer_qps(search, nq: int, reps: int = 3) -> float:
    """Queries/s of the blocking host-pointer entry point: queries copied in,
    results copied out (PCIe included), after one untimed call."""
    search()
    t = time.perf_counter()
    for _ in range(reps):
        search()
    return nq * reps / (time.perf_counter() - t)


def scanned_entries(index, probes: np.ndarray) -> int:
    return int(index.list_sizes[probes.astype(np.int64)].sum())


def giant_list_queries(index, probes: np.ndarray) -> np.ndarray:
    """Rows whose probes include a list of more than GIANT_LIST entries."""
    big = index.list_sizes[probes.astype(np.int64)] > GIANT_LIST
    return np.flatnonzero(big.any(axis=1))


def recall_report(w, found_ids, nsample: int = 200, seed: int = 2005):
    """1-recall@k (R@k) and k-recall@k (intersection) of the search against
    the oracle's exact brute force over the database vectors, on a seeded
    sample of the queries (the two measures of "Billion-scale similarity
    search with GPUs", experiments section)."""
    from oracle import oracle as O
    if w.vectors is None:
        return None
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(len(w.queries), min(nsample, len(w.queries)), replace=False))
    # the generated indexes give database row r the id r
    _, true_ids = O.bruteforce(w.vectors, w.queries[rows], w.k)
    found = found_ids[rows]
    return {"queries": int(len(rows)), "k": int(w.k),
            "recall_1_at_k": O.recall_1_at_k(found, true_ids),
            "recall_k_at_k": O.recall_k_at_k(found, true_ids)}


def cpu_baseline(w, lut_mode, budget_s: float, probes=None):
    """The oracle, as it stands, on a bounded leading sample of the queries
    (their natural mix: on the 1B Zipf index about 4% of the queries probe a
    list above 10^6 entries, and the sample holds them at that rate)."""
    from oracle import oracle as O
    threads = O.default_threads()
    probe_n = min(len(w.queries), max(threads, 16))
    t = time.perf_counter()
    O.search(w.index, w.queries[:probe_n], w.nprobe, w.k, lut_mode=lut_mode, nthreads=threads)
    per_q = (time.perf_counter() - t) / probe_n
    n = int(min(len(w.queries), max(probe_n, budget_s / max(per_q, 1e-9))))
    t = time.perf_counter()
    od, oi, op = O.search(w.index, w.queries[:n], w.nprobe, w.k, lut_mode=lut_mode,
                          nthreads=threads)
    wall = time.perf_counter() - t
    extra = ""
    if probes is not None:
        g = int(np.sum(giant_list_queries(w.index, probes[:n]) < n))
        extra = f" ({g} of them probe a list above {GIANT_LIST:,} entries)"
    return dict(value=n / wall, unit="queries/s", cores=threads, kind="oracle",
                sample=f"first {n} of {len(w.queries)} queries{extra}, full search (fp64), "
                       f"{wall:.1f} s wall"), (n, od, oi, op)


FLAT_WORKLOAD = "flat_bf16_n1000000_d128"
BF16_MFMA_PEAK_TFLOPS = 2500.0


def bench_flat(args):
    """Exact k-NN over a flat bfloat16 database (1M x 128, 10,000 queries,
    k = 1024): one step = one search of the whole query batch."""
    import torch
    import approximate_nearest_neighbour_amd as A
    from approximate_nearest_neighbour_amd import datagen as G
    from oracle import check
    from oracle import oracle as O

    t0 = time.time()
    w = G.flat_bf16_workload()
    log(f"workload {w.name}: built in {time.time() - t0:.1f} s")
    db, qbits = w.vectors, w.queries
    n, d = db.shape
    nq, k = qbits.shape[0], w.k
    f = A.ivfpq_flat_load_bf16(db)
    q = torch.from_numpy(qbits.view(np.int16)).cuda()
    out = (torch.empty((nq, k), dtype=torch.float32, device="cuda"),
           torch.empty((nq, k), dtype=torch.int64, device="cuda"))

    def step():
        A.ivfpq_flat_search_bf16_ex(f, q, k, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    A.ivfpq_flat_profile_begin(f, args.steps)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    prof = A.ivfpq_flat_profile_end(f)
    ms_step = 1e3 * elapsed / args.steps
    calls = max(prof["calls"], 1)
    stages = {s: prof[f"{s}_ms"] / calls
              for s in ("minima", "kth", "collect", "select", "fallback")}
    log(f"step {ms_step:.3f} ms  " + "  ".join(f"{s} {v:.3f} ms" for s, v in stages.items()))
    flops = 2.0 * nq * n * d  # the distance matrix's products, counted once
    # over the whole search (every pass; the minima pass alone is reported too)
    achieved = flops / (ms_step * 1e-3) / 1e12
    minima_tflops = flops / (stages["minima"] * 1e-3) / 1e12

    host_qps = host_pointer_qps(lambda: A.ivfpq_flat_search_bf16(f, qbits, k), nq)
    log(f"host-pointer entry point: {host_qps:.0f} queries/s (PCIe copies included)")

    pn = min(args.parity_queries, nq, 64)
    rep = check.compare_flat(db, qbits[:pn], k, out[0][:pn].cpu().numpy(),
                             out[1][:pn].cpu().numpy())
    log("parity", rep.summary())
    cpu = None
    if not args.no_cpu_baseline:
        threads = O.default_threads()
        t = time.perf_counter()
        O.bruteforce_bf16(db, qbits[:threads], k, nthreads=threads)
        per_q = (time.perf_counter() - t) / threads
        m = int(min(nq, max(threads, args.cpu_seconds / max(per_q, 1e-9))))
        t = time.perf_counter()
        O.bruteforce_bf16(db, qbits[:m], k, nthreads=threads)
        wall = time.perf_counter() - t
        cpu = dict(value=m / wall, unit="queries/s", cores=threads, kind="oracle",
                   sample=f"first {m} of {nq} queries, exact brute force (fp64, full sort), "
                          f"{wall:.1f} s wall")
        log("cpu baseline", cpu)
    res = {
        "metric": METRIC,
        "value": nq / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 products, fp32 sums",
        "data": "synthetic (seeded uniform [-1, 1] rounded to bf16)",
        "config": {"workload": w.name, "n": n, "d": d, "nq": nq, "k": k},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                     "traffic": None, "kernel": "whole search (all passes, end to end)",
                     "kernel_ms": ms_step, "algorithmic_flops_per_launch": flops,
                     "minima_pass": {"kernel": "flat_gemm_kernel", "ms": stages["minima"],
                                     "achieved": minima_tflops,
                                     "frac": minima_tflops / BF16_MFMA_PEAK_TFLOPS}},
        "cpu_baseline": cpu,
        "stages_ms": stages,
        "host_pointer_qps": host_qps,
        "parity": rep.summary(),
    }
    print(json.dumps(res), flush=True)
    f.close()


ENCODE_WORKLOAD = "encode_n1m_d128_m16_nlist1024"
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32: matrix cores and (packed) vector ALU alike


def bench_encode(args):
    """Index building on the device: list assignment (coarse step, nprobe 1)
    and PQ codes of the 1M x 128 workload's 1M database vectors with its
    trained centroids (nlist 1024) and codebooks (m 16): one step = one call
    over all 1M vectors."""
    import torch
    import approximate_nearest_neighbour_amd as A
    from approximate_nearest_neighbour_amd import datagen as G
    from oracle import check
    from oracle import oracle as O

    t0 = time.time()
    w = G.gmm1m(keep_vectors=True)
    log(f"workload {ENCODE_WORKLOAD}: built in {time.time() - t0:.1f} s")
    ix = A.ivfpq_load_index_host(w.index, device=0)
    x = torch.from_numpy(w.vectors).cuda()
    n, d = x.shape
    nlist, m = ix.info["nlist"], ix.info["m"]
    dsub = d // m

    def step():
        return A.ivfpq_assign_encode_ex(ix, x)

    def timed(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        lists, codes = step()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t) / args.steps
    # the two kernels on the call's stream: the whole call, then the coarse
    # step alone (the same kernel the call launches first)
    call_ms = timed(step, args.steps)
    coarse_ms = timed(lambda: A.ivfpq_coarse_ex(ix, x, 1), args.steps)
    encode_ms = max(call_ms - coarse_ms, 1e-6)
    coarse_flops = 2.0 * n * nlist * d          # x.c for every (vector, centroid)
    encode_flops = 3.0 * n * m * 256 * dsub     # (r - C)^2 summed: sub, mul, add
    log(f"step {ms_step:.3f} ms  call {call_ms:.3f} ms  coarse {coarse_ms:.3f} ms  "
        f"encode {encode_ms:.3f} ms")
    if coarse_ms >= encode_ms:
        roof = {"bound": "mfma", "achieved": coarse_flops / (coarse_ms * 1e-3) / 1e12,
                "kernel": "coarse_argmin_kernel (nprobe 1)", "kernel_ms": coarse_ms,
                "algorithmic_flops_per_launch": coarse_flops}
    else:
        roof = {"bound": "alu", "achieved": encode_flops / (encode_ms * 1e-3) / 1e12,
                "kernel": "encode_kernel", "kernel_ms": encode_ms,
                "algorithmic_flops_per_launch": encode_flops}
    roof.update(peak=FP32_PEAK_TFLOPS, unit="TFLOP/s", frac=roof["achieved"] / FP32_PEAK_TFLOPS,
                traffic=None)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, 254), replace=False)]))
    xs = w.vectors[rows]
    rep = check.compare_encode(xs, w.index.centroids, w.index.codebooks,
                               lists.cpu().numpy()[rows], codes.cpu().numpy()[rows])
    log("parity", rep.summary())
    cpu = None
    if not args.no_cpu_baseline:
        threads = O.default_threads()
        t = time.perf_counter()
        O.assign_encode(w.vectors[:4 * threads], w.index.centroids, w.index.codebooks,
                        nthreads=threads)
        per_v = (time.perf_counter() - t) / (4 * threads)
        cnt = int(min(n, max(4 * threads, args.cpu_seconds / max(per_v, 1e-9))))
        t = time.perf_counter()
        O.assign_encode(w.vectors[:cnt], w.index.centroids, w.index.codebooks, nthreads=threads)
        wall = time.perf_counter() - t
        cpu = dict(value=cnt / wall, unit="vectors/s", cores=threads, kind="oracle",
                   sample=f"first {cnt} of {n} vectors, assignment and encoding in double "
                          f"precision, {wall:.1f} s wall")
        log("cpu baseline", cpu)
    res = {
        "metric": "database vectors assigned and PQ-encoded per second",
        "value": n / (ms_step * 1e-3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded Gaussian mixture, CPU-trained centroids and codebooks)",
        "config": {"workload": ENCODE_WORKLOAD, "n": n, "d": d, "nlist": nlist, "m": m},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages_ms": {"call": call_ms, "coarse": coarse_ms, "encode": encode_ms},
        "parity": rep.summary(),
    }
    print(json.dumps(res), flush=True)
    ix.close()


KMEANS_WORKLOAD = "kmeans_n262144_d128_k1024"


def bench_kmeans(args):
    """k-means on the device at the 1M x 128 workload's coarse training shape:
    262,144 of its vectors (seeded sample), 1,024 centers initialised with
    1,024 distinct sampled vectors; one step = one call of 10 Lloyd iterations."""
    import torch
    import approximate_nearest_neighbour_amd as A
    from approximate_nearest_neighbour_amd import datagen as G
    from oracle import check
    from oracle import oracle as O

    iters = 10
    t0 = time.time()
    w = G.gmm1m(keep_vectors=True)
    rng = np.random.default_rng(2003)
    xs = w.vectors[np.sort(rng.choice(len(w.vectors), 262_144, replace=False))]
    init = xs[rng.choice(len(xs), 1024, replace=False)]
    log(f"workload {KMEANS_WORKLOAD}: built in {time.time() - t0:.1f} s")
    x = torch.from_numpy(xs).cuda()
    c0 = torch.from_numpy(init).cuda()
    c = c0.clone()
    n, d = xs.shape
    k = init.shape[0]

    def step(count=iters):
        c.copy_(c0)
        return A.ivfpq_kmeans_ex(x, c, count)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t) / args.steps
    ms_iter = ms_step / iters
    flops = 2.0 * n * k * d                       # the assignment's x.c per iteration
    achieved = flops / (ms_iter * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms = {iters} iterations, {ms_iter:.3f} ms per iteration")
    # parity: the first iteration, checked in full against the oracle
    a1, n1 = step(1)
    rep = check.compare_kmeans_iteration(xs, init, a1.cpu().numpy(), c.cpu().numpy(),
                                         n1.cpu().numpy())
    log("parity (iteration 1)", rep.summary())
    cpu = None
    if not args.no_cpu_baseline:
        threads = O.default_threads()
        t = time.perf_counter()
        O.kmeans(xs, init, 1, nthreads=threads)
        wall = time.perf_counter() - t
        cpu = dict(value=1.0 / wall, unit="iterations/s", cores=threads, kind="oracle",
                   sample=f"one iteration over all {n} vectors (assignment in double precision, "
                          f"full sort per vector; double-precision means), {wall:.1f} s wall")
        log("cpu baseline", cpu)
    res = {
        "metric": "k-means (Lloyd) iterations per second",
        "value": 1e3 / ms_iter,
        "unit": "iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (double-precision sums)",
        "data": "synthetic (seeded Gaussian mixture sample)",
        "config": {"workload": KMEANS_WORKLOAD, "n": n, "d": d, "k": k,
                   "iterations_per_step": iters},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_PEAK_TFLOPS, "traffic": None,
                     "kernel": "one iteration (coarse assignment + update), assignment flops",
                     "kernel_ms": ms_iter, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu,
        "parity": rep.summary(),
    }
    print(json.dumps(res), flush=True)


BUILD_WORKLOAD = "build_n1m_d128_m16_nlist1024"


def bench_build(args):
    """Index built on the device: the 1M x 128 workload's 1M vectors with its
    trained centroids (nlist 1024) and codebooks (m 16), assigned, encoded and
    laid out list-major by one ivfpq_build_index_ex call (scratch allocation
    and the final synchronisation included): one step = one build."""
    import torch
    import approximate_nearest_neighbour_amd as A
    from approximate_nearest_neighbour_amd import datagen as G
    from oracle import check
    from oracle import oracle as O

    t0 = time.time()
    w = G.gmm1m(keep_vectors=True)
    log(f"workload {BUILD_WORKLOAD}: built in {time.time() - t0:.1f} s")
    x = torch.from_numpy(w.vectors).cuda()
    cent = torch.from_numpy(w.index.centroids).cuda()
    books = torch.from_numpy(w.index.codebooks).cuda()
    n, d = x.shape
    nlist, m = cent.shape[0], books.shape[0]
    for _ in range(args.warmup):
        A.ivfpq_build_index_ex(x, cent, books).close()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        ix = A.ivfpq_build_index_ex(x, cent, books)
        ix.close()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t) / args.steps
    flops = 2.0 * n * nlist * d + 3.0 * n * m * 256 * (d // m)
    achieved = flops / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms per build of {n} vectors")
    ix = A.ivfpq_build_index_ex(x, cent, books)
    got = A.ivfpq_index_export(ix)
    ix.close()
    owner = np.repeat(np.arange(nlist), got["list_sizes"])
    lists = np.empty(n, np.int32)
    codes = np.empty((n, m), np.uint8)
    lists[got["ids"]] = owner
    codes[got["ids"]] = got["codes"]
    layout_ok = bool(np.all(np.diff(got["ids"])[np.diff(owner) == 0] > 0))
    rng = np.random.default_rng(2005)
    rows = np.sort(rng.choice(n, 256, replace=False))
    rep = check.compare_encode(w.vectors[rows], w.index.centroids, w.index.codebooks,
                               lists[rows], codes[rows])
    summary = dict(rep.summary(), layout_stable=layout_ok)
    log("parity", summary)
    cpu = None
    if not args.no_cpu_baseline:
        threads = O.default_threads()
        cnt = int(min(n, 16 * threads))
        t = time.perf_counter()
        O.assign_encode(w.vectors[:cnt], w.index.centroids, w.index.codebooks, nthreads=threads)
        per_v = (time.perf_counter() - t) / cnt
        cnt = int(min(n, max(cnt, args.cpu_seconds / max(per_v, 1e-9))))
        t = time.perf_counter()
        O.assign_encode(w.vectors[:cnt], w.index.centroids, w.index.codebooks, nthreads=threads)
        wall = time.perf_counter() - t
        cpu = dict(value=cnt / wall, unit="vectors/s", cores=threads, kind="oracle",
                   sample=f"assignment and encoding of the first {cnt} of {n} vectors "
                          f"(double precision; the layout is a sort), {wall:.1f} s wall")
        log("cpu baseline", cpu)
    res = {
        "metric": "database vectors indexed per second (assignment, encoding, list-major layout)",
        "value": n / (ms_step * 1e-3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded Gaussian mixture, CPU-trained centroids and codebooks)",
        "config": {"workload": BUILD_WORKLOAD, "n": n, "d": d, "nlist": nlist, "m": m},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_PEAK_TFLOPS, "traffic": None,
                     "kernel": "whole build call (assignment and encoding flops)",
                     "kernel_ms": ms_step, "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu,
        "parity": summary,
    }
    print(json.dumps(res), flush=True)


KNN_GRAPH_WORKLOAD = "knn_graph_n1m_d128_k10"


def bench_knn_graph(args):
    """The k-NN graph of the 1M x 128 workload ("Billion-scale similarity
    search with GPUs", k-NN graph experiment: every database vector searched
    for its k = 10 nearest neighbours): one step = one IVF-PQ search of all
    1M database vectors (nprobe 32, float32 tables) against the workload's
    index; a vector's own entry is among its results like any other."""
    import torch
    import approximate_nearest_neighbour_amd as A
    from approximate_nearest_neighbour_amd import datagen as G
    from oracle import check
    from oracle import oracle as O

    t0 = time.time()
    w = G.gmm1m(keep_vectors=True)
    log(f"workload {KNN_GRAPH_WORKLOAD}: built in {time.time() - t0:.1f} s")
    k, nprobe = 10, w.nprobe
    ix = A.ivfpq_load_index_host(w.index, device=0)
    q = torch.from_numpy(w.vectors).cuda()
    nq = q.shape[0]
    out = (torch.empty((nq, k), dtype=torch.float32, device="cuda"),
           torch.empty((nq, k), dtype=torch.int64, device="cuda"),
           torch.empty((nq, nprobe), dtype=torch.int32, device="cuda"))

    def step():
        A.ivfpq_search_ex(ix, q, nprobe, k, return_probes=True, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    entries = scanned_entries(w.index, out[2].cpu().numpy())
    code_bytes = entries * w.index.m
    A.ivfpq_profile_begin(ix, args.steps)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t) / args.steps
    prof = A.ivfpq_profile_end(ix)
    calls = max(prof["calls"], 1)
    scan_ms, coarse_ms = prof["scan_ms"] / calls, prof["coarse_ms"] / calls
    achieved = code_bytes / (scan_ms * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms  coarse {coarse_ms:.3f} ms  scan {scan_ms:.3f} ms  "
        f"code bytes/launch {code_bytes / 1e9:.3f} GB")
    rng = np.random.default_rng(2004)
    rows = np.sort(rng.choice(nq, min(nq, args.parity_queries), replace=False))
    rep = check.compare_search(w.index, w.vectors[rows], nprobe, k, out[0].cpu().numpy()[rows],
                               out[1].cpu().numpy()[rows], out[2].cpu().numpy()[rows])
    log("parity", rep.summary())
    # graph quality: the fraction of the 10 found within the exact 10 nearest
    # (oracle brute force, double precision) on a sample of vectors
    qs = np.sort(rng.choice(nq, 500, replace=False))
    _, true_ids = O.bruteforce(w.vectors, w.vectors[qs], k)
    recall = O.recall_k_at_k(out[1].cpu().numpy()[qs], true_ids)
    log(f"10-recall@10 on 500 sampled vectors: {recall:.4f}")
    cpu = None
    if not args.no_cpu_baseline:
        gw = G.Workload(KNN_GRAPH_WORKLOAD, w.index, w.vectors, nprobe, k)
        cpu, _ = cpu_baseline(gw, O.LUT_F64, args.cpu_seconds)
        cpu["unit"] = "vectors/s"
        log("cpu baseline", cpu)
    res = {
        "metric": "k-NN graph construction: database vectors searched per second (k 10)",
        "value": nq / (ms_step * 1e-3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded Gaussian mixture, CPU-built IVF-PQ index)",
        "config": {"workload": KNN_GRAPH_WORKLOAD, "n": nq, "d": w.index.d,
                   "nlist": w.index.nlist, "m": w.index.m, "nprobe": nprobe, "k": k},
        "roofline": {"bound": "hbm" if int(w.index.ntotal) * w.index.m > MALL_BYTES
                     else "effective", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "scan_items_kernel",
                     "kernel_ms": scan_ms, "algorithmic_bytes_per_launch": code_bytes},
        "cpu_baseline": cpu,
        "stages_ms": {"coarse": coarse_ms, "scan": scan_ms},
        "recall_10_at_10": recall,
        "parity": rep.summary(),
    }
    print(json.dumps(res), flush=True)
    ix.close()


EXTRA_WORKLOADS = [FLAT_WORKLOAD, ENCODE_WORKLOAD, KMEANS_WORKLOAD, KNN_GRAPH_WORKLOAD,
                   BUILD_WORKLOAD]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=ZIPF_WORKLOAD)
    ap.add_argument("--lut", choices=["f32", "f16"], default="f32")
    ap.add_argument("--metric", choices=["l2", "ip"], default="l2",
                    help="ranking metric of the IVF-PQ search (squared L2 or inner product)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--parity-queries", type=int, default=200)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size (counter calibration)")
    ap.add_argument("--summarize-counters", nargs="+", help="print rocprofv3 counter CSVs")
    ap.add_argument("--summarize-stats", nargs="+", help="print rocprofv3 kernel_stats CSVs")
    args = ap.parse_args()
    if args.summarize_counters or args.summarize_stats:
        summarize_counters(args.summarize_counters or [])
        summarize_stats(args.summarize_stats or [])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the multi-GPU path (replicas/shards joined by "
              "one gather) is not built; run with --gpus 1", file=sys.stderr)
        raise SystemExit(2)

    import torch
    import approximate_nearest_neighbour_amd as A
    from oracle import check
    from oracle import oracle as O

    if not os.path.exists(A.binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if args.workload == FLAT_WORKLOAD:
        return bench_flat(args)
    if args.workload == ENCODE_WORKLOAD:
        return bench_encode(args)
    if args.workload == KMEANS_WORKLOAD:
        return bench_kmeans(args)
    if args.workload == KNN_GRAPH_WORKLOAD:
        return bench_knn_graph(args)
    if args.workload == BUILD_WORKLOAD:
        return bench_build(args)

    t0 = time.time()
    w = workload(args.workload)
    log(f"workload {w.name}: built in {time.time() - t0:.1f} s")
    dev = torch.device("cuda:0")
    ix = A.ivfpq_load_index_host(w.index, device=0)
    q = torch.from_numpy(w.queries).to(dev)
    nq = q.shape[0]
    out = (torch.empty((nq, w.k), dtype=torch.float32, device=dev),
           torch.empty((nq, w.k), dtype=torch.int64, device=dev),
           torch.empty((nq, w.nprobe), dtype=torch.int32, device=dev))

    def step():
        A.ivfpq_search_ex(ix, q, w.nprobe, w.k, lut=args.lut, return_probes=True, out=out,
                          metric=args.metric)

    if args.copy_calibration_mib:
        # known traffic for the counters: a fill writes N bytes, a sum reads N
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        float(src.sum())
        torch.cuda.synchronize()
        del src
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    probes = out[2].cpu().numpy()
    entries = scanned_entries(w.index, probes)
    code_bytes = entries * w.index.m

    A.ivfpq_profile_begin(ix, args.steps)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    prof = A.ivfpq_profile_end(ix)

    ms_step = 1e3 * elapsed / args.steps
    scan_ms = prof["scan_ms"] / max(prof["calls"], 1)
    coarse_ms = prof["coarse_ms"] / max(prof["calls"], 1)
    achieved = code_bytes / (scan_ms * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms  coarse {coarse_ms:.3f} ms  scan {scan_ms:.3f} ms  "
        f"entries/query {entries / nq:.0f}  code bytes/launch {code_bytes / 1e9:.3f} GB")

    # k-select cost: same scan with the top-k replaced by a running minimum
    so = (torch.empty((nq, w.k), dtype=torch.float32, device=dev), out[1], out[2])
    A.ivfpq_search_ex(ix, q, w.nprobe, w.k, lut=args.lut, mode=1, out=so, return_probes=True,
                      metric=args.metric)
    A.ivfpq_profile_begin(ix, args.steps)
    for _ in range(args.steps):
        A.ivfpq_search_ex(ix, q, w.nprobe, w.k, lut=args.lut, mode=1, out=so, return_probes=True,
                          metric=args.metric)
    torch.cuda.synchronize()
    scan_only_ms = A.ivfpq_profile_end(ix)["scan_ms"] / args.steps

    host_qps = None
    if args.metric == "l2":   # the host-pointer entry point ranks by squared L2
        host_qps = host_pointer_qps(lambda: A.ivfpq_search(ix, w.queries, w.nprobe, w.k), nq)
        log(f"host-pointer entry point: {host_qps:.0f} queries/s (PCIe copies included)")
    read_gbs = measured_read_gbs(torch, A)
    log(f"measured streaming read: {read_gbs:.0f} GB/s")

    # parity on a sample of the timed configuration: the leading queries plus
    # (1B Zipf index) up to 8 queries that probe a list above 10^6 entries
    step()
    torch.cuda.synchronize()
    pn = min(args.parity_queries, nq)
    rows = np.arange(pn)
    giants = giant_list_queries(w.index, probes)
    rows = np.unique(np.concatenate([rows, giants[giants >= pn][:8]])).astype(np.int64)
    lut_mode = O.IP if args.metric == "ip" else (O.LUT_F16 if args.lut == "f16" else O.LUT_F64)
    decomposed = bool(A.ivfpq_index_info(ix)["flags"] & 1) and args.lut == "f32" \
        and args.metric == "l2"
    split = bool(A.ivfpq_index_info(ix)["flags"] & 2) and 1 < w.nprobe <= 128
    rep = check.compare_search(w.index, w.queries[rows], w.nprobe, w.k,
                               out[0].cpu().numpy()[rows], out[1].cpu().numpy()[rows],
                               out[2].cpu().numpy()[rows], lut_mode=lut_mode,
                               decomposed=decomposed, split_bf16=split)
    log("parity", rep.summary(), f"({len(rows) - pn} giant-list queries among {len(rows)})")
    recall = None
    if args.metric == "l2":
        recall = recall_report(w, out[1].cpu().numpy())
        if recall:
            log("recall", recall)

    cpu = None
    if not args.no_cpu_baseline:
        cpu, _ = cpu_baseline(w, lut_mode, args.cpu_seconds, probes=probes)
        log("cpu baseline", cpu)
    code_array = int(w.index.ntotal) * w.index.m
    bound = "hbm" if code_array > MALL_BYTES else "effective"
    traffic = stored_traffic(w.name, args.lut) if args.metric == "l2" else None
    # the measured L2-miss bytes' own rate: below `achieved` when code bytes
    # are served from L2 (the giant-list order), above it when tables and
    # staging add reads
    traffic_gbs = traffic / (scan_ms * 1e-3) / 1e9 if traffic else None

    res = {
        "metric": METRIC,
        "value": nq / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if args.lut == "f32" else "fp32 (binary16 tables)",
        "data": ("synthetic (seeded N(0,1) centroids, codebooks and queries; uniform random "
                 "codes; Zipf(1.1) list sizes)" if "zipf" in w.name else
                 "synthetic (seeded Gaussian mixture, CPU-built IVF-PQ index)"),
        "config": {"workload": w.name, "n": int(w.index.ntotal), "d": w.index.d,
                   "nlist": w.index.nlist, "m": w.index.m, "nq": nq, "nprobe": w.nprobe,
                   "k": w.k, "lut": args.lut, "metric": args.metric},
        "roofline": {"bound": bound, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_gbs": traffic_gbs,
                     "traffic_frac": traffic_gbs / HBM_PEAK_GBS if traffic_gbs else None,
                     "kernel": "scan_items_kernel", "kernel_ms": scan_ms,
                     "algorithmic_bytes_per_launch": code_bytes,
                     "code_array_bytes": code_array,
                     "measured_read_gbs": read_gbs, "frac_of_measured_read": achieved / read_gbs},
        "cpu_baseline": cpu,
        "stages_ms": {"coarse": coarse_ms, "scan": scan_ms, "scan_only": scan_only_ms,
                      "kselect_overhead": scan_ms / scan_only_ms - 1 if scan_only_ms else None},
        "host_pointer_qps": host_qps,
        "recall": recall,
        "parity": rep.summary(),
    }
    print(json.dumps(res), flush=True)
    ix.close()


if __name__ == "__main__":
    main()
