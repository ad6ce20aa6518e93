"""Python front of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It builds and loads ``liboracle.so`` (plain C, double
precision, see ``ivfpq_oracle.c``) and wraps its entry points with ctypes.
It has its own reader of the index file and imports nothing from the GPU
package.
"""
from __future__ import annotations

import ctypes
import os
import struct
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ivfpq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

LUT_F64 = 0
LUT_F16 = 1
IP = 2        # inner-product metric (double-precision tables), passed as lut_mode

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread", "-o", tmp, SRC,
                               "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_round_binary16.argtypes = [ctypes.c_float]
        L.oracle_round_binary16.restype = ctypes.c_double
        L.oracle_coarse.argtypes = [P, P, i32, i32, i32, P, P]
        L.oracle_lut.argtypes = [P, P, P, i32, i32, i32, P]
        L.oracle_coarse_ip.argtypes = [P, P, i32, i32, i32, P, P]
        L.oracle_lut_ip.argtypes = [P, P, i32, i32, P]
        L.oracle_search.argtypes = [P, P, P, P, P, i32, i32, i32, P, i64, i32, i32, i32, P, P, P,
                                    P, i32]
        L.oracle_entry_distances.argtypes = [P, P, P, i32, i32, i32, P, P, i64, P]
        L.oracle_bruteforce.argtypes = [P, P, i64, i32, P, i64, i32, P, P, i32]
        L.oracle_bruteforce_bf16.argtypes = [P, i64, i32, P, i64, i32, P, P, i32]
        for f in ("oracle_coarse", "oracle_lut", "oracle_coarse_ip", "oracle_lut_ip",
                  "oracle_search", "oracle_entry_distances",
                  "oracle_bruteforce",
                  "oracle_bruteforce_bf16"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# the oracle's own index-file reader
# ---------------------------------------------------------------------------

def read_index_file(path: str) -> dict:
    with open(path, "rb") as f:
        head = f.read(32)
        magic, d, nlist, m, nbits, ntotal = struct.unpack("<8sIIIIQ", head)
        if magic != b"IVFPQ01\x00" or nbits != 8 or m < 1 or d % m:
            raise ValueError("bad index file")
        dsub = d // m
        raw = np.fromfile(f, dtype=np.uint8)
    o = 0
    cent = raw[o:o + 4 * nlist * d].view("<f4").reshape(nlist, d)
    o += 4 * nlist * d
    books = raw[o:o + 4 * m * 256 * dsub].view("<f4").reshape(m, 256, dsub)
    o += 4 * m * 256 * dsub
    sizes = raw[o:o + 8 * nlist].view("<u8").astype(np.int64)
    o += 8 * nlist
    codes = raw[o:o + ntotal * m].reshape(ntotal, m)
    o += ntotal * m
    ids = raw[o:o + 8 * ntotal].view("<i8")
    return dict(centroids=cent, codebooks=books, list_sizes=sizes, codes=codes, ids=ids)


# ---------------------------------------------------------------------------
# wrappers
# ---------------------------------------------------------------------------

def round_binary16(x: float) -> float:
    return lib().oracle_round_binary16(float(x))


def coarse(x, centroids, nprobe):
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    probes = np.empty(nprobe, dtype=np.int32)
    dists = np.empty(nprobe, dtype=np.float64)
    rc = lib().oracle_coarse(_p(x), _p(c), c.shape[1], c.shape[0], nprobe, _p(probes), _p(dists))
    if rc:
        raise ValueError(f"oracle_coarse failed ({rc})")
    return probes, dists


def coarse_ip(x, centroids, nprobe):
    """Inner-product coarse step: the nprobe lists of largest <x, c_l>
    (ties to the smaller list number) and those inner products."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    probes = np.empty(nprobe, dtype=np.int32)
    ips = np.empty(nprobe, dtype=np.float64)
    rc = lib().oracle_coarse_ip(_p(x), _p(c), c.shape[1], c.shape[0], nprobe, _p(probes), _p(ips))
    if rc:
        raise ValueError(f"oracle_coarse_ip failed ({rc})")
    return probes, ips


def lut_ip(x, codebooks):
    """Inner-product tables T_j(v) = <x_j, C_j[v]> (float64 [m, 256])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = np.ascontiguousarray(codebooks, dtype=np.float32)
    m = b.shape[0]
    out = np.empty((m, 256), dtype=np.float64)
    rc = lib().oracle_lut_ip(_p(x), _p(b), x.shape[0], m, _p(out))
    if rc:
        raise ValueError(f"oracle_lut_ip failed ({rc})")
    return out


def lut(x, centroid, codebooks, lut_mode=LUT_F64):
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.ascontiguousarray(centroid, dtype=np.float32)
    b = np.ascontiguousarray(codebooks, dtype=np.float32)
    m = b.shape[0]
    out = np.empty((m, 256), dtype=np.float64)
    rc = lib().oracle_lut(_p(x), _p(c), _p(b), x.shape[0], m, lut_mode, _p(out))
    if rc:
        raise ValueError(f"oracle_lut failed ({rc})")
    return out


def entry_distances(index, x, positions, lut_mode=LUT_F64):
    """ADC distance of the entries at the given list-major positions."""
    get = (lambda n: index[n]) if isinstance(index, dict) else (lambda n: getattr(index, n))
    cent = np.ascontiguousarray(get("centroids"), dtype=np.float32)
    books = np.ascontiguousarray(get("codebooks"), dtype=np.float32)
    sizes = np.asarray(get("list_sizes"), dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(sizes)])
    pos = np.asarray(positions, dtype=np.int64)
    lists = (np.searchsorted(off, pos, side="right") - 1).astype(np.int32)
    rows = np.ascontiguousarray(np.asarray(get("codes"))[pos], dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(len(pos), dtype=np.float64)
    rc = lib().oracle_entry_distances(_p(x), _p(cent), _p(books), x.shape[0], books.shape[0],
                                      lut_mode, _p(lists), _p(rows), len(pos), _p(out))
    if rc:
        raise ValueError(f"oracle_entry_distances failed ({rc})")
    return out, lists


def search(index, queries, nprobe, k, lut_mode=LUT_F64, probes=None, nthreads=None):
    """Returns (distances float64 [nq,k], ids int64 [nq,k], probes int32 [nq,nprobe]).

    ``index`` is any object with centroids, codebooks, list_sizes, codes and
    ids attributes or keys."""
    get = (lambda n: index[n]) if isinstance(index, dict) else (lambda n: getattr(index, n))
    cent = np.ascontiguousarray(get("centroids"), dtype=np.float32)
    books = np.ascontiguousarray(get("codebooks"), dtype=np.float32)
    sizes = np.ascontiguousarray(get("list_sizes"), dtype=np.int64)
    codes = np.ascontiguousarray(get("codes"), dtype=np.uint8)
    ids = np.ascontiguousarray(get("ids"), dtype=np.int64)
    q = np.ascontiguousarray(queries, dtype=np.float32)
    nq, d = q.shape
    nlist = cent.shape[0]
    m = books.shape[0]
    if probes is not None:
        probes = np.ascontiguousarray(probes, dtype=np.int32)
        assert probes.shape == (nq, nprobe)
    od = np.empty((nq, k), dtype=np.float64)
    oi = np.empty((nq, k), dtype=np.int64)
    op = np.empty((nq, nprobe), dtype=np.int32)
    rc = lib().oracle_search(_p(cent), _p(books), _p(sizes), _p(codes), _p(ids), d, nlist, m, _p(q),
                             nq, nprobe, k, lut_mode, _p(probes), _p(od), _p(oi), _p(op),
                             nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_search failed ({rc})")
    return od, oi, op


def assign_encode(vectors, centroids, codebooks, nthreads=None):
    """Index building: list assignment and PQ encoding of database vectors.

    The index-building steps of "Custom 8-bit floating point value format for
    reducing shared memory bank conflict in ANN search" (IVFPQ section, steps
    1-3: a vector belongs to the cluster of its nearest centroid, its residual
    to that centroid is cut into sub-vectors, each sub-vector is quantized),
    with the quantizers of "Billion-scale similarity search with GPUs"
    (IVFADC section: the coarse quantizer q1, and on the residual a product
    of m quantizers with 256 reproduction values each).  A quantizer maps its
    input to the nearest reproduction value in squared L2, ties to the
    smaller index.

    Both decisions reuse the oracle's search steps: the list is the first of
    the coarse order (``coarse``: distance, then list number), and the code
    of sub-quantizer j is the smallest entry of row j of the table of that
    list (``lut``: F_j(v) = |r_j - C_j[v]|^2 with r = x - c_list, double
    precision), the first one on ties.

    Returns (lists int32 [n], codes uint8 [n, m], list_gap float64 [n],
    code_gap float64 [n, m]): the gaps are the second-smallest minus the
    smallest distance of each decision (+inf when there is one list), i.e.
    how far the decision is from a tie.
    """
    x = np.ascontiguousarray(vectors, dtype=np.float32)
    cent = np.ascontiguousarray(centroids, dtype=np.float32)
    books = np.ascontiguousarray(codebooks, dtype=np.float32)
    n = x.shape[0]
    nlist, m = cent.shape[0], books.shape[0]
    lists = np.empty(n, dtype=np.int32)
    codes = np.empty((n, m), dtype=np.uint8)
    list_gap = np.empty(n, dtype=np.float64)
    code_gap = np.empty((n, m), dtype=np.float64)
    take = 2 if nlist > 1 else 1

    def one(i):
        pr, dist = coarse(x[i], cent, take)
        lists[i] = pr[0]
        list_gap[i] = dist[1] - dist[0] if take == 2 else np.inf
        table = lut(x[i], cent[pr[0]], books)
        codes[i] = np.argmin(table, axis=1)
        two = np.partition(table, 1, axis=1)
        code_gap[i] = two[:, 1] - two[:, 0]

    def run(lo, hi):
        for i in range(lo, hi):
            one(i)

    nt = max(1, min(nthreads or default_threads(), n))
    if nt == 1:
        run(0, n)
    else:
        from concurrent.futures import ThreadPoolExecutor
        step = (n + nt - 1) // nt
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda s: run(s, min(n, s + step)), range(0, n, step)))
    return lists, codes, list_gap, code_gap


def kmeans_update(vectors, assign, centers):
    """The update step of Lloyd's algorithm (k-means: the clustering of the
    index-building step 1 of the IVFPQ section of "Custom 8-bit floating
    point value format for reducing shared memory bank conflict in ANN
    search"; exact k-means in "Billion-scale similarity search with GPUs"):
    each center becomes the mean of the vectors assigned to it, a center
    with no vector keeps its value.  Sums and means in double precision; the
    new centers are then rounded to float32, the type the index stores
    centroids in.

    Returns (centers float32 [k, d], means float64 [k, d], counts int64 [k]).
    """
    x = np.asarray(vectors, dtype=np.float64)
    a = np.asarray(assign, dtype=np.int64)
    old = np.asarray(centers, dtype=np.float32)
    k, d = old.shape
    sums = np.zeros((k, d), dtype=np.float64)
    np.add.at(sums, a, x)
    counts = np.bincount(a, minlength=k).astype(np.int64)
    means = np.where(counts[:, None] > 0, sums / np.maximum(counts, 1)[:, None],
                     old.astype(np.float64))
    return means.astype(np.float32), means, counts


def nearest_lists(vectors, centers, nthreads=None):
    """The assignment step: for each vector the first of the coarse order
    (nearest center, ties to the smaller index).  Returns (lists int32 [n],
    gap float64 [n]: second-nearest minus nearest distance, +inf with one
    center)."""
    x = np.ascontiguousarray(vectors, dtype=np.float32)
    cent = np.ascontiguousarray(centers, dtype=np.float32)
    n, k = x.shape[0], cent.shape[0]
    lists = np.empty(n, dtype=np.int32)
    gap = np.empty(n, dtype=np.float64)
    take = 2 if k > 1 else 1

    def run(lo, hi):
        for i in range(lo, hi):
            pr, dist = coarse(x[i], cent, take)
            lists[i] = pr[0]
            gap[i] = dist[1] - dist[0] if take == 2 else np.inf

    nt = max(1, min(nthreads or default_threads(), n))
    if nt == 1:
        run(0, n)
    else:
        from concurrent.futures import ThreadPoolExecutor
        step = (n + nt - 1) // nt
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda s: run(s, min(n, s + step)), range(0, n, step)))
    return lists, gap


def kmeans(vectors, init, iters, nthreads=None):
    """Lloyd's algorithm from the given float32 initial centers: `iters`
    iterations of assignment (``nearest_lists``) then update
    (``kmeans_update``).  Returns (centers float32 [k, d], the last iteration's
    assignment int32 [n], its counts int64 [k])."""
    c = np.ascontiguousarray(init, dtype=np.float32)
    a = np.zeros(len(vectors), dtype=np.int32)
    counts = np.zeros(c.shape[0], dtype=np.int64)
    for _ in range(iters):
        a, _ = nearest_lists(vectors, c, nthreads=nthreads)
        c, _, counts = kmeans_update(vectors, a, c)
    return c, a, counts


def bruteforce(db, queries, k, db_ids=None, nthreads=None):
    db = np.ascontiguousarray(db, dtype=np.float32)
    q = np.ascontiguousarray(queries, dtype=np.float32)
    ids = None if db_ids is None else np.ascontiguousarray(db_ids, dtype=np.int64)
    od = np.empty((q.shape[0], k), dtype=np.float64)
    oi = np.empty((q.shape[0], k), dtype=np.int64)
    rc = lib().oracle_bruteforce(_p(db), _p(ids), db.shape[0], db.shape[1], _p(q), q.shape[0], k,
                                 _p(od), _p(oi), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_bruteforce failed ({rc})")
    return od, oi


def bruteforce_bf16(db_bits, query_bits, k, nthreads=None):
    db = np.ascontiguousarray(db_bits, dtype=np.uint16)
    q = np.ascontiguousarray(query_bits, dtype=np.uint16)
    od = np.empty((q.shape[0], k), dtype=np.float64)
    oi = np.empty((q.shape[0], k), dtype=np.int64)
    rc = lib().oracle_bruteforce_bf16(_p(db), db.shape[0], db.shape[1], _p(q), q.shape[0], k,
                                      _p(od), _p(oi), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_bruteforce_bf16 failed ({rc})")
    return od, oi


# ---------------------------------------------------------------------------
# recall (two readings of the pages' measures)
# ---------------------------------------------------------------------------

def recall_1_at_k(found_ids, true_ids, n=None):
    """R@n ("Billion-scale similarity search with GPUs", experiments section):
    the fraction of queries whose true nearest neighbour (column 0 of
    true_ids) is among the first n ids found (n defaults to every column of
    found_ids).  A padding id (-1) never counts."""
    found = np.asarray(found_ids)
    true = np.asarray(true_ids)
    n = found.shape[1] if n is None else n
    hits = [int(t[0]) >= 0 and int(t[0]) in set(f[:n].tolist()) for f, t in zip(found, true)]
    return float(np.mean(hits)) if hits else 0.0


def recall_k_at_k(found_ids, true_ids, k=None):
    """The intersection measure of the same section: for each query the
    number of the first k ids found that are among the true k nearest,
    divided by k, averaged over the queries (k defaults to every column of
    found_ids; only the first k columns of true_ids count).  Padding ids (-1)
    never count."""
    found = np.asarray(found_ids)
    true = np.asarray(true_ids)
    k = found.shape[1] if k is None else k
    fr = []
    for f, t in zip(found, true):
        tk = set(int(v) for v in t[:k].tolist() if v >= 0)
        fk = set(int(v) for v in f[:k].tolist() if v >= 0)
        fr.append(len(fk & tk) / k)
    return float(np.mean(fr)) if fr else 0.0
