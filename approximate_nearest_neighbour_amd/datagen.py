"""Seeded synthetic inputs and a CPU IVF-PQ index builder.

This module is the one source of inputs shared by the GPU path and by the
CPU oracle.  It draws database vectors and queries, trains the coarse
quantizer and the product quantizer on the CPU (index construction is allowed
to run on the host), encodes the database, and writes/reads the index file.
It holds none of the search arithmetic: no lookup tables, no ADC sums, no
top-k selection.

Index construction follows the build phase of "Custom 8-bit floating point
value format for reducing shared memory bank conflict in ANN search"
(IVFPQ section, index-building steps 1-4): k-means clusters, residuals to the
assigned centroid, product quantization of the residual over contiguous
sub-vectors, and storage of list membership, codes and codebooks.

Random numbers come from numpy's PCG64 ``default_rng``.  Seeds per workload
number ``c``: data = 1000*c + 1, queries = 1000*c + 2, build = 1000*c + 3.
"""
from __future__ import annotations

import dataclasses
import os
import struct

import numpy as np

MAGIC = b"IVFPQ01\x00"
HEADER = struct.Struct("<8sIIIIQ")  # magic, d, nlist, m, nbits, ntotal


@dataclasses.dataclass
class HostIndex:
    """An IVF-PQ index in host memory, list-major.

    centroids  float32 [nlist, d]
    codebooks  float32 [m, 256, d // m]   (sub-vector j = dims j*dsub .. j*dsub+dsub-1)
    list_sizes int64   [nlist]
    codes      uint8   [ntotal, m]        entries of list 0, then list 1, ...
    ids        int64   [ntotal]           same order as codes
    """

    centroids: np.ndarray
    codebooks: np.ndarray
    list_sizes: np.ndarray
    codes: np.ndarray
    ids: np.ndarray

    @property
    def d(self) -> int:
        return int(self.centroids.shape[1])

    @property
    def nlist(self) -> int:
        return int(self.centroids.shape[0])

    @property
    def m(self) -> int:
        return int(self.codebooks.shape[0])

    @property
    def ntotal(self) -> int:
        return int(self.codes.shape[0])

    def list_offsets(self) -> np.ndarray:
        off = np.zeros(self.nlist + 1, dtype=np.int64)
        np.cumsum(self.list_sizes, out=off[1:])
        return off


@dataclasses.dataclass
class Workload:
    """A named synthetic workload: index, queries, search parameters and
    (where the workload has them) the raw database vectors."""

    name: str
    index: HostIndex | None
    queries: np.ndarray
    nprobe: int
    k: int
    vectors: np.ndarray | None = None
    extra: dict = dataclasses.field(default_factory=dict)


# --------------------------------------------------------------------------
# raw draws
# --------------------------------------------------------------------------

def gmm_centers(rng: np.random.Generator, ncomp: int, d: int) -> np.ndarray:
    return rng.standard_normal((ncomp, d), dtype=np.float32)


def gmm_draw(rng: np.random.Generator, centers: np.ndarray, n: int, sigma: float,
             chunk: int = 1 << 16) -> np.ndarray:
    """n points: a uniformly drawn component center plus sigma * N(0, I)."""
    ncomp, d = centers.shape
    out = np.empty((n, d), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        comp = rng.integers(0, ncomp, size=e - s)
        blk = out[s:e]
        rng.standard_normal(out=blk, dtype=np.float32)
        blk *= np.float32(sigma)
        blk += centers[comp]
    return out


# --------------------------------------------------------------------------
# index construction (host only)
# --------------------------------------------------------------------------

def nearest(x: np.ndarray, c: np.ndarray, chunk: int = 1 << 13) -> np.ndarray:
    """Index of the nearest row of c for each row of x (ties -> lowest index).

    Build-time helper; float32 BLAS with the norm expansion is plenty for
    training and encoding."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    cn = (c ** 2).sum(1)
    ct = np.ascontiguousarray(c.T)
    out = np.empty(len(x), dtype=np.int64)
    buf = np.empty((min(chunk, max(len(x), 1)), len(c)), dtype=np.float32)
    for s in range(0, len(x), chunk):
        xs = x[s:s + chunk]
        b = buf[:len(xs)]
        np.matmul(xs, ct, out=b)
        b *= np.float32(-2.0)
        b += cn[None, :]
        out[s:s + chunk] = np.argmin(b, axis=1)
    return out


def kmeans(x: np.ndarray, k: int, iters: int, rng: np.random.Generator) -> np.ndarray:
    """Lloyd k-means; init = k distinct random points; an empty cluster keeps
    its previous centroid."""
    n, d = x.shape
    if k > n:
        raise ValueError("kmeans: more clusters than points")
    c = x[rng.choice(n, size=k, replace=False)].astype(np.float32).copy()
    for _ in range(iters):
        a = nearest(x, c)
        counts = np.bincount(a, minlength=k)
        sums = np.empty((k, d), dtype=np.float64)
        for t in range(d):
            sums[:, t] = np.bincount(a, weights=x[:, t], minlength=k)
        ok = counts > 0
        c[ok] = (sums[ok] / counts[ok, None]).astype(np.float32)
    return c


def train_pq(resid: np.ndarray, m: int, iters: int, rng: np.random.Generator) -> np.ndarray:
    n, d = resid.shape
    dsub = d // m
    books = np.empty((m, 256, dsub), dtype=np.float32)
    for j in range(m):
        books[j] = kmeans(np.ascontiguousarray(resid[:, j * dsub:(j + 1) * dsub]), 256, iters, rng)
    return books


def encode_pq(resid: np.ndarray, books: np.ndarray) -> np.ndarray:
    m, _, dsub = books.shape
    codes = np.empty((len(resid), m), dtype=np.uint8)
    for j in range(m):
        sub = np.ascontiguousarray(resid[:, j * dsub:(j + 1) * dsub])
        codes[:, j] = nearest(sub, books[j]).astype(np.uint8)
    return codes


def build_ivfpq(x: np.ndarray, nlist: int, m: int, rng: np.random.Generator, iters: int = 10,
                coarse_train: int | None = None, pq_train: int | None = None,
                chunk: int = 1 << 20) -> HostIndex:
    """CPU IVF-PQ build: coarse k-means, residual PQ, list-major layout."""
    n, d = x.shape
    if d % m:
        raise ValueError("d must be a multiple of m")
    tr = x if coarse_train is None or coarse_train >= n else x[rng.choice(n, coarse_train, replace=False)]
    cent = kmeans(tr, nlist, iters, rng)
    sample = np.arange(n) if pq_train is None or pq_train >= n else np.sort(rng.choice(n, pq_train, replace=False))
    a_s = nearest(x[sample], cent)
    books = train_pq(x[sample] - cent[a_s], m, iters, rng)
    assign = np.empty(n, dtype=np.int64)
    codes = np.empty((n, m), dtype=np.uint8)
    for s in range(0, n, chunk):
        xs = x[s:s + chunk]
        a = nearest(xs, cent)
        assign[s:s + chunk] = a
        codes[s:s + chunk] = encode_pq(xs - cent[a], books)
    order = np.argsort(assign, kind="stable")
    sizes = np.bincount(assign, minlength=nlist).astype(np.int64)
    return HostIndex(cent, books, sizes, np.ascontiguousarray(codes[order]), order.astype(np.int64))


# --------------------------------------------------------------------------
# index file (little-endian): header, centroids, codebooks, list sizes,
# codes (list-major), ids
# --------------------------------------------------------------------------

def write_index(path: str, idx: HostIndex) -> None:
    with open(path, "wb") as f:
        f.write(HEADER.pack(MAGIC, idx.d, idx.nlist, idx.m, 8, idx.ntotal))
        f.write(np.ascontiguousarray(idx.centroids, dtype="<f4").tobytes())
        f.write(np.ascontiguousarray(idx.codebooks, dtype="<f4").tobytes())
        f.write(np.ascontiguousarray(idx.list_sizes, dtype="<u8").tobytes())
        np.ascontiguousarray(idx.codes, dtype=np.uint8).tofile(f)
        np.ascontiguousarray(idx.ids, dtype="<i8").tofile(f)


def read_index(path: str) -> HostIndex:
    with open(path, "rb") as f:
        magic, d, nlist, m, nbits, ntotal = HEADER.unpack(f.read(HEADER.size))
        if magic != MAGIC or nbits != 8 or m == 0 or d % m:
            raise ValueError("not an IVF-PQ v1 index file")
        cent = np.fromfile(f, dtype="<f4", count=nlist * d).reshape(nlist, d)
        books = np.fromfile(f, dtype="<f4", count=m * 256 * (d // m)).reshape(m, 256, d // m)
        sizes = np.fromfile(f, dtype="<u8", count=nlist).astype(np.int64)
        codes = np.fromfile(f, dtype=np.uint8, count=ntotal * m).reshape(ntotal, m)
        ids = np.fromfile(f, dtype="<i8", count=ntotal)
    return HostIndex(cent, books, sizes, codes, ids)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def seeds(c: int) -> tuple[int, int, int]:
    return 1000 * c + 1, 1000 * c + 2, 1000 * c + 3


def gmm_workload(name: str, c: int, n: int, d: int, ncomp: int, sigma: float, nq: int,
                 nlist: int, m: int, nprobe: int, k: int, coarse_train=None, pq_train=None,
                 keep_vectors: bool = True) -> Workload:
    sd, sq, sb = seeds(c)
    rd = np.random.default_rng(sd)
    centers = gmm_centers(rd, ncomp, d)
    x = gmm_draw(rd, centers, n, sigma)
    q = gmm_draw(np.random.default_rng(sq), centers, nq, sigma)
    idx = build_ivfpq(x, nlist, m, np.random.default_rng(sb), iters=10,
                      coarse_train=coarse_train, pq_train=pq_train)
    return Workload(name, idx, q, nprobe, k, x if keep_vectors else None)


def tiny() -> Workload:
    """10,000 x 32 from a 16-component mixture (sigma 0.3); nlist 16; m 4;
    100 queries; nprobe 4; k 10."""
    return gmm_workload("ivfpq_tiny_n10k_d32_m4", 1, 10_000, 32, 16, 0.3, 100, 16, 4, 4, 10)


def gmm1m(keep_vectors: bool = False) -> Workload:
    """1M x 128 from a 1,000-component mixture (sigma 0.2); nlist 1024; m 16;
    10,000 queries; nprobe 32; k 100."""
    return gmm_workload("ivfpq_n1m_d128_m16_nlist1024", 2, 1_000_000, 128, 1000, 0.2, 10_000,
                        1024, 16, 32, 100, coarse_train=262_144, pq_train=65_536,
                        keep_vectors=keep_vectors)


def gmm10m(keep_vectors: bool = False) -> Workload:
    """10M x 96 from a 4,096-component mixture (sigma 0.2, chosen); nlist 4096;
    m 32; 10,000 queries; nprobe 64; k 100."""
    return gmm_workload("ivfpq_n10m_d96_m32_nlist4096", 4, 10_000_000, 96, 4096, 0.2, 10_000,
                        4096, 32, 64, 100, coarse_train=1_048_576, pq_train=131_072,
                        keep_vectors=keep_vectors)


def zipf_sizes(n: int, nlist: int, s: float = 1.1) -> np.ndarray:
    """List sizes by rank: floor(n * r^-s / H), H = sum_r r^-s; the remainder
    goes +1 to the largest lists in rank order."""
    r = np.arange(1, nlist + 1, dtype=np.float64)
    w = r ** -s
    h = w.sum()
    sizes = np.floor(n * w / h).astype(np.int64)
    rem = n - int(sizes.sum())
    sizes[:rem] += 1
    return sizes


def zipf_workload(n: int = 1_000_000_000, nlist: int = 262_144, d: int = 96, m: int = 8,
                  nq: int = 10_000, nprobe: int = 128, k: int = 100, permute_ids: bool = True,
                  c: int = 5) -> Workload:
    """Codes drawn uniform i.i.d. (no training), list sizes Zipf(1.1) by rank,
    centroids / codebooks / queries ~ N(0, 1)."""
    sd, sq, _ = seeds(c)
    rd = np.random.default_rng(sd)
    cent = rd.standard_normal((nlist, d), dtype=np.float32)
    books = rd.standard_normal((m, 256, d // m), dtype=np.float32)
    sizes = zipf_sizes(n, nlist)
    codes = np.empty((n, m), dtype=np.uint8)
    step = 1 << 26
    for s in range(0, n, step):
        e = min(n, s + step)
        codes[s:e] = rd.integers(0, 256, size=(e - s, m), dtype=np.uint8)
    ids = rd.permutation(n) if permute_ids else np.arange(n, dtype=np.int64)
    q = np.random.default_rng(sq).standard_normal((nq, d), dtype=np.float32)
    return Workload(f"ivfpq_zipf_n{n}_d{d}_m{m}_nlist{nlist}", HostIndex(cent, books, sizes, codes, ids),
                    q, nprobe, k)


def flat_bf16_workload(n: int = 1_000_000, d: int = 128, nq: int = 10_000, k: int = 1024,
                       c: int = 3) -> Workload:
    """Uniform [-1, 1] database and queries rounded to bfloat16 (round to
    nearest even), kept as the raw uint16 bit patterns."""
    sd, sq, _ = seeds(c)
    x = np.random.default_rng(sd).uniform(-1.0, 1.0, size=(n, d)).astype(np.float32)
    q = np.random.default_rng(sq).uniform(-1.0, 1.0, size=(nq, d)).astype(np.float32)
    return Workload(f"flat_bf16_n{n}_d{d}", None, to_bf16_bits(q), 0, k, to_bf16_bits(x))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def random_index(rng: np.random.Generator, nlist: int, d: int, m: int, sizes, scale: float = 1.0,
                 codebook_scale: float = 1.0) -> HostIndex:
    """An index with random centroids, codebooks and codes (no training):
    handy for parity cases of arbitrary shape."""
    sizes = np.asarray(sizes, dtype=np.int64)
    n = int(sizes.sum())
    cent = (scale * rng.standard_normal((nlist, d))).astype(np.float32)
    books = (codebook_scale * rng.standard_normal((m, 256, d // m))).astype(np.float32)
    codes = rng.integers(0, 256, size=(n, m), dtype=np.uint8)
    ids = rng.permutation(n).astype(np.int64)
    return HostIndex(cent, books, sizes, codes, ids)


def cache_dir() -> str:
    return os.environ.get("IVFPQ_DATA_CACHE", os.path.join(os.path.dirname(__file__), "..", "_data"))
