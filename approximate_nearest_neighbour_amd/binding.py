"""Thin ctypes binding over ``libivfpq.so`` (declared in include/ivfpq.h).

Argument marshalling only: every step of the search runs in the library's
HIP kernels.  PyTorch supplies device memory and the HIP stream; it is
imported before the library is loaded so both share one HIP runtime.  There
is no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libivfpq.so")

OK, E_INVALID_ARG, E_IO, E_FORMAT, E_NO_DEVICE, E_OUT_OF_MEMORY, E_DEVICE = range(7)
METRIC_L2, METRIC_IP = 0, 1
LUT_F32, LUT_F16 = 0, 1
MODE_NORMAL, MODE_SCAN_ONLY = 0, 1


class IVFPQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class SearchParams(ctypes.Structure):
    _fields_ = [("nprobe", ctypes.c_int32), ("k", ctypes.c_int32), ("lut", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("metric", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("nlist", ctypes.c_int32), ("m", ctypes.c_int32),
                ("nbits", ctypes.c_int32), ("ntotal", ctypes.c_int64),
                ("max_list", ctypes.c_int64), ("device", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("device_bytes", ctypes.c_int64)]


class HostIndexStruct(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("nlist", ctypes.c_int32), ("m", ctypes.c_int32),
                ("nbits", ctypes.c_int32), ("ntotal", ctypes.c_int64),
                ("centroids", ctypes.c_void_p), ("codebooks", ctypes.c_void_p),
                ("list_sizes", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("ids", ctypes.c_void_p)]


class Timings(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("coarse_ms", ctypes.c_double), ("worklist_ms", ctypes.c_double),
                ("scan_ms", ctypes.c_double), ("merge_ms", ctypes.c_double),
                ("total_ms", ctypes.c_double), ("scanned_entries", ctypes.c_int64),
                ("work_items", ctypes.c_int64)]


class FlatTimings(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("minima_ms", ctypes.c_double), ("kth_ms", ctypes.c_double),
                ("collect_ms", ctypes.c_double), ("select_ms", ctypes.c_double),
                ("fallback_ms", ctypes.c_double), ("total_ms", ctypes.c_double)]


EXPORTS = ("ivfpq_validate_index_file", "ivfpq_validate_host_index", "ivfpq_load_index",
           "ivfpq_load_index_host", "ivfpq_free_index", "ivfpq_index_info", "ivfpq_search",
           "ivfpq_search_ex", "ivfpq_search_noalloc_ex", "ivfpq_coarse_ex", "ivfpq_assign_encode_ex", "ivfpq_kmeans_ex",
           "ivfpq_build_index_ex", "ivfpq_index_export",
           "ivfpq_compute_luts_ex",
           "ivfpq_select_topk_ex",
           "ivfpq_profile_begin",
           "ivfpq_profile_end", "ivfpq_flat_load_bf16", "ivfpq_flat_free",
           "ivfpq_flat_search_bf16_ex", "ivfpq_flat_search_bf16", "ivfpq_flat_profile_begin",
           "ivfpq_flat_profile_end", "ivfpq_stream_read", "ivfpq_last_error",
           "ivfpq_status_string")

_lib = None


def lib():
    """Load libivfpq.so (built in-tree by build_lib.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(the IVF-PQ search has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        st = ctypes.c_int
        sig = {
            "ivfpq_validate_index_file": ([ctypes.c_char_p], st),
            "ivfpq_validate_host_index": ([P], st),
            "ivfpq_load_index": ([ctypes.c_char_p, i32, P], st),
            "ivfpq_load_index_host": ([P, i32, P], st),
            "ivfpq_free_index": ([P], None),
            "ivfpq_index_info": ([P, P], st),
            "ivfpq_search": ([P, P, i64, i32, i32, P, P], st),
            "ivfpq_search_ex": ([P, P, P, i64, P, P, P, P], st),
            "ivfpq_search_noalloc_ex": ([P, P, P, i64, P, P, P, P], st),
            "ivfpq_coarse_ex": ([P, P, i64, i32, P, P, P], st),
            "ivfpq_assign_encode_ex": ([P, P, i64, P, P, P], st),
            "ivfpq_kmeans_ex": ([P, i64, i32, i32, i32, P, P, P, P], st),
            "ivfpq_build_index_ex": ([P, P, i64, i32, i32, i32, P, P, i32, P], st),
            "ivfpq_index_export": ([P, P, P, P, P, P], st),
            "ivfpq_compute_luts_ex": ([P, P, i64, P, i32, i32, P, P], st),
            "ivfpq_select_topk_ex": ([P, i64, i64, i32, P, P, P], st),
            "ivfpq_profile_begin": ([P, i32], st),
            "ivfpq_profile_end": ([P, P], st),
            "ivfpq_flat_load_bf16": ([P, i64, i32, i32, P], st),
            "ivfpq_flat_free": ([P], None),
            "ivfpq_flat_search_bf16_ex": ([P, P, i64, i32, P, P, P], st),
            "ivfpq_flat_search_bf16": ([P, P, i64, i32, P, P], st),
            "ivfpq_flat_profile_begin": ([P, i32], st),
            "ivfpq_flat_profile_end": ([P, P], st),
            "ivfpq_stream_read": ([P, ctypes.c_size_t, P, i32, P], st),
            "ivfpq_last_error": ([], ctypes.c_char_p),
            "ivfpq_status_string": ([i32], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise IVFPQError(status, lib().ivfpq_last_error().decode())


def ivfpq_last_error() -> str:
    return lib().ivfpq_last_error().decode()


def ivfpq_status_string(status: int) -> str:
    return lib().ivfpq_status_string(status).decode()


def ivfpq_validate_index_file(path: str) -> int:
    """Host-only validation; returns the status code (0 = valid)."""
    return lib().ivfpq_validate_index_file(os.fsencode(path))


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _host_struct(index, keep: list) -> HostIndexStruct:
    get = (lambda n: index[n]) if isinstance(index, dict) else (lambda n: getattr(index, n))
    cent = np.ascontiguousarray(get("centroids"), dtype=np.float32)
    books = np.ascontiguousarray(get("codebooks"), dtype=np.float32)
    sizes = np.ascontiguousarray(get("list_sizes"), dtype=np.int64)
    codes = np.ascontiguousarray(get("codes"), dtype=np.uint8)
    ids = np.ascontiguousarray(get("ids"), dtype=np.int64)
    keep.extend([cent, books, sizes, codes, ids])
    s = HostIndexStruct()
    s.d, s.nlist = cent.shape[1], cent.shape[0]
    s.m = books.shape[0]
    s.nbits = 8
    s.ntotal = codes.shape[0]
    s.centroids, s.codebooks, s.list_sizes = _np_ptr(cent), _np_ptr(books), _np_ptr(sizes)
    s.codes, s.ids = _np_ptr(codes), _np_ptr(ids)
    return s


def ivfpq_validate_host_index(index) -> int:
    keep: list = []
    s = _host_struct(index, keep)
    return lib().ivfpq_validate_host_index(ctypes.byref(s))


class Index:
    """Owner of a device index handle."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle
        self.info = ivfpq_index_info(self)

    @property
    def handle(self):
        if not self._h:
            raise ValueError("index is closed")
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            lib().ivfpq_free_index(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def search(self, queries, nprobe, k, **kw):
        return ivfpq_search_ex(self, queries, nprobe, k, **kw)


def ivfpq_load_index(path: str, device: int = 0) -> Index:
    h = ctypes.c_void_p()
    _check(lib().ivfpq_load_index(os.fsencode(path), device, ctypes.byref(h)))
    return Index(h)


def ivfpq_load_index_host(index, device: int = 0) -> Index:
    keep: list = []
    s = _host_struct(index, keep)
    h = ctypes.c_void_p()
    _check(lib().ivfpq_load_index_host(ctypes.byref(s), device, ctypes.byref(h)))
    return Index(h)


def ivfpq_build_index_ex(vectors: torch.Tensor, centroids: torch.Tensor,
                         codebooks: torch.Tensor, ids: torch.Tensor = None,
                         device: int = 0) -> Index:
    """Build an index on the device from device tensors: vectors [n, d]
    float32, centroids [nlist, d] float32, codebooks [m, 256, d/m] float32,
    ids [n] int64 (None: row numbers)."""
    x = _dev(vectors, torch.float32)
    c = _dev(centroids, torch.float32)
    b = _dev(codebooks, torch.float32)
    if x.dim() != 2 or c.dim() != 2 or b.dim() != 3 or c.shape[1] != x.shape[1] or \
            b.shape[1] != 256 or b.shape[0] * b.shape[2] != x.shape[1]:
        raise ValueError("expected vectors [n, d], centroids [nlist, d], codebooks [m, 256, d/m]")
    idp = 0
    if ids is not None:
        ids = _dev(ids, torch.int64)
        if ids.shape != (x.shape[0],):
            raise ValueError("expected ids [n]")
        idp = ids.data_ptr()
    h = ctypes.c_void_p()
    _check(lib().ivfpq_build_index_ex(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(idp),
                                      x.shape[0], x.shape[1], c.shape[0], b.shape[0],
                                      ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                      device, ctypes.byref(h)))
    return Index(h)


def ivfpq_index_export(index: Index) -> dict:
    """The index's arrays in host memory: centroids, codebooks, list_sizes,
    codes (list-major) and ids (numpy arrays, the host index layout)."""
    i = index.info
    d, nlist, m, n = i["d"], i["nlist"], i["m"], i["ntotal"]
    out = dict(centroids=np.empty((nlist, d), np.float32),
               codebooks=np.empty((m, 256, d // m), np.float32),
               list_sizes=np.empty(nlist, np.int64), codes=np.empty((n, m), np.uint8),
               ids=np.empty(n, np.int64))
    _check(lib().ivfpq_index_export(index.handle, *(_np_ptr(out[k]) for k in
                                                    ("centroids", "codebooks", "list_sizes",
                                                     "codes", "ids"))))
    return out


def ivfpq_free_index(index: Index) -> None:
    index.close()


def ivfpq_index_info(index: Index) -> dict:
    i = Info()
    _check(lib().ivfpq_index_info(index.handle, ctypes.byref(i)))
    return {f: getattr(i, f) for f, _ in Info._fields_ if f != "reserved"}


def ivfpq_search(index: Index, queries: np.ndarray, nprobe: int, k: int):
    """Blocking search on host arrays; returns (distances float32, ids int64)."""
    q = np.ascontiguousarray(queries, dtype=np.float32)
    nq = q.shape[0]
    d = np.empty((nq, k), dtype=np.float32)
    i = np.empty((nq, k), dtype=np.int64)
    _check(lib().ivfpq_search(index.handle, _np_ptr(q), nq, nprobe, k, _np_ptr(d), _np_ptr(i)))
    return d, i


def _dev(t: torch.Tensor, dtype) -> torch.Tensor:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"expected a contiguous {dtype} device tensor")
    return t


def _stream_ptr(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def ivfpq_search_ex(index: Index, queries: torch.Tensor, nprobe: int, k: int, lut: str = "f32",
                    mode: int = MODE_NORMAL, chunk_len: int = 0, return_probes: bool = False,
                    out=None, stream=None, metric: str = "l2", noalloc: bool = False):
    """Asynchronous device search on the current (or given) torch stream.
    metric "l2" (squared L2, ascending) or "ip" (inner product, descending).
    noalloc: call ivfpq_search_noalloc_ex (workspace in the library's fixed
    device scratch; pass `out` too so that nothing is allocated here either).

    Returns (distances [nq,k] float32, ids [nq,k] int64[, probes [nq,nprobe] int32])."""
    if metric not in ("l2", "ip"):
        raise ValueError("metric must be 'l2' or 'ip'")
    q = _dev(queries, torch.float32)
    nq = q.shape[0]
    if out is None:
        dist = torch.empty((nq, k), dtype=torch.float32, device=q.device)
        ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
        probes = torch.empty((nq, nprobe), dtype=torch.int32, device=q.device) \
            if return_probes else None
    else:
        dist, ids, probes = out
    p = SearchParams(nprobe, k, LUT_F16 if lut == "f16" else LUT_F32, mode, chunk_len,
                     METRIC_IP if metric == "ip" else METRIC_L2)
    fn = lib().ivfpq_search_noalloc_ex if noalloc else lib().ivfpq_search_ex
    _check(fn(index.handle, ctypes.byref(p), ctypes.c_void_p(q.data_ptr()),
              nq, ctypes.c_void_p(dist.data_ptr()),
              ctypes.c_void_p(ids.data_ptr()),
              ctypes.c_void_p(probes.data_ptr() if probes is not None else 0),
              _stream_ptr(stream)))
    return (dist, ids, probes) if return_probes else (dist, ids)


def ivfpq_coarse_ex(index: Index, queries: torch.Tensor, nprobe: int, stream=None):
    q = _dev(queries, torch.float32)
    nq = q.shape[0]
    probes = torch.empty((nq, nprobe), dtype=torch.int32, device=q.device)
    dist = torch.empty((nq, nprobe), dtype=torch.float32, device=q.device)
    _check(lib().ivfpq_coarse_ex(index.handle, ctypes.c_void_p(q.data_ptr()), nq, nprobe,
                                 ctypes.c_void_p(probes.data_ptr()),
                                 ctypes.c_void_p(dist.data_ptr()), _stream_ptr(stream)))
    return probes, dist


def ivfpq_assign_encode_ex(index: Index, vectors: torch.Tensor, stream=None):
    """List assignment and PQ codes of database vectors with the index's
    centroids and codebooks: (lists [n] int32, codes [n, m] uint8)."""
    x = _dev(vectors, torch.float32)
    if x.dim() != 2 or x.shape[1] != index.info["d"]:
        raise ValueError(f"expected vectors of shape [n, {index.info['d']}]")
    n = x.shape[0]
    lists = torch.empty(n, dtype=torch.int32, device=x.device)
    codes = torch.empty((n, index.info["m"]), dtype=torch.uint8, device=x.device)
    _check(lib().ivfpq_assign_encode_ex(index.handle, ctypes.c_void_p(x.data_ptr()), n,
                                        ctypes.c_void_p(lists.data_ptr()),
                                        ctypes.c_void_p(codes.data_ptr()), _stream_ptr(stream)))
    return lists, codes


def ivfpq_kmeans_ex(vectors: torch.Tensor, centers: torch.Tensor, iters: int, stream=None):
    """Lloyd's algorithm on the device: `centers` ([k, d] float32, updated in
    place) from `vectors` ([n, d] float32).  Returns the last round's
    (assignment [n] int32, counts [k] int32)."""
    x = _dev(vectors, torch.float32)
    c = _dev(centers, torch.float32)
    if x.dim() != 2 or c.dim() != 2 or x.shape[1] != c.shape[1]:
        raise ValueError("expected vectors [n, d] and centers [k, d]")
    n, (k, d) = x.shape[0], c.shape
    assign = torch.full((n,), -1, dtype=torch.int32, device=x.device)
    counts = torch.zeros(k, dtype=torch.int32, device=x.device)
    _check(lib().ivfpq_kmeans_ex(ctypes.c_void_p(x.data_ptr()), n, d, k, iters,
                                 ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(assign.data_ptr()),
                                 ctypes.c_void_p(counts.data_ptr()), _stream_ptr(stream)))
    return assign, counts


def ivfpq_compute_luts_ex(index: Index, queries: torch.Tensor, probes: torch.Tensor,
                          lut: str = "f32", stream=None):
    q = _dev(queries, torch.float32)
    pr = _dev(probes, torch.int32)
    nq, nprobe = pr.shape
    m = index.info["m"]
    out = torch.empty((nq, nprobe, m, 256), dtype=torch.float32, device=q.device)
    _check(lib().ivfpq_compute_luts_ex(index.handle, ctypes.c_void_p(q.data_ptr()), nq,
                                       ctypes.c_void_p(pr.data_ptr()), nprobe,
                                       LUT_F16 if lut == "f16" else LUT_F32,
                                       ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
    return out


def ivfpq_select_topk_ex(keys: torch.Tensor, k: int, stream=None):
    """Row-wise k smallest of a [rows, n] float32 device tensor:
    (values [rows,k] float32, column numbers [rows,k] int32)."""
    x = _dev(keys, torch.float32)
    rows, n = x.shape
    d = torch.empty((rows, k), dtype=torch.float32, device=x.device)
    p = torch.empty((rows, k), dtype=torch.int32, device=x.device)
    _check(lib().ivfpq_select_topk_ex(ctypes.c_void_p(x.data_ptr()), rows, n, k,
                                      ctypes.c_void_p(d.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                                      _stream_ptr(stream)))
    return d, p


def ivfpq_stream_read(data: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue the reference streaming read of a contiguous device tensor
    (measurement support); sink: an int32 device tensor of scratch words."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    s = _dev(sink, torch.int32)
    _check(lib().ivfpq_stream_read(ctypes.c_void_p(data.data_ptr()),
                                   data.numel() * data.element_size(),
                                   ctypes.c_void_p(s.data_ptr()), s.numel(), _stream_ptr(stream)))


def ivfpq_profile_begin(index: Index, max_calls: int) -> None:
    _check(lib().ivfpq_profile_begin(index.handle, max_calls))


def ivfpq_profile_end(index: Index) -> dict:
    t = Timings()
    _check(lib().ivfpq_profile_end(index.handle, ctypes.byref(t)))
    return {f: getattr(t, f) for f, _ in Timings._fields_ if f != "reserved"}


# ---------------------------------------------------------------------------
# exact search over a flat bfloat16 database
# ---------------------------------------------------------------------------

class FlatIndex:
    """Owner of a device flat-database handle."""

    def __init__(self, handle: ctypes.c_void_p, n: int, d: int):
        self._h = handle
        self.n, self.d = n, d

    @property
    def handle(self):
        if not self._h:
            raise ValueError("flat index is closed")
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            lib().ivfpq_flat_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ivfpq_flat_load_bf16(vectors: np.ndarray, device: int = 0) -> FlatIndex:
    """Upload [n, d] bfloat16 bit patterns (uint16, host)."""
    v = np.ascontiguousarray(vectors, dtype=np.uint16)
    h = ctypes.c_void_p()
    _check(lib().ivfpq_flat_load_bf16(_np_ptr(v), v.shape[0], v.shape[1], device,
                                      ctypes.byref(h)))
    return FlatIndex(h, v.shape[0], v.shape[1])


def ivfpq_flat_free(flat: FlatIndex) -> None:
    flat.close()


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return _dev(t, torch.int16)


def ivfpq_flat_search_bf16_ex(flat: FlatIndex, queries: torch.Tensor, k: int, out=None,
                              stream=None):
    """Asynchronous exact search; queries: [nq, d] device tensor of bfloat16 (or
    its bit patterns as int16).  Returns (distances [nq,k] float32, ids [nq,k]
    int64 row numbers)."""
    q = _bf16_bits(queries)
    nq = q.shape[0]
    if out is None:
        dist = torch.empty((nq, k), dtype=torch.float32, device=q.device)
        ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
    else:
        dist, ids = out
    _check(lib().ivfpq_flat_search_bf16_ex(flat.handle, ctypes.c_void_p(q.data_ptr()), nq, k,
                                           ctypes.c_void_p(dist.data_ptr()),
                                           ctypes.c_void_p(ids.data_ptr()), _stream_ptr(stream)))
    return dist, ids


def ivfpq_flat_search_bf16(flat: FlatIndex, queries: np.ndarray, k: int):
    """Blocking exact search on host bfloat16 bit patterns (uint16 [nq, d])."""
    q = np.ascontiguousarray(queries, dtype=np.uint16)
    nq = q.shape[0]
    d = np.empty((nq, k), dtype=np.float32)
    i = np.empty((nq, k), dtype=np.int64)
    _check(lib().ivfpq_flat_search_bf16(flat.handle, _np_ptr(q), nq, k, _np_ptr(d), _np_ptr(i)))
    return d, i


def ivfpq_flat_profile_begin(flat: FlatIndex, max_calls: int) -> None:
    _check(lib().ivfpq_flat_profile_begin(flat.handle, max_calls))


def ivfpq_flat_profile_end(flat: FlatIndex) -> dict:
    t = FlatTimings()
    _check(lib().ivfpq_flat_profile_end(flat.handle, ctypes.byref(t)))
    return {f: getattr(t, f) for f, _ in FlatTimings._fields_ if f != "reserved"}
