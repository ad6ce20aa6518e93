"""The allocation-free search (ivfpq_search_noalloc_ex) against the search
with a handle-owned workspace (ivfpq_search_ex), through the C ABI.

Two calls in a row, the second with a smaller batch (the fixed scratch keeps
the first call's contents): the rows must equal ivfpq_search_ex's (the same
kernels; distances bit for bit, ids up to exact ties at the k-th distance)
and pass the oracle's acceptance rules.  The call must not change the
device's free memory, and a batch whose workspace exceeds the fixed scratch
must be rejected before any device work.
"""
import numpy as np
import pytest
import torch

import approximate_nearest_neighbour_amd as A
from approximate_nearest_neighbour_amd import binding as B
from approximate_nearest_neighbour_amd import datagen as G
from oracle import check
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def skewed_index(seed):
    rng = np.random.default_rng(seed)
    nlist, d, m = 256, 96, 8
    sizes = rng.multinomial(300_000, rng.dirichlet(np.full(nlist, 0.3)))
    return G.random_index(rng, nlist, d, m, sizes, codebook_scale=0.3), rng


def outputs(nq, nprobe, k):
    return (torch.empty((nq, k), dtype=torch.float32, device="cuda"),
            torch.empty((nq, k), dtype=torch.int64, device="cuda"),
            torch.empty((nq, nprobe), dtype=torch.int32, device="cuda"))


def same_rows(d_na, i_na, d_ref, i_ref):
    """Distances bit for bit; ids equal except members of an exact tie at
    the row's k-th distance."""
    assert np.array_equal(d_na, d_ref)
    for r in range(len(d_na)):
        a, b = i_na[r], i_ref[r]
        if np.array_equal(a, b):
            continue
        kth = d_ref[r][-1]
        assert set(a[d_na[r] < kth].tolist()) == set(b[d_ref[r] < kth].tolist()), r
        assert len(set(a.tolist())) == len(a), r


@pytest.mark.parametrize("metric", ["l2", "ip"])
def test_noalloc_equals_search_ex_on_two_calls(metric):
    idx, rng = skewed_index(77 if metric == "l2" else 78)
    ix = A.ivfpq_load_index_host(idx)
    lut_mode = O.IP if metric == "ip" else O.LUT_F64
    # one call first: the fixed scratch's address is looked up on the first
    # call on a device (the code object may be loaded then)
    q0 = torch.from_numpy(rng.standard_normal((8, idx.d)).astype(np.float32)).cuda()
    A.ivfpq_search_ex(ix, q0, 4, 10, out=outputs(8, 4, 10)[:2] + (None,), metric=metric,
                      noalloc=True)
    torch.cuda.synchronize()
    for nq, nprobe, k, chunk in [(4000, 24, 100, 0), (900, 16, 64, 512)]:
        q = (idx.centroids[rng.integers(0, idx.nlist, nq)]
             + 0.5 * rng.standard_normal((nq, idx.d))).astype(np.float32)
        qd = torch.from_numpy(q).cuda()
        out = outputs(nq, nprobe, k)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        A.ivfpq_search_ex(ix, qd, nprobe, k, chunk_len=chunk, return_probes=True, out=out,
                          metric=metric, noalloc=True)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        d_na, i_na, p_na = (t.cpu().numpy() for t in out)
        d_ref, i_ref, p_ref = (t.cpu().numpy() for t in A.ivfpq_search_ex(
            ix, qd, nprobe, k, chunk_len=chunk, return_probes=True, metric=metric))
        assert np.array_equal(p_na, p_ref)
        same_rows(d_na, i_na, d_ref, i_ref)
        rows = np.sort(rng.choice(nq, 40, replace=False))
        rep = check.compare_search(idx, q[rows], nprobe, k, d_na[rows], i_na[rows], p_na[rows],
                                   lut_mode=lut_mode)
        assert rep.ok(), rep.failures[:3]
    ix.close()


def test_noalloc_with_giant_lists():
    """An index with lists of 2^20 entries or more: the allocation-free search
    also carves the giant-list order's arrays (rank-major order, item keys,
    bucket counters) from the fixed scratch and lays the queries' sequences
    out region-aligned; two calls in a row (the second smaller) must equal
    ivfpq_search_ex's rows."""
    rng = np.random.default_rng(2027)
    nlist, d, m = 40, 16, 4
    sizes = rng.integers(50, 400, nlist).astype(np.int64)
    sizes[5], sizes[11] = 1_300_000, 1_050_000
    idx = G.random_index(rng, nlist, d, m, sizes, codebook_scale=0.3)
    cent = idx.centroids.copy()
    cent[5] = 0.0  # probed by most queries
    idx = G.HostIndex(cent, idx.codebooks, idx.list_sizes, idx.codes, idx.ids)
    ix = A.ivfpq_load_index_host(idx)
    for nq, nprobe, k, chunk in [(600, 6, 50, 0), (150, 4, 20, 65536)]:
        q = (cent[rng.integers(0, nlist, nq)] + 0.5 * rng.standard_normal((nq, d))).astype(np.float32)
        qd = torch.from_numpy(q).cuda()
        out = outputs(nq, nprobe, k)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        A.ivfpq_search_ex(ix, qd, nprobe, k, chunk_len=chunk, return_probes=True, out=out,
                          noalloc=True)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        d_na, i_na, p_na = (t.cpu().numpy() for t in out)
        assert np.mean(np.any(p_na == 5, axis=1)) > 0.5
        d_ref, i_ref, p_ref = (t.cpu().numpy() for t in A.ivfpq_search_ex(
            ix, qd, nprobe, k, chunk_len=chunk, return_probes=True))
        assert np.array_equal(p_na, p_ref)
        same_rows(d_na, i_na, d_ref, i_ref)
        rows = np.sort(rng.choice(nq, 12, replace=False))
        rep = check.compare_search(idx, q[rows], nprobe, k, d_na[rows], i_na[rows], p_na[rows])
        assert rep.ok(), rep.failures[:3]
    ix.close()


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    idx, rng = skewed_index(79)
    ix = A.ivfpq_load_index_host(idx)
    nq, nprobe, k = 1_200_000, 32, 10      # probes alone: 154 MB > 128 MiB
    qd = torch.zeros((nq, idx.d), dtype=torch.float32, device="cuda")
    out = outputs(nq, nprobe, k)
    with pytest.raises(B.IVFPQError) as e:
        A.ivfpq_search_ex(ix, qd, nprobe, k, return_probes=False, out=out[:2] + (None,),
                          noalloc=True)
    assert e.value.status == B.E_INVALID_ARG and "scratch" in str(e.value)
    ix.close()
