"""Full-size IVF-PQ parity: the benchmark shapes (1M x 128 / m 16, 10M x 96 /
m 32, 1B entries / m 8 with Zipf lists), all 10,000 queries searched in the
launch configuration the benchmark times (the 10M and 1B shapes also with the
inner-product metric), a sample of the queries checked against the oracle
(exact, double precision) one by one."""
import time

import numpy as np
import pytest

from approximate_nearest_neighbour_amd import datagen as G
from oracle import check
from oracle import oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import approximate_nearest_neighbour_amd as A
    return A


def sample_rows(nq, count, seed):
    rng = np.random.default_rng(seed)
    rows = set([0, nq - 1]) | set(rng.choice(nq, size=count - 2, replace=False).tolist())
    return np.array(sorted(rows))


def search_and_check(A, w, runs=(("f32", "l2"),), sample=16, giant=0):
    """runs: (table type, metric[, sample, giant]) searched on one upload of
    the index; sample rows are checked against the oracle, plus (giant)
    rows whose probes include a list of more than 10^6 entries (the longest
    lists of a skewed index)."""
    t = time.time()
    ix = A.ivfpq_load_index_host(w.index, device=0)
    q = torch.from_numpy(w.queries).cuda()
    print(f"  {w.name}: index uploaded ({time.time() - t:.1f} s)", flush=True)
    for run in runs:
        lut, metric = run[:2]
        n_sample, n_giant = (run[2], run[3]) if len(run) > 2 else (sample, giant)
        t = time.time()
        d, i, p = A.ivfpq_search_ex(ix, q, w.nprobe, w.k, lut=lut, metric=metric,
                                    return_probes=True)
        torch.cuda.synchronize()
        print(f"  {w.name} lut={lut} metric={metric}: searched {len(w.queries)} queries "
              f"({time.time() - t:.1f} s)", flush=True)
        rows = sample_rows(len(w.queries), n_sample, 11)
        if n_giant:
            big = np.flatnonzero(np.asarray(w.index.list_sizes) > 1_000_000)
            hits = np.flatnonzero(np.isin(p.cpu().numpy(), big).any(axis=1))
            print(f"  {len(hits)} queries probe one of the {len(big)} lists above 10^6 "
                  f"entries; checking {min(n_giant, len(hits))} of them", flush=True)
            rows = np.unique(np.concatenate([rows, hits[:n_giant]]))
        mode = O.IP if metric == "ip" else O.LUT_F16 if lut == "f16" else O.LUT_F64
        t = time.time()
        decomposed = bool(A.ivfpq_index_info(ix)["flags"] & 1) and lut == "f32" \
            and metric == "l2"
        split = bool(A.ivfpq_index_info(ix)["flags"] & 2) and 1 < w.nprobe <= 128
        rep = check.compare_search(w.index, w.queries[rows], w.nprobe, w.k,
                                   d.cpu().numpy()[rows], i.cpu().numpy()[rows],
                                   p.cpu().numpy()[rows], lut_mode=mode, decomposed=decomposed,
                                   split_bf16=split)
        print(f"  parity {rep.summary()} on {len(rows)} rows ({time.time() - t:.1f} s)",
              flush=True)
        assert rep.ok(), rep.failures[:5]
    ix.close()


def test_fullsize_gmm_1m(A):
    print("full size: 1M x 128, nlist 1024, m 16, nprobe 32, k 100", flush=True)
    w = G.gmm1m()
    search_and_check(A, w)


def test_fullsize_10m_shape(A):
    # the 10M x 96 / nlist 4096 / m 32 shape with random centroids, codebooks
    # and codes (a trained index of this size takes minutes of host time;
    # the kernels and launch shapes are the same)
    print("full size: 10M entries, d 96, nlist 4096, m 32, nprobe 64, k 100", flush=True)
    rng = np.random.default_rng(404)
    nlist, n = 4096, 10_000_000
    sizes = np.bincount(rng.integers(0, nlist, size=n), minlength=nlist)
    index = G.random_index(rng, nlist, 96, 32, sizes, codebook_scale=0.3)
    queries = rng.standard_normal((10_000, 96), dtype=np.float32)
    w = G.Workload("ivfpq_shape_n10m_d96_m32_nlist4096", index, queries, 64, 100)
    # float32 and binary16 tables, and the inner-product metric
    search_and_check(A, w, runs=(("f32", "l2"), ("f16", "l2"), ("f32", "ip")))


def test_fullsize_zipf_1b(A):
    print("full size: 1B entries, d 96, nlist 262144 (Zipf), m 8, nprobe 128, k 100",
          flush=True)
    w = G.zipf_workload()
    # squared L2 (float32 and binary16 tables) and the inner-product metric
    # (the lists were built for L2, which the metric does not assume)
    search_and_check(A, w, runs=(("f32", "l2", 200, 40), ("f16", "l2", 48, 8),
                                 ("f32", "ip", 48, 8)))


def test_fullsize_flat_bf16(A):
    print("full size: flat bf16 1M x 128, 10,000 queries, k 1024", flush=True)
    w = G.flat_bf16_workload()
    f = A.ivfpq_flat_load_bf16(w.vectors)
    q = torch.from_numpy(w.queries.view(np.int16)).cuda()
    d, i = A.ivfpq_flat_search_bf16_ex(f, q, w.k)
    torch.cuda.synchronize()
    rows = sample_rows(len(w.queries), 12, 13)
    rep = check.compare_flat(w.vectors, w.queries[rows], w.k, d.cpu().numpy()[rows],
                             i.cpu().numpy()[rows])
    print(f"  parity {rep.summary()}", flush=True)
    f.close()
    assert rep.ok(), rep.failures[:5]


def test_fullsize_knn_graph_1m(A):
    # the k-NN graph of the 1M x 128 workload: all 1M database vectors
    # searched with k = 10 in one call (the benchmark's configuration),
    # sampled rows checked against the oracle
    print("full size: k-NN graph, 1M x 128 queries against the 1M index, k 10", flush=True)
    w = G.gmm1m(keep_vectors=True)
    gw = G.Workload("knn_graph_n1m_d128_k10", w.index, w.vectors, w.nprobe, 10)
    search_and_check(A, gw, sample=24)
