"""The coarse step with split bfloat16 products (indexes with d <= 96 and
nlist >= 16,384, nprobe 2..128): x.c formed from three bfloat16 parts of each
operand on the bfloat16 matrix cores ("Leveraging the bfloat16 artificial
intelligence datatype for higher-precision computations", Henry, Tang and
Heinecke), against the oracle's exact coarse distances.

* Exact: integer queries in [-300, 300] (two bfloat16 parts each: 8 bits do not
  hold them) and integer centroids in [-3, 3].  Every partial product and
  every sum is an integer below 2^24, exact in float32 in any order, so the
  device's distances must equal the oracle's to the bit, its probes the
  oracle's except inside an exact tie at the nprobe-th distance; and the
  float32 kernel (test switch IVFPQ_TEST_COARSE_FP32) must return the same
  distances.  Ragged tiles (nlist not a multiple of 64), d not a multiple of
  32, one and several centroid splits, both metrics.
* Random N(0, 1) data at the shape of the 1B workload's coarse step: probes
  within rule 1's band for split products, and the float32 kernel's distances
  of the same lists within the sum of the two bands.
"""
import os
import sys

import numpy as np
import pytest

import approximate_nearest_neighbour_amd as A
from oracle import check
from oracle import oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def flat_index(cent):
    nlist, d = cent.shape
    return dict(centroids=cent, codebooks=np.zeros((1, 256, d), np.float32),
                list_sizes=np.zeros(nlist, np.int64), codes=np.zeros((0, 1), np.uint8),
                ids=np.zeros(0, np.int64))


def coarse(ix, q, nprobe, fp32=False):
    old = os.environ.get("IVFPQ_TEST_COARSE_FP32")
    if fp32:
        os.environ["IVFPQ_TEST_COARSE_FP32"] = "1"
    else:
        os.environ.pop("IVFPQ_TEST_COARSE_FP32", None)
    try:
        p, dist = A.ivfpq_coarse_ex(ix, torch.from_numpy(q).cuda(), nprobe)
        torch.cuda.synchronize()
        return p.cpu().numpy(), dist.cpu().numpy()
    finally:
        if old is None:
            os.environ.pop("IVFPQ_TEST_COARSE_FP32", None)
        else:
            os.environ["IVFPQ_TEST_COARSE_FP32"] = old


def oracle_rows(q, cent, ip):
    nlist = cent.shape[0]
    if ip:
        out = []
        for r in range(len(q)):
            allp, ips = O.coarse_ip(q[r], cent, nlist)
            out.append((allp, -ips))
        return out
    return [O.coarse(q[r], cent, nlist) for r in range(len(q))]


def assert_exact(p, dist, ref, nprobe):
    for r, (allp, alld) in enumerate(ref):
        want = np.asarray(alld[:nprobe], dtype=np.float64)
        assert np.array_equal(dist[r].astype(np.float64), want), (r, dist[r][:5], want[:5])
        edge = alld[nprobe - 1]
        below = set(int(l) for l, v in zip(allp, alld) if v < edge)
        tie = set(int(l) for l, v in zip(allp, alld) if v == edge)
        got = set(int(l) for l in p[r])
        assert len(got) == nprobe and below <= got and got - below <= tie, r


SHAPES = [  # nlist, d, nq, nprobe
    (16400, 96, 70, 128),
    (16384, 70, 33, 64),
    (20000, 32, 130, 2),
    (17000, 17, 64, 100),
]


@pytest.mark.parametrize("nlist,d,nq,nprobe", SHAPES)
@pytest.mark.parametrize("metric", ["l2", "ip"])
def test_split_products_exact_on_integer_data(nlist, d, nq, nprobe, metric):
    say(f"coarse split exact nlist={nlist} d={d} nq={nq} nprobe={nprobe} {metric}")
    rng = np.random.default_rng(nlist + d + nq)
    cent = rng.integers(-3, 4, (nlist, d)).astype(np.float32)
    q = rng.integers(-300, 301, (nq, d)).astype(np.float32)
    # exact ties at and around the nprobe-th distance: duplicated centroids
    cent[nlist // 2: nlist // 2 + 40] = cent[7]
    ix = A.ivfpq_load_index_host(flat_index(cent))
    assert A.ivfpq_index_info(ix)["flags"] & 2
    ip = metric == "ip"
    if ip:
        p, dist = A.ivfpq_search_ex(ix, torch.from_numpy(q).cuda(), nprobe, 1, metric="ip",
                                    return_probes=True)[2], None
        # the search returns probes only; the coarse entry point is L2, so the
        # inner product is checked through its probe set
        ref = oracle_rows(q, cent, True)
        pr = p.cpu().numpy()
        for r, (allp, alld) in enumerate(ref):
            edge = alld[nprobe - 1]
            below = set(int(l) for l, v in zip(allp, alld) if v < edge)
            tie = set(int(l) for l, v in zip(allp, alld) if v == edge)
            got = set(int(l) for l in pr[r])
            assert len(got) == nprobe and below <= got and got - below <= tie, r
    else:
        p, dist = coarse(ix, q, nprobe)
        assert_exact(p, dist, oracle_rows(q, cent, False), nprobe)
        p32, dist32 = coarse(ix, q, nprobe, fp32=True)
        assert np.array_equal(dist, dist32)
    ix.close()


def test_split_products_random_data_at_the_1b_coarse_shape():
    nlist, d, nq, nprobe = 65536, 96, 200, 128
    say(f"coarse split random nlist={nlist} d={d} nq={nq} nprobe={nprobe}")
    rng = np.random.default_rng(5)
    cent = rng.standard_normal((nlist, d)).astype(np.float32)
    q = rng.standard_normal((nq, d)).astype(np.float32)
    index = flat_index(cent)
    ix = A.ivfpq_load_index_host(index)
    p, dist = coarse(ix, q, nprobe)
    p32, dist32 = coarse(ix, q, nprobe, fp32=True)
    op = np.stack([O.coarse(q[r], cent, nprobe)[0] for r in range(nq)])
    for probes, split in ((p, True), (p32, False)):
        rep = check.Report()
        check.check_probes(index, q, probes, op, rep, split_bf16=split)
        assert rep.ok(), rep.failures[:5]
    cmax = float(np.max(np.sum(cent.astype(np.float64) ** 2, axis=1)))
    g_split = check.gamma(check.coarse_gamma_n(d, True))
    g_f32 = check.gamma(check.coarse_gamma_n(d, False))
    worst = 0.0
    for r in range(nq):
        x2 = float(np.sum(q[r].astype(np.float64) ** 2))
        allp, alld = O.coarse(q[r], cent, nlist)
        ref = dict(zip(allp.tolist(), alld.tolist()))
        a = dict(zip(p[r].tolist(), dist[r].tolist()))
        b = dict(zip(p32[r].tolist(), dist32[r].tolist()))
        for l, v in a.items():
            assert abs(v - ref[l]) <= 2 * g_split * (x2 + cmax)
            worst = max(worst, abs(v - ref[l]) / (x2 + cmax))
            if l in b:
                assert abs(v - b[l]) <= 2 * (g_split + g_f32) * (x2 + cmax)
    # the observed error is far inside the bound: about float32 rounding
    say(f"  largest |error| / (|x|^2 + max |c|^2): {worst:.3g}")
    assert worst < 1e-6
    ix.close()
