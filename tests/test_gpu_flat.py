"""Exact search over a flat bfloat16 database on the GPU against the oracle's
brute force (exact, double precision), through the C ABI."""
import numpy as np
import pytest

from approximate_nearest_neighbour_amd import datagen as G
from oracle import check

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import approximate_nearest_neighbour_amd as A
    return A


def uniform_bits(rng, n, d):
    return G.to_bf16_bits(rng.uniform(-1.0, 1.0, size=(n, d)).astype(np.float32))


def run(A, db, q, k):
    f = A.ivfpq_flat_load_bf16(db)
    qd = torch.from_numpy(q.view(np.int16)).cuda()
    dist, ids = A.ivfpq_flat_search_bf16_ex(f, qd, k)
    torch.cuda.synchronize()
    out = dist.cpu().numpy(), ids.cpu().numpy()
    f.close()
    return out


SHAPES = [  # n, d, nq, k: several tiles, ragged tails, d not a multiple of 32
    (1000, 32, 50, 10),
    (5003, 100, 37, 100),
    (20000, 128, 300, 1024),
    (64, 8, 5, 100),
    (3000, 256, 20, 64),
    (1, 4, 3, 5),
    (70001, 96, 129, 257),
]


@pytest.mark.parametrize("n,d,nq,k", SHAPES)
def test_flat_matches_oracle(A, n, d, nq, k):
    print(f"flat parity n={n} d={d} nq={nq} k={k}", flush=True)
    rng = np.random.default_rng(n * 7 + d)
    db, q = uniform_bits(rng, n, d), uniform_bits(rng, nq, d)
    gd, gi = run(A, db, q, k)
    rep = check.compare_flat(db, q, k, gd, gi)
    assert rep.ok(), (rep.summary(), rep.failures[:5])


def test_flat_integer_data_is_exact(A):
    # small integers are exact in bf16 and every distance is an exact integer
    # in float32: the sorted distances must equal the oracle's bit for bit
    rng = np.random.default_rng(3)
    n, d, nq, k = 9000, 64, 40, 300
    db = G.to_bf16_bits(rng.integers(-3, 4, size=(n, d)).astype(np.float32))
    q = G.to_bf16_bits(rng.integers(-3, 4, size=(nq, d)).astype(np.float32))
    gd, gi = run(A, db, q, k)
    from oracle import oracle as O
    od, oi = O.bruteforce_bf16(db, q, k)
    assert np.array_equal(gd.astype(np.float64), od)
    rep = check.compare_flat(db, q, k, gd, gi, tau=0.0)
    assert rep.ok(), rep.failures[:5]


def test_flat_many_ties_take_the_fallback(A):
    # 6000 copies of one row: every query's bound sits on the tie, more rows
    # than the candidate buffer holds qualify, and the exact fallback answers
    rng = np.random.default_rng(4)
    d, k = 16, 50
    base = rng.integers(-2, 3, size=(1, d)).astype(np.float32)
    other = rng.integers(-2, 3, size=(3000, d)).astype(np.float32) + 5.0
    db = G.to_bf16_bits(np.vstack([np.repeat(base, 6000, axis=0), other]))
    q = G.to_bf16_bits(np.vstack([base, base + 1.0, other[:3]]))
    gd, gi = run(A, db, q, k)
    rep = check.compare_flat(db, q, k, gd, gi, tau=0.0)
    assert rep.ok(), rep.failures[:5]
    assert np.all(gd[0] == 0.0) and np.all(gi[0] < 6000)


def test_flat_chunked_batches_match(A, monkeypatch):
    rng = np.random.default_rng(5)
    db, q = uniform_bits(rng, 4000, 32), uniform_bits(rng, 70, 32)
    full = run(A, db, q, 20)
    # slot minima, bound, counter line, flag, |x|^2, candidates, -2x row
    per_query = 16 * 63 * 4 + 12 + 128 + 4096 * 8 + 32 * 2
    monkeypatch.setenv("IVFPQ_TEST_FLAT_WS_BYTES", str(per_query * 16 + 300))
    chunked = run(A, db, q, 20)
    assert np.array_equal(full[0], chunked[0])
    rep = check.compare_flat(db, q, 20, *chunked)
    assert rep.ok(), rep.failures[:5]


RECOMPUTE_SHAPES = [  # more than one query block (2048), ragged segments, k = 1024
    (20000, 128, 300, 1024),
    (70001, 96, 129, 257),
    (5003, 100, 2500, 100),
    (3000, 256, 20, 64),
    (1, 4, 3, 5),
]


@pytest.mark.parametrize("n,d,nq,k", RECOMPUTE_SHAPES)
def test_flat_recompute_equals_full_collect(A, monkeypatch, n, d, nq, k):
    # The collect pass recomputes only the slots whose minimum is under the
    # bound; the earlier form (a second full GEMM with the bound test, behind
    # a test switch) must give the same k distances to the bit, and the same
    # rows wherever a distance is not tied with another row's.
    print(f"flat recompute vs full collect n={n} d={d} nq={nq} k={k}", flush=True)
    rng = np.random.default_rng(n + 13 * d + nq)
    db, q = uniform_bits(rng, n, d), uniform_bits(rng, nq, d)
    gd, gi = run(A, db, q, k)
    monkeypatch.setenv("IVFPQ_TEST_FLAT_FULL_COLLECT", "1")
    fd, fi = run(A, db, q, k)
    monkeypatch.delenv("IVFPQ_TEST_FLAT_FULL_COLLECT")
    assert np.array_equal(gd.view(np.uint32), fd.view(np.uint32))
    for row in range(nq):
        vals, counts = np.unique(gd[row], return_counts=True)
        single = set(vals[counts == 1].tolist())
        for j in range(k):
            if gd[row, j] in single and gd[row, j] != gd[row, -1]:
                assert gi[row, j] == fi[row, j], (row, j)
    rep = check.compare_flat(db, q, k, gd, gi)
    assert rep.ok(), (rep.summary(), rep.failures[:5])


def test_flat_empty_database_and_host_api(A):
    rng = np.random.default_rng(6)
    q = uniform_bits(rng, 4, 8)
    gd, gi = run(A, np.zeros((0, 8), np.uint16), q, 3)
    assert np.all(gi == -1) and np.all(np.isinf(gd))
    db = uniform_bits(rng, 500, 8)
    f = A.ivfpq_flat_load_bf16(db)
    hd, hi = A.ivfpq_flat_search_bf16(f, q, 7)
    dd, di = A.ivfpq_flat_search_bf16_ex(f, torch.from_numpy(q.view(np.int16)).cuda(), 7)
    assert np.array_equal(hd, dd.cpu().numpy()) and np.array_equal(hi, di.cpu().numpy())
    with pytest.raises(A.IVFPQError):
        A.ivfpq_flat_search_bf16(f, q, 0)
    with pytest.raises(A.IVFPQError):
        A.ivfpq_flat_search_bf16(f, q, 1025)
    f.close()


def test_flat_profile_reports_every_pass(A):
    rng = np.random.default_rng(7)
    db, q = uniform_bits(rng, 20000, 128), uniform_bits(rng, 64, 128)
    f = A.ivfpq_flat_load_bf16(db)
    qd = torch.from_numpy(q.view(np.int16)).cuda()
    A.ivfpq_flat_profile_begin(f, 3)
    for _ in range(3):
        A.ivfpq_flat_search_bf16_ex(f, qd, 100)
    t = A.ivfpq_flat_profile_end(f)
    assert t["calls"] == 3
    for key in ("minima_ms", "kth_ms", "collect_ms", "select_ms", "fallback_ms", "total_ms"):
        assert t[key] > 0, key
    f.close()
