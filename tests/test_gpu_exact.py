"""Bit-exact parity of every compiled scan shape on integer data.

Integer centroids and codewords in [-3, 3] and integer queries in [-6, 6]:
every residual, table entry (difference form and, with float32 tables, the
decomposed form; binary16 storage of the difference form: entries stay below
2048) and sum is an exact small integer in float32, and so is every
inner-product score.  The device must therefore
return the oracle's distances exactly, the same ids below the k-th distance
and only members of the k-th distance's tie group at it.

Each case plants what the method's edge cases need (the IVFPQ section of
"Custom 8-bit floating point value format for reducing shared memory bank
conflict in ANN search": R = sum_j F_j(code_j) = |x - (c_l + decode(code))|^2):
queries equal to an entry's reconstruction (distance 0), entries with
duplicated codes in one list and across lists (exact ties, several of them
at the k-th distance), and far more candidates than k.  Each shape runs with
one work item per query (the scan writes the result) and with many (the
cross-item merge), at float32 and binary16 tables and the inner-product
metric; the (m 16, dsub 8) shape also with its decomposed tables switched
off at index load.

Compiled shapes (m, dsub): (4, 8), (16, 8), (32, 3), (8, 12); (5, 4) runs the
run-time-shape kernel for comparison.
"""
import sys

import numpy as np
import pytest

import approximate_nearest_neighbour_amd as A
from approximate_nearest_neighbour_amd import datagen as G
from oracle import oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHAPES = [(4, 8), (16, 8), (32, 3), (8, 12), (5, 4)]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def exact_case(m, dsub, seed, nlist=10, n=6000, nq=24):
    rng = np.random.default_rng(seed)
    d = m * dsub
    cent = rng.integers(-3, 4, (nlist, d)).astype(np.float32)
    books = rng.integers(-3, 4, (m, 256, dsub)).astype(np.float32)
    sizes = rng.multinomial(n, np.ones(nlist) / nlist).astype(np.int64)
    codes = rng.integers(0, 256, (n, m), dtype=np.uint8)
    off = np.concatenate([[0], np.cumsum(sizes)])
    # exact ties: rows copied inside a list (identical reconstruction) and
    # across lists (identical code, another centroid)
    for _ in range(60):
        a, b = rng.integers(0, n, 2)
        codes[b] = codes[a]
    big = int(np.argmax(sizes))
    for r in range(off[big], off[big] + min(40, sizes[big])):
        codes[r] = codes[off[big]]          # 40 equal entries in one list
    ids = rng.permutation(n).astype(np.int64)
    idx = G.HostIndex(cent, books, sizes, codes, ids)
    q = rng.integers(-6, 7, (nq, d)).astype(np.float32)
    # zero distances: queries on reconstructions (values stay in [-6, 6])
    for t in range(0, nq, 3):
        pos = int(off[big]) if t == 0 else int(rng.integers(0, n))
        l = int(np.searchsorted(off, pos, side="right") - 1)
        q[t] = cent[l] + np.concatenate([books[j, codes[pos, j]] for j in range(m)])
    return idx, q


def run(idx, q, nprobe, k, lut="f32", metric="l2", chunk_len=0, expect_decomposed=None):
    ix = A.ivfpq_load_index_host(idx)
    if expect_decomposed is not None:
        assert bool(A.ivfpq_index_info(ix)["flags"] & 1) == expect_decomposed
    qd = torch.from_numpy(q).cuda()
    d, i, p = A.ivfpq_search_ex(ix, qd, nprobe, k, lut=lut, metric=metric, chunk_len=chunk_len,
                                return_probes=True)
    torch.cuda.synchronize()
    out = d.cpu().numpy(), i.cpu().numpy(), p.cpu().numpy()
    ix.close()
    return out


def assert_exact(idx, q, nprobe, k, d, i, p, metric="l2"):
    """Distances equal the oracle's bit for bit; ids equal below the k-th
    value, tie-group members at it; probe sets equal (integer coarse
    distances are exact too)."""
    n = int(idx.ntotal)
    mode = O.IP if metric == "ip" else O.LUT_F64
    od, oi, op = O.search(idx, q, nprobe, n, lut_mode=mode)      # every candidate, sorted
    sgn = -1.0 if metric == "ip" else 1.0
    # probe sets: equal, except lists tied exactly with the nprobe-th coarse
    # value (any member of a tie is a correct choice); those rows are then
    # compared with the oracle run on the device's probes
    differ = []
    cent = idx.centroids.astype(np.float64)
    for r in range(len(q)):
        g, o = set(p[r].tolist()), set(op[r].tolist())
        assert len(g) == nprobe
        if g == o:
            continue
        xr = q[r].astype(np.float64)
        key = -(cent @ xr) if metric == "ip" else np.sum((xr - cent) ** 2, axis=1)
        edge = np.sort(key)[nprobe - 1]
        assert all(key[l] == edge for l in g ^ o), (r, sorted(g), sorted(o))
        differ.append(r)
    if differ:
        say(f"{len(differ)} rows with a tie at the nprobe-th coarse value")
        rows = np.asarray(differ)
        od2, oi2, _ = O.search(idx, q[rows], nprobe, n, lut_mode=mode, probes=p[rows])
        od, oi = od.copy(), oi.copy()
        od[rows], oi[rows] = od2, oi2
    for r in range(len(q)):
        valid = int(np.sum(oi[r] >= 0))
        kk = min(k, valid)
        assert np.array_equal(d[r, :kk], od[r, :kk].astype(np.float32)), r
        assert np.all(i[r, kk:] == -1)
        if kk < k:
            assert np.all(np.isinf(d[r, kk:]))
        if kk == 0:
            continue
        kth = od[r, kk - 1]
        key = sgn * od[r]                 # ascending ranking key
        kk_key = sgn * kth
        below = set(oi[r][key < kk_key].tolist())
        got = i[r, :kk]
        gkey = sgn * d[r, :kk].astype(np.float64)
        assert set(got[gkey < kk_key].tolist()) == below, r
        tie = set(oi[r][od[r] == kth].tolist())
        at = got[gkey == kk_key]
        assert len(set(at.tolist())) == len(at) and set(at.tolist()) <= tie, r
        dist_of = dict(zip(oi[r].tolist(), od[r].tolist()))
        assert all(dist_of[int(a)] == float(b) for a, b in zip(got, d[r, :kk])), r


@pytest.mark.parametrize("m,dsub", SHAPES)
@pytest.mark.parametrize("lut", ["f32", "f16"])
def test_exact_l2(m, dsub, lut):
    idx, q = exact_case(m, dsub, seed=100 * m + dsub)
    nlist = idx.nlist
    for nprobe, k, chunk in [(nlist, 100, 0), (nlist, 100, 256), (3, 100, 0), (nlist, 1, 64),
                             (2, 1024, 0)]:
        say(f"exact l2 m={m} dsub={dsub} lut={lut} nprobe={nprobe} k={k} chunk={chunk}")
        d, i, p = run(idx, q, nprobe, k, lut=lut, chunk_len=chunk)
        assert_exact(idx, q, nprobe, k, d, i, p)
        if nprobe == nlist:         # planted zero distances (their lists probed)
            assert np.all(d[0::3, 0] == 0.0)
    # the 40 equal entries of one list tie at the k-th distance for the query
    # placed on them (k = 10 < 40: only tie members may be returned)
    d, i, p = run(idx, q[:1], nlist, 10, lut=lut)
    assert np.all(d[0] == 0.0)
    assert_exact(idx, q[:1], nlist, 10, d, i, p)


@pytest.mark.parametrize("wide_min", ["1", "300", "100000000"])
def test_exact_l2_m8_table_forms(monkeypatch, wide_min):
    """The (m 8, dsub 12) scan with every piece in the replicated table form
    (wide_min 1), a mix of both forms (300: lists of this index hold about
    600 entries, cut into pieces of any size by the items), and none."""
    monkeypatch.setenv("IVFPQ_SCAN_WIDE_MIN", wide_min)
    idx, q = exact_case(8, 12, seed=812)
    nlist = idx.nlist
    for nprobe, k, chunk in [(nlist, 100, 0), (nlist, 100, 256), (nlist, 100, 700), (3, 100, 0),
                             (nlist, 1, 64), (2, 1024, 0)]:
        say(f"exact l2 m=8 dsub=12 wide_min={wide_min} nprobe={nprobe} k={k} chunk={chunk}")
        d, i, p = run(idx, q, nprobe, k, chunk_len=chunk)
        assert_exact(idx, q, nprobe, k, d, i, p)
        if nprobe == nlist:
            assert np.all(d[0::3, 0] == 0.0)


@pytest.mark.parametrize("m,dsub", SHAPES)
def test_exact_inner_product(m, dsub):
    idx, q = exact_case(m, dsub, seed=7 * m + dsub)
    nlist = idx.nlist
    for nprobe, k, chunk in [(nlist, 100, 0), (nlist, 100, 256), (3, 50, 0)]:
        say(f"exact ip m={m} dsub={dsub} nprobe={nprobe} k={k} chunk={chunk}")
        s, i, p = run(idx, q, nprobe, k, metric="ip", chunk_len=chunk)
        assert_exact(idx, q, nprobe, k, s, i, p, metric="ip")


@pytest.mark.parametrize("lut", ["f32", "f16"])
def test_exact_m16_both_table_forms(monkeypatch, lut):
    """(m 16, dsub 8): decomposed tables (default for this shape) and the
    difference form (test hook at index load) give the same exact rows."""
    idx, q = exact_case(16, 8, seed=1608)
    for decomposed in (True, False):
        if decomposed:
            monkeypatch.delenv("IVFPQ_TEST_NO_LIST_TERM", raising=False)
        else:
            monkeypatch.setenv("IVFPQ_TEST_NO_LIST_TERM", "1")
        say(f"exact m16 decomposed={decomposed} lut={lut}")
        for nprobe, k, chunk in [(idx.nlist, 100, 0), (4, 100, 512)]:
            d, i, p = run(idx, q, nprobe, k, lut=lut, chunk_len=chunk,
                          expect_decomposed=decomposed)
            assert_exact(idx, q, nprobe, k, d, i, p)


def test_repeat_is_bitwise_identical_at_1m_shape():
    """The 1M x 128 shape (nlist 1024, m 16, nprobe 32, k 100, 10,000
    queries) with codes drawn from a pool of 4,000, so that every row has
    deep exact ties at its k-th distance and work items of one query run
    concurrently: three searches return the same bits, and the first is the
    oracle's on sampled queries."""
    rng = np.random.default_rng(1_000_001)
    nlist, d, m, n, nq = 1024, 128, 16, 1_000_000, 10_000
    sizes = rng.multinomial(n, np.ones(nlist) / nlist)
    idx = G.random_index(rng, nlist, d, m, sizes, codebook_scale=0.3)
    pool = rng.integers(0, 256, (4000, m), dtype=np.uint8)
    idx = G.HostIndex(idx.centroids, idx.codebooks, idx.list_sizes,
                      pool[rng.integers(0, len(pool), n)], idx.ids)
    q = (idx.centroids[rng.integers(0, nlist, nq)]
         + 0.3 * rng.standard_normal((nq, d))).astype(np.float32)
    ix = A.ivfpq_load_index_host(idx)
    qd = torch.from_numpy(q).cuda()
    runs = []
    for rep in range(3):
        for chunk in (0, 2048):
            d_, i_ = A.ivfpq_search_ex(ix, qd, 32, 100, chunk_len=chunk)
            torch.cuda.synchronize()
            runs.append((chunk, d_.cpu().numpy(), i_.cpu().numpy()))
    ix.close()
    for chunk in (0, 2048):
        rr = [r for r in runs if r[0] == chunk]
        for _, d_, i_ in rr[1:]:
            assert np.array_equal(d_, rr[0][1])
            nd = int(np.sum(i_ != rr[0][2]))
            say(f"repeat chunk={chunk}: {nd} ids differ")
            assert nd == 0
    from oracle import check
    rows = np.sort(rng.choice(nq, 24, replace=False))
    rep = check.compare_search(idx, q[rows], 32, 100, runs[0][1][rows], runs[0][2][rows],
                               decomposed=True)
    assert rep.ok(), rep.failures[:3]
