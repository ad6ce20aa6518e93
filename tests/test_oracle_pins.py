"""Pins of the CPU oracle against things other than itself.

* a hand-worked case (tests/golden/hand_case.json);
* the identity stated after Eq. (1) of the IVFPQ section of "Custom 8-bit
  floating point value format for reducing shared memory bank conflict in
  ANN search": the table sum R equals the squared L2 norm of the query minus
  the reconstructed database vector (centroid + decoded residual);
* PQ-exact integer data, where IVF-PQ with every list probed must equal exact
  brute-force k-NN bit for bit;
* textbook routines: numpy argsort for the coarse step, numpy float16 for
  binary16 rounding, pure-Python loops for brute force.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from oracle import check

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def hand_index(extra=None):
    g = json.load(open(os.path.join(GOLDEN, "hand_case.json")))
    m, d = g["m"], g["d"]
    books = np.empty((m, 256, d // m), dtype=np.float32)
    books[:] = np.asarray(g["default_codeword"], dtype=np.float32)
    for j, words in g["codewords"].items():
        for v, w in words.items():
            books[int(j), int(v)] = w
    lists = [list(l) for l in g["lists"]]
    if extra is not None:
        lists[0] = lists[0] + [extra]
    codes = np.array([c for l in lists for _, c in l], dtype=np.uint8).reshape(-1, m)
    ids = np.array([i for l in lists for i, _ in l], dtype=np.int64)
    sizes = np.array([len(l) for l in lists], dtype=np.int64)
    idx = dict(centroids=np.asarray(g["centroids"], dtype=np.float32), codebooks=books,
               list_sizes=sizes, codes=codes, ids=ids)
    return g, idx


def inf_list(v):
    return [math.inf if x == "inf" else float(x) for x in v]


def reconstruct(idx):
    """Centroid of the entry's list plus the concatenated codewords."""
    cent, books = idx["centroids"], idx["codebooks"]
    m = books.shape[0]
    lists = np.repeat(np.arange(len(idx["list_sizes"])), idx["list_sizes"])
    dec = np.concatenate([books[j][idx["codes"][:, j]] for j in range(m)], axis=1)
    return cent[lists].astype(np.float64) + dec.astype(np.float64)


def numpy_knn(db, q, k, ids=None):
    ids = np.arange(len(db)) if ids is None else ids
    d = ((q[:, None, :].astype(np.float64) - db[None, :, :].astype(np.float64)) ** 2).sum(-1)
    out_d = np.full((len(q), k), np.inf)
    out_i = np.full((len(q), k), -1, dtype=np.int64)
    for r in range(len(q)):
        order = np.lexsort((ids, d[r]))[:k]
        out_d[r, :len(order)] = d[r][order]
        out_i[r, :len(order)] = ids[order]
    return out_d, out_i


# ---------------------------------------------------------------------------
# hand-worked case
# ---------------------------------------------------------------------------

def test_hand_case_coarse_and_tables():
    g, idx = hand_index()
    x = np.asarray(g["query"], dtype=np.float32)
    probes, dists = O.coarse(x, idx["centroids"], 2)
    assert probes.tolist() == [0, 1]
    assert dists.tolist() == g["coarse_distances"]
    t0 = O.lut(x, idx["centroids"][0], idx["codebooks"])
    assert t0[:, :3].tolist() == g["lut_list0_first3"]
    t1 = O.lut(x, idx["centroids"][1], idx["codebooks"])
    assert [t1[0, 0], t1[1, 0]] == g["lut_list1_code0"]


@pytest.mark.parametrize("case", [0, 1])
def test_hand_case_search(case):
    g, idx = hand_index()
    c = g["cases"][case]
    d, i, p = O.search(idx, np.asarray([g["query"]], np.float32), c["nprobe"], c["k"])
    assert i[0].tolist() == c["ids"]
    assert d[0].tolist() == inf_list(c["dist"])


def test_hand_case_tie_order():
    g, _ = hand_index()
    t = g["tie_case"]
    _, idx = hand_index(extra=t["add_to_list0"])
    d, i, _ = O.search(idx, np.asarray([g["query"]], np.float32), t["nprobe"], t["k"])
    assert i[0].tolist() == t["ids"]
    assert d[0].tolist() == inf_list(t["dist"])


def test_coarse_tie_goes_to_lower_list_number():
    cent = np.array([[1, 0], [0, 1], [-1, 0], [5, 5]], dtype=np.float32)
    p, d = O.coarse(np.zeros(2, np.float32), cent, 3)
    assert p.tolist() == [0, 1, 2] and d.tolist() == [1, 1, 1]


# ---------------------------------------------------------------------------
# the table-sum identity, random indexes of several shapes
# ---------------------------------------------------------------------------

def random_idx(seed, nlist, d, m, n):
    rng = np.random.default_rng(seed)
    sizes = rng.multinomial(n, np.ones(nlist) / nlist).astype(np.int64)
    return dict(centroids=rng.standard_normal((nlist, d)).astype(np.float32),
                codebooks=(0.5 * rng.standard_normal((m, 256, d // m))).astype(np.float32),
                list_sizes=sizes, codes=rng.integers(0, 256, (n, m), dtype=np.uint8),
                ids=rng.permutation(n).astype(np.int64)), rng


@pytest.mark.parametrize("nlist,d,m,n", [(4, 8, 2, 300), (6, 12, 4, 500), (3, 24, 8, 257),
                                         (5, 16, 16, 200)])
def test_adc_equals_reconstruction_distance(nlist, d, m, n):
    idx, rng = random_idx(1 + nlist * d, nlist, d, m, n)
    q = rng.standard_normal((5, d)).astype(np.float32)
    dist, ids, _ = O.search(idx, q, nlist, n)          # every list, every entry
    recon = reconstruct(idx)
    pos_of = np.empty(n, dtype=np.int64)
    pos_of[idx["ids"]] = np.arange(n)
    for r in range(len(q)):
        expl = ((q[r].astype(np.float64) - recon[pos_of[ids[r]]]) ** 2).sum(1)
        np.testing.assert_allclose(dist[r], expl, rtol=1e-5, atol=0)
        assert np.max(np.abs(dist[r] - expl) / expl) < 1e-10


def test_entry_distances_equal_reconstruction_distance():
    idx, rng = random_idx(17, 5, 12, 3, 400)
    x = rng.standard_normal(12).astype(np.float32)
    pos = rng.choice(400, 50, replace=False)
    got, lists = O.entry_distances(idx, x, pos)
    off = np.concatenate([[0], np.cumsum(idx["list_sizes"])])
    assert np.all((off[lists] <= pos) & (pos < off[lists + 1]))
    expl = ((x.astype(np.float64) - reconstruct(idx)[pos]) ** 2).sum(1)
    np.testing.assert_allclose(got, expl, rtol=1e-12)


def test_adc_single_list_matches_reconstruction():
    idx, rng = random_idx(7, 3, 16, 4, 120)
    q = rng.standard_normal((1, 16)).astype(np.float32)
    probes, _ = O.coarse(q[0], idx["centroids"], 1)
    dist, ids, p = O.search(idx, q, 1, 200)
    assert p[0].tolist() == probes.tolist()
    l = int(probes[0])
    off = np.concatenate([[0], np.cumsum(idx["list_sizes"])])
    in_list = set(idx["ids"][off[l]:off[l + 1]].tolist())
    valid = ids[0] >= 0
    assert set(ids[0][valid].tolist()) == in_list
    assert valid.sum() == idx["list_sizes"][l]
    assert np.all(np.isinf(dist[0][~valid])) and np.all(ids[0][~valid] == -1)


# ---------------------------------------------------------------------------
# coarse step against numpy's argsort
# ---------------------------------------------------------------------------

def test_coarse_matches_numpy_argsort():
    rng = np.random.default_rng(11)
    cent = rng.standard_normal((300, 24)).astype(np.float32)
    for _ in range(10):
        x = rng.standard_normal(24).astype(np.float32)
        ref = ((x.astype(np.float64) - cent.astype(np.float64)) ** 2).sum(1)
        order = np.argsort(ref, kind="stable")[:17]
        p, d = O.coarse(x, cent, 17)
        assert p.tolist() == order.tolist()
        np.testing.assert_allclose(d, ref[order], rtol=1e-13)


# ---------------------------------------------------------------------------
# PQ-exact integer data: IVF-PQ (all lists) == exact k-NN, bit for bit
# ---------------------------------------------------------------------------

def pq_exact(seed, nlist=5, d=8, m=4, n=400, nq=6):
    rng = np.random.default_rng(seed)
    cent = rng.integers(-3, 4, (nlist, d)).astype(np.float32)
    books = rng.integers(-3, 4, (m, 256, d // m)).astype(np.float32)
    sizes = rng.multinomial(n, np.ones(nlist) / nlist).astype(np.int64)
    codes = rng.integers(0, 256, (n, m), dtype=np.uint8)
    ids = rng.permutation(n).astype(np.int64)
    idx = dict(centroids=cent, codebooks=books, list_sizes=sizes, codes=codes, ids=ids)
    db = reconstruct(idx).astype(np.float32)     # exact: small integers
    q = rng.integers(-6, 7, (nq, d)).astype(np.float32)
    return idx, db, q


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_pq_exact_integer_equals_bruteforce(seed):
    idx, db, q = pq_exact(seed)
    k = 25
    d, i, _ = O.search(idx, q, 5, k)
    bd, bi = numpy_knn(db, q, k, ids=idx["ids"])
    assert np.array_equal(i, bi)
    assert np.array_equal(d, bd)
    cd, ci = O.bruteforce(db, q, k, db_ids=idx["ids"])
    assert np.array_equal(ci, bi) and np.array_equal(cd, bd)
    # heavy ties exist at these sizes: the (distance, id) order decides them
    assert any(len(set(r.tolist())) < k for r in d)
    assert O.recall_1_at_k(i, bi) == 1.0 and O.recall_k_at_k(i, bi) == 1.0


# ---------------------------------------------------------------------------
# brute force against pure-Python loops; bf16 widening against numpy
# ---------------------------------------------------------------------------

def test_bruteforce_pure_python():
    rng = np.random.default_rng(5)
    db = rng.standard_normal((40, 3)).astype(np.float32)
    q = rng.standard_normal((4, 3)).astype(np.float32)
    d, i = O.bruteforce(db, q, 7)
    for r in range(4):
        allp = sorted((sum((float(q[r][t]) - float(db[j][t])) ** 2 for t in range(3)), j)
                      for j in range(40))
        assert [j for _, j in allp[:7]] == i[r].tolist()
        np.testing.assert_allclose(d[r], [v for v, _ in allp[:7]], rtol=1e-14)


def test_bruteforce_bf16_widening():
    rng = np.random.default_rng(6)
    db = rng.integers(0, 1 << 16, (64, 8)).astype(np.uint16)
    db &= ~np.uint16(0x7F80)            # keep exponents small: finite, no inf/nan
    db |= np.uint16(0x3F00)
    q = db[:3].copy()
    d, i = O.bruteforce_bf16(db, q, 5)
    dbf = (db.astype(np.uint32) << 16).view(np.float32)
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    bd, bi = numpy_knn(dbf, qf, 5)
    assert np.array_equal(i, bi) and np.allclose(d, bd, rtol=1e-14)
    assert np.all(d[:, 0] == 0)


def test_padding_when_fewer_candidates_than_k():
    idx, rng = random_idx(3, 4, 8, 2, 30)
    q = rng.standard_normal((3, 8)).astype(np.float32)
    d, i, p = O.search(idx, q, 2, 64)
    for r in range(3):
        n = int(sum(idx["list_sizes"][l] for l in p[r]))
        assert np.all(i[r, :n] >= 0) and np.all(i[r, n:] == -1)
        assert np.all(np.isfinite(d[r, :n])) and np.all(np.isinf(d[r, n:]))


def test_empty_lists_are_allowed():
    idx, rng = random_idx(4, 6, 8, 2, 50)
    idx["list_sizes"] = np.array([0, 20, 0, 30, 0, 0], dtype=np.int64)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    d, i, _ = O.search(idx, q, 6, 60)
    assert (i >= 0).sum(1).tolist() == [50, 50]


# ---------------------------------------------------------------------------
# binary16 rounding against numpy's float16
# ---------------------------------------------------------------------------

def test_round_binary16_matches_numpy():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25,
                        3 * 2.0 ** -25, 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
                        2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 6.1e-5, 1e-8, 1e6],
                       dtype=np.float32)
    # exponents spread over the binary16 range as well
    spread = (rng.standard_normal(20000) * np.exp2(rng.uniform(-26, 17, 20000))).astype(np.float32)
    for v in itertools.chain(special, -special, vals[:5000], spread):
        with np.errstate(over="ignore"):
            ref = float(np.float32(v).astype(np.float16))
        got = O.round_binary16(float(v))
        assert got == ref or (math.isnan(got) and math.isnan(ref)), (v, got, ref)


def test_fp16_table_mode_rounds_each_entry():
    idx, rng = random_idx(12, 2, 16, 4, 10)
    x = rng.standard_normal(16).astype(np.float32)
    full = O.lut(x, idx["centroids"][1], idx["codebooks"], O.LUT_F64)
    half = O.lut(x, idx["centroids"][1], idx["codebooks"], O.LUT_F16)
    # explicit table from the definition, then numpy's float32 -> float16
    r = x.astype(np.float64) - idx["centroids"][1].astype(np.float64)
    books = idx["codebooks"].astype(np.float64)
    expl = np.stack([((r[j * 4:(j + 1) * 4][None, :] - books[j]) ** 2).sum(1) for j in range(4)])
    np.testing.assert_allclose(full, expl, rtol=1e-14)
    assert np.array_equal(half, expl.astype(np.float32).astype(np.float16).astype(np.float64))


# ---------------------------------------------------------------------------
# the acceptance checker itself
# ---------------------------------------------------------------------------

def test_checker_accepts_oracle_and_rejects_perturbations():
    idx, rng = random_idx(21, 8, 16, 4, 2000)
    q = rng.standard_normal((8, 16)).astype(np.float32)
    d, i, p = O.search(idx, q, 3, 20)
    rep = check.compare_search(idx, q, 3, 20, d.astype(np.float32), i, p)
    assert rep.ok(), rep.failures
    far_d, far_i, _ = O.search(idx, q[:1], 3, 2000)
    bad = i.copy()
    bad[0, 5] = far_i[0][int(np.sum(far_i[0] >= 0)) - 1]     # the farthest probed entry
    rep = check.compare_search(idx, q, 3, 20, d.astype(np.float32), bad, p)
    assert not rep.ok()
    dd = d.astype(np.float32).copy()
    dd[1, 3] *= 1.001
    dd[1] = np.sort(dd[1])
    rep = check.compare_search(idx, q, 3, 20, dd, i, p)
    assert not rep.ok()
    pp = p.copy()
    pp[2, 0] = [l for l in range(8) if l not in p[2]][0]
    rep = check.compare_search(idx, q, 3, 20, d.astype(np.float32), i, pp)
    assert not rep.ok()


# ---------------------------------------------------------------------------
# index building: list assignment and PQ encoding
# ---------------------------------------------------------------------------

def test_encode_recovers_the_codewords_a_vector_was_made_of():
    # x = c_l + (C_0[v_0], ..., C_{m-1}[v_{m-1}]) with far-apart centroids and
    # small codewords: the encoder must return l and the v_j
    rng = np.random.default_rng(31)
    nlist, d, m = 8, 16, 4
    cent = (10.0 * rng.standard_normal((nlist, d))).astype(np.float32)
    books = (0.1 * rng.standard_normal((m, 256, d // m))).astype(np.float32)
    n = 300
    lst = rng.integers(0, nlist, n)
    code = rng.integers(0, 256, (n, m))
    x = (cent[lst] + np.concatenate([books[j][code[:, j]] for j in range(m)], axis=1))
    lists, codes, lgap, cgap = O.assign_encode(x.astype(np.float32), cent, books)
    assert np.array_equal(lists, lst)
    assert np.array_equal(codes, code)
    assert np.all(lgap > 0) and np.all(cgap > 0)


def test_encode_is_the_joint_optimum_by_enumeration():
    # the per-sub-quantizer choice must minimise the whole reconstruction
    # error |x - c_l - (C_0[v_0], C_1[v_1])|^2 over all 256^2 code pairs, and
    # the list must be the nearest centroid (numpy, double precision)
    rng = np.random.default_rng(32)
    nlist, d = 3, 4
    cent = rng.standard_normal((nlist, d)).astype(np.float32)
    books = rng.standard_normal((2, 256, 2)).astype(np.float32)
    x = rng.standard_normal((40, d)).astype(np.float32)
    lists, codes, _, _ = O.assign_encode(x, cent, books)
    v0, v1 = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    recon = np.concatenate([books[0][v0.ravel()], books[1][v1.ravel()]], axis=1).astype(np.float64)
    for i in range(len(x)):
        dc = ((x[i].astype(np.float64) - cent.astype(np.float64)) ** 2).sum(1)
        assert lists[i] == int(np.argmin(dc))
        r = x[i].astype(np.float64) - cent[lists[i]].astype(np.float64)
        err = ((r[None, :] - recon) ** 2).sum(1)
        best = int(np.argmin(err))
        assert (int(codes[i, 0]), int(codes[i, 1])) == (best // 256, best % 256)


def test_encode_ties_go_to_the_smaller_index():
    cent = np.array([[0, 0, 0, 0], [5, 5, 5, 5], [0, 0, 0, 0]], dtype=np.float32)
    books = np.full((2, 256, 2), 100.0, dtype=np.float32)
    books[0, 7] = books[0, 3] = (0.5, 0.5)
    books[1, 200] = books[1, 9] = (1.0, 1.0)
    x = np.array([[0.4, 0.6, 1.1, 0.9]], dtype=np.float32)
    lists, codes, lgap, cgap = O.assign_encode(x, cent, books)
    assert lists[0] == 0 and lgap[0] == 0.0
    assert codes[0].tolist() == [3, 9] and cgap[0].tolist() == [0.0, 0.0]


def test_encode_agrees_with_the_index_builder_where_decisions_are_clear():
    # the CPU index builder (float32 norm expansion, numpy) is an independent
    # encoder: it must agree wherever the decision is not a near-tie
    from approximate_nearest_neighbour_amd import datagen as G
    rng = np.random.default_rng(33)
    nlist, d, m = 16, 32, 4
    cent = rng.standard_normal((nlist, d)).astype(np.float32)
    books = (0.3 * rng.standard_normal((m, 256, d // m))).astype(np.float32)
    x = (cent[rng.integers(0, nlist, 500)] + 0.3 * rng.standard_normal((500, d))).astype(np.float32)
    lists, codes, lgap, cgap = O.assign_encode(x, cent, books)
    gl = G.nearest(x, cent)
    gc = G.encode_pq(x - cent[lists], books)
    clear_l = lgap > 1e-3
    assert np.array_equal(lists[clear_l], gl[clear_l])
    clear_c = cgap > 1e-3
    assert np.array_equal(codes[clear_c], gc[clear_c])
    assert clear_l.mean() > 0.95 and clear_c.mean() > 0.95


def test_encode_checker_accepts_oracle_and_rejects_perturbations():
    rng = np.random.default_rng(34)
    nlist, d, m = 12, 24, 4
    cent = rng.standard_normal((nlist, d)).astype(np.float32)
    books = (0.4 * rng.standard_normal((m, 256, d // m))).astype(np.float32)
    x = (cent[rng.integers(0, nlist, 200)] + 0.4 * rng.standard_normal((200, d))).astype(np.float32)
    out = O.assign_encode(x, cent, books)
    lists, codes, lgap, cgap = out
    assert check.compare_encode(x, cent, books, lists, codes, oracle_out=out).ok()
    i = int(np.argmax(cgap[:, 1]))                     # the clearest decision of sub-quantizer 1
    bad = codes.copy()
    table = O.lut(x[i], cent[lists[i]], books)
    bad[i, 1] = int(np.argmax(table[1]))
    assert not check.compare_encode(x, cent, books, lists, bad, oracle_out=out).ok()
    i = int(np.argmax(lgap))
    far = lists.copy()
    far[i] = int(O.coarse(x[i], cent, nlist)[0][-1])   # the farthest list
    assert not check.compare_encode(x, cent, books, far, codes, oracle_out=out).ok()
    assert not check.compare_encode(x, cent, books, np.full(200, nlist), codes, oracle_out=out).ok()


# ---------------------------------------------------------------------------
# k-means (Lloyd's algorithm)
# ---------------------------------------------------------------------------

def test_kmeans_update_pure_python():
    rng = np.random.default_rng(51)
    x = rng.standard_normal((37, 3)).astype(np.float32)
    a = rng.integers(0, 5, 37)
    a[a == 4] = 3                                  # center 4 gets nothing
    c0 = rng.standard_normal((5, 3)).astype(np.float32)
    got, means, counts = O.kmeans_update(x, a, c0)
    for c in range(5):
        members = [x[i] for i in range(37) if a[i] == c]
        assert counts[c] == len(members)
        for t in range(3):
            if members:
                want = math.fsum(float(v[t]) for v in members) / len(members)
            else:
                want = float(c0[c, t])
            assert abs(means[c, t] - want) <= 1e-15 * max(1.0, abs(want))
            assert got[c, t] == np.float32(want)


def test_kmeans_update_closed_forms():
    # identical members: their value; symmetric pairs: the midpoint; shifting
    # every vector shifts every mean
    p = np.array([1.5, -2.25, 3.0], dtype=np.float32)
    q = np.array([0.5, 0.5, -0.5], dtype=np.float32)
    x = np.stack([p, p, p, q + 1, q - 1])
    a = np.array([0, 0, 0, 1, 1])
    c0 = np.zeros((3, 3), dtype=np.float32)
    got, _, counts = O.kmeans_update(x, a, c0)
    assert np.array_equal(got[0], p) and np.array_equal(got[1], q)
    assert np.array_equal(got[2], c0[2]) and counts.tolist() == [3, 2, 0]
    rng = np.random.default_rng(52)
    y = rng.standard_normal((200, 4))
    b = rng.integers(0, 6, 200)
    _, m1, _ = O.kmeans_update(y, b, np.zeros((6, 4), dtype=np.float32))
    _, m2, _ = O.kmeans_update(y + 7.0, b, np.zeros((6, 4), dtype=np.float32))
    np.testing.assert_allclose(m2, m1 + 7.0, rtol=0, atol=1e-12)


def test_kmeans_lloyd_decreases_the_objective_and_finds_separated_clusters():
    rng = np.random.default_rng(53)
    k, d = 6, 8
    true = 20.0 * rng.standard_normal((k, d))
    lab = rng.integers(0, k, 600)
    x = (true[lab] + rng.standard_normal((600, d))).astype(np.float32)
    init = x[[int(np.flatnonzero(lab == c)[0]) for c in range(k)]]   # one point per cluster

    def objective(c, a):
        return float(np.sum((x.astype(np.float64) - c.astype(np.float64)[a]) ** 2))

    c, prev = init, None
    for it in range(4):
        a, _ = O.nearest_lists(x, c)
        if prev is not None:
            assert objective(c, a) <= prev * (1 + 1e-9)
        c, _, counts = O.kmeans_update(x, a, c)
        prev = objective(c, a)
    # one point per true cluster to start: the first assignment is the
    # clustering itself, and the centers are the cluster means
    assert np.array_equal(a, lab)
    for j in range(k):
        assert np.array_equal(c[j], x[lab == j].astype(np.float64).mean(0).astype(np.float32))
    c2, a2, n2 = O.kmeans(x, init, 4)
    assert np.array_equal(c2, c) and np.array_equal(a2, a) and np.array_equal(n2, counts)


def test_kmeans_checker_accepts_oracle_and_rejects_perturbations():
    rng = np.random.default_rng(54)
    x = rng.standard_normal((300, 6)).astype(np.float32)
    c0 = x[:10].copy()
    a, _ = O.nearest_lists(x, c0)
    c1, means, counts = O.kmeans_update(x, a, c0)
    assert check.compare_kmeans_iteration(x, c0, a, c1, counts).ok()
    other = c1.copy()
    c, t = 3, 2
    other[c, t] = np.nextafter(c1[c, t], np.float32(np.inf if means[c, t] > c1[c, t] else -np.inf))
    assert check.compare_kmeans_iteration(x, c0, a, other, counts).ok()      # the other neighbour
    far = c1.copy()
    far[c, t] = np.nextafter(c1[c, t], np.float32(-np.inf if means[c, t] > c1[c, t] else np.inf))
    assert not check.compare_kmeans_iteration(x, c0, a, far, counts).ok()
    bad = a.copy()
    i = int(np.argmax([np.sum((x[j] - c0[a[j]]) ** 2) for j in range(300)]))
    bad[i] = int(O.coarse(x[i], c0, 10)[0][-1])
    assert not check.compare_kmeans_iteration(x, c0, bad, c1, counts).ok()
    assert not check.compare_kmeans_iteration(x, c0, a, c1, counts + 1).ok()


# ---------------------------------------------------------------------------
# inner-product metric
# ---------------------------------------------------------------------------

def test_ip_coarse_matches_numpy_argsort():
    rng = np.random.default_rng(71)
    c = rng.standard_normal((300, 24)).astype(np.float32)
    c[17] = c[5]                                       # an exact tie: 5 before 17
    for _ in range(5):
        x = rng.standard_normal(24).astype(np.float32)
        ip = c.astype(np.float64) @ x.astype(np.float64)
        order = np.argsort(-ip, kind="stable")
        probes, ips = O.coarse_ip(x, c, 40)
        assert np.array_equal(probes, order[:40])
        np.testing.assert_allclose(ips, ip[order[:40]], rtol=1e-14)
    x = c[5] * 3
    probes, _ = O.coarse_ip(x, c, 2)
    assert probes.tolist() == [5, 17]


@pytest.mark.parametrize("nlist,d,m,n", [(4, 8, 2, 300), (6, 12, 4, 500), (5, 16, 16, 200)])
def test_ip_scores_equal_inner_product_with_reconstruction(nlist, d, m, n):
    idx, rng = random_idx(2 + nlist * d, nlist, d, m, n)
    q = rng.standard_normal((4, d)).astype(np.float32)
    score, ids, _ = O.search(idx, q, nlist, n, lut_mode=O.IP)     # every list, every entry
    recon = reconstruct(idx)
    pos_of = np.empty(n, dtype=np.int64)
    pos_of[idx["ids"]] = np.arange(n)
    for r in range(len(q)):
        expl = recon[pos_of[ids[r]]] @ q[r].astype(np.float64)
        np.testing.assert_allclose(score[r], expl, rtol=1e-10, atol=1e-12)
        assert np.all(np.diff(score[r]) <= 0)


@pytest.mark.parametrize("seed", [1, 2])
def test_ip_pq_exact_integer_equals_bruteforce(seed):
    # integer data, every list probed: the scores are exact integers and the
    # result must be the brute-force maximum inner product, ties by id
    idx, db, q = pq_exact(seed)
    k = 25
    score, ids, _ = O.search(idx, q, len(idx["list_sizes"]), k, lut_mode=O.IP)
    pos_of = np.empty(len(db), dtype=np.int64)
    pos_of[idx["ids"]] = np.arange(len(db))
    for r in range(len(q)):
        s = db.astype(np.float64) @ q[r].astype(np.float64)
        order = sorted(range(len(db)), key=lambda i: (-s[pos_of[i]], i))[:k]
        assert ids[r].tolist() == order
        assert score[r].tolist() == [s[pos_of[i]] for i in order]


def test_ip_padding_and_entry_scores():
    idx, rng = random_idx(73, 4, 8, 2, 30)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    score, ids, probes = O.search(idx, q, 1, 50, lut_mode=O.IP)
    for r in range(2):
        valid = int(np.sum(ids[r] >= 0))
        assert valid == idx["list_sizes"][probes[r][0]]
        assert np.all(np.isneginf(score[r][valid:])) and np.all(ids[r][valid:] == -1)
    pos_of = np.empty(30, dtype=np.int64)
    pos_of[idx["ids"]] = np.arange(30)
    got, _ = O.entry_distances(idx, q[0], pos_of[ids[0][:3]], lut_mode=O.IP)
    np.testing.assert_allclose(got, score[0][:3], rtol=1e-14)


def test_ip_checker_accepts_oracle_and_rejects_perturbations():
    idx, rng = random_idx(74, 8, 16, 4, 2000)
    q = rng.standard_normal((6, 16)).astype(np.float32)
    s, i, p = O.search(idx, q, 3, 20, lut_mode=O.IP)
    rep = check.compare_search(idx, q, 3, 20, s.astype(np.float32), i, p, lut_mode=O.IP)
    assert rep.ok(), rep.failures
    far_s, far_i, _ = O.search(idx, q[:1], 3, 2000, lut_mode=O.IP)
    bad = i.copy()
    bad[0, 5] = far_i[0][int(np.sum(far_i[0] >= 0)) - 1]        # the lowest-scoring entry
    assert not check.compare_search(idx, q, 3, 20, s.astype(np.float32), bad, p,
                                    lut_mode=O.IP).ok()
    ss = s.astype(np.float32).copy()
    ss[1, 3] += 1e-3
    ss[1] = -np.sort(-ss[1])
    assert not check.compare_search(idx, q, 3, 20, ss, i, p, lut_mode=O.IP).ok()
    pp = p.copy()
    pp[2, 0] = int(O.coarse_ip(q[2], idx["centroids"], 8)[0][-1])
    assert not check.compare_search(idx, q, 3, 20, s.astype(np.float32), i, pp,
                                    lut_mode=O.IP).ok()


# ---------------------------------------------------------------------------
# recall measures ("Billion-scale similarity search with GPUs", experiments
# section: R@n, the fraction of queries whose true nearest neighbour is among
# the first n results, and the intersection measure, the fraction of the k
# found that are among the true k nearest), worked by hand
# ---------------------------------------------------------------------------

# four queries, three ids found each (-1 = padding); the truth lists five
# neighbours per query, nearest first, so that a measure reading past k
# columns of the truth or one that tests the wrong membership changes value
RECALL_FOUND = np.array([[5, 3, 9], [1, 2, 4], [7, 8, 6], [0, -1, -1]])
RECALL_TRUE = np.array([[3, 5, 2, 9, 4], [9, 1, 2, 4, 0], [8, 6, 7, 1, 2], [4, 0, 1, 2, 3]])


def test_recall_at_n_hand_worked():
    # true nearest: 3, 9, 8, 4.  Found in the first n:
    #   n = 1: 5, 1, 7, 0        -> none                      -> 0
    #   n = 2: {5,3} {1,2} {7,8} {0} -> q0 and q2             -> 1/2
    #   n = 3: adds 9, 4, 6      -> still q0 and q2           -> 1/2
    assert O.recall_1_at_k(RECALL_FOUND, RECALL_TRUE, n=1) == 0.0
    assert O.recall_1_at_k(RECALL_FOUND, RECALL_TRUE, n=2) == 0.5
    assert O.recall_1_at_k(RECALL_FOUND, RECALL_TRUE) == 0.5
    # (the reversed membership test, "the first id found is among the true
    # ones", would give 1 at n = 1: 5, 1, 7 and 0 are all in their truth rows)


def test_recall_intersection_hand_worked():
    # |found ∩ true[:3]| per query: {5,3,9}∩{3,5,2} = 2, {1,2,4}∩{9,1,2} = 2,
    # {7,8,6}∩{8,6,7} = 3, {0}∩{4,0,1} = 1 -> (2 + 2 + 3 + 1) / (4 * 3) = 2/3
    assert abs(O.recall_k_at_k(RECALL_FOUND, RECALL_TRUE) - 2.0 / 3.0) < 1e-15
    # against all five true neighbours it would be (3 + 3 + 3 + 1) / 12
    # k = 1: 5 vs 3, 1 vs 9, 7 vs 8, 0 vs 4 -> 0
    assert O.recall_k_at_k(RECALL_FOUND, RECALL_TRUE, k=1) == 0.0
    # k = 2: {5,3}∩{3,5} = 2, {1,2}∩{9,1} = 1, {7,8}∩{8,6} = 1, {0}∩{4,0} = 1 -> 5/8
    assert O.recall_k_at_k(RECALL_FOUND, RECALL_TRUE, k=2) == 5 / 8
    # padding never matches padding
    pad = np.array([[-1, -1, -1]])
    assert O.recall_k_at_k(pad, pad) == 0.0 and O.recall_1_at_k(pad, pad) == 0.0


def test_recall_on_bruteforce_neighbours():
    # the exact neighbours of a small set found again with one of them
    # replaced: recall drops by exactly one id out of k for that query
    rng = np.random.default_rng(11)
    db = rng.standard_normal((300, 6)).astype(np.float32)
    q = rng.standard_normal((20, 6)).astype(np.float32)
    _, ti = O.bruteforce(db, q, 10)
    fi = ti.copy()
    fi[3, 9] = -1                       # the 10th of query 3 lost
    fi[7, 0] = next(j for j in range(300) if j not in set(ti[7].tolist()))  # nearest of q7 wrong
    assert abs(O.recall_k_at_k(fi, ti) - (1 - 2 / 200)) < 1e-12
    assert O.recall_1_at_k(fi, ti) == 19 / 20


# ---------------------------------------------------------------------------
# absolute error terms of rule 3 near a zero distance: a float32 evaluation
# (numpy float32, the device's order of operations) of both table forms for
# queries placed on a reconstruction must stay inside half of each band (the
# checker allows twice the bound), and the checker must accept an error
# inside the band and reject one past it
# ---------------------------------------------------------------------------

def _rand_index(rng, nlist, d, m, sizes, codebook_scale=1.0):
    sizes = np.asarray(sizes, dtype=np.int64)
    n = int(sizes.sum())
    return dict(centroids=rng.standard_normal((nlist, d)).astype(np.float32),
                codebooks=(codebook_scale * rng.standard_normal((m, 256, d // m)))
                .astype(np.float32),
                list_sizes=sizes, codes=rng.integers(0, 256, (n, m), dtype=np.uint8),
                ids=rng.permutation(n).astype(np.int64))


def _f32_difference_form(x, c, books, codes):
    """sum_j sum_s (fl(x - c)_s - C)^2 in float32, s and j ascending."""
    m, _, dsub = books.shape
    r = (x.astype(np.float32) - c.astype(np.float32)).astype(np.float32)
    tot = np.float32(0)
    for j in range(m):
        e = np.float32(0)
        for s in range(dsub):
            df = np.float32(r[j * dsub + s] - books[j, codes[j], s])
            e = np.float32(e + np.float32(df * df))
        tot = np.float32(tot + e)
    return float(tot)


def _f32_decomposed_form(x, c, books, codes):
    """fl(fl(t1 + t2) [+ |x - c|^2]) per sub-quantizer, t1 from double."""
    m, _, dsub = books.shape
    x32 = x.astype(np.float32)
    cst = np.float32(0)
    for t in range(len(x)):
        df = np.float32(x32[t] - np.float32(c[t]))
        cst = np.float32(cst + np.float32(df * df))
    tot = np.float32(0)
    for j in range(m):
        cw = books[j, codes[j]].astype(np.float64)
        t1 = np.float32(np.dot(cw, cw) + 2.0 * np.dot(c[j * dsub:(j + 1) * dsub]
                                                       .astype(np.float64), cw))
        acc = np.float32(0)
        for s in range(dsub):
            acc = np.float32(acc + np.float32(x32[j * dsub + s] * np.float32(cw[s])))
        e = np.float32(t1 + np.float32(np.float32(-2.0) * acc))
        if j == 0:
            e = np.float32(e + cst)
        tot = np.float32(tot + e)
    return float(tot)


@pytest.mark.parametrize("m,dsub", [(16, 8), (8, 12), (4, 8)])
def test_l2_bands_bound_float32_evaluations_near_zero(m, dsub):
    rng = np.random.default_rng(17 + m)
    d, nlist, n = m * dsub, 6, 60
    idx = _rand_index(rng, nlist, d, m, [10] * nlist, codebook_scale=0.5)
    off = np.concatenate([[0], np.cumsum(idx["list_sizes"])])
    worst_diff = worst_dec = 0.0
    for t in range(12):
        pos = int(rng.integers(0, n))
        l = int(np.searchsorted(off, pos, side="right") - 1)
        code = idx["codes"][pos]
        recon = idx["centroids"][l].astype(np.float64) + np.concatenate(
            [idx["codebooks"][j, code[j]] for j in range(m)]).astype(np.float64)
        eps = [0.0, 1e-6, 1e-4, 1e-2][t % 4]
        x = (recon + eps * rng.standard_normal(d)).astype(np.float32)
        exact, _ = O.entry_distances(idx, x, np.array([pos]))
        exact = float(exact[0])
        kth = np.array([exact])
        b_diff = check.l2_abs_tol(idx, x[None], [[l]], kth)[0] / 2
        b_dec = check.l2_abs_tol(idx, x[None], [[l]], kth, decomposed=True)[0] / 2
        rel = check.gamma(dsub + m + 2) * exact
        e_diff = abs(_f32_difference_form(x, idx["centroids"][l], idx["codebooks"], code) - exact)
        e_dec = abs(_f32_decomposed_form(x, idx["centroids"][l], idx["codebooks"], code) - exact)
        assert e_diff <= b_diff + rel, (eps, e_diff, b_diff)
        assert e_dec <= b_dec + rel, (eps, e_dec, b_dec)
        worst_diff = max(worst_diff, e_diff)
        worst_dec = max(worst_dec, e_dec)
    # the decomposed form really does lose to cancellation near zero
    assert worst_dec > 10 * worst_diff


def test_checker_band_near_zero_accepts_and_rejects():
    rng = np.random.default_rng(23)
    m, dsub, nlist = 8, 4, 4
    idx = _rand_index(rng, nlist, m * dsub, m, [40] * nlist, codebook_scale=0.5)
    pos = 7
    code = idx["codes"][pos]
    x = (idx["centroids"][0].astype(np.float64) + np.concatenate(
        [idx["codebooks"][j, code[j]] for j in range(m)])).astype(np.float32)[None]
    k = 10
    od, oi, op = O.search(idx, x, nlist, k)
    base = od.astype(np.float32)
    kth = od[:, k - 1]
    checked = 0
    for decomposed in (False, True):
        band = check.l2_abs_tol(idx, x, op, kth, decomposed=decomposed)[0]
        assert band > 0
        for scale, ok in ((0.5, True), (3.0, False)):
            g = base.copy()
            g[0, 0] = np.float32(od[0, 0] + scale * band + check.TAU_F32 * od[0, 0])
            if g[0, 0] > g[0, 1]:      # keep the row ascending (and the ids with it)
                continue
            rep = check.compare_search(idx, x, nlist, k, g, oi, op, decomposed=decomposed)
            assert rep.ok() == ok, (decomposed, scale, rep.failures[:2])
            checked += 1
    assert checked == 4
