"""The search's work plan on the CPU: the functions the device plan and scan
kernels call (csrc/plan.hpp), compiled for the host with the HIP headers and
run by tests/plan_driver.cpp.

Checked against what the plan must be ("Billion-scale similarity search
with GPUs", IVFADC section: every (query, list) entry is scanned by exactly
one piece of work): a query's items cover its probed entries [0, E) once, in
order, each at most `chunk` entries, at most imax of them, one empty item for
a query with no entries; each item's pieces are exactly its intersections
with the probed lists (empty lists contribute none); the persistent grid is
at least one workgroup and never more than the items there can be.  Plus the
hand-worked case of the index with lists {7, 3, 5} and {9}."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "approximate_nearest_neighbour_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", CSRC, os.path.join(ROOT, "tests", "plan_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"host compiler could not build the plan driver: {r.stderr[:300]}")
    return exe


def run(driver, cases):
    """cases: list of dicts(sizes, probes [nq][nprobe], kw, target, per_cu, cus)."""
    lines = [str(len(cases))]
    for c in cases:
        probes = np.asarray(c["probes"], dtype=np.int64)
        lines.append(f"{len(c['sizes'])} {probes.shape[0]} {probes.shape[1]} {c['kw']} "
                     f"{c['target']} {c['per_cu']} {c['cus']} {c.get('align', 1)}")
        lines.append(" ".join(str(int(v)) for v in c["sizes"]))
        lines.append(" ".join(str(int(v)) for v in probes.ravel()))
    out = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, check=True).stdout.split("\n")
    res, cur = [], None
    for line in out:
        f = line.split()
        if not f:
            continue
        if f[0] == "case":
            cur = dict(imax=int(f[1]), max_items=int(f[2]), grid=int(f[3]), queries=[])
            res.append(cur)
        elif f[0] == "query":
            cur["queries"].append(dict(total=int(f[1]), chunk=int(f[2]), count=int(f[3]),
                                       items=[]))
        else:
            vals = list(map(int, f[1:]))
            n = vals[2]
            pieces = [tuple(vals[3 + 3 * j:6 + 3 * j]) for j in range(n)]
            cur["queries"][-1]["items"].append(dict(start=vals[0], stop=vals[1], pieces=pieces))
    return res


def check_case(c, r):
    sizes = np.asarray(c["sizes"], dtype=np.int64)
    probes = np.asarray(c["probes"], dtype=np.int64)
    nq = probes.shape[0]
    assert len(r["queries"]) == nq
    assert 2 <= r["imax"] <= 64 and r["max_items"] == nq * r["imax"]
    assert 1 <= r["grid"] <= max(r["max_items"], 1)
    assert r["grid"] <= max(c["per_cu"], 1) * max(c["cus"], 1)
    for q, pq in enumerate(r["queries"]):
        lists = [int(l) for l in probes[q] if 0 <= l < len(sizes)]
        # the query's entries laid end to end, probe order
        seq = [(l, j) for l in lists for j in range(int(sizes[l]))]
        assert pq["total"] == len(seq)
        assert 1 <= pq["count"] <= r["imax"]
        assert pq["chunk"] >= c["target"] and pq["chunk"] >= 1
        assert pq["chunk"] % c.get("align", 1) == 0
        if seq:
            assert pq["count"] == -(-len(seq) // pq["chunk"])
        else:
            assert pq["count"] == 1
        covered = []
        prev = 0
        for it in pq["items"]:
            assert it["start"] == prev and it["stop"] - it["start"] <= pq["chunk"]
            prev = it["stop"]
            got = [(l, j) for (l, b, e) in it["pieces"] for j in range(b, e)]
            assert got == seq[it["start"]:it["stop"]]
            # one piece per list met, none empty, none for an empty list
            assert all(e > b for (_, b, e) in it["pieces"])
            assert len({l for (l, _, _) in it["pieces"]}) == len(it["pieces"]) or \
                len(lists) != len(set(lists))
            covered += got
        assert prev == len(seq) and covered == seq


HAND_SIZES = [3, 1]


def test_hand_case_plan(driver):
    base = dict(sizes=HAND_SIZES, kw=64, target=131072, per_cu=2, cus=256)
    r = run(driver, [dict(base, probes=[[0, 1]]), dict(base, probes=[[0]]),
                     dict(base, probes=[[0, 1]], target=1)])
    one, first, fine = r
    # nprobe 2: one item of 4 entries, pieces list 0 [0, 3) and list 1 [0, 1)
    q = one["queries"][0]
    assert (q["total"], q["count"]) == (4, 1)
    assert q["items"][0]["pieces"] == [(0, 0, 3), (1, 0, 1)]
    # one query with imax 64 items at most: 64 workgroups, not one per resident slot
    assert one["imax"] == 64 and one["max_items"] == 64 and one["grid"] == 64
    # nprobe 1: list 0 only
    assert first["queries"][0]["items"][0]["pieces"] == [(0, 0, 3)]
    # one entry per item: four items, the last one in list 1
    q = fine["queries"][0]
    assert q["count"] == 4
    assert [it["pieces"] for it in q["items"]] == [[(0, 0, 1)], [(0, 1, 2)], [(0, 2, 3)],
                                                   [(1, 0, 1)]]
    for c, rr in zip([dict(base, probes=[[0, 1]]), dict(base, probes=[[0]]),
                      dict(base, probes=[[0, 1]], target=1)], r):
        check_case(c, rr)


def test_empty_lists_plan(driver):
    # lists 1 and 3 empty; query 0 probes only empty lists, query 1 mixes
    sizes = [5, 0, 7, 0]
    cases = [dict(sizes=sizes, probes=[[1, 3], [1, 0], [3, 2]], kw=128, target=4, per_cu=2,
                  cus=4),
             dict(sizes=[0, 0], probes=[[0, 1]], kw=64, target=1, per_cu=1, cus=1)]
    r = run(driver, cases)
    q0 = r[0]["queries"][0]
    assert q0["total"] == 0 and q0["count"] == 1 and q0["items"][0]["pieces"] == []
    q1 = r[0]["queries"][1]
    assert q1["items"][0]["pieces"] == [(0, 0, 4)] and q1["items"][1]["pieces"] == [(0, 4, 5)]
    q2 = r[0]["queries"][2]
    assert [it["pieces"] for it in q2["items"]] == [[(2, 0, 4)], [(2, 4, 7)]]
    assert r[1]["grid"] == 1
    for c, rr in zip(cases, r):
        check_case(c, rr)


def test_random_and_skewed_plans(driver):
    rng = np.random.default_rng(3)
    cases = []
    for t in range(40):
        nlist = int(rng.integers(1, 40))
        if t % 3 == 0:   # heavy-tailed sizes (a few lists dominate)
            sizes = (1000 * rng.pareto(1.1, nlist)).astype(np.int64)
        else:
            sizes = rng.integers(0, 50, nlist)
        nq = int(rng.integers(1, 6))
        nprobe = int(rng.integers(1, nlist + 1))
        probes = np.stack([rng.permutation(nlist)[:nprobe] for _ in range(nq)])
        cases.append(dict(sizes=sizes, probes=probes,
                          kw=int(rng.choice([64, 128, 1024])),
                          target=int(rng.choice([1, 3, 16, 1000, 131072])),
                          per_cu=int(rng.integers(1, 4)), cus=int(rng.choice([1, 8, 256]))))
    # many queries: imax falls to its floor of 2 and the chunks grow
    nl = 50
    cases.append(dict(sizes=rng.integers(0, 30, nl),
                      probes=np.stack([rng.permutation(nl)[:10] for _ in range(1 << 17)]),
                      kw=1024, target=1, per_cu=2, cus=256))
    # chunks rounded up to whole regions (the scan's region-aligned layout
    # of queries that probe giant lists): 7, 64 and 2^18 entries
    cases += [dict(c, align=int(rng.choice([7, 64, 1 << 18]))) for c in cases[:40]]
    r = run(driver, cases)
    assert r[40]["imax"] == 2
    for c, rr in zip(cases, r):
        check_case(c, rr)


def test_large_totals_do_not_wrap(driver):
    # 3e9 entries in one query (below 2^32): items of ceil(E / 64) entries
    sizes = [1_500_000_007, 1_499_999_993]
    r = run(driver, [dict(sizes=sizes, probes=[[0, 1]], kw=128, target=131072, per_cu=2,
                          cus=256)])
    q = r[0]["queries"][0]
    assert q["total"] == 3_000_000_000 and q["count"] == 64
    assert q["chunk"] == -(-3_000_000_000 // 64)
    assert q["items"][-1]["stop"] == 3_000_000_000
    assert sum(it["stop"] - it["start"] for it in q["items"]) == 3_000_000_000
    mid = [it for it in q["items"] if len(it["pieces"]) == 2]
    assert len(mid) == 1 and mid[0]["pieces"][0][2] == 1_500_000_007

