"""GPU-vs-oracle acceptance rules (TEST INFRASTRUCTURE ONLY).

The oracle is exact (double precision); the device computes in float32.  The
rules below say when a device result counts as the oracle's result:

1. Probe sets.  A device probe set may differ from the oracle's only by lists
   whose oracle coarse distance lies within delta_c of the oracle's
   nprobe-th smallest, delta_c(q) = 4 * gamma_{d+2} * (|x_q|^2 + max_l |c_l|^2),
   gamma_n = n u / (1 - n u), u = 2^-24: a forward-error bound of any float32
   evaluation of |x - c|^2 (direct or through the norm expansion), times two.
   Where the sets differ the oracle is re-run on the device's probe set.
   Split bfloat16 products (split_bf16=True: the device forms x.c from three
   bfloat16 parts of each operand, x = x0 + x1 + x2 exactly, as six exact
   partial products per dimension, x2 c0 + x0 c2 + x1 c1 + x1 c0 + x0 c1 +
   x0 c0, summed in float32 by the matrix cores, "Leveraging the bfloat16
   artificial intelligence datatype for higher-precision computations",
   Henry, Tang and Heinecke): the sum has 6 * 32 * ceil(d/32) products and
   the start value, so a sequential float32 evaluation of it errs by at most
   gamma_{192 ceil(d/32)} times the sum of the terms' magnitudes (<= 1.01 times
   those of the float32 expansion), the norms by gamma_d each, and the three
   dropped products by 2u |x_i c_i|; together within
   2 gamma_n (|x|^2 + |c|^2) with n = 192 ceil(d/32) + d + 2, so delta_c uses
   that n in place of d + 2.
2. Result ids.  The device id set may differ from the oracle's only by ids
   whose oracle distance is within tau * D_o[k-1] of the oracle's k-th
   distance; no duplicates; distances non-decreasing; the padding (+inf, -1)
   matches.
3. Distances.  Every returned id's distance is within tau relative of the
   oracle's distance for that id (tau = 1e-4 float32 tables, 1e-2 fp16),
   plus an absolute term for the residual's rounding: the device forms
   r = fl(x - c_l) in float32 (search step 2 of the IVFPQ section of "Custom
   8-bit floating point value format for reducing shared memory bank conflict
   in ANN search"), |fl(r_s) - r_s| <= u |x_s - c_s|, and squaring
   (r_s - C_s) turns that into |R^ - R| <= 2 u X sqrt(R) + u^2 X^2 beyond the
   relative error of the table arithmetic, X = |x - c_l|.  The checker allows
   twice that with X the largest |x - c_l| over the row's probed lists and R
   the row's k-th oracle distance (an upper bound for every returned id).
   It matters only near R = 0 (a query on a reconstruction), where no
   relative bound can hold.
   Decomposed tables (the list-term/query-term split of the IVFADC section of
   "Billion-scale similarity search with GPUs"): the device computes
   F_j(v) = fl(fl(t1 + t2) [+ |x - c_l|^2 for j = 0]) with
   t1 = |C_j[v]|^2 + 2 <c_l,j, C_j[v]> (double precision, rounded once) and
   t2 = -2 fl(<x_j, C_j[v]>), then sums the m entries in float32.  Each term
   is bounded by |t1| <= B_j^2 + 2 |c_l,j| B_j and |t2| <= 2 |x_j| B_j
   (B_j = max_v |C_j[v]|, Cauchy-Schwarz), so
   |R^ - R| <= gamma_{dsub+m+4} (sum_j (B_j^2 + 2 (|c_l,j| + |x_j|) B_j)
   + |x - c_l|^2) + gamma_{d+2} |x - c_l|^2; the checker allows twice that,
   maximised over the row's probed lists.  Unlike the difference form this
   cancels: near R = 0 the error is of the order of u times the norms.

Inner-product metric: rules 1-3 on the negated scores (so that rows ascend),
with absolute bands in place of the relative ones (a score can be near zero):
delta_c(q) = 4 gamma_{d+2} |x_q| max_l |c_l| for the probes, and for ids and
scores delta_s(q) = 4 gamma_{d+m+2} |x_q| (max_l |c_l| + sum_j max_v |C_j[v]|),
a forward-error bound of the float32 score <x, c_l> + sum_j <x_j, C_j[v_j]>
(Cauchy-Schwarz on each term), times two.

Index building (assignment and encoding of database vectors):

4. Lists.  A device list may differ from the oracle's (the nearest centroid)
   only by a list whose oracle coarse distance is within delta_c of the
   nearest one (delta_c as in rule 1).
5. Codes.  With l the device's list and F the oracle's table of l (the same
   F_j(v) as the search's, r = x - c_l), each device code v of sub-quantizer j
   satisfies F_j(v) <= min_w F_j(w) + delta_e(j), delta_e(j) = 4
   gamma_{dsub+3} sum_s (2 |r_s| + max_w |C_j[w][s]|)^2 over the dsub dims s
   of sub-vector j: a forward-error bound of a float32 evaluation of
   sum_s (fl(x_s - c_s) - C_j[w][s])^2, times two.  Where no other code is
   that close, the codes must be equal.

k-means (Lloyd's algorithm on the device):

6. One iteration.  The device assignment obeys rule 4 against the iteration's input
   centers; with that assignment the oracle's update (double-precision means)
   gives the counts exactly, and each device center equals the float32
   rounding of the oracle's mean or its float32 neighbour on the other side
   of the exact mean (the device sums in double precision in another order).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import oracle as O

TAU_F32 = 1e-4
TAU_F16 = 1e-2


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


@dataclasses.dataclass
class Report:
    nq: int = 0
    probe_flips: int = 0
    queries_reprobed: int = 0
    tie_swaps: int = 0
    max_rel_err: float = 0.0
    failures: list = dataclasses.field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> dict:
        return dict(nq=self.nq, probe_flips=self.probe_flips, queries_reprobed=self.queries_reprobed,
                    tie_swaps=self.tie_swaps, max_rel_err=self.max_rel_err,
                    failures=len(self.failures))


def _get(index, name):
    return index[name] if isinstance(index, dict) else getattr(index, name)


def coarse_gamma_n(d: int, split_bf16: bool = False) -> int:
    """n of the gamma_n in rule 1's band: d + 2 for a float32 evaluation of
    the norm expansion; 192 ceil(d/32) + d + 2 for split bfloat16 products."""
    return 192 * ((d + 31) // 32) + d + 2 if split_bf16 else d + 2


def check_probes(index, queries, gpu_probes, oracle_probes, report: Report, ip=False,
                 split_bf16=False):
    """Rule 1.  Returns the list of query rows whose probe set differs."""
    cent = np.asarray(_get(index, "centroids"), dtype=np.float32)
    nlist, d = cent.shape
    gn = coarse_gamma_n(d, split_bf16)
    cmax = float(np.max(np.sum(cent.astype(np.float64) ** 2, axis=1)))
    differ = []
    for qi in range(len(queries)):
        g = set(int(v) for v in gpu_probes[qi])
        o = set(int(v) for v in oracle_probes[qi])
        if len(g) != len(gpu_probes[qi]):
            report.failures.append((qi, "duplicate probe"))
            continue
        if g == o:
            continue
        nprobe = len(oracle_probes[qi])
        x2 = float(np.sum(np.asarray(queries[qi], dtype=np.float64) ** 2))
        if ip:
            allp, ips = O.coarse_ip(queries[qi], cent, nlist)
            alld = -ips
            delta = 4.0 * gamma(gn) * math.sqrt(x2 * cmax)
        else:
            allp, alld = O.coarse(queries[qi], cent, nlist)
            delta = 4.0 * gamma(gn) * (x2 + cmax)
        dist_of = {int(p): float(v) for p, v in zip(allp, alld)}
        edge = float(alld[nprobe - 1])
        for lst in g ^ o:
            if lst not in dist_of or abs(dist_of[lst] - edge) > delta:
                report.failures.append((qi, f"probe {lst} outside the coarse tie band"))
                break
        report.probe_flips += len(g - o)
        differ.append(qi)
    return differ


def check_results(gpu_d, gpu_i, ora_d, ora_i, k, tau, report: Report, rows=None, lookup=None,
                  abs_tol=None):
    """Rules 2 and 3 for each row; ora_* hold at least k columns (more give
    the distances of ids just past the k-th).  lookup(row, ids) -> oracle
    distances (or None where the id is not a candidate) resolves ids past the
    oracle's columns (deep ties).  abs_tol[row], when given, widens both
    tolerances by an absolute term (the norm-expansion error near zero)."""
    rows = range(len(gpu_d)) if rows is None else rows
    for r in rows:
        at = 0.0 if abs_tol is None else float(abs_tol[r])
        gd = np.asarray(gpu_d[r], dtype=np.float64)
        gi = np.asarray(gpu_i[r], dtype=np.int64)
        od = np.asarray(ora_d[r], dtype=np.float64)
        oi = np.asarray(ora_i[r], dtype=np.int64)
        valid_o = int(np.sum(oi[:k] >= 0))
        valid_g = int(np.sum(gi >= 0))
        if valid_g != valid_o:
            report.failures.append((r, f"valid count {valid_g} != {valid_o}"))
            continue
        if np.any(gi[valid_g:] != -1) or np.any(np.isfinite(gd[valid_g:])):
            report.failures.append((r, "bad padding"))
            continue
        if np.any(gi[:valid_g] < 0):
            report.failures.append((r, "sentinel inside the valid prefix"))
            continue
        if len(set(gi[:valid_g].tolist())) != valid_g:
            report.failures.append((r, "duplicate ids"))
            continue
        if valid_g > 1 and np.any(np.diff(gd[:valid_g]) < 0):
            report.failures.append((r, "distances not ascending"))
            continue
        if valid_g == 0:
            continue
        dist_of = {int(i): float(v) for i, v in zip(oi, od) if i >= 0}
        unknown = [int(i) for i in gi[:valid_g] if int(i) not in dist_of]
        if unknown and lookup is not None:
            for i, v in zip(unknown, lookup(r, unknown)):
                if v is not None:
                    dist_of[i] = float(v)
        kth = float(od[valid_o - 1])
        band = tau * kth + at
        gset, oset = set(gi[:valid_g].tolist()), set(oi[:valid_o].tolist())
        bad = False
        for i in gset ^ oset:
            v = dist_of.get(int(i))
            if v is None or abs(v - kth) > band:
                report.failures.append((r, f"id {i} outside the k-th distance tie band"))
                bad = True
                break
        if bad:
            continue
        report.tie_swaps += len(gset - oset)
        for i, v in zip(gi[:valid_g], gd[:valid_g]):
            ref = dist_of.get(int(i))
            if ref is None:
                report.failures.append((r, f"id {i} is not a candidate of the probed lists"))
                break
            err = abs(float(v) - ref)
            if err > tau * abs(ref) + at:
                report.failures.append((r, f"id {i}: distance {v} vs oracle {ref}"))
                break
            if ref != 0:
                report.max_rel_err = max(report.max_rel_err, err / abs(ref))


def l2_abs_tol(index, queries, probes, kth, decomposed=False):
    """Absolute term of rule 3 per query row (squared L2): the residual's
    float32 rounding, and with decomposed tables their forward-error bound
    (the module docstring derives both); maximised over the row's probed
    lists.  kth: the row's k-th oracle distance."""
    u = 2.0 ** -24
    cent = np.asarray(_get(index, "centroids"), dtype=np.float64)
    books = np.asarray(_get(index, "codebooks"), dtype=np.float64)
    d, m = cent.shape[1], books.shape[0]
    dsub = d // m
    bj = np.sqrt(np.max(np.sum(books ** 2, axis=2), axis=1))          # [m]
    q = np.asarray(queries, dtype=np.float64)
    out = np.zeros(len(q))
    for r in range(len(q)):
        ls = np.asarray(probes[r], dtype=np.int64)
        ls = ls[(ls >= 0) & (ls < len(cent))]
        if len(ls) == 0:
            continue
        c = cent[ls]                                                    # [p][d]
        x2 = np.sum((q[r] - c) ** 2, axis=1)                           # |x - c_l|^2
        rk = max(float(kth[r]), 0.0) if np.isfinite(kth[r]) else 0.0
        tol = 2.0 * (2.0 * u * np.sqrt(x2) * np.sqrt(rk) + u * u * x2)
        if decomposed:
            cj = np.sqrt(np.sum(c.reshape(len(ls), m, dsub) ** 2, axis=2))    # [p][m]
            xj = np.sqrt(np.sum(q[r].reshape(m, dsub) ** 2, axis=1))          # [m]
            terms = np.sum(bj ** 2 + 2.0 * (cj + xj) * bj, axis=1)             # [p]
            tol = tol + 2.0 * (gamma(dsub + m + 4) * (terms + x2) + gamma(d + 2) * x2)
        out[r] = float(np.max(tol))
    return out


def compare_search(index, queries, nprobe, k, gpu_d, gpu_i, gpu_probes=None, lut_mode=O.LUT_F64,
                   tau=None, k_extra=32, nthreads=None, decomposed=False,
                   split_bf16=False) -> Report:
    """Full acceptance check of a device IVF-PQ search against the oracle
    (lut_mode O.IP: the inner-product metric, scores in decreasing order).
    decomposed: the device built its tables from the per-list term (squared
    L2 only); rule 3's absolute term then includes their error bound.
    split_bf16: the device's coarse products came from split bfloat16 parts
    (rule 1's band with its n)."""
    ip = lut_mode == O.IP
    tau = (TAU_F32 if lut_mode in (O.LUT_F64, O.IP) else TAU_F16) if tau is None else tau
    queries = np.ascontiguousarray(queries, dtype=np.float32)
    rep = Report(nq=len(queries))
    kx = k + k_extra
    od, oi, op = O.search(index, queries, nprobe, kx, lut_mode=lut_mode, nthreads=nthreads)
    if gpu_probes is not None:
        differ = check_probes(index, queries, gpu_probes, op, rep, ip=ip, split_bf16=split_bf16)
        if differ:
            rep.queries_reprobed = len(differ)
            sub = np.asarray(differ)
            d2, i2, _ = O.search(index, queries[sub], nprobe, kx, lut_mode=lut_mode,
                                 probes=np.asarray(gpu_probes)[sub], nthreads=nthreads)
            od[sub], oi[sub] = d2, i2
    ids = np.asarray(_get(index, "ids"), dtype=np.int64)
    pos_of = np.full(int(ids.max()) + 1 if len(ids) else 1, -1, dtype=np.int64)
    pos_of[ids] = np.arange(len(ids))
    sizes = np.asarray(_get(index, "list_sizes"), dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(sizes)])
    probes_used = op if gpu_probes is None else np.asarray(gpu_probes)

    def lookup(row, id_list):
        """Exact oracle distance of ids outside the oracle's returned columns,
        provided they lie in one of the lists the row probed."""
        pos = np.array([pos_of[i] if 0 <= i < len(pos_of) else -1 for i in id_list])
        ok = pos >= 0
        lists = np.searchsorted(off, np.where(ok, pos, 0), side="right") - 1
        probed = set(int(l) for l in probes_used[row])
        ok &= np.array([int(l) in probed for l in lists], dtype=bool)
        out = [None] * len(id_list)
        if ok.any():
            vals, _ = O.entry_distances(index, queries[row], pos[ok], lut_mode=lut_mode)
            for j, v in zip(np.flatnonzero(ok), vals):
                out[j] = -v if ip else v
        return out

    if ip:
        cent = np.asarray(_get(index, "centroids"), dtype=np.float64)
        books = np.asarray(_get(index, "codebooks"), dtype=np.float64)
        d, m = cent.shape[1], books.shape[0]
        cmax = float(np.sqrt(np.max(np.sum(cent ** 2, axis=1))))
        bsum = float(np.sum(np.sqrt(np.max(np.sum(books ** 2, axis=2), axis=1))))
        xn = np.sqrt(np.sum(queries.astype(np.float64) ** 2, axis=1))
        abs_tol = 4.0 * gamma(d + m + 2) * xn * (cmax + bsum)
        check_results(-np.asarray(gpu_d, dtype=np.float64), gpu_i, -od, oi, k, 0.0, rep,
                      lookup=lookup, abs_tol=abs_tol)
    else:
        kth = np.array([row[min(k, int(np.sum(np.isfinite(row)))) - 1]
                        if np.any(np.isfinite(row)) else 0.0 for row in od[:, :k]])
        abs_tol = l2_abs_tol(index, queries, probes_used, kth, decomposed=decomposed)
        check_results(gpu_d, gpu_i, od, oi, k, tau, rep, lookup=lookup, abs_tol=abs_tol)
    return rep


def compare_flat(db_bits, query_bits, k, gpu_d, gpu_i, tau=TAU_F32, k_extra=32,
                 nthreads=None) -> Report:
    """Acceptance check of a device exact search over bfloat16 rows against
    the oracle's brute force (exact, double precision).  The device evaluates
    |x|^2 + |y|^2 - 2 x.y in float32, so next to the relative tolerance each
    row allows the absolute forward-error term 4 gamma_{d+2} (|x|^2 + max |y|^2)
    (bf16 products are exact in float32; the sums carry the error)."""
    db = np.ascontiguousarray(db_bits, dtype=np.uint16)
    q = np.ascontiguousarray(query_bits, dtype=np.uint16)
    rep = Report(nq=len(q))
    od, oi = O.bruteforce_bf16(db, q, k + k_extra, nthreads=nthreads)
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dbf = widen(db)
    qf = widen(q)
    d = db.shape[1]
    ymax = float(np.max(np.sum(dbf * dbf, axis=1))) if len(db) else 0.0
    abs_tol = 4.0 * gamma(d + 2) * (np.sum(qf * qf, axis=1) + ymax)

    def lookup(row, id_list):
        ids = np.asarray(id_list, dtype=np.int64)
        ok = (ids >= 0) & (ids < len(db))
        out = [None] * len(ids)
        for j in np.flatnonzero(ok):
            diff = qf[row] - dbf[ids[j]]
            out[j] = float(np.dot(diff, diff))
        return out

    check_results(gpu_d, gpu_i, od, oi, k, tau, rep, lookup=lookup, abs_tol=abs_tol)
    return rep



@dataclasses.dataclass
class EncodeReport:
    n: int = 0
    list_flips: int = 0
    code_flips: int = 0
    failures: list = dataclasses.field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> dict:
        return dict(n=self.n, list_flips=self.list_flips, code_flips=self.code_flips,
                    failures=len(self.failures))


def compare_encode(vectors, centroids, codebooks, gpu_lists, gpu_codes, oracle_out=None,
                   nthreads=None) -> EncodeReport:
    """Rules 4 and 5: device list assignment and PQ codes against the oracle.
    oracle_out: a precomputed ``O.assign_encode`` result for the same inputs."""
    x = np.ascontiguousarray(vectors, dtype=np.float32)
    cent = np.ascontiguousarray(centroids, dtype=np.float32)
    books = np.ascontiguousarray(codebooks, dtype=np.float32)
    gl = np.asarray(gpu_lists).reshape(-1).astype(np.int64)
    gc = np.asarray(gpu_codes).reshape(len(x), -1)
    n, d = x.shape
    nlist, m, dsub = cent.shape[0], books.shape[0], books.shape[2]
    rep = EncodeReport(n=n)
    if gl.shape[0] != n or gc.shape[1] != m:
        rep.failures.append((-1, "output shape"))
        return rep
    lists, codes, _, _ = (O.assign_encode(x, cent, books, nthreads=nthreads)
                          if oracle_out is None else oracle_out)
    cmax = float(np.max(np.sum(cent.astype(np.float64) ** 2, axis=1))) if nlist else 0.0
    bmax = np.max(np.abs(books.astype(np.float64)), axis=1)           # [m, dsub]
    for i in range(n):
        li = int(gl[i])
        if not 0 <= li < nlist:
            rep.failures.append((i, f"list {li} out of range"))
            continue
        if li != lists[i]:
            allp, alld = O.coarse(x[i], cent, nlist)
            dist_of = dict(zip(allp.tolist(), alld.tolist()))
            x2 = float(np.sum(x[i].astype(np.float64) ** 2))
            delta = 4.0 * gamma(d + 2) * (x2 + cmax)
            if dist_of[li] - float(alld[0]) > delta:
                rep.failures.append((i, f"list {li} outside the coarse tie band"))
                continue
            rep.list_flips += 1
        elif np.array_equal(gc[i], codes[i]):
            continue
        table = O.lut(x[i], cent[li], books)
        r = np.abs(x[i].astype(np.float64) - cent[li].astype(np.float64)).reshape(m, dsub)
        delta_e = 4.0 * gamma(dsub + 3) * np.sum((2.0 * r + bmax) ** 2, axis=1)
        best = table.min(axis=1)
        for j in range(m):
            v = int(gc[i, j])
            if table[j, v] - best[j] > delta_e[j]:
                rep.failures.append((i, f"code {v} of sub-quantizer {j} is not the nearest"))
            elif li == lists[i] and v != codes[i, j]:
                rep.code_flips += 1
    return rep


@dataclasses.dataclass
class KmeansReport:
    n: int = 0
    k: int = 0
    assign_flips: int = 0
    ulp_diffs: int = 0
    failures: list = dataclasses.field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> dict:
        return dict(n=self.n, k=self.k, assign_flips=self.assign_flips, ulp_diffs=self.ulp_diffs,
                    failures=len(self.failures))


def compare_kmeans_iteration(vectors, centers_in, gpu_assign, gpu_centers, gpu_counts=None,
                         nthreads=None) -> KmeansReport:
    """Rule 6: one device iteration (assignment + update) from centers_in."""
    x = np.ascontiguousarray(vectors, dtype=np.float32)
    c0 = np.ascontiguousarray(centers_in, dtype=np.float32)
    ga = np.asarray(gpu_assign).reshape(-1).astype(np.int64)
    gc = np.asarray(gpu_centers, dtype=np.float32)
    n, d = x.shape
    k = c0.shape[0]
    rep = KmeansReport(n=n, k=k)
    if ga.shape[0] != n or gc.shape != c0.shape:
        rep.failures.append((-1, "output shape"))
        return rep
    if n and (ga.min() < 0 or ga.max() >= k):
        rep.failures.append((-1, "assignment out of range"))
        return rep
    ol, _ = O.nearest_lists(x, c0, nthreads=nthreads)
    cmax = float(np.max(np.sum(c0.astype(np.float64) ** 2, axis=1)))
    for i in np.flatnonzero(ga != ol):
        allp, alld = O.coarse(x[i], c0, k)
        dist_of = dict(zip(allp.tolist(), alld.tolist()))
        delta = 4.0 * gamma(d + 2) * (float(np.sum(x[i].astype(np.float64) ** 2)) + cmax)
        if dist_of[int(ga[i])] - float(alld[0]) > delta:
            rep.failures.append((int(i), f"assigned to {int(ga[i])}, outside the tie band"))
        else:
            rep.assign_flips += 1
    want, means, counts = O.kmeans_update(x, ga, c0)
    if gpu_counts is not None and not np.array_equal(np.asarray(gpu_counts).reshape(-1), counts):
        rep.failures.append((-1, "counts differ"))
    same = gc == want
    if not same.all():
        # the other float32 neighbour of the exact mean
        other = np.where(want.astype(np.float64) < means,
                         np.nextafter(want, np.float32(np.inf)),
                         np.nextafter(want, np.float32(-np.inf)))
        near = (gc == other) & (want.astype(np.float64) != means)
        rep.ulp_diffs = int(np.sum(~same & near))
        for c, t in zip(*np.nonzero(~same & ~near)):
            rep.failures.append((int(c), f"center {int(c)} dim {int(t)}: {gc[c, t]!r} "
                                          f"against mean {means[c, t]!r}"))
            if len(rep.failures) > 20:
                break
    return rep
