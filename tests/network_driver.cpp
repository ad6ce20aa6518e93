// Host model of the register k-selection's networks and of WaveTopK, run on
// the schedules and lane masks of csrc/network.hpp (the tables the device code
// runs).  Each check prints "ok <name>" or "FAIL <name> <detail>"; the Python
// test asserts on the lines.
//
// The model of a step follows the device's semantics: lane-stride arrays of
// 64*R elements (element e in register e / 64 of lane e % 64); for S < 64 the
// partner is lane l ^ S of the same register and a lane keeps the smaller key
// when its bit of keep_min_mask is set, taking the partner's pair only when
// the partner's key is strictly smaller (resp. larger), so equal keys never
// move; for S >= 64 registers r and r | S/64 of one lane are exchanged when
// strictly out of order for the block's direction.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "network.hpp"

using namespace ivfpq;

struct Arr {
    int R;
    std::vector<float> k;
    std::vector<uint32_t> v;
    explicit Arr(int r) : R(r), k(64 * r), v(64 * r) {}
};

static void step(Arr &a, int B, int S, bool desc)
{
    if (S >= 64) {
        const int RS = S / 64;
        for (int r = 0; r < a.R; ++r) {
            if (r & RS)
                continue;
            const bool up = block_ascending(B, desc, r);
            for (int l = 0; l < 64; ++l) {
                const int i = r * 64 + l, j = (r | RS) * 64 + l;
                const bool swap = up ? (a.k[j] < a.k[i]) : (a.k[i] < a.k[j]);
                if (swap) {
                    std::swap(a.k[i], a.k[j]);
                    std::swap(a.v[i], a.v[j]);
                }
            }
        }
        return;
    }
    Arr out = a;
    for (int r = 0; r < a.R; ++r) {
        uint64_t keep = keep_min_mask(S, B, desc, r);
#ifdef PLANT_MASK_BIT
        if (S == 2 && r == 0)
            keep ^= 1ull << 5;
#endif
        for (int l = 0; l < 64; ++l) {
            const int i = r * 64 + l, p = r * 64 + (l ^ S);
            const bool km = (keep >> l) & 1;
            const bool take = km ? (a.k[p] < a.k[i]) : (a.k[p] > a.k[i]);
            if (take) {
                out.k[i] = a.k[p];
                out.v[i] = a.v[p];
            }
        }
    }
    a = out;
}

// Planted mistakes (the test builds the driver with each and expects a FAIL):
// PLANT_SKIP_STEP drops a schedule's last step, PLANT_MASK_BIT flips one lane
// of one step's keep mask, PLANT_NO_FOLD replaces W's last register by the
// sorted buffer instead of taking the element-wise minimum.
template <size_t N>
static void run(Arr &a, const std::array<NetStep, N> &sched, bool desc)
{
#ifdef PLANT_SKIP_STEP
    for (size_t i = 0; i + 1 < N; ++i)
        step(a, sched[i].B, sched[i].S, desc);
#else
    for (const NetStep &s : sched)
        step(a, s.B, s.S, desc);
#endif
}

static int fails = 0;
static void report(bool ok, const char *name, const char *detail = "")
{
    if (ok)
        std::printf("ok %s\n", name);
    else {
        std::printf("FAIL %s %s\n", name, detail);
        ++fails;
    }
}

static bool sorted_by(const Arr &a, bool desc)
{
    for (size_t i = 1; i < a.k.size(); ++i)
        if (desc ? a.k[i - 1] < a.k[i] : a.k[i - 1] > a.k[i])
            return false;
    return true;
}

// the (key, value) pairs are a permutation of the input's
static bool same_pairs(const Arr &a, const Arr &b)
{
    std::vector<std::pair<float, uint32_t>> x, y;
    for (size_t i = 0; i < a.k.size(); ++i) {
        x.emplace_back(a.k[i], a.v[i]);
        y.emplace_back(b.k[i], b.v[i]);
    }
    std::sort(x.begin(), x.end());
    std::sort(y.begin(), y.end());
    return x == y;
}

// ---- depth closed forms -------------------------------------------------
static void check_depths()
{
    bool ok = kSort64.size() == 21 && sort_steps(64) == 6 * 7 / 2;
    for (int n = 1; n <= 10; ++n)
        ok = ok && sort_steps(1 << n) == n * (n + 1) / 2 && merge_steps(1 << n) == n;
    ok = ok && kMergeUp<1>.size() == 6 && kMergeUp<2>.size() == 7 && kMergeUp<4>.size() == 8 &&
         kMergeUp<8>.size() == 9 && kMergeUp<16>.size() == 10;
    // the sort's blocks grow 2, 4, ..., 64 and each block's half-cleaners
    // shrink B/2 .. 1; the merge's S halve from 32R to 1
    int i = 0;
    for (int B = 2; B <= 64; B *= 2)
        for (int S = B / 2; S >= 1; S /= 2, ++i)
            ok = ok && kSort64[i].S == S && kSort64[i].B == (B == 64 ? 0 : B);
    report(ok, "depth_closed_forms");
}

// ---- 0-1 principle ------------------------------------------------------
// The 64-element sort, both directions: every 0-1 input with at most three
// runs (all of them), and random 0-1 inputs; then float inputs with ties.
static void check_sort64()
{
    std::mt19937_64 rng(1);
    for (int desc = 0; desc < 2; ++desc) {
        bool ok = true;
        auto try_bits = [&](uint64_t bits) {
            Arr a(1);
            for (int l = 0; l < 64; ++l) {
                a.k[l] = (float)((bits >> l) & 1);
                a.v[l] = l;
            }
            Arr in = a;
            run(a, kSort64, desc);
            ok = ok && sorted_by(a, desc) && same_pairs(a, in);
        };
        for (int x = 0; x <= 64; ++x)
            for (int y = x; y <= 64; ++y)
                for (int z = y; z <= 64; ++z) {
                    uint64_t bits = 0;
                    for (int l = 0; l < 64; ++l)
                        if ((l >= x && l < y) || l >= z)
                            bits |= 1ull << l;
                    try_bits(bits);
                }
        for (int t = 0; t < 200000; ++t)
            try_bits(rng());
        for (int t = 0; t < 20000 && ok; ++t) {
            Arr a(1);
            for (int l = 0; l < 64; ++l) {
                a.k[l] = (float)(rng() % 9);
                a.v[l] = l;
            }
            Arr in = a;
            run(a, kSort64, desc);
            ok = ok && sorted_by(a, desc) && same_pairs(a, in);
        }
        report(ok, desc ? "sort64_desc_zero_one" : "sort64_asc_zero_one");
    }
}

// The merge of 64*R elements: bitonic 0-1 inputs (rotations of 0^a 1^b 0^c
// and of 1^a 0^b 1^c: by the 0-1 principle these cover every bitonic input),
// all of them for R <= 4 and `samples` drawn at random for larger R.
template <int R>
static void check_merge(int samples = 0)
{
    constexpr int N = 64 * R;
    bool ok = true;
    std::mt19937_64 rng(100 + R);
    const long total = (long)(N + 1) * N * 2;
    for (long t = 0; t < (samples ? samples : total); ++t) {
        const long c = samples ? (long)(rng() % total) : t;
        const int ones = (int)(c / (2L * N)), rot = (int)((c / 2) % N), inv = (int)(c % 2);
        Arr a(R);
        for (int e = 0; e < N; ++e) {
            const int pos = (e + rot) % N;
            a.k[e] = (float)((pos < ones) ^ inv);
            a.v[e] = e;
        }
        Arr in = a;
        run(a, kMergeUp<R>, false);
        ok = ok && sorted_by(a, false) && same_pairs(a, in);
    }
    char name[32];
    std::snprintf(name, sizeof name, "merge_bitonic_zero_one_R%d", R);
    report(ok, name);
}

// ---- WaveTopK model and the WarpSelect invariants -----------------------
struct TopK {
    int NW, k;
    Arr W;
    std::vector<float> bk;
    std::vector<uint32_t> bv;
    float thr = INFINITY, kth = INFINITY;
    TopK(int nw, int k_) : NW(nw), k(k_), W(nw)
    {
        std::fill(W.k.begin(), W.k.end(), INFINITY);
        std::fill(W.v.begin(), W.v.end(), 0xFFFFFFFFu);
    }
    void flush()
    {
        if (bk.empty())
            return;
        Arr b(1);
        for (int l = 0; l < 64; ++l) {
            b.k[l] = l < (int)bk.size() ? bk[l] : INFINITY;
            b.v[l] = l < (int)bk.size() ? bv[l] : 0xFFFFFFFFu;
        }
        run(b, kSort64, true); // descending
        // first step of the bitonic merge of W (ascending) with the buffer
        // (descending, padded with +inf): element-wise min into W's last
        // register, which leaves a bitonic sequence of the kw smallest
        for (int l = 0; l < 64; ++l) {
            const int i = (NW - 1) * 64 + l;
#ifdef PLANT_NO_FOLD
            if (true) {
#else
            if (b.k[l] < W.k[i]) {
#endif
                W.k[i] = b.k[l];
                W.v[i] = b.v[l];
            }
        }
        switch (NW) {
        case 1: run(W, kMergeUp<1>, false); break;
        case 2: run(W, kMergeUp<2>, false); break;
        case 4: run(W, kMergeUp<4>, false); break;
        case 8: run(W, kMergeUp<8>, false); break;
        default: run(W, kMergeUp<16>, false); break;
        }
        bk.clear();
        bv.clear();
        kth = W.k[k - 1];
        thr = std::min(thr, kth);
    }
    // one candidate per lane, lanes with no candidate pass +inf
    void push(const float *key, const uint32_t *val)
    {
        int n = 0;
        for (int l = 0; l < 64; ++l)
            n += key[l] < thr;
        if (n == 0)
            return;
        if ((int)bk.size() + n > 64) {
            flush();
            n = 0;
            for (int l = 0; l < 64; ++l)
                n += key[l] < thr;
        }
        for (int l = 0; l < 64; ++l)
            if (key[l] < thr) {
                bk.push_back(key[l]);
                bv.push_back(val[l]);
            }
    }
};

static void check_topk(int NW, int k, int nsteps, int distinct, uint64_t seed, const char *name)
{
    std::mt19937_64 rng(seed);
    TopK t(NW, k);
    std::vector<float> seen;
    bool sorted_ok = true, kept_ok = true, thr_ok = true;
    for (int s = 0; s < nsteps; ++s) {
        float key[64];
        uint32_t val[64];
        for (int l = 0; l < 64; ++l) {
            key[l] = distinct ? (float)(rng() % distinct) : (float)(rng() >> 40) * 0x1p-24f;
            val[l] = (uint32_t)(s * 64 + l);
            seen.push_back(key[l]);
        }
        t.push(key, val);
        // invariant 1: W ascending
        sorted_ok = sorted_ok && sorted_by(t.W, false);
        // invariant 2: the k smallest keys seen so far are all in W or the
        // buffer (as a multiset, up to the k-th value)
        std::vector<float> s_all = seen;
        std::sort(s_all.begin(), s_all.end());
        const int kk = std::min<int>(k, (int)s_all.size());
        std::vector<float> held(t.W.k.begin(), t.W.k.end());
        held.insert(held.end(), t.bk.begin(), t.bk.end());
        std::sort(held.begin(), held.end());
        for (int i = 0; i < kk && kept_ok; ++i)
            kept_ok = held[i] <= s_all[i];
        // invariant 3: the threshold never excludes a value below the k-th
        // smallest seen so far
        if ((int)s_all.size() >= k)
            thr_ok = thr_ok && t.thr >= s_all[k - 1];
    }
    t.flush();
    std::vector<float> s_all = seen;
    std::sort(s_all.begin(), s_all.end());
    bool final_ok = true;
    for (int i = 0; i < k; ++i)
        final_ok = final_ok && t.W.k[i] == s_all[i];
    // values: distinct positions whose keys are the reported keys
    std::vector<uint32_t> ids(t.W.v.begin(), t.W.v.begin() + k);
    std::sort(ids.begin(), ids.end());
    final_ok = final_ok && std::adjacent_find(ids.begin(), ids.end()) == ids.end();
    for (int i = 0; i < k && final_ok; ++i)
        final_ok = t.W.v[i] < seen.size() && seen[t.W.v[i]] == t.W.k[i];
    char buf[128];
    std::snprintf(buf, sizeof buf, "sorted=%d kept=%d thr=%d final=%d", sorted_ok, kept_ok, thr_ok,
                  final_ok);
    report(sorted_ok && kept_ok && thr_ok && final_ok, name, buf);
}

int main()
{
    check_depths();
    check_sort64();
    check_merge<1>();
    check_merge<2>();
    check_merge<4>();
    check_merge<8>(4000);
    check_merge<16>(2000);
    check_topk(1, 1, 200, 0, 11, "topk_nw1_k1");
    check_topk(1, 10, 400, 0, 12, "topk_nw1_k10");
    check_topk(1, 64, 300, 0, 13, "topk_nw1_k64");
    check_topk(2, 100, 300, 0, 14, "topk_nw2_k100");
    check_topk(2, 128, 300, 5, 15, "topk_nw2_k128_heavy_ties");
    check_topk(16, 1000, 100, 0, 16, "topk_nw16_k1000");
    check_topk(16, 1024, 60, 3, 17, "topk_nw16_k1024_three_values");
    std::printf("done %d\n", fails);
    return fails ? 1 : 0;
}
