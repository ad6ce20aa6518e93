// Register-resident k-selection for one wave64.
//
// Follows the structure of WarpSelect ("Billion-scale similarity search with
// GPUs", k-selection section: a warp queue W of the k smallest values seen,
// kept sorted ascending in a lane-stride register array, sentinel +inf,
// values carried with their indices, and a per-step filter that rejects a
// value that cannot be among the k smallest), re-shaped for wave64:
//
//  * The filter threshold is W[k-1] (the k-th smallest so far), optionally
//    tightened by an external bound (another wave's W[k-1]: its k values
//    already beat anything above it).  A value >= threshold is dropped.
//  * Survivors are compacted, in lane order, into a 64-slot staging buffer
//    of the wave in LDS: ballot + mbcnt give each survivor its slot and it
//    writes itself there (a store nobody waits for; a pass with survivors
//    costs a few instructions and no round trip).  This replaces the per-lane
//    thread queues of the paper: on wave64 it merges once per 64 survivors
//    instead of whenever one lane's queue fills.
//  * When the buffer would overflow (and at the end) it is read back one
//    element per lane, sorted descending by a 64-element bitonic network in
//    registers, folded into W's last register with an
//    element-wise min (the first step of a bitonic merge of W with the
//    reversed buffer keeps exactly the kw smallest), and W is re-sorted by
//    a bitonic merge (log2(kw) steps).  All of it is data-independent.
//
// Invariant: every value seen so far that belongs to the k smallest (ties
// aside) is in W or in the buffer; W is sorted ascending.
#pragma once

#include "wave_ops.hpp"

namespace ivfpq {

template <int NW> // W holds kw = 64 * NW elements, kw >= k
struct WaveTopK {
    float wk[NW];
    uint32_t wv[NW];
    float *sk;    // 64-slot candidate staging buffer of this wave (LDS)
    uint32_t *sv;
    int bcount; // filled buffer slots (wave-uniform)
    int k;
    int rk;     // rank whose value the wave publishes for the union bound
    float kth;  // W[k-1] (wave-uniform)
    float part; // W[rk-1] (wave-uniform)
    float thr;  // filter threshold = min(kth, external bounds)

    // stage: 64 keys then 64 values of LDS owned by this wave
    __device__ __forceinline__ void init(int k_, uint32_t *stage, int rk_ = 0)
    {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            wk[r] = INFINITY;
            wv[r] = kSentinel;
        }
        sk = reinterpret_cast<float *>(stage);
        sv = stage + 64;
        bcount = 0;
        k = k_;
        rk = rk_ > 0 ? rk_ : k_;
        kth = INFINITY;
        part = INFINITY;
        thr = INFINITY;
    }

    // W[e] (wave-uniform), e < 64 * NW
    __device__ __forceinline__ float read_rank(int e) const
    {
        const int lane = e & 63;
        float out = INFINITY;
#pragma unroll
        for (int r = 0; r < NW; ++r)
            if (r == (e >> 6))
                out = __uint_as_float(
                    (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(wk[r]), lane));
        return out;
    }

    // Wave-uniform values kept in scalar registers.
    __device__ __forceinline__ static float uni(float x)
    {
        return __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(x)));
    }
    __device__ __forceinline__ static int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

    // Merge the buffer into W.
    __device__ __forceinline__ void flush()
    {
        if (bcount == 0)
            return;
        const int lane = lane_id();
        float bk = INFINITY;
        uint32_t bv = kSentinel;
        if (lane < bcount) {
            bk = sk[lane];
            bv = sv[lane];
        }
        sort64<true>(bk, bv);
        // first step of the bitonic merge of W (ascending) with the buffer
        // (descending, padded with +inf to kw): keep the element-wise min
        {
            const bool take = bk < wk[NW - 1];
            wk[NW - 1] = take ? bk : wk[NW - 1];
            wv[NW - 1] = take ? bv : wv[NW - 1];
        }
        bitonic_merge_up<NW>(wk, wv);
        bcount = 0;
        kth = uni(read_rank(k - 1));
        part = uni(read_rank(rk - 1));
        thr = uni(fminf(thr, kth));
    }

    // Tighten the filter with an external bound (another wave's k-th value).
    __device__ __forceinline__ void bound(float ext) { thr = uni(fminf(thr, ext)); }

    // Whether any lane's key would pass the filter now (wave-uniform).
    __device__ __forceinline__ bool any_below(float key) const
    {
        return wave_ballot(key < thr) != 0;
    }

    // One candidate per lane; lanes without a candidate pass key = +inf.
    __device__ __forceinline__ void push(float key, uint32_t val)
    {
        bool pass = key < thr;
        uint64_t mask = wave_ballot(pass);
        if (mask == 0)
            return;
        int n = uni((int)__popcll(mask));
        if (bcount + n > 64) {
            flush();
            pass = key < thr;
            mask = wave_ballot(pass);
            if (mask == 0)
                return;
            n = uni((int)__popcll(mask));
        }
        if (pass) {
            const int slot = bcount + mbcnt64(mask);
            sk[slot] = key;
            sv[slot] = val;
        }
        bcount = uni(bcount + n);
    }

    // Write W (kw elements, lane-stride order) to memory.
    __device__ __forceinline__ void store(float *keys, uint32_t *vals) const
    {
        const int lane = lane_id();
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            keys[r * 64 + lane] = wk[r];
            vals[r * 64 + lane] = wv[r];
        }
    }

    // Merge another sorted kw-array (ascending, in memory) into W: the
    // element-wise min of W and the reversed other array holds the kw
    // smallest of both and is bitonic; one bitonic merge sorts it.
    __device__ __forceinline__ void merge_sorted(const float *keys, const uint32_t *vals)
    {
        const int lane = lane_id();
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int src = (NW - 1 - r) * 64 + (63 - lane);
            const float ok = keys[src];
            const uint32_t ov = vals[src];
            const bool take = ok < wk[r];
            wk[r] = take ? ok : wk[r];
            wv[r] = take ? ov : wv[r];
        }
        bitonic_merge_up<NW>(wk, wv);
        kth = read_rank(k - 1);
        part = read_rank(rk - 1);
        thr = fminf(thr, kth);
    }
};

} // namespace ivfpq
