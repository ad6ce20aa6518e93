// IVF-PQ search kernels for gfx950: work planning, table build + code scan +
// first-pass top-k, cross-item merge.
//
// Definitions ("Custom 8-bit floating point value format for reducing shared
// memory bank conflict in ANN search", IVFPQ section, search steps 2-5 and
// Eq. (1)):  for each probed list l of query x, r = x - c_l,
//   F_j(v) = sum_{t<dsub} (r[j dsub + t] - C_j[v][t])^2      (table, in LDS)
//   R_i    = sum_{j<m} F_j(code_i[j])                          (per entry)
// and the k smallest R over all probed lists are returned.
//
// Work decomposition ("Billion-scale similarity search with GPUs", IVFADC
// section: (query, list) pairs are independent; a first k-selection pass per
// piece of work reduces to f*k partial results, a second pass reduces those
// to k):
//  * plan:  per query, E = total entries of its probed lists; the query's
//           entries (lists in probe order, one after the other) are cut into
//           ceil(E / chunk) work items of chunk entries, chunk = max(target,
//           ceil(E / imax)), so a query has at most imax items whatever the
//           list-size skew;
//  * scan:  persistent workgroups take items from an atomic counter.  For an
//           item the workgroup lays out its pieces (list, entry range), then
//           per piece builds the m x 256 table in LDS (double-buffered: the
//           next piece's table is built while the current one is scanned)
//           and its waves scan the piece, one entry per lane, code rows read
//           as wide coalesced loads one step ahead, each wave keeping a
//           register top-k (WaveTopK).  A per-query bound (the smallest k-th
//           value any wave of any item of the query holds) is shared through
//           LDS and global memory.  An item that is its query's only item
//           writes the final result; otherwise its sorted top-k goes to a
//           partial slot;
//  * merge: per query with several items, bitonic merges of the sorted
//           partials, then the id gather.
//
// The codebook lives in registers: thread v of group g holds codeword v of
// the m/G sub-quantizers of group g, so a table build reads no memory but the
// residual (an LDS broadcast).  The difference form (sum of squares) is used:
// no cancellation, every entry and every sum is a sum of non-negative terms.
#include "common.hpp"
#include "internal.hpp"
#include "plan.hpp"

#include <cstdlib>

namespace ivfpq {

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------

// Region-aligned layout of a query's sequence when the index has giant lists
// (the scan order groups the work items that read the same region of a
// giant list; aligned, those items read the same lines in step): the small
// lists first, in probe order, then, from the next multiple of kRegion, the
// giant lists in probe order, each taking its size rounded up to a multiple
// of kRegion (the padding holds no entries and no piece meets it).  Item
// boundaries, multiples of a chunk that is itself a multiple of kRegion,
// then fall on region boundaries of every giant list.
__host__ __device__ inline uint64_t region_round(uint64_t n)
{
    return (n + kRegion - 1) / kRegion * kRegion;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t *__restrict__ probes, int nprobe,
                                                    int64_t nq, int nlist,
                                                    const uint32_t *__restrict__ list_off,
                                                    uint32_t target, uint32_t imax,
                                                    uint32_t *__restrict__ qtotal,
                                                    uint32_t *__restrict__ qchunk,
                                                    uint32_t *__restrict__ qcount,
                                                    uint32_t *__restrict__ qbound,
                                                    uint32_t *__restrict__ counter,
                                                    unsigned long long *__restrict__ prof,
                                                    const uint32_t *__restrict__ gbucket,
                                                    uint32_t *__restrict__ bcur, uint32_t nbucket)
{
    // one wave per query (16 per workgroup): its lanes read the probes 64 at
    // a time and the sums meet by shuffles
    __shared__ unsigned long long wsum[16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t gt = (int64_t)blockIdx.x * 1024 + threadIdx.x;
    const int64_t q = (int64_t)blockIdx.x * 16 + wave;
    if (gt == 0)
        *counter = 0;
    if (bcur) // the giant-list buckets' counters (order_* kernels)
        for (int64_t i = gt; i <= (int64_t)nbucket; i += (int64_t)gridDim.x * 1024)
            bcur[i] = 0;
    uint64_t e = 0, small = 0, giant = 0;
    for (int p = lane; q < nq && p < nprobe; p += 64) {
        const int l = probes[q * nprobe + p];
        if ((unsigned)l < (unsigned)nlist) {
            const uint32_t sz = list_off[l + 1] - list_off[l];
            e += sz;
            if (gbucket && gbucket[l] != kNoBucket)
                giant += region_round(sz);
            else
                small += sz;
        }
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) {
        e += __shfl_xor(e, sh);
        small += __shfl_xor(small, sh);
        giant += __shfl_xor(giant, sh);
    }
    if (prof) {
        // entries scanned: one atomic per workgroup (a same-address atomic
        // per query would queue behind each other)
        if (lane == 0)
            wsum[wave] = e;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long t = 0;
            for (int w = 0; w < 16; ++w)
                t += wsum[w];
            if (t)
                atomicAdd(prof, t);
        }
    }
    if (lane != 0 || q >= nq)
        return;
    // the query's sequence: its entries (with giant lists, the region-aligned
    // layout of the scan order)
    const uint32_t total = (uint32_t)(giant ? region_round(small) + giant : e);
    const QueryPlan qp = plan_query(total, target, imax, gbucket ? kRegion : 1u);
    qtotal[q] = total;
    qchunk[q] = qp.chunk;
    qcount[q] = qp.count;
    qbound[q] = float_order_key(INFINITY);
}

// Exclusive prefix sum of qcount into base[0..nq]; one workgroup of 1024.
__global__ __launch_bounds__(1024) void item_scan_kernel(const uint32_t *__restrict__ qcount,
                                                         int64_t nq, uint32_t *__restrict__ base,
                                                         unsigned long long *__restrict__ prof)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    if (tid == 0)
        carry_s = 0;
    __syncthreads();
    for (int64_t s = 0; s < nq; s += 1024) {
        const int64_t i = s + tid;
        const uint32_t v = i < nq ? qcount[i] : 0u;
        const uint32_t incl = wave_inclusive_sum(v);
        if (lane == 63)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t before = carry_s;
        for (int w = 0; w < wave; ++w)
            before += wsum[w];
        if (i < nq)
            base[i] = before + incl - v;
        __syncthreads();
        if (tid == 1023)
            carry_s = before + incl;
        __syncthreads();
    }
    if (tid == 0) {
        base[nq] = carry_s;
        if (prof)
            atomicAdd(prof + 1, (unsigned long long)carry_s);
    }
}

// Scan order of the work items, rank-major: item 0 of every query (queries
// in order), then item 1 of every query that has one, and so on.  The items
// of one query then start at different times, and a later one begins with
// the bound its query's earlier items have published (their k-th values
// bound the query's), so its k-selection admits few candidates; with the
// items of a query side by side in the order, all of them would start from
// an empty top-k at once.  Two kernels, one workgroup per rank r < imax:
// the number of queries with more than r items, then the positions.
__global__ __launch_bounds__(1024) void rank_count_kernel(const uint32_t *__restrict__ qcount,
                                                          int64_t nq, uint32_t *__restrict__ rank_n)
{
    __shared__ uint32_t wsum[16];
    const uint32_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t c = 0;
    for (int64_t i = tid; i < nq; i += 1024)
        c += qcount[i] > r ? 1u : 0u;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1)
        c += (uint32_t)__shfl_xor((int)c, sh);
    if (lane == 0)
        wsum[wave] = c;
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
        for (int w = 0; w < 16; ++w)
            t += wsum[w];
        rank_n[r] = t;
    }
}

__global__ __launch_bounds__(1024) void rank_order_kernel(const uint32_t *__restrict__ qcount,
                                                          int64_t nq,
                                                          const uint32_t *__restrict__ rank_n,
                                                          uint32_t *__restrict__ item_q,
                                                          uint32_t *__restrict__ item_r)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry_s;
    const uint32_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0) {
        uint32_t b = 0;
        for (uint32_t s = 0; s < r; ++s)
            b += rank_n[s];
        carry_s = b;
    }
    __syncthreads();
    for (int64_t s = 0; s < nq; s += 1024) {
        const int64_t i = s + tid;
        const uint32_t v = (i < nq && qcount[i] > r) ? 1u : 0u;
        const uint32_t incl = wave_inclusive_sum(v);
        if (lane == 63)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t before = carry_s;
        for (int w = 0; w < wave; ++w)
            before += wsum[w];
        if (v) {
            item_q[before + incl - 1] = (uint32_t)i;
            item_r[before + incl - 1] = r;
        }
        __syncthreads();
        if (tid == 1023)
            carry_s = before + incl;
        __syncthreads();
    }
}

// Scan order with giant lists (kGiantList entries or more).  The lists
// nearest to many queries are probed by many of them: at the 1B Zipf shape
// the regions of the giant lists are read by about 20 work items each, and
// in rank-major order those reads are spread over the whole scan.  The items
// past a query's first with a piece of a giant list are therefore taken out
// of the rank-major order and run after the others, bucket by bucket, a
// bucket being the region (kRegion entries) of a giant list where the item's
// largest such piece starts: items that read the same region then run side
// by side, and all but the first find its lines in the cache.  The other
// items keep their rank-major order and run first, the first item of every
// query (its nearest lists) among them, so a query's bound is published
// before its giant pieces are scanned.  The result does not depend on the
// order.
//
// item_key_kernel: each item's bucket (kNoBucket: none), counted into
// bcur[bucket + 1] (bcur zeroed by the plan kernel).
__global__ __launch_bounds__(256) void item_key_kernel(
    const uint32_t *__restrict__ item_base, int64_t nq, const uint32_t *__restrict__ rm_q,
    const uint32_t *__restrict__ rm_r, const uint32_t *__restrict__ qchunk,
    const uint32_t *__restrict__ qtotal, const int32_t *__restrict__ probes, int nprobe,
    int nlist, const uint32_t *__restrict__ list_off, const uint32_t *__restrict__ gbucket,
    uint32_t *__restrict__ ikey, uint32_t *__restrict__ bcur)
{
    // one wave per item, the items of the rank-major order in turn: the
    // lanes take the query's probes 64 at a time; the offsets of the giant
    // lists in the region-aligned sequence come from a prefix sum over the
    // lanes, the longest piece (the first probe among equals) from a maximum
    const int lane = threadIdx.x & 63;
    const int64_t total = item_base[nq];
    const int64_t nw = (int64_t)gridDim.x * 4;
    for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < total; i += nw) {
        const int64_t q = rm_q[i];
        const uint32_t r = rm_r[i];
        uint32_t key = kNoBucket;
        // a query's first item (its nearest lists) keeps its rank-major
        // place: the bound it publishes is the one its other items start from
        if (r > 0) {
            uint32_t start, stop;
            item_range(r, qchunk[q], qtotal[q], &start, &stop);
            uint64_t small = 0;
            for (int p = lane; p < nprobe; p += 64) {
                const int l = probes[q * nprobe + p];
                if ((unsigned)l < (unsigned)nlist && gbucket[l] == kNoBucket)
                    small += list_off[l + 1] - list_off[l];
            }
#pragma unroll
            for (int sh = 32; sh >= 1; sh >>= 1)
                small += __shfl_xor(small, sh);
            uint32_t acc = (uint32_t)region_round(small); // the giant lists start here
            uint64_t best = 0; // (piece length, ~probe) of this lane's longest piece
            uint32_t bkey = kNoBucket;
            for (int p0 = 0; p0 < nprobe; p0 += 64) {
                const int p = p0 + lane;
                int l = 0;
                uint32_t sz = 0;
                bool g = false;
                if (p < nprobe) {
                    l = probes[q * nprobe + p];
                    g = (unsigned)l < (unsigned)nlist && gbucket[l] != kNoBucket;
                    sz = g ? list_off[l + 1] - list_off[l] : 0u;
                }
                const uint32_t w = (uint32_t)region_round(sz);
                uint32_t x = w; // inclusive prefix over the lanes
#pragma unroll
                for (int dd = 1; dd < 64; dd <<= 1) {
                    const uint32_t y = __shfl_up(x, dd);
                    x += lane >= dd ? y : 0u;
                }
                const uint32_t lo = acc + x - w;
                uint32_t b, e;
                if (g && piece_of(lo, lo + sz, start, stop, &b, &e)) {
                    const uint64_t c = ((uint64_t)(e - b) << 32) | (0xFFFFFFFFu - (uint32_t)p);
                    if (c > best) {
                        best = c;
                        bkey = gbucket[l] + b / kRegion;
                    }
                }
                acc += __shfl(x, 63);
            }
            uint64_t m = best;
#pragma unroll
            for (int sh = 32; sh >= 1; sh >>= 1) {
                const uint64_t o = __shfl_xor(m, sh);
                m = o > m ? o : m;
            }
            if (m != 0) {
                const uint32_t pb = 0xFFFFFFFFu - (uint32_t)m;
                key = (uint32_t)__shfl((int)bkey, (int)(pb & 63));
            }
        }
        if (lane == 0) {
            ikey[i] = key;
            if (key != kNoBucket)
                atomicAdd(&bcur[key + 1], 1u);
        }
    }
}

// One workgroup: the items without a bucket, compacted in rank-major order to
// the front of the final order; then bcur[b] becomes the first position of
// bucket b (an inclusive prefix over bcur[0..nbucket], whose bcur[b + 1]
// held bucket b's count, plus the number of items placed first).
__global__ __launch_bounds__(1024) void order_scan_kernel(
    const uint32_t *__restrict__ item_base, int64_t nq, const uint32_t *__restrict__ rm_q,
    const uint32_t *__restrict__ rm_r, const uint32_t *__restrict__ ikey,
    uint32_t *__restrict__ bcur, uint32_t nbucket, uint32_t *__restrict__ item_q,
    uint32_t *__restrict__ item_r)
{
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t carry_s;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t total = item_base[nq];
    if (tid == 0)
        carry_s = 0;
    __syncthreads();
    for (int64_t s = 0; s < total; s += 1024) {
        const int64_t i = s + tid;
        const uint32_t v = (i < total && ikey[i] == kNoBucket) ? 1u : 0u;
        const uint32_t incl = wave_inclusive_sum(v);
        if (lane == 63)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t before = carry_s;
        for (int w = 0; w < wave; ++w)
            before += wsum[w];
        if (v) {
            item_q[before + incl - 1] = rm_q[i];
            item_r[before + incl - 1] = rm_r[i];
        }
        __syncthreads();
        if (tid == 1023)
            carry_s = before + incl;
        __syncthreads();
    }
    const uint32_t placed = carry_s;
    __syncthreads();
    if (tid == 0)
        carry_s = placed;
    __syncthreads();
    for (int64_t s = 0; s <= (int64_t)nbucket; s += 1024) {
        const int64_t i = s + tid;
        const uint32_t v = i <= (int64_t)nbucket ? bcur[i] : 0u;
        const uint32_t incl = wave_inclusive_sum(v);
        if (lane == 63)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t before = carry_s;
        for (int w = 0; w < wave; ++w)
            before += wsum[w];
        if (i <= (int64_t)nbucket)
            bcur[i] = before + incl;
        __syncthreads();
        if (tid == 1023)
            carry_s = before + incl;
        __syncthreads();
    }
}

// The items with a bucket, each to the next free position of its bucket.
__global__ __launch_bounds__(256) void order_scatter_kernel(
    const uint32_t *__restrict__ item_base, int64_t nq, const uint32_t *__restrict__ rm_q,
    const uint32_t *__restrict__ rm_r, const uint32_t *__restrict__ ikey,
    uint32_t *__restrict__ bcur, uint32_t *__restrict__ item_q, uint32_t *__restrict__ item_r)
{
    const uint32_t total = item_base[nq];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)total)
        return;
    const uint32_t key = ikey[i];
    if (key == kNoBucket)
        return;
    const uint32_t pos = atomicAdd(&bcur[key], 1u);
    item_q[pos] = rm_q[i];
    item_r[pos] = rm_r[i];
}

// ---------------------------------------------------------------------------
// scan
// ---------------------------------------------------------------------------

struct ScanArgs {
    const float *queries;
    int d, m, dsub, nlist, nprobe, k, kw;
    int pg; // tables per group
    const float *centroids;
    const float *codebooks;
    const float *t1; // list term of the decomposed tables (PRE)
    const uint32_t *list_off;
    const uint8_t *codes;
    const int64_t *ids;
    const int32_t *probes;
    const uint32_t *qtotal, *qchunk, *item_base, *item_q, *item_r;
    uint32_t *qbound;
    uint32_t *counter;
    int64_t nq;
    float *part_d;
    uint32_t *part_p;
    float *out_d;
    int64_t *out_i;
    int ip;      // inner-product metric (tables of the run-time shape)
    float osign; // sign of the reported values: +1 squared L2, -1 inner product
    uint32_t wide_min; // pieces of at least this many entries get a replicated table
    const uint32_t *gbucket; // giant lists' buckets (region-aligned sequence), or nullptr
};

// A code row of M bytes read with the widest loads its size allows.
template <int M>
struct CodeRow {
    static constexpr int W = M / 4;
    uint32_t w[W];
    __device__ __forceinline__ void load(const uint8_t *p)
    {
        if constexpr (M % 16 == 0) {
#pragma unroll
            for (int i = 0; i < M / 16; ++i) {
                const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
                w[4 * i] = v.x;
                w[4 * i + 1] = v.y;
                w[4 * i + 2] = v.z;
                w[4 * i + 3] = v.w;
            }
        } else if constexpr (M % 8 == 0) {
#pragma unroll
            for (int i = 0; i < M / 8; ++i) {
                const uint2 v = reinterpret_cast<const uint2 *>(p)[i];
                w[2 * i] = v.x;
                w[2 * i + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i)
                w[i] = reinterpret_cast<const uint32_t *>(p)[i];
        }
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < W; ++i)
            w[i] = 0;
    }
};

// Sum of M values: j ascending, or (TREE, M a power of two) as a balanced
// pairwise tree, ((t0 + t1) + (t2 + t3)) + ...  The tree gives the same bits
// for any order t[k] = F_{k ^ s} (each node adds the same two values, and a
// float sum of two values does not depend on their order), which the
// replicated-table scan relies on.
template <int M, bool TREE>
__device__ __forceinline__ float sum_terms(float (&t)[M])
{
    if constexpr (TREE) {
#pragma unroll
        for (int w = 1; w < M; w *= 2)
#pragma unroll
            for (int j = 0; j < M; j += 2 * w)
                t[j] = t[j] + t[j + w];
        return t[0];
    } else {
        float r = t[0];
#pragma unroll
        for (int j = 1; j < M; ++j)
            r += t[j];
        return r;
    }
}

// R = sum_{j<M} F_j(code[j]) for the M code bytes in the M/4 words w.  The M
// table reads are all issued before the first add (they are independent), so
// one entry costs one LDS round trip rather than M of them.
template <int M, bool F16, bool TREE = false>
__device__ __forceinline__ float adc_words(const uint32_t *w, const void *lut)
{
    float t[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const uint32_t c = (w[j >> 2] >> (8 * (j & 3))) & 255u;
        t[j] = Table<F16>::get(lut, j * 256 + (int)c);
    }
    return sum_terms<M, TREE>(t);
}

// Run-time m (any m, byte loads when m % 4 != 0).
template <bool F16>
__device__ __forceinline__ float adc_rt(const uint8_t *__restrict__ code, int m, const void *lut)
{
    float r = 0.f;
    if ((m & 3) == 0) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(code);
        for (int j4 = 0; j4 < (m >> 2); ++j4) {
            const uint32_t word = w[j4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                r += Table<F16>::get(lut, (j4 * 4 + b) * 256 + ((word >> (8 * b)) & 255u));
        }
    } else {
        for (int j = 0; j < m; ++j)
            r += Table<F16>::get(lut, j * 256 + code[j]);
    }
    return r;
}

struct Piece {
    int32_t list;
    uint32_t b, e;
};

// Shapes: M > 0 compile-time m and dsub with the codebook in registers
// (G groups of 256 threads, each holding m/G sub-quantizers); M == 0 run-time
// m and dsub, codebook read from memory, G == 1.
//
// PRE (M > 0): decomposed tables.  With r = x - c_l,
//   F_j(v) = |r_j - C_j[v]|^2 = |r_j|^2 + t1[l][j][v] - 2 <x_j, C_j[v]>,
// t1[l][j][v] = |C_j[v]|^2 + 2 <c_l,j, C_j[v]> held per list in memory, and
// sum_j |r_j|^2 = |x - c_l|^2.  A thread keeps t2[jj] = -2 <x_j, C_j[v]> of
// its sub-quantizers (computed once per item, no codebook in registers); a
// table entry is t1 + t2, with |x - c_l|^2 (computed per piece) added to the
// entries of sub-quantizer 0, so that sum_j F_j is unchanged and the scan
// is the same.  The sums now cancel where |x - c_l - C(code)| is small
// against |x - c_l| and |C(code)|: float32 rounding of order 1e-7 of those
// norms, against the same order of the result in the difference form.
//
// IP: inner-product metric.  The scan ranks entries by the negated score,
// -(<x, c_l> + sum_j <x_j, C_j[v_j]>): table entries are -<x_j, C_j[v]>, and
// -<x, c_l> (computed per piece) is added to the entries of sub-quantizer 0.
// With a compile-time shape the query term is held in registers as in PRE
// (no list term, no codebook slice).  The reported values are negated back.
template <int M, int DSUB, int G, int NW, bool F16, bool SO, bool PRE, bool IP = false>
// Register budget: 128 VGPRs, i.e. four waves per SIMD, so that two
// workgroups of eight waves share a CU and their table-build and scan
// phases overlap.
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(4)))
void scan_items_kernel(ScanArgs a)
{
    constexpr int WAVES = 4 * G;
    constexpr int THREADS = 256 * G;
    constexpr int JG = M > 0 ? M / G : 1;
    extern __shared__ __align__(16) unsigned char smem[];

    const int d = a.d;
    const int m = M > 0 ? M : a.m;
    const int dsub = M > 0 ? DSUB : a.dsub;
    const int dpad = (d + 3) & ~3;
    const size_t tbytes = (size_t)m * 256 * (F16 ? 2 : 4);

    static_assert(!PRE || M > 0, "decomposed tables need a compile-time shape");
    static_assert(!IP || !PRE, "one table form at a time");
    // codebook slice in registers (difference form) or the query term (PRE,
    // IP with a compile-time shape)
    constexpr bool QT = M > 0 && (PRE || IP);

    // Row tables (m 8, float32 tables of the difference form or the inner
    // product; not the decomposed tables): both table buffers share a
    // 64 KiB region at LDS offset 0 of 256 rows (code value c) x 256 bytes,
    // buffer b in bytes [128 b, 128 b + 128) of every row, so that a table
    // address is (c << 8) | byte0 and one v_perm_b32 assembles it from the
    // code byte and a per-lane column byte.  In step t of an entry lane l
    // reads sub-quantizer j = s ^ t, s = (l & 31) >> 2 (it byte-permutes its
    // code row once so that the code of step t sits in byte t):
    //  * a group of up to 4 short pieces: table p in columns 8p .. 8p + 7,
    //    column 8p + j, one copy (a half-wave's lanes meet at most 4 to a
    //    bank, about what random 8-bit indices into one table give);
    //  * a long piece (at least a.wide_min entries) alone in the buffer: four
    //    copies, column 4j + r holding copy r of sub-quantizer j; lane l reads
    //    copy l & 3, i.e. column (l & 31) ^ 4t: the 32 lanes of a half-wave
    //    read 32 different banks whatever the codes ("Custom 8-bit floating
    //    point value format for reducing shared memory bank conflict in ANN
    //    search", bank-conflict analysis: random 8-bit indices into one table
    //    collide in the banks; replication spreads them).
    constexpr bool WIDE = M == 8 && !F16 && !PRE && G == 2;

    // Pieces (list, entry range) are handled in groups of PG: one barrier per
    // group, tables of the next group built while the current one is
    // scanned (two buffers of PG tables, two of PG residuals).
    const int PG = a.pg;
    // LDS layout by byte offsets from smem (pointer arithmetic on the LDS
    // array keeps every access a DS instruction).  Row tables come first, at
    // offset 0; otherwise the tables come last.
    const uint32_t o_base = WIDE ? 2u * (uint32_t)PG * (uint32_t)tbytes : 0u;
    const uint32_t o_misc = o_base + (1u + 2u * (uint32_t)PG) * dpad * 4u;
    const uint32_t o_pieces = o_misc + 64u;
    const uint32_t o_stage = (o_pieces + (uint32_t)a.nprobe * (uint32_t)sizeof(Piece) + 15u) & ~15u;
    const uint32_t o_tab = WIDE ? 0u : o_stage + WAVES * 512u;
    float *xs = reinterpret_cast<float *>(smem + o_base);
    // misc: [0] item [1] pieces [2] min bound [4 .. 4+WAVES) per-wave rank values
    uint32_t *misc = reinterpret_cast<uint32_t *>(smem + o_misc);
    uint32_t *pub = misc + 4;
    Piece *pieces = reinterpret_cast<Piece *>(smem + o_pieces);
    unsigned char *tab = smem + o_tab;
    auto rsbuf = [&](int b, int p) { return xs + dpad + (b * PG + p) * dpad; };
    auto tabp = [&](int b, int p) {
        if constexpr (WIDE)   // the row-table buffer's first byte, plus the table's columns
            return reinterpret_cast<void *>(tab + 128 * b + 32 * p);
        else
            return reinterpret_cast<void *>(tab + (size_t)(b * PG + p) * tbytes);
    };
    float *mk = reinterpret_cast<float *>(tab);
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (WAVES - 1) * 64 * NW);

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave number is the same in all lanes: say so, so that what derives
    // from it (piece rotation, loop bounds) is scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // thread -> (group g, codeword v); with WIDE a half-wave holds 16
    // threads of each group, and thread v holds sub-quantizer
    // g * JG + ((jj + v) % JG) in register slot jj, so that the 16-byte stores
    // of a half-wave's replicated entries cover all 32 banks
    const int v = WIDE ? ((tid & 15) | ((tid >> 5) << 4)) : (tid & 255);
    const int g = WIDE ? ((tid >> 4) & 1) : (tid >> 8);
    auto jsub = [&](int jj) { return WIDE ? g * JG + ((jj + v) & (JG - 1)) : g * JG + jj; };

    // byte selectors of v_perm_b32 that move code byte t ^ s of a lane's
    // 8-byte row into byte t (s = (l & 31) >> 2), low and high word
    uint32_t perm_lo = 0, perm_hi = 0;
    if constexpr (WIDE) {
        const uint32_t sx = (uint32_t)((lane & 31) >> 2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            perm_lo |= ((uint32_t)t ^ sx) << (8 * t);
            perm_hi |= ((uint32_t)(t + 4) ^ sx) << (8 * t);
        }
    }
    float cb[(M > 0 && !QT) ? JG * DSUB : 1];
    float t2[QT ? JG : 1];
    if constexpr (M > 0 && !QT) {
#pragma unroll
        for (int jj = 0; jj < JG; ++jj)
#pragma unroll
            for (int s = 0; s < DSUB; ++s)
                cb[jj * DSUB + s] = a.codebooks[((size_t)jsub(jj) * 256 + v) * DSUB + s];
    }

    // rs: the piece's residual (difference form) or, in rs[0], |x - c_l|^2
    // (PRE); list: the piece's list; wide: the replicated layout
    auto build = [&](const float *rs, int list, void *lut, bool wide) {
        if constexpr (IP && M > 0) {
            const float cst = rs[0];
#pragma unroll
            for (int jj = 0; jj < JG; ++jj) {
                const int j = jsub(jj);
                const float e = j == 0 ? t2[jj] + cst : t2[jj];
                unsigned char *row = reinterpret_cast<unsigned char *>(lut) + (v << 8);
                if (WIDE && wide)   // the four copies of (j, v): one 16-byte store
                    *reinterpret_cast<float4 *>(row + 16 * j) = make_float4(e, e, e, e);
                else if (WIDE)      // row table, one copy
                    *reinterpret_cast<float *>(row + 4 * j) = e;
                else
                    Table<F16>::put(lut, j * 256 + v, e);
            }
            (void)list;
        } else if constexpr (IP) {
            const float cst = rs[0];
            for (int j = 0; j < m; ++j) {
                const float *cw = a.codebooks + ((size_t)j * 256 + v) * dsub;
                float acc = 0.f;
                for (int s = 0; s < dsub; ++s)
                    acc = fmaf(xs[j * dsub + s], cw[s], acc);
                Table<F16>::put(lut, j * 256 + v, j == 0 ? cst - acc : -acc);
            }
            (void)list;
        } else if constexpr (PRE) {
            const float cst = rs[0];
            const float *t1l = a.t1 + (size_t)list * M * 256;
#pragma unroll
            for (int jj = 0; jj < JG; ++jj) {
                const int j = g * JG + jj;
                float e = t1l[j * 256 + v] + t2[jj];
                if (j == 0)
                    e += cst;
                Table<F16>::put(lut, j * 256 + v, e);
            }
        } else if constexpr (M > 0) {
#pragma unroll
            for (int jj = 0; jj < JG; ++jj) {
                const int j = jsub(jj);
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < DSUB; ++s) {
                    const float df = rs[j * DSUB + s] - cb[jj * DSUB + s];
                    acc = fmaf(df, df, acc);
                }
                unsigned char *row = reinterpret_cast<unsigned char *>(lut) + (v << 8);
                if (WIDE && wide)   // the four copies of (j, v): one 16-byte store
                    *reinterpret_cast<float4 *>(row + 16 * j) = make_float4(acc, acc, acc, acc);
                else if (WIDE)      // row table, one copy
                    *reinterpret_cast<float *>(row + 4 * j) = acc;
                else
                    Table<F16>::put(lut, j * 256 + v, acc);
            }
        } else {
            for (int j = 0; j < m; ++j) {
                const float *cw = a.codebooks + ((size_t)j * 256 + v) * dsub;
                float acc = 0.f;
                for (int s = 0; s < dsub; ++s) {
                    const float df = rs[j * dsub + s] - cw[s];
                    acc = fmaf(df, df, acc);
                }
                Table<F16>::put(lut, j * 256 + v, acc);
            }
        }
    };
    // Pieces of an item: nn narrow ones in slots [0, nn), taken PG to a group
    // (ngn groups), then nw wide ones, one per group, in slots counted down
    // from nprobe - 1.
    int nn = 0, nw = 0, ngn = 0;
    auto group_size = [&](int grp) {
        return grp >= ngn ? 1 : (nn - grp * PG < PG ? nn - grp * PG : PG);
    };
    auto group_wide = [&](int grp) { return grp >= ngn; };
    auto piece_index = [&](int grp, int p) {
        return grp >= ngn ? a.nprobe - 1 - (grp - ngn) : grp * PG + p;
    };
    // residuals x - c_l of the pieces of group grp into residual buffer b
    // (PRE: their squared norms, one wave per piece, into the buffer's first
    // word)
    auto residual_group = [&](int grp, int b) {
        const int pn = group_size(grp);
        if constexpr (PRE || IP) {
            // PRE: |x - c_l|^2; IP: -<x, c_l>
            for (int p = wave; p < pn; p += WAVES) {
                const float *c = a.centroids + (size_t)pieces[piece_index(grp, p)].list * d;
                float acc = 0.f;
                for (int t = lane; t < d; t += 64) {
                    if constexpr (IP) {
                        acc = fmaf(xs[t], c[t], acc);
                    } else {
                        const float df = xs[t] - c[t];
                        acc = fmaf(df, df, acc);
                    }
                }
#pragma unroll
                for (int sh = 32; sh >= 1; sh >>= 1)
                    acc += __shfl_xor(acc, sh);
                if (lane == 0)
                    rsbuf(b, p)[0] = IP ? -acc : acc;
            }
        } else {
            for (int i = tid; i < pn * d; i += THREADS) {
                const int p = i / d, t = i - p * d;
                const float *c = a.centroids + (size_t)pieces[piece_index(grp, p)].list * d;
                rsbuf(b, p)[t] = xs[t] - c[t];
            }
        }
    };
    auto build_group = [&](int grp, int b) {
        const int pn = group_size(grp);
        const bool wide = group_wide(grp);
        for (int p = 0; p < pn; ++p)
            build(rsbuf(b, p), pieces[piece_index(grp, p)].list, tabp(b, p), wide);
    };

    const uint32_t total_items = a.item_base[a.nq];
    for (;;) {
        if (tid == 0)
            misc[0] = atomicAdd(a.counter, 1u);
        __syncthreads();
        // values read from LDS that every lane shares: scalar registers, so
        // the control flow that depends on them stays uniform
        const uint32_t item = (uint32_t)__builtin_amdgcn_readfirstlane((int)misc[0]);
        if (item >= total_items)
            break;
        // the query and item number at this position of the scan order
        const int64_t q = (int64_t)__builtin_amdgcn_readfirstlane((int)a.item_q[item]);
        const uint32_t rk = (uint32_t)__builtin_amdgcn_readfirstlane((int)a.item_r[item]);
        const uint32_t first = a.item_base[q];
        const uint32_t count = a.item_base[q + 1] - first;
        const uint32_t slot = first + rk; // the item's partial top-k
        uint32_t start, stop;
        item_range(rk, a.qchunk[q], a.qtotal[q], &start, &stop);

        for (int t = tid; t < d; t += THREADS)
            xs[t] = a.queries[q * d + t];
        // pieces of [start, stop) of the query's concatenated probed lists
        if (wave == 0) {
            uint32_t acc = 0, cn = 0, cw = 0;
            // with giant lists (a.gbucket), the region-aligned sequence: small
            // lists in pass 0, giant ones from the next region in pass 1
            bool any_giant = false;
            for (int pass = 0; pass < (a.gbucket ? 2 : 1); ++pass) {
            if (pass == 1) {
                if (!any_giant)
                    break;
                acc = (uint32_t)region_round(acc);
            }
            for (int p0 = 0; p0 < a.nprobe; p0 += 64) {
                const int p = p0 + lane;
                int l = -1;
                uint32_t sz = 0, off = 0;
                bool giant = false;
                if (p < a.nprobe) {
                    l = a.probes[q * a.nprobe + p];
                    if ((unsigned)l < (unsigned)a.nlist) {
                        off = a.list_off[l];
                        sz = a.list_off[l + 1] - off;
                        giant = a.gbucket && a.gbucket[l] != kNoBucket;
                    }
                }
                any_giant = any_giant || wave_ballot(giant) != 0;
                // this pass's lists: their places in the sequence, their entries
                const bool mine = giant == (pass == 1);
                const uint32_t seq = mine ? (giant ? (uint32_t)region_round(sz) : sz) : 0u;
                sz = mine ? sz : 0u;
                const uint32_t incl = wave_inclusive_sum(seq);
                Piece pc;
                const uint32_t lo = acc + incl - seq;
                const bool take = piece_of(lo, lo + sz, start, stop, &pc.b, &pc.e);
                const bool wide = WIDE && take && pc.e - pc.b >= a.wide_min;
                const uint64_t mn = wave_ballot(take && !wide), mw = wave_ballot(wide);
                if (take) {
                    pc.list = l;
                    const int slot = wide ? a.nprobe - 1 - (int)(cw + mbcnt64(mw))
                                          : (int)(cn + mbcnt64(mn));
                    pieces[slot] = pc;
                }
                cn += (uint32_t)__popcll(mn);
                cw += (uint32_t)__popcll(mw);
                acc += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            }
            } // passes
            if (lane == 0) {
                misc[1] = cn;
                misc[3] = cw;
                misc[2] = a.qbound[q];
            }
            if (lane < WAVES)
                pub[lane] = float_order_key(INFINITY);
        }
        __syncthreads();
        nn = __builtin_amdgcn_readfirstlane((int)misc[1]);
        nw = __builtin_amdgcn_readfirstlane((int)misc[3]);
        ngn = (nn + PG - 1) / PG;
        if constexpr (QT) {
            // the query term of this thread's sub-quantizers and code value
            // (the codebook pointer made opaque here: loads the compiler
            // could hoist out of the item loop would keep the codebook
            // slice in registers again)
            uint64_t cbase = reinterpret_cast<uint64_t>(a.codebooks);
            __asm__ volatile("" : "+s"(cbase));
            using gfloat = __attribute__((address_space(1))) const float;
            gfloat *cbk = reinterpret_cast<gfloat *>(cbase);
#pragma unroll
            for (int jj = 0; jj < JG; ++jj) {
                const int j = jsub(jj);
                gfloat *cw = cbk + ((size_t)j * 256 + v) * DSUB;
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < DSUB; ++s)
                    acc = fmaf(xs[j * DSUB + s], cw[s], acc);
                t2[jj] = (PRE ? -2.f : -1.f) * acc;
                // materialised here (the compiler would otherwise recompute
                // it in every table build and keep the codebook values live)
                __asm__ volatile("" : "+v"(t2[jj]));
            }
        }

        // Union bound: wave w publishes its rk-th smallest value, rk =
        // ceil(k / WAVES); each wave then holds >= rk values <= the largest
        // published value, so together >= k: that maximum bounds the item's
        // k-th distance from above and filters every wave.
        WaveTopK<NW> sel;
        sel.init(a.k, reinterpret_cast<uint32_t *>(smem + o_stage) + wave * 128,
                 (a.k + WAVES - 1) / WAVES);
        float sink = INFINITY, published = INFINITY;

        const int ng = ngn + nw;
        if (ng > 0) {
            residual_group(0, 0);
            __syncthreads();
            build_group(0, 0);
            if (ng > 1)
                residual_group(1, 1);
            __syncthreads();
        }
        for (int grp = 0; grp < ng; ++grp) {
            if (grp + 1 < ng)
                build_group(grp + 1, (grp + 1) & 1);
            if (grp + 2 < ng)
                residual_group(grp + 2, grp & 1);
            if constexpr (!SO)
                sel.bound(read_bound(&misc[2]));
            const int pn = group_size(grp);
            const bool gwide = group_wide(grp);
            for (int pp = 0; pp < pn; ++pp) {
            const int pi = piece_index(grp, pp);
            void *lut = tabp(grp & 1, pp);
            // the wave that starts a piece rotates, so that a group of short
            // lists spreads over the waves
            const int rank = (wave - pi) & (WAVES - 1);
            Piece pc = pieces[pi];
            pc.list = __builtin_amdgcn_readfirstlane(pc.list);
            pc.b = (uint32_t)__builtin_amdgcn_readfirstlane((int)pc.b);
            pc.e = (uint32_t)__builtin_amdgcn_readfirstlane((int)pc.e);
            const uint32_t off = a.list_off[pc.list];
            const uint8_t *base = a.codes + (size_t)off * m;
            constexpr uint32_t STRIDE = 64 * WAVES;
            uint32_t i0 = pc.b + rank * 64;
            if constexpr (M > 0) {
                // Each lane takes EPL consecutive entries per step (32 bytes
                // of code rows at m <= 32: more bytes in flight per wave).
                // Full steps need no per-lane bounds and read one step
                // ahead; then at most one partial step.
                constexpr int EPL = M >= 32 ? 1 : 32 / M;
                constexpr uint32_t SPAN = 64 * EPL;          // entries per wave-step
                constexpr uint32_t WSTRIDE = SPAN * WAVES;   // entries per workgroup-step
                constexpr size_t PSTEP = (size_t)WSTRIDE * M;
                using Row = CodeRow<M * EPL>;
                // row tables: byte 0 of the address of step t (its column
                // and buffer half), four steps per word
                uint32_t zlo = 0, zhi = 0;
                if constexpr (WIDE) {
                    const uint32_t l5 = (uint32_t)(lane & 31), sx = l5 >> 2;
                    const uint32_t col0 =
                        (uint32_t)(reinterpret_cast<unsigned char *>(lut) - tab);  // 128 b + 32 p
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const uint32_t z = gwide ? ((col0 & 128u) | ((l5 << 2) ^ (uint32_t)(t << 4)))
                                                 : (col0 | (((uint32_t)t ^ sx) << 2));
                        if (t < 4)
                            zlo |= z << (8 * t);
                        else
                            zhi |= z << (8 * (t - 4));
                    }
                }
                // FULL: every entry of the step exists (no per-lane bound)
                // The lane's EPL entries of a step are all formed first (their
                // table reads overlap) and then tested against the filter
                // threshold with one comparison of their minimum: the usual
                // step has no value under it in any lane and pushes nothing.
                // Otherwise each entry is pushed in order, as one at a time
                // would be (the threshold only falls in between, so a skipped
                // step would have pushed nothing either).
                auto consume = [&](auto full, const Row &row, uint32_t first, uint32_t limit) {
                    constexpr bool FULL = decltype(full)::value;
                    float r[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        if constexpr (WIDE) {
                            // code of sub-quantizer t ^ s into byte t (s = (l & 31) >> 2)
                            const uint32_t lo = row.w[2 * e], hi = row.w[2 * e + 1];
                            const uint32_t nl = __builtin_amdgcn_perm(hi, lo, perm_lo);
                            const uint32_t nh = __builtin_amdgcn_perm(hi, lo, perm_hi);
                            float tv[8];
#pragma unroll
                            for (int t = 0; t < 8; ++t) {
                                // address = (c << 8) | z_t: byte 1 <- code byte t & 3 of
                                // the permuted word, byte 0 <- byte t & 3 of z, bytes 2-3 <- 0
                                const uint32_t SEL = (uint32_t)(t & 3) |
                                                         ((uint32_t)(4 + (t & 3)) << 8) |
                                                         (0x0cu << 16) | (0x0cu << 24);
                                const uint32_t ad = __builtin_amdgcn_perm(t < 4 ? nl : nh,
                                                                          t < 4 ? zlo : zhi, SEL);
                                // the row tables sit at LDS address 0: read through an
                                // LDS pointer made from the address itself (a DS read with
                                // no add for the array base)
                                tv[t] = *reinterpret_cast<const __attribute__((address_space(3))) float *>(
                                    (uintptr_t)ad);
                            }
                            r[e] = sum_terms<8, true>(tv);
                        } else {
                            r[e] = adc_words<M, F16>(row.w + e * (M / 4), lut);
                        }
                        if constexpr (!FULL)
                            r[e] = first + e < limit ? r[e] : INFINITY;
                    }
                    if constexpr (SO) {
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            sink = fminf(sink, r[e]);
                    } else {
                        float mn = r[0];
#pragma unroll
                        for (int e = 1; e < EPL; ++e)
                            mn = fminf(mn, r[e]);
                        if (sel.any_below(mn)) {
#pragma unroll
                            for (int e = 0; e < EPL; ++e)
                                sel.push(r[e], off + first + e);
                        }
                    }
                };
                uint32_t s0 = pc.b + rank * SPAN;
                const uint8_t *p = base + ((size_t)s0 + (size_t)lane * EPL) * M;
                if (s0 + SPAN <= pc.e) {
                    Row cur;
                    cur.load(p);
                    for (;;) {
                        const uint32_t n0 = s0 + WSTRIDE;
                        const bool more = n0 + SPAN <= pc.e;
                        // unconditional (the current step again when there is
                        // no next one), so that the wait before the scan of
                        // this step leaves the next step's load in flight
                        Row nxt;
                        nxt.load(more ? p + PSTEP : p);
                        // keep the next step's loads ahead of this step's scan:
                        // the scheduler would otherwise sink them below it into
                        // the current step's registers, and every step would
                        // wait for its own load with nothing in flight
                        __builtin_amdgcn_sched_barrier(0);
                        consume(std::true_type{}, cur, s0 + lane * EPL, 0u);
                        s0 = n0;
                        p += PSTEP;
                        if (!more)
                            break;
                        cur = nxt;
                    }
                }
                if (s0 < pc.e) {
                    const uint32_t first = s0 + lane * EPL;
                    Row cur;
                    if (first + EPL <= pc.e) {
                        cur.load(p);
                    } else {
                        cur.zero();
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            if (first + e < pc.e)
#pragma unroll
                                for (int wi = 0; wi < M / 4; ++wi)
                                    cur.w[e * (M / 4) + wi] =
                                        reinterpret_cast<const uint32_t *>(p + e * M)[wi];
                    }
                    consume(std::false_type{}, cur, first, pc.e);
                }
            } else {
                for (; i0 < pc.e; i0 += STRIDE) {
                    const uint32_t i = i0 + lane;
                    const float r =
                        i < pc.e ? adc_rt<F16>(base + (size_t)i * m, m, lut) : INFINITY;
                    if constexpr (SO)
                        sink = fminf(sink, r);
                    else
                        sel.push(r, off + i);
                }
            }
            } // pieces of the group
            if constexpr (!SO) {
                // union bound, once per group (per step it cost more than it
                // saved): the wave publishes its rank value; the maximum over
                // the waves enters the item's bound (misc[2], read by every
                // wave after the barrier) and the query's.  A wave whose
                // current value tid 0 does not see yet counts with an older,
                // larger one: still a bound.
                if (sel.part < published) {
                    published = sel.part;
                    if (lane == 0)
                        pub[wave] = float_order_key(published);
                }
                publish_bound(&misc[2], sel.kth);
                if (tid == 0) {
                    uint32_t mx = 0;
                    for (int w = 0; w < WAVES; ++w)
                        mx = mx > pub[w] ? mx : pub[w];
                    const uint32_t mine = misc[2] < mx ? misc[2] : mx;
                    const uint32_t old = atomicMin(&a.qbound[q], mine);
                    atomicMin(&misc[2], old < mine ? old : mine);
                }
            }
            __syncthreads();
        }

        if constexpr (SO) {
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1)
                sink = fminf(sink, __shfl_xor(sink, s));
            if (tid == 0)
                a.out_d[q * a.k] = sink;
            __syncthreads();
        } else {
            sel.flush();
            merge_waves<NW, WAVES>(sel, mk, mv);
            if (wave == 0) {
                if (count == 1) {
#pragma unroll
                    for (int r = 0; r < NW; ++r) {
                        const int e = r * 64 + lane;
                        if (e < a.k) {
                            a.out_d[q * a.k + e] = a.osign * sel.wk[r];
                            a.out_i[q * a.k + e] =
                                sel.wv[r] == kSentinel ? -1 : a.ids[sel.wv[r]];
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < NW; ++r) {
                        const size_t e = (size_t)slot * (64 * NW) + r * 64 + lane;
                        a.part_d[e] = sel.wk[r];
                        a.part_p[e] = sel.wv[r];
                    }
                    // the item's own k-th value (merged over its waves) bounds
                    // the query's: its items that start later filter against
                    // it instead of the looser union bound
                    publish_bound(&a.qbound[q], sel.kth);
                }
            }
            __syncthreads(); // merge scratch aliases the tables
        }
    }
}

// ---------------------------------------------------------------------------
// merge of the partial top-k of a query's items
// ---------------------------------------------------------------------------

template <int NW>
__global__ __launch_bounds__(256) void merge_items_kernel(const uint32_t *__restrict__ item_base,
                                                          const float *__restrict__ part_d,
                                                          const uint32_t *__restrict__ part_p,
                                                          const int64_t *__restrict__ ids, int k,
                                                          float osign, float *__restrict__ out_d,
                                                          int64_t *__restrict__ out_i)
{
    __shared__ __align__(16) float mk[3 * 64 * NW];
    __shared__ __align__(16) uint32_t mv[3 * 64 * NW];
    const int64_t q = blockIdx.x;
    const uint32_t first = item_base[q], count = item_base[q + 1] - first;
    if (count <= 1)
        return;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    WaveTopK<NW> sel; // merges sorted arrays only: no staging buffer
    sel.init(k, nullptr);
    for (uint32_t it = wave; it < count; it += 4)
        sel.merge_sorted(part_d + (size_t)(first + it) * 64 * NW,
                         part_p + (size_t)(first + it) * 64 * NW);
    merge_waves<NW, 4>(sel, mk, mv);
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int e = r * 64 + lane;
            if (e < k) {
                out_d[q * k + e] = osign * sel.wk[r];
                out_i[q * k + e] = sel.wv[r] == kSentinel ? -1 : ids[sel.wv[r]];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int nw_of(int k)
{
    int nw = 1;
    while (nw * 64 < k)
        nw *= 2;
    return nw;
}

static int cu_count()
{
    static int n = 0;
    if (!n) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
    }
    return n;
}

// Pieces of at least this many entries get the replicated table of the m 8
// scan (its build writes four copies of every entry, which a short piece's
// lookups do not repay); IVFPQ_SCAN_WIDE_MIN overrides it, read at every
// search (tuning, and tests that force either table form).
static uint32_t wide_min_entries()
{
    const char *e = std::getenv("IVFPQ_SCAN_WIDE_MIN");
    const long long x = e ? std::atoll(e) : 4096;
    return x < 1 ? 1u : (x > 0x7FFFFFFFll ? 0x7FFFFFFFu : (uint32_t)x);
}

// Tables per group: as many as 32 KiB holds (1..8), two groups resident.
static int tables_per_group(int m, bool f16)
{
    const int t = 32768 / (m * 256 * (f16 ? 2 : 4));
    return t < 1 ? 1 : (t > 8 ? 8 : t);
}

size_t scan_lds_bytes(int d, int m, int nprobe, bool f16, int nw, int g)
{
    const int pg = tables_per_group(m, f16);
    const size_t dpad = (size_t)((d + 3) & ~3);
    const size_t table = 2 * (size_t)pg * m * 256 * (f16 ? 2 : 4);
    const size_t merge = (size_t)(4 * g - 1) * 64 * nw * 8;
    const size_t o_tab =
        ((dpad * 4 * (1 + 2 * (size_t)pg) + 64 + (size_t)nprobe * sizeof(Piece) + 15) &
         ~(size_t)15) +
        (size_t)4 * g * 512;
    return o_tab + (table > merge ? table : merge);
}

template <int M, int DSUB, int G, int NW, bool F16, bool SO, bool PRE = false, bool IP = false>
static hipError_t scan_variant(const ScanArgs &a, const SearchPlan &pl, hipStream_t stream)
{
    auto kern = scan_items_kernel<M, DSUB, G, NW, F16, SO, PRE, IP>;
    const size_t lds = scan_lds_bytes(a.d, a.m, a.nprobe, F16, NW, G);
    if (lds > 160 * 1024)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256 * G, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t grid = scan_grid(per_cu, cu_count(), pl.max_items);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256 * G), lds, stream, a);
    return hipGetLastError();
}

template <int M, int DSUB, int G, int NW>
static hipError_t scan_shape(const ScanArgs &a, const SearchPlan &pl, int f16, int so,
                             hipStream_t stream)
{
    if (a.ip) // inner product: float32 tables
        return so ? scan_variant<M, DSUB, G, NW, false, true, false, true>(a, pl, stream)
                  : scan_variant<M, DSUB, G, NW, false, false, false, true>(a, pl, stream);
    if constexpr (M == 16 && DSUB == 8) {
        if (a.t1) {
            if (so)
                return f16 ? scan_variant<M, DSUB, G, NW, true, true, true>(a, pl, stream)
                           : scan_variant<M, DSUB, G, NW, false, true, true>(a, pl, stream);
            return f16 ? scan_variant<M, DSUB, G, NW, true, false, true>(a, pl, stream)
                       : scan_variant<M, DSUB, G, NW, false, false, true>(a, pl, stream);
        }
    }
    if (so)
        return f16 ? scan_variant<M, DSUB, G, NW, true, true>(a, pl, stream)
                   : scan_variant<M, DSUB, G, NW, false, true>(a, pl, stream);
    return f16 ? scan_variant<M, DSUB, G, NW, true, false>(a, pl, stream)
               : scan_variant<M, DSUB, G, NW, false, false>(a, pl, stream);
}

template <int NW>
static hipError_t scan_nw(const ScanArgs &a, const SearchPlan &pl, int f16, int so,
                          hipStream_t stream)
{
    if (a.m == 4 && a.dsub == 8)
        return scan_shape<4, 8, 1, NW>(a, pl, f16, so, stream);
    if (a.m == 16 && a.dsub == 8)
        return scan_shape<16, 8, 2, NW>(a, pl, f16, so, stream);
    if (a.m == 32 && a.dsub == 3)
        return scan_shape<32, 3, 2, NW>(a, pl, f16, so, stream);
    if (a.m == 8 && a.dsub == 12)
        return scan_shape<8, 12, 2, NW>(a, pl, f16, so, stream);
    return scan_shape<0, 0, 1, NW>(a, pl, f16, so, stream);
}

template <int NW>
static hipError_t merge_nw(const SearchArgs &s, const SearchPlan &pl, const DeviceIndex &ix,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(merge_items_kernel<NW>, dim3((unsigned)s.nq), dim3(256), 0, stream,
                       pl.item_base, pl.part_d, pl.part_p, ix.ids, s.k,
                       s.metric ? -1.f : 1.f, s.out_d, s.out_i);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// list term of the decomposed tables (index load)
// ---------------------------------------------------------------------------

// t1[l][j][c] = |C_j[c]|^2 + 2 <c_l,j, C_j[c]> in double precision, rounded
// once; one thread per entry.
__global__ __launch_bounds__(256) void list_term_kernel(const float *__restrict__ centroids,
                                                        const float *__restrict__ codebooks,
                                                        int nlist, int m, int dsub,
                                                        float *__restrict__ t1)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)nlist * m * 256;
    if (i >= total)
        return;
    const int c = (int)(i & 255);
    const int j = (int)((i >> 8) % m);
    const int64_t l = (i >> 8) / m;
    const float *cw = codebooks + ((size_t)j * 256 + c) * dsub;
    const float *cl = centroids + (size_t)l * m * dsub + (size_t)j * dsub;
    double acc = 0.0;
    for (int s = 0; s < dsub; ++s)
        acc += (double)cw[s] * ((double)cw[s] + 2.0 * (double)cl[s]);
    t1[i] = (float)acc;
}

// The shape with the compiled decomposed-table scan (m 16, dsub 8), while the
// list term stays small enough to be cache resident (<= 64 MiB).
bool scan_uses_list_term(int m, int d, int nlist)
{
    return m == 16 && d == 128 && (size_t)nlist * m * 256 * 4 <= ((size_t)64 << 20);
}

hipError_t launch_list_term(const DeviceIndex &ix, hipStream_t stream)
{
    if (!ix.t1 || ix.nlist == 0)
        return hipSuccess;
    const int64_t total = (int64_t)ix.nlist * ix.m * 256;
    hipLaunchKernelGGL(list_term_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, ix.centroids, ix.codebooks, ix.nlist, ix.m, ix.d / ix.m, ix.t1);
    return hipGetLastError();
}

// Whether a search over this index uses the giant-list order and the
// region-aligned sequences: the index has giant lists and a query's padded
// sequence (at most nprobe + 1 regions of padding) stays below 2^32 entries.
static bool giant_order(const DeviceIndex &ix, int nprobe)
{
    return ix.nbucket > 0 && ix.gbucket &&
           (uint64_t)ix.ntotal + (uint64_t)(nprobe + 1) * kRegion < (1ull << 32);
}

hipError_t launch_plan(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                       hipStream_t stream)
{
    const unsigned blocks = (unsigned)((s.nq + 15) / 16); // a wave per query
    const bool reorder = giant_order(ix, s.nprobe) && pl.bcur && pl.rm_q && pl.rm_r && pl.ikey;
    hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(1024), 0, stream, s.probes, s.nprobe, s.nq,
                       ix.nlist, ix.list_off, pl.target, pl.imax, pl.qtotal, pl.qchunk, pl.qcount,
                       pl.qbound, pl.counter, pl.prof, reorder ? ix.gbucket : nullptr,
                       reorder ? pl.bcur : nullptr, ix.nbucket);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(item_scan_kernel, dim3(1), dim3(1024), 0, stream, pl.qcount, s.nq,
                       pl.item_base, pl.prof);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(rank_count_kernel, dim3(pl.imax), dim3(1024), 0, stream, pl.qcount, s.nq,
                       pl.rank_n);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(rank_order_kernel, dim3(pl.imax), dim3(1024), 0, stream, pl.qcount, s.nq,
                       pl.rank_n, reorder ? pl.rm_q : pl.item_q, reorder ? pl.rm_r : pl.item_r);
    e = hipGetLastError();
    if (e != hipSuccess || !reorder)
        return e;
    const unsigned iblocks = (unsigned)((pl.max_items + 255) / 256);
    // a wave per item, at most 8,192 waves looping over the items
    const int64_t kb = (pl.max_items + 3) / 4;
    const unsigned kblocks = (unsigned)(kb < 2048 ? kb : 2048);
    hipLaunchKernelGGL(item_key_kernel, dim3(kblocks), dim3(256), 0, stream, pl.item_base, s.nq,
                       pl.rm_q, pl.rm_r, pl.qchunk, pl.qtotal, s.probes, s.nprobe, ix.nlist,
                       ix.list_off, ix.gbucket, pl.ikey, pl.bcur);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(order_scan_kernel, dim3(1), dim3(1024), 0, stream, pl.item_base, s.nq,
                       pl.rm_q, pl.rm_r, pl.ikey, pl.bcur, ix.nbucket, pl.item_q, pl.item_r);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(order_scatter_kernel, dim3(iblocks), dim3(256), 0, stream, pl.item_base,
                       s.nq, pl.rm_q, pl.rm_r, pl.ikey, pl.bcur, pl.item_q, pl.item_r);
    return hipGetLastError();
}

hipError_t launch_scan(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                       hipStream_t stream)
{
    if (s.nq == 0)
        return hipSuccess;
    ScanArgs a;
    a.queries = s.queries;
    a.d = ix.d;
    a.m = ix.m;
    a.dsub = ix.d / ix.m;
    a.nlist = ix.nlist;
    a.nprobe = s.nprobe;
    a.k = s.k;
    a.kw = 64 * nw_of(s.k);
    a.pg = tables_per_group(ix.m, s.lut != 0);
    a.centroids = ix.centroids;
    a.codebooks = ix.codebooks;
    // decomposed tables for squared L2 with float32 tables only: binary16
    // storage would round entries the size of |x - c_l|^2 instead of F_j
    a.t1 = (s.metric || s.lut) ? nullptr : ix.t1;
    a.list_off = ix.list_off;
    a.codes = ix.codes;
    a.ids = ix.ids;
    // the plan's layout (launch_plan: the same condition and workspace)
    a.gbucket = giant_order(ix, s.nprobe) && pl.bcur ? ix.gbucket : nullptr;
    a.probes = s.probes;
    a.qtotal = pl.qtotal;
    a.qchunk = pl.qchunk;
    a.item_base = pl.item_base;
    a.item_q = pl.item_q;
    a.item_r = pl.item_r;
    a.qbound = pl.qbound;
    a.counter = pl.counter;
    a.nq = s.nq;
    a.part_d = pl.part_d;
    a.part_p = pl.part_p;
    a.out_d = s.out_d;
    a.out_i = s.out_i;
    a.ip = s.metric;
    a.osign = s.metric ? -1.f : 1.f;
    a.wide_min = wide_min_entries();
    switch (nw_of(s.k)) {
    case 1: return scan_nw<1>(a, pl, s.lut, s.mode, stream);
    case 2: return scan_nw<2>(a, pl, s.lut, s.mode, stream);
    case 4: return scan_nw<4>(a, pl, s.lut, s.mode, stream);
    case 8: return scan_nw<8>(a, pl, s.lut, s.mode, stream);
    default: return scan_nw<16>(a, pl, s.lut, s.mode, stream);
    }
}

hipError_t launch_merge(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                        hipStream_t stream)
{
    if (s.nq == 0)
        return hipSuccess;
    switch (nw_of(s.k)) {
    case 1: return merge_nw<1>(s, pl, ix, stream);
    case 2: return merge_nw<2>(s, pl, ix, stream);
    case 4: return merge_nw<4>(s, pl, ix, stream);
    case 8: return merge_nw<8>(s, pl, ix, stream);
    default: return merge_nw<16>(s, pl, ix, stream);
    }
}

} // namespace ivfpq
