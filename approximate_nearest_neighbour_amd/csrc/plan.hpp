// Work-plan arithmetic of a search, shared by the device plan and scan
// kernels and the host (the host launcher, and a CPU test that checks it).
//
// "Billion-scale similarity search with GPUs", IVFADC section: the (query,
// list) pairs are independent, a first k-selection reduces each piece of work
// to k partial results and a second one reduces a query's partials to k.
// Here a query's probed lists are laid end to end (in probe order) into one
// sequence of E entries, cut into work items of `chunk` entries; an item
// meets each list in at most one contiguous piece.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ivfpq {

// Entries per item and item count of a query with `total` probed entries:
// chunk = max(target, ceil(total / imax)) rounded up to a multiple of
// `align`, so a query never has more than imax items whatever its lists'
// sizes; a query with no entries still gets one (empty) item, which writes
// its padded result.
struct QueryPlan {
    uint32_t chunk, count;
};

__host__ __device__ inline QueryPlan plan_query(uint32_t total, uint32_t target, uint32_t imax,
                                                uint32_t align = 1)
{
    uint32_t chunk = (uint32_t)(((uint64_t)total + imax - 1) / imax);
    chunk = chunk > target ? chunk : target;
    // a multiple of `align` (item boundaries on region boundaries)
    chunk = (uint32_t)(((uint64_t)chunk + align - 1) / align * align);
    const uint32_t count = (uint32_t)(((uint64_t)total + chunk - 1) / chunk);
    return QueryPlan{chunk, count > 0 ? count : 1u};
}

// Entry range [start, stop) of item number `i` (0-based within its query).
__host__ __device__ inline void item_range(uint32_t i, uint32_t chunk, uint32_t total,
                                           uint32_t *start, uint32_t *stop)
{
    const uint64_t s = (uint64_t)i * chunk;
    const uint64_t e = s + chunk;
    *start = (uint32_t)(s < total ? s : total);
    *stop = (uint32_t)(e < total ? e : total);
}

// The piece of a list that occupies [lo, hi) of the query's sequence inside
// an item [start, stop): entries [*b, *e) of the list.  False if they do not
// meet (or the list is empty).
__host__ __device__ inline bool piece_of(uint32_t lo, uint32_t hi, uint32_t start, uint32_t stop,
                                         uint32_t *b, uint32_t *e)
{
    if (hi <= lo || lo >= stop || hi <= start)
        return false;
    *b = (start > lo ? start : lo) - lo;
    *e = (stop < hi ? stop : hi) - lo;
    return true;
}

// Work items per query: as many as a 1 GiB partial top-k buffer holds, 2 to
// 64 (kw = k rounded up to 64 times a power of two).  With heavy-tailed list
// sizes a query that probes the largest lists holds many times the average
// work; more items keep the largest item small against the work per
// workgroup (the persistent workgroups otherwise wait on one long item).
inline uint32_t items_per_query(int64_t nq, int kw)
{
    const double per = (1024.0 * 1024 * 1024) / ((double)(nq > 0 ? nq : 1) * kw * 8);
    if (per < 2)
        return 2;
    return per > 64 ? 64u : (uint32_t)per;
}

// Persistent grid of the scan: every resident workgroup, but never more
// workgroups than there can be items (an idle workgroup only takes the
// counter once and leaves).
inline int64_t scan_grid(int per_cu, int cus, int64_t max_items)
{
    int64_t g = (int64_t)(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (g > max_items)
        g = max_items > 0 ? max_items : 1;
    return g;
}

} // namespace ivfpq
