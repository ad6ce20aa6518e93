// Internal interface between the C-ABI host code (api.hip) and the kernel
// launchers (kernels_*.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ivfpq {

// Device-resident index.  Positions (row numbers in the list-major code
// array) are 32-bit: ntotal < 2^32, and 0xFFFFFFFF is the empty sentinel.
struct DeviceIndex {
    int d = 0, nlist = 0, m = 0;
    int64_t ntotal = 0;
    int64_t max_list = 0;
    float *centroids = nullptr;  // [nlist][d]
    int d4 = 0;                  // K-steps of the coarse MFMA: ceil(d/4) padded to 8/16/24/32
    int nblk = 0;                // 16-centroid blocks, a multiple of 4 (whole 64-wide tiles)
    float *cblk = nullptr;       // centroids in MFMA B-operand order [nblk][d4/4][64][4]
    float *cnorm_pad = nullptr;  // [nblk * 16] |c_l|^2, +inf past nlist
    // centroids as three bfloat16 parts for the bf16x6 coarse kernel (only
    // where it runs: d <= 96, nlist >= 16,384; else nullptr):
    // [nblk/4 tiles][4][x6_kb][3][64][8]
    uint16_t *cx6 = nullptr;
    int x6_kb = 0;               // 32-dim K-blocks: ceil(d / 32)
    float *codebooks = nullptr;  // [m][256][dsub]
    uint32_t *list_off = nullptr; // [nlist + 1]
    uint8_t *codes = nullptr;    // [ntotal][m]
    int64_t *ids = nullptr;      // [ntotal]
    // list term of the decomposed tables (only for the shapes and sizes that
    // use them, else nullptr): t1[l][j][c] = |C_j[c]|^2 + 2 <c_l,j, C_j[c]>
    float *t1 = nullptr;         // [nlist][m][256]
    // Regions of the giant lists (kGiantList entries or more): list l's
    // region j (entries [j kRegion, (j + 1) kRegion)) is bucket gbucket[l] + j
    // of the scan order (kNoBucket for the other lists); nbucket in all.
    uint32_t *gbucket = nullptr; // [nlist], nullptr when nbucket == 0
    uint32_t nbucket = 0;
};

constexpr uint32_t kGiantList = 1u << 20;
constexpr uint32_t kRegion = 1u << 19;
constexpr uint32_t kNoBucket = 0xFFFFFFFFu;

struct SearchArgs {
    const float *queries;
    int64_t nq;
    int nprobe;
    int k;
    int lut;  // 0 = float32 table, 1 = binary16 table
    int mode; // 0 normal, 1 scan only
    int chunk_len;
    float *out_d;
    int64_t *out_i;
    int metric = 0;  // 0 squared L2, 1 inner product
    int32_t *probes; // [nq][nprobe] (workspace or caller buffer)
    float *probe_d;  // [nq][nprobe] or nullptr
};

// Work plan of one search (device workspace): per query the total probed
// entries, the entries per work item, the item count and its exclusive
// prefix (item_base[nq] = number of items), a shared top-k bound, the item
// counter of the persistent scan, and the partial top-k of every item.
struct SearchPlan {
    uint32_t target = 0;   // minimum entries per work item
    uint32_t imax = 0;     // maximum work items per query
    int64_t max_items = 0; // nq * imax
    uint32_t *qtotal = nullptr, *qchunk = nullptr, *qcount = nullptr, *item_base = nullptr;
    uint32_t *qbound = nullptr, *counter = nullptr;
    // scan order of the items, rank-major: position i holds query item_q[i]'s
    // item number item_r[i]; rank_n[r] = queries with more than r items
    uint32_t *item_q = nullptr, *item_r = nullptr, *rank_n = nullptr;
    // with giant lists: the rank-major order (rm_q, rm_r), each item's bucket
    // (ikey) and the buckets' cursors (bcur, nbucket + 1 words); item_q and
    // item_r then receive the final order (scan_order_kernel)
    uint32_t *rm_q = nullptr, *rm_r = nullptr, *ikey = nullptr, *bcur = nullptr;
    float *part_d = nullptr;   // [max_items][kw]
    uint32_t *part_p = nullptr; // [max_items][kw]
    // when not null: [0] += entries of the probed lists, [1] += work items
    // (profiling)
    unsigned long long *prof = nullptr;
};

// Each launcher enqueues on `stream` and returns the launch status.
// ip: rank the lists by -<x, c_l> (inner-product metric) instead of |x - c_l|^2
hipError_t launch_coarse(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                         void *ws, int32_t *probes, float *probe_d, hipStream_t stream,
                         bool ip = false);
hipError_t launch_coarse_valu(const DeviceIndex &ix, const float *queries, int64_t nq,
                              int nprobe, int32_t *probes, float *probe_d, hipStream_t stream,
                              bool ip = false);
size_t coarse_ws_bytes(const DeviceIndex &ix, int64_t nq, int nprobe);
hipError_t launch_centroid_blocks(const DeviceIndex &ix, hipStream_t stream);
// whether an index of this shape gets the bfloat16 parts of its centroids
// (the bf16x6 coarse kernel: d <= 96, nlist >= 16,384)
bool coarse_uses_x6(int d, int nlist);
hipError_t launch_plan(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                       hipStream_t stream);
// Decomposed tables for this index? (compiled shape, list term small enough
// to stay cache resident)
bool scan_uses_list_term(int m, int d, int nlist);
hipError_t launch_list_term(const DeviceIndex &ix, hipStream_t stream);
// PQ codes of n vectors (x [n][d]) given their lists (index building)
hipError_t launch_encode(const DeviceIndex &ix, const float *x, int64_t n, const int32_t *lists,
                         uint8_t *codes, hipStream_t stream);
// list-major layout of n encoded entries (index building): counts [nlist],
// keys_out, perm_in, perm_out [n] scratch; sort_tmp == nullptr asks for the
// sort's scratch size in *sort_tmp_bytes
hipError_t launch_list_layout(const int32_t *lists, int64_t n, int nlist, int m,
                              const uint8_t *codes_in, const int64_t *ids_in, uint32_t *counts,
                              int32_t *keys_out, int32_t *perm_in, int32_t *perm_out,
                              void *sort_tmp, size_t *sort_tmp_bytes, uint8_t *codes_out,
                              int64_t *ids_out, hipStream_t stream);
// k-means update step: centers = means of their assigned vectors (sums [k][d]
// double and counts [k] are scratch / output)
hipError_t launch_kmeans_update(const float *x, int64_t n, int d, const int32_t *assign, int k,
                                double *sums, int32_t *counts, float *centers, hipStream_t stream);
hipError_t launch_scan(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                       hipStream_t stream);
hipError_t launch_merge(const DeviceIndex &ix, const SearchArgs &s, const SearchPlan &pl,
                        hipStream_t stream);
size_t scan_lds_bytes(int d, int m, int nprobe, bool f16, int nw, int g);
hipError_t launch_luts(const DeviceIndex &ix, const float *queries, int64_t nq,
                       const int32_t *probes, int nprobe, int lut, float *out, hipStream_t stream);
hipError_t launch_stream_read(const void *data, size_t bytes, uint32_t *sink, int sink_words,
                              hipStream_t stream);
hipError_t launch_select(const float *keys, int64_t rows, int64_t n, int k, float *out_d,
                         int32_t *out_pos, hipStream_t stream);

// Flat bfloat16 database on the device: rows padded to dp = 32*ceil(d/32)
// values (zeros) and to npad = 64*ceil(n/64) rows (zero rows, norm +inf).
struct FlatDevice {
    int d = 0, dp = 0;
    int64_t n = 0, npad = 0;
    uint16_t *vec = nullptr; // [npad][dp]
    float *norms = nullptr;  // [npad] |y|^2 in float32
    float ymax = 0.f;        // max |y|^2 over the rows
};

// Shape of one flat search: 64-row tiles, segments of `seg` tiles (16 slot
// minima per query each), and the candidate capacity per query.
struct FlatPlan {
    int64_t ntile = 0;
    int seg = 1;
    int64_t nseg = 0, nslot = 0;
    uint32_t cap = 0;
    int dp = 0; // padded row length (bf16)
};

FlatPlan flat_plan(int64_t n, int k, int64_t nq, int dp);
size_t flat_ws_bytes(const FlatPlan &p, int64_t nq);
hipError_t launch_flat_pack(const uint16_t *src, int64_t n, int d, int dp, int64_t npad,
                            uint16_t *dst, float *norms, hipStream_t stream);
// stage 0: clear + slot minima, 1: k-th minimum, 2: collect, 3: select, 4: fallback
hipError_t launch_flat_stage(const FlatDevice &fx, const uint16_t *queries, int64_t nq, int k,
                             const FlatPlan &p, void *ws, float *out_d, int64_t *out_i, int stage,
                             hipStream_t stream);

// Largest k / nprobe the selection supports.
constexpr int kMaxK = 1024;

} // namespace ivfpq
