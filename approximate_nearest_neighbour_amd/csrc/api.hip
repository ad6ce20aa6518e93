// C-ABI host side of the IVF-PQ library: argument and file validation (host
// only), index upload, workspace, kernel sequencing on the caller's stream,
// per-kernel event timing.  Declarations and conventions: include/ivfpq.h.
#include "../../include/ivfpq.h"
#include "internal.hpp"
#include "plan.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

using namespace ivfpq;

namespace {

thread_local std::string g_err;

ivfpq_status fail(ivfpq_status s, const std::string &msg)
{
    g_err = msg;
    return s;
}

ivfpq_status ok()
{
    g_err.clear();
    return IVFPQ_OK;
}

// Test hook: IVFPQ_TEST_FAIL_ALLOC=n makes the n-th device allocation
// (1-based) counted from the moment the variable took its current value fail,
// to exercise the out-of-memory paths.  The count restarts whenever the
// variable's value changes (unset counts as a value), so a long-running test
// process can aim at "the n-th allocation from now"; the value is read as its
// leading integer, so "3:a" and "3:b" both mean 3 and still restart the count.
int g_alloc_count = 0;
std::string g_alloc_env;

hipError_t dev_alloc(void **p, size_t bytes)
{
    const char *env = std::getenv("IVFPQ_TEST_FAIL_ALLOC");
    const std::string now = env ? env : "";
    if (now != g_alloc_env) {
        g_alloc_env = now;
        g_alloc_count = 0;
    }
    ++g_alloc_count;
    if (env && std::atoi(env) == g_alloc_count) {
        *p = nullptr;
        return hipErrorOutOfMemory;
    }
    return hipMalloc(p, bytes ? bytes : 1);
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess)
            prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (prev >= 0)
            (void)hipSetDevice(prev);
    }
};

struct EventPair {
    hipEvent_t start = nullptr, stop = nullptr;
};

constexpr int kStages = 4; // coarse, worklist, scan, merge

// Minimum entries per scan work item when the caller passes chunk_len = 0.
// Large items amortise the top-k warm-up (every wave of an item starts from an
// empty queue); the imax cap still splits long queries across workgroups.
constexpr uint32_t kDefaultChunk = 262144;

int kw_of(int k)
{
    int kw = 64;
    while (kw < k)
        kw *= 2;
    return kw;
}

} // namespace

struct ivfpq_index {
    int device = 0;
    DeviceIndex dx;
    int64_t device_bytes = 0;
    // workspace
    void *ws = nullptr;
    size_t ws_bytes = 0;
    // profiling
    bool profiling = false;
    int prof_max = 0;
    int prof_calls = 0;
    unsigned long long *prof_counts = nullptr; // device: [entries scanned, work items]
    std::vector<EventPair> prof_events; // [call][stage]
    std::vector<int> prof_used;         // [call][stage] 0/1
    std::vector<uint32_t> host_off;     // list offsets (host copy)
};

namespace {

ivfpq_status check_shape(int64_t d, int64_t nlist, int64_t m, int64_t nbits, int64_t ntotal)
{
    if (d < 1 || d > 1024)
        return fail(IVFPQ_E_FORMAT, "d must be in [1, 1024]");
    if (nlist < 1 || nlist > (1 << 30))
        return fail(IVFPQ_E_FORMAT, "nlist must be in [1, 2^30]");
    if (m < 1 || m > 64 || d % m)
        return fail(IVFPQ_E_FORMAT, "m must be in [1, 64] and divide d");
    if (nbits != 8)
        return fail(IVFPQ_E_FORMAT, "only 8-bit sub-quantizer codes are supported");
    if (ntotal < 0 || ntotal >= (int64_t)0xFFFFFFFFll)
        return fail(IVFPQ_E_FORMAT, "ntotal must be below 2^32 - 1");
    return IVFPQ_OK;
}

ivfpq_status check_sizes(const int64_t *sizes, int64_t nlist, int64_t ntotal, int64_t *max_list)
{
    int64_t sum = 0, mx = 0;
    for (int64_t l = 0; l < nlist; ++l) {
        if (sizes[l] < 0)
            return fail(IVFPQ_E_FORMAT, "negative list size");
        // compared with the room left before the addition: a sum that wrapped
        // around could otherwise come back to ntotal
        if (sizes[l] > ntotal - sum)
            return fail(IVFPQ_E_FORMAT, "list sizes exceed ntotal");
        sum += sizes[l];
        mx = sizes[l] > mx ? sizes[l] : mx;
    }
    if (sum != ntotal)
        return fail(IVFPQ_E_FORMAT, "list sizes do not add up to ntotal");
    if (max_list)
        *max_list = mx;
    return IVFPQ_OK;
}

struct FileHeader {
    char magic[8];
    uint32_t d, nlist, m, nbits;
    uint64_t ntotal;
};
static_assert(sizeof(FileHeader) == 32, "header layout");

size_t body_bytes(const FileHeader &h)
{
    const size_t dsub = h.d / h.m;
    return (size_t)h.nlist * h.d * 4 + (size_t)h.m * 256 * dsub * 4 + (size_t)h.nlist * 8 +
           (size_t)h.ntotal * h.m + (size_t)h.ntotal * 8;
}

ivfpq_status read_header(FILE *f, FileHeader *h)
{
    if (std::fread(h, sizeof *h, 1, f) != 1)
        return fail(IVFPQ_E_FORMAT, "truncated header");
    if (std::memcmp(h->magic, "IVFPQ01\0", 8) != 0)
        return fail(IVFPQ_E_FORMAT, "bad magic");
    ivfpq_status s = check_shape(h->d, h->nlist, h->m, h->nbits, (int64_t)h->ntotal);
    if (s)
        return s;
    if (std::fseek(f, 0, SEEK_END) != 0)
        return fail(IVFPQ_E_IO, "cannot seek");
    const long end = std::ftell(f);
    if (end < 0)
        return fail(IVFPQ_E_IO, "cannot tell file size");
    if ((size_t)end != sizeof *h + body_bytes(*h))
        return fail(IVFPQ_E_FORMAT, (size_t)end < sizeof *h + body_bytes(*h)
                                        ? "truncated index file"
                                        : "trailing bytes after the index body");
    if (std::fseek(f, sizeof *h, SEEK_SET) != 0)
        return fail(IVFPQ_E_IO, "cannot seek");
    return IVFPQ_OK;
}

void release(ivfpq_index *ix)
{
    if (!ix)
        return;
    DeviceGuard g(ix->device);
    DeviceIndex &d = ix->dx;
    (void)hipFree(d.centroids);
    (void)hipFree(d.cblk);
    (void)hipFree(d.cnorm_pad);
    (void)hipFree(d.cx6);
    (void)hipFree(d.codebooks);
    (void)hipFree(d.list_off);
    (void)hipFree(d.codes);
    (void)hipFree(d.ids);
    (void)hipFree(d.t1);
    (void)hipFree(d.gbucket);
    (void)hipFree(ix->ws);
    (void)hipFree(ix->prof_counts);
    for (auto &e : ix->prof_events) {
        if (e.start)
            (void)hipEventDestroy(e.start);
        if (e.stop)
            (void)hipEventDestroy(e.stop);
    }
    delete ix;
}

ivfpq_status device_check(int device)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1)
        return fail(IVFPQ_E_NO_DEVICE, "no GPU available");
    if (device < 0 || device >= n)
        return fail(IVFPQ_E_NO_DEVICE, "device number out of range");
    return IVFPQ_OK;
}

#define ALLOC_OR_FAIL(ptr, bytes)                                                              \
    do {                                                                                       \
        if (dev_alloc(reinterpret_cast<void **>(&(ptr)), (bytes)) != hipSuccess) {             \
            (void)hipGetLastError();                                                           \
            release(ix);                                                                       \
            return fail(IVFPQ_E_OUT_OF_MEMORY, "device allocation failed");                    \
        }                                                                                      \
        ix->device_bytes += (int64_t)(bytes);                                                  \
    } while (0)

#define COPY_OR_FAIL(dst, src, bytes)                                                          \
    do {                                                                                       \
        if (hipMemcpy((dst), (src), (bytes), hipMemcpyHostToDevice) != hipSuccess) {           \
            release(ix);                                                                       \
            return fail(IVFPQ_E_DEVICE, "host to device copy failed");                         \
        }                                                                                      \
    } while (0)

// Allocate the device index; the caller fills it.
ivfpq_status alloc_index(int device, int d, int nlist, int m, int64_t ntotal,
                         const int64_t *sizes, ivfpq_index **out)
{
    ivfpq_index *ix = new (std::nothrow) ivfpq_index();
    if (!ix)
        return fail(IVFPQ_E_OUT_OF_MEMORY, "host allocation failed");
    ix->device = device;
    DeviceIndex &dx = ix->dx;
    dx.d = d;
    dx.nlist = nlist;
    dx.m = m;
    dx.ntotal = ntotal;
    ix->host_off.resize((size_t)nlist + 1);
    ix->host_off[0] = 0;
    int64_t mx = 0;
    for (int l = 0; l < nlist; ++l) {
        ix->host_off[l + 1] = ix->host_off[l] + (uint32_t)sizes[l];
        mx = sizes[l] > mx ? sizes[l] : mx;
    }
    dx.max_list = mx;
    ALLOC_OR_FAIL(dx.centroids, (size_t)nlist * d * 4);
    // K-steps padded to the coarse kernel's register blocking (8, 16, 24 or
    // 32) and blocks to whole 64-centroid tiles; the padding is zero (norm +inf)
    dx.d4 = (d + 3) / 4 <= 32 ? ((d + 31) / 32) * 8 : (d + 3) / 4;
    dx.nblk = ((nlist + 63) / 64) * 4;
    ALLOC_OR_FAIL(dx.cblk, (size_t)dx.nblk * dx.d4 * 64 * 4);
    ALLOC_OR_FAIL(dx.cnorm_pad, (size_t)dx.nblk * 16 * 4);
    if (coarse_uses_x6(d, nlist)) {
        dx.x6_kb = (d + 31) / 32;
        ALLOC_OR_FAIL(dx.cx6, (size_t)dx.nblk * 16 * dx.x6_kb * 32 * 3 * 2);
    }
    ALLOC_OR_FAIL(dx.codebooks, (size_t)d * 256 * 4);
    ALLOC_OR_FAIL(dx.list_off, ((size_t)nlist + 1) * 4);
    ALLOC_OR_FAIL(dx.codes, (size_t)ntotal * m);
    ALLOC_OR_FAIL(dx.ids, (size_t)ntotal * 8);
    // list term of the decomposed tables (test hook: IVFPQ_TEST_NO_LIST_TERM=1
    // keeps the difference form everywhere)
    const char *no_lt = std::getenv("IVFPQ_TEST_NO_LIST_TERM");
    if (scan_uses_list_term(m, d, nlist) && !(no_lt && no_lt[0] == '1'))
        ALLOC_OR_FAIL(dx.t1, (size_t)nlist * m * 256 * 4);
    COPY_OR_FAIL(dx.list_off, ix->host_off.data(), ((size_t)nlist + 1) * 4);
    *out = ix;
    return IVFPQ_OK;
}

ivfpq_status finish_load(ivfpq_index *ix)
{
    // region buckets of the giant lists, from the host copy of the list
    // offsets (the scan order runs the work items that read the same region
    // of a giant list side by side)
    {
        DeviceIndex &dx = ix->dx;
        std::vector<uint32_t> gb((size_t)dx.nlist, kNoBucket);
        uint64_t nb = 0;
        for (int l = 0; l < dx.nlist; ++l) {
            const uint64_t sz = ix->host_off[l + 1] - ix->host_off[l];
            if (sz >= kGiantList) {
                gb[l] = (uint32_t)nb;
                nb += (sz + kRegion - 1) / kRegion;
            }
        }
        if (nb > 0) {
            dx.nbucket = (uint32_t)nb;
            ALLOC_OR_FAIL(dx.gbucket, (size_t)dx.nlist * 4);
            COPY_OR_FAIL(dx.gbucket, gb.data(), (size_t)dx.nlist * 4);
        }
    }
    if (launch_centroid_blocks(ix->dx, nullptr) != hipSuccess ||
        launch_list_term(ix->dx, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        release(ix);
        return fail(IVFPQ_E_DEVICE, "centroid layout or list term kernel failed");
    }
    return IVFPQ_OK;
}

ivfpq_status ensure_ws(ivfpq_index *ix, size_t bytes)
{
    if (bytes <= ix->ws_bytes)
        return IVFPQ_OK;
    if (ix->ws) {
        (void)hipDeviceSynchronize();
        (void)hipFree(ix->ws);
        ix->ws = nullptr;
        ix->ws_bytes = 0;
    }
    if (dev_alloc(&ix->ws, bytes) != hipSuccess) {
        (void)hipGetLastError();
        ix->ws = nullptr;
        return fail(IVFPQ_E_OUT_OF_MEMORY, "workspace allocation failed");
    }
    ix->ws_bytes = bytes;
    return IVFPQ_OK;
}

ivfpq_status check_params(const ivfpq_index *ix, const ivfpq_search_params *p, int64_t nq)
{
    if (!ix)
        return fail(IVFPQ_E_INVALID_ARG, "index handle is NULL");
    if (!p)
        return fail(IVFPQ_E_INVALID_ARG, "params is NULL");
    if (nq < 0 || nq > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "nq must be in [0, 2^31)");
    if (p->nprobe < 1 || p->nprobe > ix->dx.nlist)
        return fail(IVFPQ_E_INVALID_ARG, "nprobe must be in [1, nlist]");
    if (p->nprobe > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "nprobe above 1024 is not supported");
    if (p->k < 1 || p->k > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "k must be in [1, 1024]");
    if (p->lut != IVFPQ_LUT_F32 && p->lut != IVFPQ_LUT_F16)
        return fail(IVFPQ_E_INVALID_ARG, "unknown table type");
    if (p->mode != IVFPQ_MODE_NORMAL && p->mode != IVFPQ_MODE_SCAN_ONLY)
        return fail(IVFPQ_E_INVALID_ARG, "unknown mode");
    if (p->chunk_len < 0)
        return fail(IVFPQ_E_INVALID_ARG, "chunk_len must be >= 0");
    if (p->metric != IVFPQ_METRIC_L2 && p->metric != IVFPQ_METRIC_IP)
        return fail(IVFPQ_E_INVALID_ARG, "unknown metric");
    if (p->metric == IVFPQ_METRIC_IP && p->lut != IVFPQ_LUT_F32)
        return fail(IVFPQ_E_INVALID_ARG, "the inner-product metric uses float32 tables");
    return IVFPQ_OK;
}

void prof_record(ivfpq_index *ix, int stage, bool start, hipStream_t s)
{
    if (!ix->profiling || ix->prof_calls >= ix->prof_max)
        return;
    EventPair &e = ix->prof_events[(size_t)ix->prof_calls * kStages + stage];
    (void)hipEventRecord(start ? e.start : e.stop, s);
    if (!start)
        ix->prof_used[(size_t)ix->prof_calls * kStages + stage] = 1;
}

// Flat bfloat16 database handle.
struct FlatEvent {
    int stage;
    EventPair ev;
};

} // namespace

struct ivfpq_flat {
    int device = 0;
    FlatDevice fx;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    bool profiling = false;
    int prof_max = 0, prof_calls = 0;
    size_t prof_next = 0;
    std::vector<FlatEvent> prof_pool;
    std::vector<size_t> prof_call_first; // first pool slot of each recorded call
};

namespace {

constexpr size_t kFlatWsBudget = (size_t)4 << 30; // workspace cap; larger batches run in chunks
constexpr int kFlatEventsPerCall = 64;
constexpr int kFlatStages = 5; // minima, kth, collect, select, fallback

void flat_release(ivfpq_flat *f)
{
    if (!f)
        return;
    DeviceGuard g(f->device);
    (void)hipFree(f->fx.vec);
    (void)hipFree(f->fx.norms);
    (void)hipFree(f->ws);
    for (auto &e : f->prof_pool) {
        if (e.ev.start)
            (void)hipEventDestroy(e.ev.start);
        if (e.ev.stop)
            (void)hipEventDestroy(e.ev.stop);
    }
    delete f;
}

// Event pair for one flat kernel launch while profiling, else nullptr.
EventPair *flat_prof_slot(ivfpq_flat *f, int stage)
{
    if (!f->profiling || f->prof_calls >= f->prof_max || f->prof_next >= f->prof_pool.size())
        return nullptr;
    FlatEvent &e = f->prof_pool[f->prof_next++];
    e.stage = stage;
    return &e.ev;
}

} // namespace

extern "C" {

const char *ivfpq_last_error(void) { return g_err.c_str(); }

const char *ivfpq_status_string(ivfpq_status s)
{
    // a C caller may pass any int: read the argument's bytes as one instead
    // of loading it as the C++ enumeration, whose range ends at 7
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case IVFPQ_OK: return "ok";
    case IVFPQ_E_INVALID_ARG: return "invalid argument";
    case IVFPQ_E_IO: return "i/o error";
    case IVFPQ_E_FORMAT: return "malformed index";
    case IVFPQ_E_NO_DEVICE: return "no device";
    case IVFPQ_E_OUT_OF_MEMORY: return "out of memory";
    case IVFPQ_E_DEVICE: return "device error";
    }
    return "unknown status";
}

ivfpq_status ivfpq_validate_index_file(const char *path)
{
    if (!path)
        return fail(IVFPQ_E_INVALID_ARG, "path is NULL");
    FILE *f = std::fopen(path, "rb");
    if (!f)
        return fail(IVFPQ_E_IO, std::string("cannot open ") + path);
    FileHeader h;
    ivfpq_status s = read_header(f, &h);
    if (s) {
        std::fclose(f);
        return s;
    }
    // list sizes must add up to ntotal
    const long sizes_at = (long)(sizeof h + (size_t)h.nlist * h.d * 4 + (size_t)h.d * 256 * 4);
    std::vector<int64_t> sizes(h.nlist);
    if (std::fseek(f, sizes_at, SEEK_SET) != 0 ||
        std::fread(sizes.data(), 8, h.nlist, f) != h.nlist) {
        std::fclose(f);
        return fail(IVFPQ_E_IO, "cannot read list sizes");
    }
    std::fclose(f);
    s = check_sizes(sizes.data(), h.nlist, (int64_t)h.ntotal, nullptr);
    return s ? s : ok();
}

ivfpq_status ivfpq_validate_host_index(const ivfpq_host_index *src)
{
    if (!src)
        return fail(IVFPQ_E_INVALID_ARG, "source is NULL");
    ivfpq_status s = check_shape(src->d, src->nlist, src->m, src->nbits, src->ntotal);
    if (s)
        return s;
    if (!src->centroids || !src->codebooks || !src->list_sizes ||
        (src->ntotal > 0 && (!src->codes || !src->ids)))
        return fail(IVFPQ_E_INVALID_ARG, "a required array is NULL");
    s = check_sizes(src->list_sizes, src->nlist, src->ntotal, nullptr);
    return s ? s : ok();
}

ivfpq_status ivfpq_load_index_host(const ivfpq_host_index *src, int device, ivfpq_index **out)
{
    if (!out)
        return fail(IVFPQ_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    ivfpq_status s = ivfpq_validate_host_index(src);
    if (s)
        return s;
    if ((s = device_check(device)))
        return s;
    DeviceGuard g(device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    ivfpq_index *ix = nullptr;
    if ((s = alloc_index(device, src->d, src->nlist, src->m, src->ntotal, src->list_sizes, &ix)))
        return s;
    DeviceIndex &dx = ix->dx;
    COPY_OR_FAIL(dx.centroids, src->centroids, (size_t)src->nlist * src->d * 4);
    COPY_OR_FAIL(dx.codebooks, src->codebooks, (size_t)src->d * 256 * 4);
    if (src->ntotal > 0) {
        COPY_OR_FAIL(dx.codes, src->codes, (size_t)src->ntotal * src->m);
        COPY_OR_FAIL(dx.ids, src->ids, (size_t)src->ntotal * 8);
    }
    if ((s = finish_load(ix)))
        return s;
    *out = ix;
    return ok();
}

ivfpq_status ivfpq_load_index(const char *path, int device, ivfpq_index **out)
{
    if (!out)
        return fail(IVFPQ_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    ivfpq_status s = ivfpq_validate_index_file(path);
    if (s)
        return s;
    if ((s = device_check(device)))
        return s;
    FILE *f = std::fopen(path, "rb");
    if (!f)
        return fail(IVFPQ_E_IO, "cannot open index file");
    FileHeader h;
    if ((s = read_header(f, &h))) {
        std::fclose(f);
        return s;
    }
    const int d = (int)h.d, nlist = (int)h.nlist, m = (int)h.m;
    const int64_t ntotal = (int64_t)h.ntotal;
    std::vector<float> cent((size_t)nlist * d), books((size_t)d * 256);
    std::vector<int64_t> sizes(nlist);
    bool rd = std::fread(cent.data(), 4, cent.size(), f) == cent.size() &&
              std::fread(books.data(), 4, books.size(), f) == books.size() &&
              std::fread(sizes.data(), 8, sizes.size(), f) == sizes.size();
    if (!rd) {
        std::fclose(f);
        return fail(IVFPQ_E_IO, "cannot read index header arrays");
    }
    DeviceGuard g(device);
    if (!g.ok) {
        std::fclose(f);
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    }
    ivfpq_index *ix = nullptr;
    if ((s = alloc_index(device, d, nlist, m, ntotal, sizes.data(), &ix))) {
        std::fclose(f);
        return s;
    }
    DeviceIndex &dx = ix->dx;
    COPY_OR_FAIL(dx.centroids, cent.data(), cent.size() * 4);
    COPY_OR_FAIL(dx.codebooks, books.data(), books.size() * 4);
    // stream codes and ids in chunks (the big arrays never sit whole in host memory)
    const size_t chunk = (size_t)256 << 20;
    std::vector<unsigned char> buf(chunk);
    const size_t parts[2] = {(size_t)ntotal * m, (size_t)ntotal * 8};
    unsigned char *dsts[2] = {dx.codes, reinterpret_cast<unsigned char *>(dx.ids)};
    for (int a = 0; a < 2; ++a) {
        for (size_t o = 0; o < parts[a]; o += chunk) {
            const size_t n = parts[a] - o < chunk ? parts[a] - o : chunk;
            if (std::fread(buf.data(), 1, n, f) != n) {
                std::fclose(f);
                release(ix);
                return fail(IVFPQ_E_IO, "cannot read codes or ids");
            }
            if (hipMemcpy(dsts[a] + o, buf.data(), n, hipMemcpyHostToDevice) != hipSuccess) {
                std::fclose(f);
                release(ix);
                return fail(IVFPQ_E_DEVICE, "host to device copy failed");
            }
        }
    }
    std::fclose(f);
    if ((s = finish_load(ix)))
        return s;
    *out = ix;
    return ok();
}

void ivfpq_free_index(ivfpq_index *idx) { release(idx); }

ivfpq_status ivfpq_index_info(const ivfpq_index *idx, ivfpq_info *out)
{
    if (!idx || !out)
        return fail(IVFPQ_E_INVALID_ARG, "NULL argument");
    std::memset(out, 0, sizeof *out);
    out->d = idx->dx.d;
    out->nlist = idx->dx.nlist;
    out->m = idx->dx.m;
    out->nbits = 8;
    out->ntotal = idx->dx.ntotal;
    out->max_list = idx->dx.max_list;
    out->device = idx->device;
    out->flags = (idx->dx.t1 ? IVFPQ_INDEX_DECOMPOSED_TABLES : 0) |
                 (idx->dx.cx6 ? IVFPQ_INDEX_COARSE_SPLIT_BF16 : 0);
    out->device_bytes = idx->device_bytes;
    return ok();
}

} // extern "C"

namespace {

// Workspace of one search, byte offsets: probes (unless the caller passes a
// buffer) | plan arrays | coarse scratch | partial top-k of the work items
// (imax items per query; a query with one item writes its rows from the
// scan, so imax = 1 needs no partials).
struct WsLayout {
    size_t probes, total, chunk, count, base, bound, counter, order_q, order_r, rank_n, rm_q,
        rm_r, ikey, bcur, coarse, pd, pp, bytes;
};

WsLayout ws_layout(const DeviceIndex &dx, int64_t nq, int nprobe, int k, uint32_t imax,
                   bool own_probes)
{
    WsLayout o{};
    size_t off = 0;
    auto carve = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    o.probes = own_probes ? carve((size_t)nq * nprobe * 4) : 0;
    o.total = carve((size_t)nq * 4);
    o.chunk = carve((size_t)nq * 4);
    o.count = carve((size_t)nq * 4);
    o.base = carve(((size_t)nq + 1) * 4);
    o.bound = carve((size_t)nq * 4);
    o.counter = carve(4);
    o.order_q = carve((size_t)nq * imax * 4);
    o.order_r = carve((size_t)nq * imax * 4);
    o.rank_n = carve((size_t)imax * 4);
    if (dx.nbucket > 0) { // the order by giant-list regions
        o.rm_q = carve((size_t)nq * imax * 4);
        o.rm_r = carve((size_t)nq * imax * 4);
        o.ikey = carve((size_t)nq * imax * 4);
        o.bcur = carve(((size_t)dx.nbucket + 1) * 4);
    }
    o.coarse = carve(coarse_ws_bytes(dx, nq, nprobe));
    const size_t part = imax > 1 ? (size_t)nq * imax * (size_t)kw_of(k) * 4 : 0;
    o.pd = carve(part);
    o.pp = carve(part);
    o.bytes = off;
    return o;
}

// Fixed device scratch of the allocation-free search (ivfpq_search_noalloc_ex):
// one array per GPU, created with the code object and held until the process
// ends.  Host code never uses the array's name as an address: its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in g_scratch.
constexpr size_t kScratchBytes = IVFPQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address (the caller has made `device` current).
hipError_t scratch_address(int device, unsigned char **out)
{
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    ScratchSlot &sl = g_scratch[device];
    std::call_once(sl.once, [&] {
        sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch));
    });
    *out = static_cast<unsigned char *>(sl.ptr);
    return sl.err;
}

// The search behind ivfpq_search_ex (workspace owned by the handle, grown on
// demand) and ivfpq_search_noalloc_ex (workspace in the fixed scratch; no
// allocation of any kind).
ivfpq_status search_impl(ivfpq_index *idx, const ivfpq_search_params *p, const float *queries_dev,
                         int64_t nq, float *distances_dev, int64_t *ids_dev, int32_t *probes_dev,
                         void *stream, bool noalloc)
{
    ivfpq_status s = check_params(idx, p, nq);
    if (s)
        return s;
    if (nq == 0)
        return ok();
    if (!queries_dev || !distances_dev || (!ids_dev && p->mode == IVFPQ_MODE_NORMAL))
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    DeviceGuard g(idx->device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const DeviceIndex &dx = idx->dx;
    const bool ip = p->metric == IVFPQ_METRIC_IP;
    if (scan_lds_bytes(dx.d, dx.m, p->nprobe, p->lut == IVFPQ_LUT_F16, kw_of(p->k) / 64,
                       dx.m % 2 == 0 ? 2 : 1) > 160 * 1024)
        return fail(IVFPQ_E_INVALID_ARG, "tables of this m and precision exceed the LDS");
    SearchPlan pl;
    pl.target = p->chunk_len > 0 ? (uint32_t)p->chunk_len : kDefaultChunk;
    pl.imax = items_per_query(nq, kw_of(p->k));
    WsLayout o = ws_layout(dx, nq, p->nprobe, p->k, pl.imax, !probes_dev);
    unsigned char *ws = nullptr;
    if (noalloc) {
        // as many items per query as the fixed scratch holds (down to one)
        while (o.bytes > kScratchBytes && pl.imax > 1) {
            pl.imax = pl.imax > 2 ? pl.imax / 2 : 1;
            o = ws_layout(dx, nq, p->nprobe, p->k, pl.imax, !probes_dev);
        }
        if (o.bytes > kScratchBytes)
            return fail(IVFPQ_E_INVALID_ARG,
                        "the batch needs " + std::to_string(o.bytes) +
                            " bytes of workspace, more than the allocation-free search's "
                            "fixed scratch of " + std::to_string(kScratchBytes) +
                            " bytes: split it into smaller batches");
        if (scratch_address(idx->device, &ws) != hipSuccess || !ws) {
            (void)hipGetLastError();
            return fail(IVFPQ_E_DEVICE, "cannot find the device address of the fixed scratch");
        }
    } else {
        if ((s = ensure_ws(idx, o.bytes)))
            return s;
        ws = static_cast<unsigned char *>(idx->ws);
    }
    pl.max_items = nq * (int64_t)pl.imax;
    int32_t *probes = probes_dev ? probes_dev : reinterpret_cast<int32_t *>(ws + o.probes);
    pl.qtotal = reinterpret_cast<uint32_t *>(ws + o.total);
    pl.qchunk = reinterpret_cast<uint32_t *>(ws + o.chunk);
    pl.qcount = reinterpret_cast<uint32_t *>(ws + o.count);
    pl.item_base = reinterpret_cast<uint32_t *>(ws + o.base);
    pl.qbound = reinterpret_cast<uint32_t *>(ws + o.bound);
    pl.counter = reinterpret_cast<uint32_t *>(ws + o.counter);
    pl.item_q = reinterpret_cast<uint32_t *>(ws + o.order_q);
    pl.item_r = reinterpret_cast<uint32_t *>(ws + o.order_r);
    pl.rank_n = reinterpret_cast<uint32_t *>(ws + o.rank_n);
    if (dx.nbucket > 0) {
        pl.rm_q = reinterpret_cast<uint32_t *>(ws + o.rm_q);
        pl.rm_r = reinterpret_cast<uint32_t *>(ws + o.rm_r);
        pl.ikey = reinterpret_cast<uint32_t *>(ws + o.ikey);
        pl.bcur = reinterpret_cast<uint32_t *>(ws + o.bcur);
    }
    pl.part_d = reinterpret_cast<float *>(ws + o.pd);
    pl.part_p = reinterpret_cast<uint32_t *>(ws + o.pp);
    const bool recording = idx->profiling && idx->prof_calls < idx->prof_max;
    pl.prof = recording ? idx->prof_counts : nullptr;

    prof_record(idx, 0, true, st);
    hipError_t e =
        launch_coarse(dx, queries_dev, nq, p->nprobe, ws + o.coarse, probes, nullptr, st, ip);
    prof_record(idx, 0, false, st);
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("coarse kernel: ") + hipGetErrorString(e));
    SearchArgs a;
    a.queries = queries_dev;
    a.nq = nq;
    a.nprobe = p->nprobe;
    a.k = p->k;
    a.lut = p->lut;
    a.mode = p->mode;
    a.chunk_len = p->chunk_len;
    a.metric = ip ? 1 : 0;
    a.out_d = distances_dev;
    a.out_i = ids_dev;
    a.probes = probes;
    a.probe_d = nullptr;
    prof_record(idx, 1, true, st);
    e = launch_plan(dx, a, pl, st);
    prof_record(idx, 1, false, st);
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("plan kernels: ") + hipGetErrorString(e));
    prof_record(idx, 2, true, st);
    e = launch_scan(dx, a, pl, st);
    prof_record(idx, 2, false, st);
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("scan kernel: ") + hipGetErrorString(e));
    if (p->mode == IVFPQ_MODE_NORMAL) {
        prof_record(idx, 3, true, st);
        e = launch_merge(dx, a, pl, st);
        prof_record(idx, 3, false, st);
        if (e != hipSuccess)
            return fail(IVFPQ_E_DEVICE, std::string("merge kernel: ") + hipGetErrorString(e));
    }
    if (recording)
        idx->prof_calls++;
    return ok();
}

} // namespace

extern "C" {

ivfpq_status ivfpq_search_ex(const ivfpq_index *cidx, const ivfpq_search_params *p,
                             const float *queries_dev, int64_t nq, float *distances_dev,
                             int64_t *ids_dev, int32_t *probes_dev, void *stream)
{
    return search_impl(const_cast<ivfpq_index *>(cidx), p, queries_dev, nq, distances_dev,
                       ids_dev, probes_dev, stream, false);
}

ivfpq_status ivfpq_search_noalloc_ex(const ivfpq_index *cidx, const ivfpq_search_params *p,
                                     const float *queries_dev, int64_t nq, float *distances_dev,
                                     int64_t *ids_dev, int32_t *probes_dev, void *stream)
{
    return search_impl(const_cast<ivfpq_index *>(cidx), p, queries_dev, nq, distances_dev,
                       ids_dev, probes_dev, stream, true);
}

ivfpq_status ivfpq_search(const ivfpq_index *idx, const float *queries, int64_t nq, int nprobe,
                          int k, float *distances, int64_t *ids)
{
    ivfpq_search_params p;
    std::memset(&p, 0, sizeof p);
    p.nprobe = nprobe;
    p.k = k;
    ivfpq_status s = check_params(idx, &p, nq);
    if (s)
        return s;
    if (nq == 0)
        return ok();
    if (!queries || !distances || !ids)
        return fail(IVFPQ_E_INVALID_ARG, "a required pointer is NULL");
    DeviceGuard g(idx->device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    const size_t qb = (size_t)nq * idx->dx.d * 4, db = (size_t)nq * k * 4, ib = (size_t)nq * k * 8;
    void *buf = nullptr;
    if (dev_alloc(&buf, qb + db + ib) != hipSuccess) {
        (void)hipGetLastError();
        return fail(IVFPQ_E_OUT_OF_MEMORY, "device allocation failed");
    }
    unsigned char *b = static_cast<unsigned char *>(buf);
    float *dq = reinterpret_cast<float *>(b);
    int64_t *di = reinterpret_cast<int64_t *>(b + qb);
    float *dd = reinterpret_cast<float *>(b + qb + ib);
    if (hipMemcpy(dq, queries, qb, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(buf);
        return fail(IVFPQ_E_DEVICE, "query upload failed");
    }
    s = ivfpq_search_ex(idx, &p, dq, nq, dd, di, nullptr, nullptr);
    if (s == IVFPQ_OK) {
        if (hipStreamSynchronize(nullptr) != hipSuccess ||
            hipMemcpy(distances, dd, db, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(ids, di, ib, hipMemcpyDeviceToHost) != hipSuccess)
            s = fail(IVFPQ_E_DEVICE, "search failed on the device");
    }
    (void)hipFree(buf);
    return s;
}

ivfpq_status ivfpq_coarse_ex(const ivfpq_index *idx, const float *queries_dev, int64_t nq,
                             int nprobe, int32_t *probes_dev, float *coarse_dist_dev, void *stream)
{
    if (!idx)
        return fail(IVFPQ_E_INVALID_ARG, "index handle is NULL");
    if (nq < 0 || nq > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "nq must be in [0, 2^31)");
    if (nprobe < 1 || nprobe > idx->dx.nlist || nprobe > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "nprobe must be in [1, min(nlist, 1024)]");
    if (nq == 0)
        return ok();
    if (!queries_dev || !probes_dev)
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    DeviceGuard g(idx->device);
    ivfpq_index *ix = const_cast<ivfpq_index *>(idx);
    ivfpq_status s = ensure_ws(ix, coarse_ws_bytes(ix->dx, nq, nprobe));
    if (s)
        return s;
    hipError_t e = launch_coarse(idx->dx, queries_dev, nq, nprobe, ix->ws, probes_dev,
                                 coarse_dist_dev, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("coarse kernel: ") + hipGetErrorString(e));
    return ok();
}

ivfpq_status ivfpq_assign_encode_ex(const ivfpq_index *idx, const float *vectors_dev, int64_t n,
                                    int32_t *lists_dev, uint8_t *codes_dev, void *stream)
{
    if (!idx)
        return fail(IVFPQ_E_INVALID_ARG, "index handle is NULL");
    if (n < 0 || n > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "n must be in [0, 2^31)");
    if (n == 0)
        return ok();
    if (!vectors_dev || !lists_dev || !codes_dev)
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    DeviceGuard g(idx->device);
    ivfpq_index *ix = const_cast<ivfpq_index *>(idx);
    ivfpq_status s = ensure_ws(ix, coarse_ws_bytes(ix->dx, n, 1));
    if (s)
        return s;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_coarse(idx->dx, vectors_dev, n, 1, ix->ws, lists_dev, nullptr, st);
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("coarse kernel: ") + hipGetErrorString(e));
    e = launch_encode(idx->dx, vectors_dev, n, lists_dev, codes_dev, st);
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("encode kernel: ") + hipGetErrorString(e));
    return ok();
}

ivfpq_status ivfpq_kmeans_ex(const float *vectors_dev, int64_t n, int d, int k, int iters,
                             float *centers_dev, int32_t *assign_dev, int32_t *counts_dev,
                             void *stream)
{
    if (n < 0 || n > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "n must be in [0, 2^31)");
    if (d < 1 || d > 4096 || k < 1 || k > (1 << 24) || iters < 0 || iters > 100000)
        return fail(IVFPQ_E_INVALID_ARG, "need 1 <= d <= 4096, 1 <= k <= 2^24, 0 <= iters");
    if (!centers_dev || (n > 0 && !vectors_dev))
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    if (iters == 0)
        return ok();
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess)
        return fail(IVFPQ_E_NO_DEVICE, "no current device");
    // the centers as a coarse quantizer (layout of the coarse kernel)
    DeviceIndex dx;
    dx.d = d;
    dx.nlist = k;
    dx.d4 = (d + 3) / 4 <= 32 ? ((d + 31) / 32) * 8 : (d + 3) / 4;
    dx.nblk = ((k + 63) / 64) * 4;
    dx.centroids = centers_dev;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    void *cblk = nullptr, *cnorm = nullptr, *sums = nullptr, *own_a = nullptr, *own_c = nullptr,
         *ws = nullptr;
    const size_t ws_bytes = coarse_ws_bytes(dx, n > 0 ? n : 1, 1);
    ivfpq_status s = IVFPQ_OK;
    if (dev_alloc(&cblk, (size_t)dx.nblk * dx.d4 * 64 * 4) != hipSuccess ||
        dev_alloc(&cnorm, (size_t)dx.nblk * 16 * 4) != hipSuccess ||
        dev_alloc(&sums, (size_t)k * d * 8) != hipSuccess ||
        (!assign_dev && dev_alloc(&own_a, (size_t)(n > 0 ? n : 1) * 4) != hipSuccess) ||
        (!counts_dev && dev_alloc(&own_c, (size_t)k * 4) != hipSuccess) ||
        (ws_bytes && dev_alloc(&ws, ws_bytes) != hipSuccess))
        s = fail(IVFPQ_E_OUT_OF_MEMORY, "k-means scratch allocation failed");
    dx.cblk = static_cast<float *>(cblk);
    dx.cnorm_pad = static_cast<float *>(cnorm);
    int32_t *assign = assign_dev ? assign_dev : static_cast<int32_t *>(own_a);
    int32_t *counts = counts_dev ? counts_dev : static_cast<int32_t *>(own_c);
    for (int it = 0; it < iters && s == IVFPQ_OK; ++it) {
        hipError_t e = launch_centroid_blocks(dx, st);
        if (e == hipSuccess)
            e = launch_coarse(dx, vectors_dev, n, 1, ws, assign, nullptr, st);
        if (e == hipSuccess)
            e = launch_kmeans_update(vectors_dev, n, d, assign, k, static_cast<double *>(sums),
                                     counts, centers_dev, st);
        if (e != hipSuccess)
            s = fail(IVFPQ_E_DEVICE, std::string("k-means round: ") + hipGetErrorString(e));
    }
    if (hipStreamSynchronize(st) != hipSuccess && s == IVFPQ_OK)
        s = fail(IVFPQ_E_DEVICE, "k-means failed on the device");
    for (void *p : {cblk, cnorm, sums, own_a, own_c, ws})
        if (p)
            (void)hipFree(p);
    return s;
}

ivfpq_status ivfpq_build_index_ex(const float *vectors_dev, const int64_t *ids_dev, int64_t n,
                                  int d, int nlist, int m, const float *centroids_dev,
                                  const float *codebooks_dev, int device, ivfpq_index **out)
{
    if (!out)
        return fail(IVFPQ_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (n < 0 || n > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "n must be in [0, 2^31)");
    if (check_shape(d, nlist, m, 8, n) != IVFPQ_OK) {
        const std::string msg = g_err;
        return fail(IVFPQ_E_INVALID_ARG, msg);
    }
    if (!centroids_dev || !codebooks_dev || (n > 0 && !vectors_dev))
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    ivfpq_status s = device_check(device);
    if (s)
        return s;
    DeviceGuard g(device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    std::vector<int64_t> no_sizes((size_t)nlist, 0);
    ivfpq_index *ix = nullptr;
    if ((s = alloc_index(device, d, nlist, m, n, no_sizes.data(), &ix)))
        return s;
    DeviceIndex &dx = ix->dx;
    if (hipMemcpy(dx.centroids, centroids_dev, (size_t)nlist * d * 4, hipMemcpyDeviceToDevice) !=
            hipSuccess ||
        hipMemcpy(dx.codebooks, codebooks_dev, (size_t)d * 256 * 4, hipMemcpyDeviceToDevice) !=
            hipSuccess ||
        launch_centroid_blocks(dx, nullptr) != hipSuccess) {
        release(ix);
        return fail(IVFPQ_E_DEVICE, "centroid or codebook upload failed");
    }
    if (n > 0) {
        // scratch: lists, codes in input order, sort keys and permutation,
        // list counts, the sort's own scratch
        void *lists = nullptr, *codes = nullptr, *keys = nullptr, *perm_in = nullptr,
             *perm_out = nullptr, *counts = nullptr, *tmp = nullptr;
        size_t tmp_bytes = 0;
        std::vector<uint32_t> counts_h((size_t)nlist);
        bool okay = dev_alloc(&lists, (size_t)n * 4) == hipSuccess &&
                    dev_alloc(&codes, (size_t)n * m) == hipSuccess &&
                    dev_alloc(&keys, (size_t)n * 4) == hipSuccess &&
                    dev_alloc(&perm_in, (size_t)n * 4) == hipSuccess &&
                    dev_alloc(&perm_out, (size_t)n * 4) == hipSuccess &&
                    dev_alloc(&counts, (size_t)nlist * 4) == hipSuccess;
        s = okay ? ensure_ws(ix, coarse_ws_bytes(dx, n, 1))
                 : fail(IVFPQ_E_OUT_OF_MEMORY, "build scratch allocation failed");
        auto li = static_cast<int32_t *>(lists);
        auto co = static_cast<uint8_t *>(codes);
        auto ke = static_cast<int32_t *>(keys);
        auto pi = static_cast<int32_t *>(perm_in);
        auto po = static_cast<int32_t *>(perm_out);
        auto cn = static_cast<uint32_t *>(counts);
        if (s == IVFPQ_OK &&
            (launch_coarse(dx, vectors_dev, n, 1, ix->ws, li, nullptr, nullptr) != hipSuccess ||
             launch_encode(dx, vectors_dev, n, li, co, nullptr) != hipSuccess ||
             launch_list_layout(li, n, nlist, m, co, ids_dev, cn, ke, pi, po, nullptr, &tmp_bytes,
                                dx.codes, dx.ids, nullptr) != hipSuccess))
            s = fail(IVFPQ_E_DEVICE, "assignment or encoding kernels failed");
        if (s == IVFPQ_OK && dev_alloc(&tmp, tmp_bytes) != hipSuccess)
            s = fail(IVFPQ_E_OUT_OF_MEMORY, "sort scratch allocation failed");
        if (s == IVFPQ_OK &&
            (launch_list_layout(li, n, nlist, m, co, ids_dev, cn, ke, pi, po, tmp, &tmp_bytes,
                                dx.codes, dx.ids, nullptr) != hipSuccess ||
             hipDeviceSynchronize() != hipSuccess ||
             hipMemcpy(counts_h.data(), cn, (size_t)nlist * 4, hipMemcpyDeviceToHost) !=
                 hipSuccess))
            s = fail(IVFPQ_E_DEVICE, "list layout failed");
        for (void *p : {lists, codes, keys, perm_in, perm_out, counts, tmp})
            if (p)
                (void)hipFree(p);
        if (s != IVFPQ_OK) {
            release(ix);
            return s;
        }
        // list offsets (host copy and device array) from the counts
        int64_t mx = 0;
        for (int l = 0; l < nlist; ++l) {
            ix->host_off[l + 1] = ix->host_off[l] + counts_h[l];
            mx = (int64_t)counts_h[l] > mx ? (int64_t)counts_h[l] : mx;
        }
        dx.max_list = mx;
        if ((int64_t)ix->host_off[nlist] != n) {
            release(ix);
            return fail(IVFPQ_E_DEVICE, "an entry was assigned outside the lists");
        }
        COPY_OR_FAIL(dx.list_off, ix->host_off.data(), ((size_t)nlist + 1) * 4);
    }
    if ((s = finish_load(ix)))
        return s;
    *out = ix;
    return ok();
}

ivfpq_status ivfpq_index_export(const ivfpq_index *idx, float *centroids, float *codebooks,
                                int64_t *list_sizes, uint8_t *codes, int64_t *ids)
{
    if (!idx)
        return fail(IVFPQ_E_INVALID_ARG, "index handle is NULL");
    DeviceGuard g(idx->device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    const DeviceIndex &dx = idx->dx;
    if (list_sizes)
        for (int l = 0; l < dx.nlist; ++l)
            list_sizes[l] = (int64_t)idx->host_off[l + 1] - (int64_t)idx->host_off[l];
    if ((centroids && hipMemcpy(centroids, dx.centroids, (size_t)dx.nlist * dx.d * 4,
                                hipMemcpyDeviceToHost) != hipSuccess) ||
        (codebooks && hipMemcpy(codebooks, dx.codebooks, (size_t)dx.d * 256 * 4,
                                hipMemcpyDeviceToHost) != hipSuccess) ||
        (codes && dx.ntotal > 0 &&
         hipMemcpy(codes, dx.codes, (size_t)dx.ntotal * dx.m, hipMemcpyDeviceToHost) !=
             hipSuccess) ||
        (ids && dx.ntotal > 0 &&
         hipMemcpy(ids, dx.ids, (size_t)dx.ntotal * 8, hipMemcpyDeviceToHost) != hipSuccess))
        return fail(IVFPQ_E_DEVICE, "device to host copy failed");
    return ok();
}

ivfpq_status ivfpq_compute_luts_ex(const ivfpq_index *idx, const float *queries_dev, int64_t nq,
                                   const int32_t *probes_dev, int nprobe, int lut,
                                   float *luts_dev, void *stream)
{
    if (!idx)
        return fail(IVFPQ_E_INVALID_ARG, "index handle is NULL");
    if (nq < 0 || nprobe < 1 || nprobe > idx->dx.nlist || nq * (int64_t)nprobe > 0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "bad nq or nprobe");
    if (lut != IVFPQ_LUT_F32 && lut != IVFPQ_LUT_F16)
        return fail(IVFPQ_E_INVALID_ARG, "unknown table type");
    if (nq == 0)
        return ok();
    if (!queries_dev || !probes_dev || !luts_dev)
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    DeviceGuard g(idx->device);
    hipError_t e = launch_luts(idx->dx, queries_dev, nq, probes_dev, nprobe, lut, luts_dev,
                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("table kernel: ") + hipGetErrorString(e));
    return ok();
}

ivfpq_status ivfpq_select_topk_ex(const float *keys_dev, int64_t rows, int64_t n, int k,
                                  float *out_dist_dev, int32_t *out_pos_dev, void *stream)
{
    if (rows < 0 || rows > (int64_t)0x7FFFFFFF || n < 0 || n > (int64_t)0xFFFFFFFEll)
        return fail(IVFPQ_E_INVALID_ARG, "rows must be in [0, 2^31) and n in [0, 2^32 - 1)");
    if (k < 1 || k > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "k must be in [1, 1024]");
    if (rows == 0)
        return ok();
    if ((!keys_dev && n > 0) || !out_dist_dev || !out_pos_dev)
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    hipError_t e = launch_select(keys_dev, rows, n, k, out_dist_dev, out_pos_dev,
                                 reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("select kernel: ") + hipGetErrorString(e));
    return ok();
}

ivfpq_status ivfpq_stream_read(const void *data_dev, size_t bytes, uint32_t *sink_dev,
                               int sink_words, void *stream)
{
    if (!data_dev || !sink_dev || sink_words < 1 ||
        (reinterpret_cast<uintptr_t>(data_dev) & 15) != 0)
        return fail(IVFPQ_E_INVALID_ARG,
                    "data_dev must be a 16-byte aligned device pointer and sink_words >= 1");
    hipError_t e = launch_stream_read(data_dev, bytes, sink_dev, sink_words,
                                      reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(IVFPQ_E_DEVICE, std::string("stream read kernel: ") + hipGetErrorString(e));
    return ok();
}

ivfpq_status ivfpq_profile_begin(ivfpq_index *idx, int max_calls)
{
    if (!idx || max_calls < 1 || max_calls > 100000)
        return fail(IVFPQ_E_INVALID_ARG, "bad profile arguments");
    DeviceGuard g(idx->device);
    const size_t need = (size_t)max_calls * kStages;
    while (idx->prof_events.size() < need) {
        EventPair e;
        if (hipEventCreate(&e.start) != hipSuccess || hipEventCreate(&e.stop) != hipSuccess)
            return fail(IVFPQ_E_DEVICE, "event creation failed");
        idx->prof_events.push_back(e);
    }
    if (!idx->prof_counts && dev_alloc(reinterpret_cast<void **>(&idx->prof_counts),
                                       2 * sizeof(unsigned long long)) != hipSuccess) {
        (void)hipGetLastError();
        idx->prof_counts = nullptr;
        return fail(IVFPQ_E_OUT_OF_MEMORY, "profile counter allocation failed");
    }
    if (hipMemset(idx->prof_counts, 0, 2 * sizeof(unsigned long long)) != hipSuccess)
        return fail(IVFPQ_E_DEVICE, "profile counter reset failed");
    idx->prof_used.assign(need, 0);
    idx->profiling = true;
    idx->prof_max = max_calls;
    idx->prof_calls = 0;
    return ok();
}

ivfpq_status ivfpq_profile_end(ivfpq_index *idx, ivfpq_timings *out)
{
    if (!idx || !out)
        return fail(IVFPQ_E_INVALID_ARG, "NULL argument");
    DeviceGuard g(idx->device);
    std::memset(out, 0, sizeof *out);
    double *slot[kStages] = {&out->coarse_ms, &out->worklist_ms, &out->scan_ms, &out->merge_ms};
    for (int c = 0; c < idx->prof_calls; ++c) {
        float first_start = -1.f;
        hipEvent_t t0 = nullptr, t1 = nullptr;
        for (int st = 0; st < kStages; ++st) {
            const size_t i = (size_t)c * kStages + st;
            if (!idx->prof_used[i])
                continue;
            if (hipEventSynchronize(idx->prof_events[i].stop) != hipSuccess)
                return fail(IVFPQ_E_DEVICE, "event synchronisation failed");
            float ms = 0.f;
            (void)hipEventElapsedTime(&ms, idx->prof_events[i].start, idx->prof_events[i].stop);
            *slot[st] += ms;
            if (!t0)
                t0 = idx->prof_events[i].start;
            t1 = idx->prof_events[i].stop;
            (void)first_start;
        }
        if (t0 && t1) {
            float ms = 0.f;
            (void)hipEventElapsedTime(&ms, t0, t1);
            out->total_ms += ms;
        }
    }
    out->calls = idx->prof_calls;
    unsigned long long counts[2] = {0, 0};
    if (idx->prof_counts && (hipDeviceSynchronize() != hipSuccess ||
                             hipMemcpy(counts, idx->prof_counts, sizeof counts,
                                       hipMemcpyDeviceToHost) != hipSuccess))
        return fail(IVFPQ_E_DEVICE, "profile counter read failed");
    out->scanned_entries = (int64_t)counts[0];
    out->work_items = (int64_t)counts[1];
    idx->profiling = false;
    return ok();
}


// ---------------------------------------------------------------------------
// flat bfloat16 exact search
// ---------------------------------------------------------------------------

ivfpq_status ivfpq_flat_load_bf16(const uint16_t *vectors, int64_t n, int d, int device,
                                  ivfpq_flat **out)
{
    if (!out)
        return fail(IVFPQ_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (d < 1 || d > 256)
        return fail(IVFPQ_E_INVALID_ARG, "d must be in [1, 256]");
    if (n < 0 || n >= (int64_t)0xFFFFFFFFll - 64)
        return fail(IVFPQ_E_INVALID_ARG, "n must be in [0, 2^32 - 65]");
    if (!vectors && n > 0)
        return fail(IVFPQ_E_INVALID_ARG, "vectors is NULL");
    ivfpq_status s = device_check(device);
    if (s)
        return s;
    DeviceGuard g(device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    ivfpq_flat *f = new (std::nothrow) ivfpq_flat;
    if (!f)
        return fail(IVFPQ_E_OUT_OF_MEMORY, "host allocation failed");
    f->device = device;
    FlatDevice &fx = f->fx;
    fx.d = d;
    fx.dp = (d + 31) / 32 * 32;
    fx.n = n;
    fx.npad = (n + 63) / 64 * 64;
    void *src = nullptr;
    if (dev_alloc(reinterpret_cast<void **>(&fx.vec), (size_t)fx.npad * fx.dp * 2) != hipSuccess ||
        dev_alloc(reinterpret_cast<void **>(&fx.norms), (size_t)fx.npad * 4) != hipSuccess ||
        dev_alloc(&src, (size_t)n * d * 2) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(src);
        flat_release(f);
        return fail(IVFPQ_E_OUT_OF_MEMORY, "device allocation failed");
    }
    if ((n > 0 && hipMemcpy(src, vectors, (size_t)n * d * 2, hipMemcpyHostToDevice) != hipSuccess) ||
        launch_flat_pack(static_cast<const uint16_t *>(src), n, d, fx.dp, fx.npad, fx.vec,
                         fx.norms, nullptr) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(src);
        flat_release(f);
        return fail(IVFPQ_E_DEVICE, "database upload failed");
    }
    (void)hipFree(src);
    // max |y|^2 (the rounding allowance of the collect bound)
    if (n > 0) {
        std::vector<float> nrm((size_t)n);
        if (hipMemcpy(nrm.data(), fx.norms, (size_t)n * 4, hipMemcpyDeviceToHost) != hipSuccess) {
            flat_release(f);
            return fail(IVFPQ_E_DEVICE, "database upload failed");
        }
        for (float v : nrm)
            fx.ymax = v > fx.ymax ? v : fx.ymax;
    }
    *out = f;
    return ok();
}

void ivfpq_flat_free(ivfpq_flat *f) { flat_release(f); }

ivfpq_status ivfpq_flat_search_bf16_ex(const ivfpq_flat *cf, const uint16_t *queries_dev,
                                       int64_t nq, int k, float *distances_dev,
                                       int64_t *ids_dev, void *stream)
{
    ivfpq_flat *f = const_cast<ivfpq_flat *>(cf);
    if (!f)
        return fail(IVFPQ_E_INVALID_ARG, "flat handle is NULL");
    if (nq < 0 || nq > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "nq must be in [0, 2^31)");
    if (k < 1 || k > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "k must be in [1, 1024]");
    if (nq == 0)
        return ok();
    if (!queries_dev || !distances_dev || !ids_dev)
        return fail(IVFPQ_E_INVALID_ARG, "a required device pointer is NULL");
    DeviceGuard g(f->device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const FlatDevice &fx = f->fx;
    const FlatPlan plan = flat_plan(fx.n, k, nq, fx.dp);
    const size_t per_q = flat_ws_bytes(plan, 1);
    // test hook: IVFPQ_TEST_FLAT_WS_BYTES=n caps the workspace (forces chunks)
    size_t budget = kFlatWsBudget;
    if (const char *env = std::getenv("IVFPQ_TEST_FLAT_WS_BYTES"))
        budget = (size_t)std::atoll(env);
    int64_t chunk = (int64_t)(budget / per_q);
    chunk = chunk < 1 ? 1 : chunk > nq ? nq : chunk;
    // the same plan for every chunk (the bound pass's shape depends on nq only
    // through the parts count, fixed above)
    if (f->ws_bytes < flat_ws_bytes(plan, chunk)) {
        if (f->ws) {
            (void)hipDeviceSynchronize();
            (void)hipFree(f->ws);
            f->ws = nullptr;
            f->ws_bytes = 0;
        }
        if (dev_alloc(&f->ws, flat_ws_bytes(plan, chunk)) != hipSuccess) {
            (void)hipGetLastError();
            f->ws = nullptr;
            return fail(IVFPQ_E_OUT_OF_MEMORY, "workspace allocation failed");
        }
        f->ws_bytes = flat_ws_bytes(plan, chunk);
    }
    if (f->profiling && f->prof_calls < f->prof_max)
        f->prof_call_first.push_back(f->prof_next);
    static const char *names[kFlatStages] = {"minima", "kth", "collect", "select", "fallback"};
    for (int64_t c0 = 0; c0 < nq; c0 += chunk) {
        const int64_t cn = nq - c0 < chunk ? nq - c0 : chunk;
        for (int stage = 0; stage < kFlatStages; ++stage) {
            EventPair *ev = flat_prof_slot(f, stage);
            if (ev)
                (void)hipEventRecord(ev->start, st);
            hipError_t e = launch_flat_stage(fx, queries_dev + c0 * fx.d, cn, k, plan, f->ws,
                                             distances_dev + c0 * k, ids_dev + c0 * k, stage, st);
            if (ev)
                (void)hipEventRecord(ev->stop, st);
            if (e != hipSuccess)
                return fail(IVFPQ_E_DEVICE,
                            std::string("flat ") + names[stage] + " kernel: " + hipGetErrorString(e));
        }
    }
    if (f->profiling && f->prof_calls < f->prof_max)
        f->prof_calls++;
    return ok();
}

ivfpq_status ivfpq_flat_search_bf16(const ivfpq_flat *f, const uint16_t *queries, int64_t nq,
                                    int k, float *distances, int64_t *ids)
{
    if (!f)
        return fail(IVFPQ_E_INVALID_ARG, "flat handle is NULL");
    if (nq < 0 || nq > (int64_t)0x7FFFFFFF)
        return fail(IVFPQ_E_INVALID_ARG, "nq must be in [0, 2^31)");
    if (k < 1 || k > kMaxK)
        return fail(IVFPQ_E_INVALID_ARG, "k must be in [1, 1024]");
    if (nq == 0)
        return ok();
    if (!queries || !distances || !ids)
        return fail(IVFPQ_E_INVALID_ARG, "a required pointer is NULL");
    DeviceGuard g(f->device);
    if (!g.ok)
        return fail(IVFPQ_E_NO_DEVICE, "cannot select device");
    const size_t qb = ((size_t)nq * f->fx.d * 2 + 255) & ~(size_t)255;
    const size_t db = (size_t)nq * k * 4, ib = (size_t)nq * k * 8;
    void *buf = nullptr;
    if (dev_alloc(&buf, qb + db + ib) != hipSuccess) {
        (void)hipGetLastError();
        return fail(IVFPQ_E_OUT_OF_MEMORY, "device allocation failed");
    }
    unsigned char *b = static_cast<unsigned char *>(buf);
    uint16_t *dq = reinterpret_cast<uint16_t *>(b);
    int64_t *di = reinterpret_cast<int64_t *>(b + qb);
    float *dd = reinterpret_cast<float *>(b + qb + ib);
    if (hipMemcpy(dq, queries, (size_t)nq * f->fx.d * 2, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(buf);
        return fail(IVFPQ_E_DEVICE, "query upload failed");
    }
    ivfpq_status s = ivfpq_flat_search_bf16_ex(f, dq, nq, k, dd, di, nullptr);
    if (s == IVFPQ_OK) {
        if (hipStreamSynchronize(nullptr) != hipSuccess ||
            hipMemcpy(distances, dd, db, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(ids, di, ib, hipMemcpyDeviceToHost) != hipSuccess)
            s = fail(IVFPQ_E_DEVICE, "search failed on the device");
    }
    (void)hipFree(buf);
    return s;
}

ivfpq_status ivfpq_flat_profile_begin(ivfpq_flat *f, int max_calls)
{
    if (!f || max_calls < 1 || max_calls > 100000)
        return fail(IVFPQ_E_INVALID_ARG, "bad profile arguments");
    DeviceGuard g(f->device);
    const size_t need = (size_t)max_calls * kFlatEventsPerCall;
    while (f->prof_pool.size() < need) {
        FlatEvent e{0, {}};
        if (hipEventCreate(&e.ev.start) != hipSuccess || hipEventCreate(&e.ev.stop) != hipSuccess)
            return fail(IVFPQ_E_DEVICE, "event creation failed");
        f->prof_pool.push_back(e);
    }
    f->profiling = true;
    f->prof_max = max_calls;
    f->prof_calls = 0;
    f->prof_next = 0;
    f->prof_call_first.clear();
    return ok();
}

ivfpq_status ivfpq_flat_profile_end(ivfpq_flat *f, ivfpq_flat_timings *out)
{
    if (!f || !out)
        return fail(IVFPQ_E_INVALID_ARG, "NULL argument");
    DeviceGuard g(f->device);
    std::memset(out, 0, sizeof *out);
    double *slot[kFlatStages] = {&out->minima_ms, &out->kth_ms, &out->collect_ms, &out->select_ms,
                                 &out->fallback_ms};
    for (size_t i = 0; i < f->prof_next; ++i) {
        const FlatEvent &e = f->prof_pool[i];
        if (hipEventSynchronize(e.ev.stop) != hipSuccess)
            return fail(IVFPQ_E_DEVICE, "event synchronisation failed");
        float ms = 0.f;
        (void)hipEventElapsedTime(&ms, e.ev.start, e.ev.stop);
        *slot[e.stage] += ms;
    }
    for (size_t c = 0; c < f->prof_call_first.size(); ++c) {
        const size_t a = f->prof_call_first[c];
        const size_t z = c + 1 < f->prof_call_first.size() ? f->prof_call_first[c + 1] : f->prof_next;
        if (z > a) {
            float ms = 0.f;
            (void)hipEventElapsedTime(&ms, f->prof_pool[a].ev.start, f->prof_pool[z - 1].ev.stop);
            out->total_ms += ms;
        }
    }
    out->calls = f->prof_calls;
    f->profiling = false;
    return ok();
}

} // extern "C"
