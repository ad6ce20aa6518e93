/*
 * ivfpq.h - IVF-PQ approximate nearest-neighbour search on one MI355X (gfx950).
 *
 * The problem (k-nearest-neighbour search; "Custom 8-bit floating point value
 * format for reducing shared memory bank conflict in ANN search", problem
 * statement and IVFPQ section): given a database of N d-dimensional vectors
 * compressed into an IVF-PQ index and a batch of queries, return for each
 * query the k database ids with the smallest approximate squared L2 distance
 *
 *     R = sum_{j<m} F_j(code_j),  F_j(v) = | r_j - C_j[v] |^2,  r = x - c_l
 *
 * (Eq. (1) there), searching only the nprobe inverted lists whose centroids c_l
 * are closest to the query ("Billion-scale similarity search with GPUs",
 * IVFADC section).
 *
 * Conventions, all calls:
 *  - every call returns an ivfpq_status; no exception crosses the ABI;
 *    ivfpq_last_error() gives a message for the last failing call on the
 *    calling thread (an unsupported request is an explicit error, not a
 *    silent fallback: "Support HNSW Search using GPUs", API section);
 *  - distances are squared L2, smaller is better, each result row sorted
 *    ascending; a row with fewer than k candidates is padded with
 *    (+INFINITY, -1) (the +infinity sentinel of the k-selection section of
 *    "Billion-scale similarity search with GPUs"; the -1 id of the sentinel
 *    handling in "Support HNSW Search using GPUs", Search kernel section);
 *  - arguments are validated on the host before any device work ("Support
 *    HNSW Search using GPUs", graph conversion section: the structure is
 *    checked before the GPU dereferences it); on error the output buffers
 *    are left unspecified;
 *  - inputs must be finite (documented precondition, not checked);
 *  - one search at a time per index handle (the handle owns a workspace).
 *
 * Index file, version 1 (little-endian):
 *   char magic[8] = "IVFPQ01\0"; u32 d, nlist, m, nbits (= 8); u64 ntotal;
 *   f32 centroids[nlist][d]; f32 codebooks[m][256][d/m];
 *   u64 list_sizes[nlist]; u8 codes[ntotal][m] (list after list, one row of m
 *   bytes per entry); i64 ids[ntotal] (same order).
 * Sub-vector j of a residual is dims j*(d/m) .. (j+1)*(d/m)-1.
 * Limits: 1 <= m <= 64, m divides d, d <= 1024, ntotal < 2^32.
 */
#ifndef IVFPQ_H
#define IVFPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ivfpq_index ivfpq_index; /* opaque, owned by the library */

typedef enum {
    IVFPQ_OK = 0,
    IVFPQ_E_INVALID_ARG = 1, /* a bad argument: range, null pointer, unsupported shape */
    IVFPQ_E_IO = 2,          /* the index file cannot be opened or read */
    IVFPQ_E_FORMAT = 3,      /* the index file or host arrays are malformed */
    IVFPQ_E_NO_DEVICE = 4,   /* no usable GPU, or the device number is out of range */
    IVFPQ_E_OUT_OF_MEMORY = 5,
    IVFPQ_E_DEVICE = 6       /* a HIP runtime or kernel launch error */
} ivfpq_status;

typedef enum { IVFPQ_LUT_F32 = 0, IVFPQ_LUT_F16 = 1 } ivfpq_lut_type;

/* Ranking metric of a search.  IVFPQ_METRIC_L2: squared L2 distance, smaller
 * is better, rows ascending, padding (+INFINITY, -1).  IVFPQ_METRIC_IP: inner
 * product, larger is better, rows descending, padding (-INFINITY, -1): the
 * lists probed are the nprobe of largest <x, c_l> and an entry of list l with
 * code v scores <x, c_l> + sum_j <x_j, C_j[v_j]>, the inner product of the
 * query with the entry's reconstruction (the conventions of "Support HNSW
 * Search using GPUs", Search kernel section: the kernels rank by the negated
 * value and flip its sign on output).  Float32 tables only. */
typedef enum { IVFPQ_METRIC_L2 = 0, IVFPQ_METRIC_IP = 1 } ivfpq_metric;

typedef enum {
    IVFPQ_MODE_NORMAL = 0,
    /* benchmark only: the scan computes every distance but keeps just the
     * per-wave minimum instead of the top-k (measures what the k-select
     * costs); results are not a valid search */
    IVFPQ_MODE_SCAN_ONLY = 1
} ivfpq_mode;

/* Search parameters ("Billion-scale similarity search with GPUs", IVFADC
 * section: nprobe is the number tau of lists probed, k the results kept; the
 * k-selection section bounds k near 1024).  nprobe in [1, nlist]; k in
 * [1, 1024]; lut selects the table precision (float32, or float32 computed
 * then stored as IEEE binary16 round-to-nearest-even; sums are float32 in
 * both).  chunk_len: the target number of entries of one scan work item
 * (0 = automatic, 262144).  It is a minimum, not a cap: a query whose probed
 * lists hold E entries gets ceil(E / max(chunk_len, ceil(E / imax))) items,
 * imax (2..64) chosen from nq and k, so long queries get larger items.  On an
 * index with lists of 2^20 entries or more, the sequence of a query that
 * probes one is laid out with those lists on 2^19-entry boundaries and its
 * item size is rounded up to a multiple of 2^19 entries (the work items that
 * read the same part of such a list then run together).  The result does
 * not depend on it. */
typedef struct {
    int32_t nprobe;
    int32_t k;
    int32_t lut;  /* ivfpq_lut_type */
    int32_t mode; /* ivfpq_mode */
    int32_t chunk_len;
    int32_t metric; /* ivfpq_metric (0 = squared L2) */
} ivfpq_search_params;

/* ivfpq_info.flags: the squared-L2 scan of this index with float32 tables
 * builds its tables from a list term precomputed at load plus a query term
 * (the decomposition of "Billion-scale similarity search with GPUs", IVFADC
 * section); their float32 error near a zero distance is larger than the
 * difference form's (bounded by the sum of the terms' magnitudes times a few
 * units of round-off).  Binary16 tables and the inner product always use the
 * direct form. */
#define IVFPQ_INDEX_DECOMPOSED_TABLES 1
/* ivfpq_info.flags: the top-nprobe coarse step of this index (nprobe 2..128)
 * forms x.c from three bfloat16 parts of each operand on the bfloat16 matrix
 * cores (six exact partial products per dimension summed in float32; the
 * split of "Leveraging the bfloat16 artificial intelligence datatype for
 * higher-precision computations", Henry, Tang and Heinecke): indexes with
 * d <= 96 and nlist >= 16,384.  Its forward-error bound counts
 * 192 ceil(d/32) + d + 2 float32 roundings instead of d + 2. */
#define IVFPQ_INDEX_COARSE_SPLIT_BF16 2

typedef struct {
    int32_t d, nlist, m, nbits;
    int64_t ntotal;
    int64_t max_list; /* longest inverted list */
    int32_t device;
    int32_t flags;        /* IVFPQ_INDEX_* bits */
    int64_t device_bytes; /* device memory held by the index */
} ivfpq_info;

/* Host arrays describing an index (same layout as the file body).  The
 * library copies them; the caller keeps ownership. */
typedef struct {
    int32_t d, nlist, m, nbits;
    int64_t ntotal;
    const float *centroids;    /* [nlist][d] */
    const float *codebooks;    /* [m][256][d/m] */
    const int64_t *list_sizes; /* [nlist], sum = ntotal */
    const uint8_t *codes;      /* [ntotal][m], list after list */
    const int64_t *ids;        /* [ntotal] */
} ivfpq_host_index;

/* Per-kernel device time, milliseconds, summed over the searches run between
 * ivfpq_profile_begin and ivfpq_profile_end (HIP events recorded on the
 * search stream around each kernel). */
typedef struct {
    int32_t calls;
    int32_t reserved;
    double coarse_ms;   /* coarse distances + top-nprobe */
    double worklist_ms; /* work-item builder */
    double scan_ms;     /* LUT + code scan + first-pass select */
    double merge_ms;    /* cross-item merge + id gather */
    double total_ms;    /* first kernel start to last kernel end */
    int64_t scanned_entries; /* entries of the probed lists, i.e. entries scanned
                                (sum over calls; counted on the device) */
    int64_t work_items;      /* scan work items (sum over calls; counted on the device) */
} ivfpq_timings;

/* Host-only check of an index file's header and size (no GPU needed): the
 * validation "Support HNSW Search using GPUs" (graph conversion section) asks
 * for before a structure reaches the device.  The file layout is the index
 * of "Custom 8-bit floating point value format for reducing shared memory
 * bank conflict in ANN search", IVFPQ section, index-building step 4 (lists,
 * codes, codebooks saved).  IVFPQ_E_IO if unreadable, IVFPQ_E_FORMAT if the
 * magic, nbits, d % m, the list sizes or the length is wrong. */
ivfpq_status ivfpq_validate_index_file(const char *path);

/* Host-only check of host index arrays (no GPU needed), as
 * ivfpq_validate_index_file: IVFPQ_E_INVALID_ARG for a NULL pointer,
 * IVFPQ_E_FORMAT for a bad shape or list sizes that do not sum to ntotal. */
ivfpq_status ivfpq_validate_host_index(const ivfpq_host_index *src);

/* Read an index file and upload it to GPU `device`.  Codes and centroids stay
 * resident in HBM for the handle's life ("Billion-scale similarity search
 * with GPUs", multi-GPU/system section: the index lives on the device, only
 * queries travel).  *out receives the handle. */
ivfpq_status ivfpq_load_index(const char *path, int device, ivfpq_index **out);

/* As ivfpq_load_index, from host arrays (copied). */
ivfpq_status ivfpq_load_index_host(const ivfpq_host_index *src, int device, ivfpq_index **out);

/* Release the handle and its device memory.  NULL is allowed.  The device
 * index is search-only ("Support HNSW Search using GPUs", API section: the
 * GPU index is built from a host index and not copied back into one); the
 * handle owns every device allocation it made, and this frees all of them. */
void ivfpq_free_index(ivfpq_index *idx);

/* Shape and device footprint of a loaded index (host-only read of the
 * handle): d, nlist, m, nbits, ntotal, the longest list, the device and the
 * bytes of device memory the handle holds.  IVFPQ_E_INVALID_ARG for NULL. */
ivfpq_status ivfpq_index_info(const ivfpq_index *idx, ivfpq_info *out);

/* Blocking search with host buffers (the search of "Custom 8-bit floating
 * point value format for reducing shared memory bank conflict in ANN search",
 * IVFPQ section, search steps 1-5): queries [nq][d] float32 row-major in,
 * distances [nq][k] float32 and ids [nq][k] int64 out.  Copies queries to the
 * device and results back (PCIe included).  nq = 0 is a no-op. */
ivfpq_status ivfpq_search(const ivfpq_index *idx, const float *queries, int64_t nq, int nprobe,
                          int k, float *distances, int64_t *ids);

/* Asynchronous search with device buffers on `stream` (a hipStream_t; NULL =
 * the null stream).  The path of "Billion-scale similarity search with
 * GPUs", IVFADC section: coarse distances and the nprobe nearest lists, a
 * table per (query, list), the scan of the lists' codes summing m table
 * entries per entry, a first k-selection per piece of work and a second one
 * across a query's pieces; the tables and sums are those of Eq. (1) of the
 * IVFPQ section of "Custom 8-bit floating point value format for reducing
 * shared memory bank conflict in ANN search".  params: see
 * ivfpq_search_params (its metric picks squared L2 or inner product).  queries_dev [nq][d] float32, distances_dev [nq][k] float32,
 * ids_dev [nq][k] int64; probes_dev, when not NULL, receives the probed list
 * numbers [nq][nprobe] int32 in ascending coarse distance.  No host
 * synchronisation happens between the kernels; the call returns once they are
 * enqueued.  The buffers must stay valid until the stream reaches them. */
ivfpq_status ivfpq_search_ex(const ivfpq_index *idx, const ivfpq_search_params *params,
                             const float *queries_dev, int64_t nq, float *distances_dev,
                             int64_t *ids_dev, int32_t *probes_dev, void *stream);

/* Allocation-free search, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and kernels as ivfpq_search_ex, but the
 * workspace (probes unless probes_dev is given, the work plan, the coarse
 * step's scratch and the partial top-k of the work items) lives in a fixed
 * device array of IVFPQ_NOALLOC_SCRATCH_BYTES per GPU, created with the
 * library's code object and held until the process ends; the call allocates
 * and frees nothing (no hipMalloc, no library routine that allocates).
 * Items per query are reduced (64 down to 1) until the workspace fits; a
 * batch that does not fit even then (about nq * (4 nprobe + 8 nprobe-rounded
 * coarse partials + 24) bytes) is rejected with IVFPQ_E_INVALID_ARG before
 * any device work: split it.  Every call on a GPU uses that GPU's single
 * array, so calls that overlap on one GPU (two streams, two threads, two
 * handles) race and must be serialised by the caller; the array keeps the
 * last call's contents, and the kernels set everything they read before
 * reading it. */
#define IVFPQ_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ivfpq_status ivfpq_search_noalloc_ex(const ivfpq_index *idx, const ivfpq_search_params *params,
                                     const float *queries_dev, int64_t nq, float *distances_dev,
                                     int64_t *ids_dev, int32_t *probes_dev, void *stream);

/* The coarse step alone (device buffers, asynchronous; the coarse quantizer
 * q1 of "Billion-scale similarity search with GPUs", IVFADC section, and
 * search step 1 of the IVFPQ section of "Custom 8-bit floating point value
 * format for reducing shared memory bank conflict in ANN search"): for each query the
 * nprobe lists of smallest |x - c_l|^2, ascending: probes_dev [nq][nprobe]
 * int32 and, when not NULL, coarse_dist_dev [nq][nprobe] float32. */
ivfpq_status ivfpq_coarse_ex(const ivfpq_index *idx, const float *queries_dev, int64_t nq,
                             int nprobe, int32_t *probes_dev, float *coarse_dist_dev,
                             void *stream);

/* Index building, list assignment and PQ encoding of database vectors
 * (device buffers, asynchronous on `stream`).  "Custom 8-bit floating point
 * value format for reducing shared memory bank conflict in ANN search", IVFPQ
 * section, index-building steps 1-3, with the quantizers of "Billion-scale
 * similarity search with GPUs", IVFADC section (coarse quantizer q1, and m
 * quantizers of 256 reproduction values on the residual).
 *
 * vectors_dev [n][d] float32 row-major.  lists_dev [n] int32 receives the
 * list of smallest |x - c_l|^2 (the coarse distances of a search, float32
 * through the norm expansion; with d <= 128 equal distances go to the
 * smaller list number, above that to any of the tied lists);
 * codes_dev [n][m] uint8 receives, for each sub-quantizer j, the codeword v
 * of smallest F_j(v) = sum_s (r[j dsub + s] - C_j[v][s])^2 with r = x - c_list
 * (float32, evaluated as the search evaluates its tables; ties to the smaller
 * v).  The index's centroids and codebooks are used; the index's own lists
 * are not changed.  n = 0 is a no-op; n must be < 2^31.  Errors:
 * IVFPQ_E_INVALID_ARG (NULL handle or pointer, bad n),
 * IVFPQ_E_OUT_OF_MEMORY (coarse workspace), IVFPQ_E_DEVICE (launch).  The
 * buffers belong to the caller and must stay valid until the stream reaches
 * the kernels; the call uses the handle's workspace, so it must not overlap a
 * search on the same handle. */
ivfpq_status ivfpq_assign_encode_ex(const ivfpq_index *idx, const float *vectors_dev, int64_t n,
                                    int32_t *lists_dev, uint8_t *codes_dev, void *stream);

/* k-means by Lloyd's algorithm on the device (the clustering of "Custom 8-bit
 * floating point value format for reducing shared memory bank conflict in ANN
 * search", IVFPQ section, index-building step 1; run it on the residuals of
 * one sub-vector to train a sub-quantizer's 256 codewords).  Each of `iters`
 * iterations assigns every vector to its nearest center (the coarse step with
 * nprobe = 1: squared L2 through the float32 norm expansion on the matrix
 * cores; with d <= 128 equal distances go to the smaller center number)
 * and then moves every center to the mean of its vectors (sums in
 * double precision, the mean rounded to float32); a center with no vector
 * keeps its value.
 *
 * vectors_dev [n][d] float32 row-major; centers_dev [k][d] float32: the
 * initial centers on entry, the centers after the last iteration on return.
 * assign_dev [n] int32 and counts_dev [k] int32, when not NULL, receive the
 * last iteration's assignment and cluster sizes.  On the current device and
 * `stream`; scratch is allocated and freed inside, and the call returns after
 * the device work is done.  iters = 0 changes nothing; n = 0 leaves the centers
 * as they are.  Errors: IVFPQ_E_INVALID_ARG (n outside [0, 2^31), d outside
 * [1, 4096], k outside [1, 2^24], iters < 0, NULL centers, NULL vectors with
 * n > 0), IVFPQ_E_OUT_OF_MEMORY, IVFPQ_E_NO_DEVICE, IVFPQ_E_DEVICE. */
ivfpq_status ivfpq_kmeans_ex(const float *vectors_dev, int64_t n, int d, int k, int iters,
                             float *centers_dev, int32_t *assign_dev, int32_t *counts_dev,
                             void *stream);

/* Index building: an index built on `device` from n database vectors in
 * device memory and trained centroids and codebooks (device memory too, for
 * instance from ivfpq_kmeans_ex).  Each vector goes to the list of its nearest
 * centroid and is PQ-encoded on its residual (ivfpq_assign_encode_ex); the
 * entries are then laid out list after list, keeping their input order inside
 * a list ("Custom 8-bit floating point value format for reducing shared memory
 * bank conflict in ANN search", IVFPQ section, index-building steps 1-4;
 * "Billion-scale similarity search with GPUs", IVFADC section: the codes of a
 * list are stored contiguously).
 *
 * vectors_dev [n][d] float32; ids_dev [n] int64 or NULL (the ids are then the
 * row numbers 0..n-1); centroids_dev [nlist][d] float32; codebooks_dev
 * [m][256][d/m] float32.  The library copies what it keeps; the caller keeps
 * ownership of its buffers.  Its kernels run on the null stream, so buffers
 * written on another stream must be complete before the call; it returns when
 * the index is ready (it synchronises the device).  Errors: IVFPQ_E_INVALID_ARG (NULL out or pointer,
 * n outside [0, 2^31), a shape ivfpq_load_index would reject), IVFPQ_E_NO_DEVICE,
 * IVFPQ_E_OUT_OF_MEMORY, IVFPQ_E_DEVICE. */
ivfpq_status ivfpq_build_index_ex(const float *vectors_dev, const int64_t *ids_dev, int64_t n,
                                  int d, int nlist, int m, const float *centroids_dev,
                                  const float *codebooks_dev, int device, ivfpq_index **out);

/* Copy an index back to host memory (for saving it, or checking it): any
 * pointer may be NULL to skip that array.  Sizes from ivfpq_index_info:
 * centroids [nlist][d] float32, codebooks [m][256][d/m] float32, list_sizes
 * [nlist] int64, codes [ntotal][m] uint8 (list after list), ids [ntotal]
 * int64.  Blocking.  Errors: IVFPQ_E_INVALID_ARG (NULL handle),
 * IVFPQ_E_NO_DEVICE, IVFPQ_E_DEVICE. */
ivfpq_status ivfpq_index_export(const ivfpq_index *idx, float *centroids, float *codebooks,
                                int64_t *list_sizes, uint8_t *codes, int64_t *ids);

/* The table step alone (device buffers, asynchronous, for verification): for
 * each query q and each of its nprobe lists probes_dev[q][p], writes the
 * m x 256 table F_j(v) to luts_dev[q][p][j][v] as float32 (values of the fp16
 * variant are the binary16 numbers widened to float32). */
ivfpq_status ivfpq_compute_luts_ex(const ivfpq_index *idx, const float *queries_dev, int64_t nq,
                                   const int32_t *probes_dev, int nprobe, int lut,
                                   float *luts_dev, void *stream);

/* The k-selection on its own (device buffers, asynchronous): for each of
 * `rows` rows of n float32 keys (keys_dev [rows][n]) the k smallest, ascending,
 * with their column numbers: out_dist_dev [rows][k] float32, out_pos_dev
 * [rows][k] int32, padded with (+INFINITY, -1) when n < k.  Ties between equal
 * keys may resolve to any of the tied columns.  ("Billion-scale similarity
 * search with GPUs", k-selection section: the k least values of a sequence,
 * their indices carried along.) */
ivfpq_status ivfpq_select_topk_ex(const float *keys_dev, int64_t rows, int64_t n, int k,
                                  float *out_dist_dev, int32_t *out_pos_dev, void *stream);

/* Measurement support (not part of the search path): start summing
 * per-kernel times (HIP events on the search stream, no host
 * synchronisation during searches) and counting the entries and work items
 * scanned (device counters).  Up to max_calls searches are recorded.
 * Errors: IVFPQ_E_INVALID_ARG (NULL handle, max_calls outside [1, 100000]),
 * IVFPQ_E_OUT_OF_MEMORY, IVFPQ_E_DEVICE. */
ivfpq_status ivfpq_profile_begin(ivfpq_index *idx, int max_calls);

/* Wait for the recorded searches, write the sums to *out, stop recording. */
ivfpq_status ivfpq_profile_end(ivfpq_index *idx, ivfpq_timings *out);

/* ---- exact k-NN over a flat bfloat16 database --------------------------
 *
 * Brute-force search ("Billion-scale similarity search with GPUs", exact
 * search section): the exact k nearest database rows of each query by squared
 * L2 distance, evaluated as |x|^2 + |y|^2 - 2 x.y with bfloat16 x bfloat16
 * products summed in float32 (matrix cores) and |x|^2, |y|^2 in float32 from
 * the bfloat16 values.  Ids are database row numbers (0-based).  Ties at the
 * k-th distance may resolve to any of the tied rows.  Limits: 1 <= d <= 256,
 * 0 <= n < 2^32 - 64, k in [1, 1024]. */
typedef struct ivfpq_flat ivfpq_flat; /* opaque, owned by the library */

/* Per-kernel device time, milliseconds, summed over the recorded searches. */
typedef struct {
    int32_t calls;
    int32_t reserved;
    double minima_ms;   /* all distances; per-lane minima over segments of rows */
    double kth_ms;      /* k-th smallest minimum per query: the collect bound */
    double collect_ms;  /* all distances again; rows under the bound kept */
    double select_ms;   /* exact top-k of the kept rows */
    double fallback_ms; /* exact streaming top-k for queries whose kept rows overflowed */
    double total_ms;    /* first kernel start to last kernel end */
} ivfpq_flat_timings;

/* Upload n rows of d bfloat16 values (bit patterns, row-major [n][d], host
 * memory; copied) to GPU `device`.  *out receives the handle. */
ivfpq_status ivfpq_flat_load_bf16(const uint16_t *vectors, int64_t n, int d, int device,
                                  ivfpq_flat **out);

/* Release the handle and its device memory.  NULL is allowed. */
void ivfpq_flat_free(ivfpq_flat *f);

/* Asynchronous exact search with device buffers on `stream` (hipStream_t,
 * NULL = null stream): queries_dev [nq][d] bfloat16 bit patterns,
 * distances_dev [nq][k] float32 ascending, ids_dev [nq][k] int64 row numbers,
 * padded with (+INFINITY, -1) when n < k.  One search at a time per handle
 * (the handle owns the workspace). */
ivfpq_status ivfpq_flat_search_bf16_ex(const ivfpq_flat *f, const uint16_t *queries_dev,
                                       int64_t nq, int k, float *distances_dev,
                                       int64_t *ids_dev, void *stream);

/* Blocking variant with host buffers (PCIe copies included). */
ivfpq_status ivfpq_flat_search_bf16(const ivfpq_flat *f, const uint16_t *queries, int64_t nq,
                                    int k, float *distances, int64_t *ids);

/* Per-kernel timing of flat searches, as ivfpq_profile_begin / _end. */
ivfpq_status ivfpq_flat_profile_begin(ivfpq_flat *f, int max_calls);
ivfpq_status ivfpq_flat_profile_end(ivfpq_flat *f, ivfpq_flat_timings *out);

/* ---- measurement support ---------------------------------------------- */

/* Reference streaming read for the bandwidth roofline (not part of the search
 * path): reads the `bytes` bytes at data_dev (device memory, 16-byte aligned;
 * a tail shorter than 16 bytes is not read) once, enqueued on `stream`
 * (NULL = default), asynchronous.  sink_dev: device scratch of sink_words >= 1
 * uint32 that the kernel may write (its contents are meaningless); the grid is
 * at most sink_words workgroups.  The caller times it with events on the same
 * stream.  Errors: IVFPQ_E_INVALID_ARG for a NULL pointer, a misaligned
 * data_dev or sink_words < 1; IVFPQ_E_DEVICE if the launch fails. */
ivfpq_status ivfpq_stream_read(const void *data_dev, size_t bytes, uint32_t *sink_dev,
                               int sink_words, void *stream);

/* Message for the last failing call on this thread ("" if none); valid until
 * the next call on this thread.  (Errors are reported, never hidden behind a
 * fallback: "Support HNSW Search using GPUs", API section.)  The string is
 * owned by the library. */
const char *ivfpq_last_error(void);

/* A fixed English name of a status code ("unknown status" for a value outside
 * the enum); a static string owned by the library. */
const char *ivfpq_status_string(ivfpq_status s);

#ifdef __cplusplus
}
#endif

#endif /* IVFPQ_H */
