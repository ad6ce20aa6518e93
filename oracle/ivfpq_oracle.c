/*
 * IVF-PQ search oracle: plain, slow, double-precision CPU code.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP path.
 *
 * What it computes follows the IVFPQ search steps of "Custom 8-bit floating
 * point value format for reducing shared memory bank conflict in ANN search"
 * (IVFPQ section, search steps 1-5 and Eq. (1)), with the coarse step of
 * "Billion-scale similarity search with GPUs" (IVFADC section: the lists
 * probed are the tau lists whose centroids are closest to the query):
 *
 *   1. coarse:  Dc[l] = sum_t (x[t] - c_l[t])^2, every list l; the nprobe
 *               smallest (distance, then list number) are probed;
 *   2. residual r = x - c_l for each probed list;
 *   3. table    F_j(v) = sum_{t < dsub} (r[j*dsub + t] - C_j[v][t])^2,
 *               sub-vector j = the dsub consecutive dims starting at j*dsub;
 *   4. ADC      R = sum_{j < m} F_j(code[j]) for every entry of the list;
 *   5. top-k    all (R, id) of all probed lists, fully sorted by (R, id);
 *               the first k are returned, missing ones padded (+inf, -1).
 *
 * Every floating-point step is in double precision.  In fp16-table mode each
 * table entry is rounded double -> float -> IEEE binary16 (round to nearest
 * even) before the sums, which is what a device that computes the table in
 * float and stores it as binary16 holds.
 *
 * Also: an exact brute-force k-NN (sum of squared differences over the raw
 * vectors, full sort by (distance, id)), the textbook definition of the
 * k-NN problem stated in the same page's problem statement.
 *
 * Inner-product metric (ORACLE_IP; the conventions of "Support HNSW Search
 * using GPUs", Search kernel section: inner product, larger is better, the
 * kernel ranks by the negated value and flips the sign on output): the lists probed are those of largest <x, c_l> (ties to the smaller
 * list number), the tables T_j(v) = <x_j, C_j[v]> depend on the query only,
 * and an entry of list l with code c scores <x, c_l> + sum_j T_j(c_j), the
 * inner product of x with the reconstructed vector c_l + (C_j[c_j])_j.  The
 * candidates are sorted by (score decreasing, id); missing ones are padded
 * (-inf, -1).
 *
 * Queries are independent; the search and brute-force entry points run them
 * on a pool of POSIX threads, one query at a time per thread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LUT_F64 0
#define ORACLE_LUT_F16 1
#define ORACLE_IP 2 /* inner-product metric, double-precision tables */

typedef struct {
    double key;
    int64_t id;
} pair_t;

static int cmp_pair(const void *pa, const void *pb)
{
    const pair_t *a = (const pair_t *)pa, *b = (const pair_t *)pb;
    if (a->key < b->key) return -1;
    if (a->key > b->key) return 1;
    if (a->id < b->id) return -1;
    if (a->id > b->id) return 1;
    return 0;
}

/* Round a float to the nearest IEEE-754 binary16 value (ties to even) and
 * return it widened to double.  binary16: 10 stored fraction bits, normal
 * exponents -14..15, subnormals are multiples of 2^-24, largest finite value
 * 65504; anything that rounds above it becomes infinity. */
double oracle_round_binary16(float f)
{
    double a = fabs((double)f);
    if (a == 0.0 || isnan(a) || isinf(a))
        return (double)f;
    int e;
    frexp(a, &e);            /* a = frac * 2^e, frac in [0.5, 1) -> floor(log2 a) = e - 1 */
    int ex = e - 1;
    if (ex < -14)
        ex = -14;            /* subnormal range: fixed quantum 2^-24 */
    double quantum = ldexp(1.0, ex - 10);
    double r = rint(a / quantum) * quantum;   /* rint: round half to even */
    if (r > 65504.0)
        r = INFINITY;
    return f < 0 ? -r : r;
}

/* Step 1: coarse distances to every centroid, sorted; writes the first
 * nprobe list numbers (and their distances when dists != NULL). */
int oracle_coarse(const float *x, const float *centroids, int d, int nlist, int nprobe,
                  int32_t *probes, double *dists)
{
    if (nprobe < 1 || nprobe > nlist)
        return -1;
    pair_t *all = (pair_t *)malloc(sizeof(pair_t) * (size_t)nlist);
    if (!all)
        return -2;
    for (int l = 0; l < nlist; l++) {
        const float *c = centroids + (size_t)l * d;
        double s = 0.0;
        for (int t = 0; t < d; t++) {
            double diff = (double)x[t] - (double)c[t];
            s += diff * diff;
        }
        all[l].key = s;
        all[l].id = l;
    }
    qsort(all, (size_t)nlist, sizeof(pair_t), cmp_pair);
    for (int p = 0; p < nprobe; p++) {
        probes[p] = (int32_t)all[p].id;
        if (dists)
            dists[p] = all[p].key;
    }
    free(all);
    return 0;
}

static double dot(const float *a, const float *b, int n)
{
    double s = 0.0;
    for (int t = 0; t < n; t++)
        s += (double)a[t] * (double)b[t];
    return s;
}

/* Inner-product step 1: the nprobe lists of largest <x, c_l> (ties to the
 * smaller list number); ips, when not NULL, receives their inner products. */
int oracle_coarse_ip(const float *x, const float *centroids, int d, int nlist, int nprobe,
                     int32_t *probes, double *ips)
{
    if (nprobe < 1 || nprobe > nlist)
        return -1;
    pair_t *all = (pair_t *)malloc(sizeof(pair_t) * (size_t)nlist);
    if (!all)
        return -2;
    for (int l = 0; l < nlist; l++) {
        all[l].key = -dot(x, centroids + (size_t)l * d, d);
        all[l].id = l;
    }
    qsort(all, (size_t)nlist, sizeof(pair_t), cmp_pair);
    for (int p = 0; p < nprobe; p++) {
        probes[p] = (int32_t)all[p].id;
        if (ips)
            ips[p] = -all[p].key;
    }
    free(all);
    return 0;
}

/* Inner-product tables: T_j(v) = <x_j, C_j[v]> over the dsub dims of
 * sub-vector j (the same for every list). */
int oracle_lut_ip(const float *x, const float *codebooks, int d, int m, double *lut)
{
    if (m < 1 || d % m)
        return -1;
    int dsub = d / m;
    for (int j = 0; j < m; j++)
        for (int v = 0; v < 256; v++)
            lut[j * 256 + v] = dot(x + j * dsub, codebooks + ((size_t)j * 256 + v) * dsub, dsub);
    return 0;
}

/* Steps 2-3: the m x 256 table for query x and the list with centroid c.
 * codebooks is [m][256][dsub] float. */
int oracle_lut(const float *x, const float *c, const float *codebooks, int d, int m, int lut_mode,
               double *lut)
{
    if (m < 1 || d % m)
        return -1;
    int dsub = d / m;
    double *r = (double *)malloc(sizeof(double) * (size_t)d);
    if (!r)
        return -2;
    for (int t = 0; t < d; t++)
        r[t] = (double)x[t] - (double)c[t];
    for (int j = 0; j < m; j++) {
        for (int v = 0; v < 256; v++) {
            const float *cw = codebooks + ((size_t)j * 256 + v) * dsub;
            double s = 0.0;
            for (int t = 0; t < dsub; t++) {
                double diff = r[j * dsub + t] - (double)cw[t];
                s += diff * diff;
            }
            if (lut_mode == ORACLE_LUT_F16)
                s = oracle_round_binary16((float)s);
            lut[j * 256 + v] = s;
        }
    }
    free(r);
    return 0;
}

/* Step 4 for one entry: sum of the m table values its code bytes select. */
static double adc_one(const double *lut, const uint8_t *code, int m)
{
    double s = 0.0;
    for (int j = 0; j < m; j++)
        s += lut[j * 256 + code[j]];
    return s;
}

/* Steps 2-4 for single entries: the ADC distance of each listed entry
 * (entry e lies in list lists[i] and has code row codes[e]) for query x. */
int oracle_entry_distances(const float *x, const float *centroids, const float *codebooks, int d,
                           int m, int lut_mode, const int32_t *lists, const uint8_t *code_rows,
                           int64_t n, double *out)
{
    if (m < 1 || d % m || n < 0)
        return -1;
    double *lut = (double *)malloc(sizeof(double) * (size_t)m * 256);
    if (!lut)
        return -2;
    if (lut_mode == ORACLE_IP && oracle_lut_ip(x, codebooks, d, m, lut)) {
        free(lut);
        return -1;
    }
    for (int64_t i = 0; i < n; i++) {
        const float *c = centroids + (size_t)lists[i] * d;
        if (lut_mode == ORACLE_IP) {
            out[i] = dot(x, c, d) + adc_one(lut, code_rows + (size_t)i * m, m);
            continue;
        }
        int rc = oracle_lut(x, c, codebooks, d, m, lut_mode, lut);
        if (rc) {
            free(lut);
            return rc;
        }
        out[i] = adc_one(lut, code_rows + (size_t)i * m, m);
    }
    free(lut);
    return 0;
}

typedef struct {
    /* index */
    const float *centroids;
    const float *codebooks;
    const int64_t *list_offsets; /* nlist + 1 */
    const uint8_t *codes;
    const int64_t *ids;
    int d, nlist, m;
    /* query batch */
    const float *queries;
    int64_t nq;
    int nprobe, k, lut_mode;
    const int32_t *probes_in;
    double *out_dist;
    int64_t *out_ids;
    int32_t *out_probes;
    /* work distribution */
    int64_t next;
    pthread_mutex_t lock;
    int error;
} search_job_t;

static int64_t take_query(int64_t *next, pthread_mutex_t *lock, int64_t nq)
{
    pthread_mutex_lock(lock);
    int64_t q = *next < nq ? (*next)++ : -1;
    pthread_mutex_unlock(lock);
    return q;
}

static int search_one(search_job_t *J, int64_t q)
{
    const float *x = J->queries + (size_t)q * J->d;
    int32_t *probes = (int32_t *)malloc(sizeof(int32_t) * (size_t)J->nprobe);
    double *lut = (double *)malloc(sizeof(double) * (size_t)J->m * 256);
    if (!probes || !lut) {
        free(probes);
        free(lut);
        return -2;
    }
    const int ip = J->lut_mode == ORACLE_IP;
    if (J->probes_in) {
        memcpy(probes, J->probes_in + (size_t)q * J->nprobe, sizeof(int32_t) * (size_t)J->nprobe);
    } else if (ip ? oracle_coarse_ip(x, J->centroids, J->d, J->nlist, J->nprobe, probes, NULL)
                  : oracle_coarse(x, J->centroids, J->d, J->nlist, J->nprobe, probes, NULL)) {
        free(probes);
        free(lut);
        return -1;
    }
    int64_t total = 0;
    for (int p = 0; p < J->nprobe; p++) {
        int l = probes[p];
        total += J->list_offsets[l + 1] - J->list_offsets[l];
    }
    pair_t *cand = (pair_t *)malloc(sizeof(pair_t) * (size_t)(total > 0 ? total : 1));
    if (!cand) {
        free(probes);
        free(lut);
        return -2;
    }
    int64_t n = 0;
    if (ip)
        oracle_lut_ip(x, J->codebooks, J->d, J->m, lut);
    for (int p = 0; p < J->nprobe; p++) {
        int l = probes[p];
        const float *c = J->centroids + (size_t)l * J->d;
        double base = 0.0;
        if (ip)
            base = dot(x, c, J->d);
        else
            oracle_lut(x, c, J->codebooks, J->d, J->m, J->lut_mode, lut);
        for (int64_t e = J->list_offsets[l]; e < J->list_offsets[l + 1]; e++) {
            double r = adc_one(lut, J->codes + (size_t)e * J->m, J->m);
            /* inner product: sort by the negated score, so that larger comes first */
            cand[n].key = ip ? -(base + r) : r;
            cand[n].id = J->ids[e];
            n++;
        }
    }
    qsort(cand, (size_t)n, sizeof(pair_t), cmp_pair);
    for (int i = 0; i < J->k; i++) {
        J->out_dist[(size_t)q * J->k + i] =
            i < n ? (ip ? -cand[i].key : cand[i].key) : (ip ? -INFINITY : INFINITY);
        J->out_ids[(size_t)q * J->k + i] = i < n ? cand[i].id : -1;
    }
    if (J->out_probes)
        memcpy(J->out_probes + (size_t)q * J->nprobe, probes, sizeof(int32_t) * (size_t)J->nprobe);
    free(cand);
    free(probes);
    free(lut);
    return 0;
}

static void *search_worker(void *arg)
{
    search_job_t *J = (search_job_t *)arg;
    int64_t q;
    while ((q = take_query(&J->next, &J->lock, J->nq)) >= 0) {
        int rc = search_one(J, q);
        if (rc) {
            pthread_mutex_lock(&J->lock);
            J->error = rc;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

static int run_pool(void *(*fn)(void *), void *job, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th)
        return -2;
    int started = 0;
    for (int i = 0; i < nthreads; i++) {
        if (pthread_create(&th[i], NULL, fn, job) == 0)
            started++;
        else
            break;
    }
    if (started == 0)
        fn(job);
    for (int i = 0; i < started; i++)
        pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/* Full IVF-PQ search (steps 1-5) for nq queries.  list_sizes[nlist] gives the
 * list lengths; entries are stored list after list.  probes_in, when not NULL,
 * replaces step 1 with the given [nq][nprobe] list numbers.  out_probes, when
 * not NULL, receives the probed lists.  Returns 0, or <0 on bad arguments or
 * allocation failure. */
int oracle_search(const float *centroids, const float *codebooks, const int64_t *list_sizes,
                  const uint8_t *codes, const int64_t *ids, int d, int nlist, int m,
                  const float *queries, int64_t nq, int nprobe, int k, int lut_mode,
                  const int32_t *probes_in, double *out_dist, int64_t *out_ids,
                  int32_t *out_probes, int nthreads)
{
    if (m < 1 || d % m || nlist < 1 || nprobe < 1 || nprobe > nlist || k < 1 || nq < 0)
        return -1;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * ((size_t)nlist + 1));
    if (!off)
        return -2;
    off[0] = 0;
    for (int l = 0; l < nlist; l++)
        off[l + 1] = off[l] + list_sizes[l];
    search_job_t J;
    memset(&J, 0, sizeof(J));
    J.centroids = centroids;
    J.codebooks = codebooks;
    J.list_offsets = off;
    J.codes = codes;
    J.ids = ids;
    J.d = d;
    J.nlist = nlist;
    J.m = m;
    J.queries = queries;
    J.nq = nq;
    J.nprobe = nprobe;
    J.k = k;
    J.lut_mode = lut_mode;
    J.probes_in = probes_in;
    J.out_dist = out_dist;
    J.out_ids = out_ids;
    J.out_probes = out_probes;
    pthread_mutex_init(&J.lock, NULL);
    run_pool(search_worker, &J, nthreads);
    pthread_mutex_destroy(&J.lock);
    free(off);
    return J.error;
}

/* ---------------------------------------------------------------------- */
/* exact brute-force k-NN                                                  */
/* ---------------------------------------------------------------------- */

typedef struct {
    const float *db;        /* float rows, or NULL when db_bf16 is used */
    const uint16_t *db_bf16; /* bfloat16 bit patterns */
    const int64_t *db_ids;  /* NULL: id = row number */
    int64_t n;
    int d;
    const float *queries;
    const uint16_t *queries_bf16;
    int64_t nq;
    int k;
    double *out_dist;
    int64_t *out_ids;
    int64_t next;
    pthread_mutex_t lock;
    int error;
} brute_job_t;

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void *brute_worker(void *arg)
{
    brute_job_t *J = (brute_job_t *)arg;
    pair_t *cand = (pair_t *)malloc(sizeof(pair_t) * (size_t)(J->n > 0 ? J->n : 1));
    double *x = (double *)malloc(sizeof(double) * (size_t)J->d);
    if (!cand || !x) {
        pthread_mutex_lock(&J->lock);
        J->error = -2;
        pthread_mutex_unlock(&J->lock);
        free(cand);
        free(x);
        return NULL;
    }
    int64_t q;
    while ((q = take_query(&J->next, &J->lock, J->nq)) >= 0) {
        for (int t = 0; t < J->d; t++)
            x[t] = J->queries ? (double)J->queries[(size_t)q * J->d + t]
                              : bf16_value(J->queries_bf16[(size_t)q * J->d + t]);
        for (int64_t i = 0; i < J->n; i++) {
            double s = 0.0;
            for (int t = 0; t < J->d; t++) {
                double y = J->db ? (double)J->db[(size_t)i * J->d + t]
                                 : bf16_value(J->db_bf16[(size_t)i * J->d + t]);
                double diff = x[t] - y;
                s += diff * diff;
            }
            cand[i].key = s;
            cand[i].id = J->db_ids ? J->db_ids[i] : i;
        }
        qsort(cand, (size_t)J->n, sizeof(pair_t), cmp_pair);
        for (int i = 0; i < J->k; i++) {
            J->out_dist[(size_t)q * J->k + i] = i < J->n ? cand[i].key : INFINITY;
            J->out_ids[(size_t)q * J->k + i] = i < J->n ? cand[i].id : -1;
        }
    }
    free(cand);
    free(x);
    return NULL;
}

static int brute_run(brute_job_t *J, int nthreads)
{
    if (J->d < 1 || J->k < 1 || J->n < 0 || J->nq < 0)
        return -1;
    pthread_mutex_init(&J->lock, NULL);
    run_pool(brute_worker, J, nthreads);
    pthread_mutex_destroy(&J->lock);
    return J->error;
}

/* Exact k-NN over float rows: squared L2, full sort by (distance, id). */
int oracle_bruteforce(const float *db, const int64_t *db_ids, int64_t n, int d,
                      const float *queries, int64_t nq, int k, double *out_dist,
                      int64_t *out_ids, int nthreads)
{
    brute_job_t J;
    memset(&J, 0, sizeof(J));
    J.db = db;
    J.db_ids = db_ids;
    J.n = n;
    J.d = d;
    J.queries = queries;
    J.nq = nq;
    J.k = k;
    J.out_dist = out_dist;
    J.out_ids = out_ids;
    return brute_run(&J, nthreads);
}

/* Exact k-NN over bfloat16 rows and queries (bit patterns), the values
 * widened exactly to double. */
int oracle_bruteforce_bf16(const uint16_t *db, int64_t n, int d, const uint16_t *queries,
                           int64_t nq, int k, double *out_dist, int64_t *out_ids, int nthreads)
{
    brute_job_t J;
    memset(&J, 0, sizeof(J));
    J.db_bf16 = db;
    J.n = n;
    J.d = d;
    J.queries_bf16 = queries;
    J.nq = nq;
    J.k = k;
    J.out_dist = out_dist;
    J.out_ids = out_ids;
    return brute_run(&J, nthreads);
}
