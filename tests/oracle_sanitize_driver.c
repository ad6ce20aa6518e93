/*
 * Runs every entry point of the C oracle (oracle/ivfpq_oracle.c) on small
 * seeded inputs and their edge cases, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: empty lists, nprobe = nlist, k above the number
 * of candidates (padding), binary16 tables, the inner-product metric, several
 * threads, rejected arguments.  It also checks the properties every result
 * must have (rows sorted, padding where candidates run out, the ADC distance
 * of a returned entry equal to its entry distance), so that a run under the
 * sanitizers exercises the real paths.  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LUT_F64 0
#define ORACLE_LUT_F16 1
#define ORACLE_IP 2

int oracle_coarse(const float *x, const float *centroids, int d, int nlist, int nprobe,
                  int32_t *probes, double *dists);
int oracle_coarse_ip(const float *x, const float *centroids, int d, int nlist, int nprobe,
                     int32_t *probes, double *ips);
int oracle_lut(const float *x, const float *c, const float *codebooks, int d, int m, int lut_mode,
               double *lut);
int oracle_lut_ip(const float *x, const float *codebooks, int d, int m, double *lut);
int oracle_entry_distances(const float *x, const float *centroids, const float *codebooks, int d,
                           int m, int lut_mode, const int32_t *lists, const uint8_t *code_rows,
                           int64_t n, double *out);
int oracle_search(const float *centroids, const float *codebooks, const int64_t *list_sizes,
                  const uint8_t *codes, const int64_t *ids, int d, int nlist, int m,
                  const float *queries, int64_t nq, int nprobe, int k, int lut_mode,
                  const int32_t *probes_in, double *out_dist, int64_t *out_ids,
                  int32_t *out_probes, int nthreads);
int oracle_bruteforce(const float *db, const int64_t *db_ids, int64_t n, int d,
                      const float *queries, int64_t nq, int k, double *out_dist,
                      int64_t *out_ids, int nthreads);
int oracle_bruteforce_bf16(const uint16_t *db, int64_t n, int d, const uint16_t *queries,
                           int64_t nq, int k, double *out_dist, int64_t *out_ids, int nthreads);

static int failures = 0;
#define CHECK(cond, what)                                                  \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAIL %s (line %d)\n", what, __LINE__);        \
            failures++;                                                    \
        }                                                                  \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uniform(void) { return (float)((next_u64() >> 40) * (1.0 / 16777216.0)) * 2.f - 1.f; }

static void fill(float *a, size_t n)
{
    for (size_t i = 0; i < n; i++)
        a[i] = uniform();
}

/* rows of k results: ascending (descending for the inner product) over the
 * valid prefix, then padding (+-inf, -1) only */
static void check_rows(const double *dist, const int64_t *ids, int64_t nq, int k, int ip,
                       int64_t expect_valid, const char *what)
{
    for (int64_t q = 0; q < nq; q++) {
        const double *dr = dist + q * k;
        const int64_t *ir = ids + q * k;
        int64_t valid = 0;
        while (valid < k && ir[valid] >= 0)
            valid++;
        CHECK(expect_valid < 0 || valid == (expect_valid < k ? expect_valid : k), what);
        for (int64_t j = 1; j < valid; j++)
            CHECK(ip ? dr[j] <= dr[j - 1] : dr[j] >= dr[j - 1], what);
        for (int64_t j = valid; j < k; j++)
            CHECK(ir[j] == -1 && isinf(dr[j]) && (ip ? dr[j] < 0 : dr[j] > 0), what);
    }
}

int main(void)
{
    enum { D = 16, M = 4, NLIST = 6, NQ = 9 };
    const int dsub = D / M;
    /* lists of sizes 0, 5, 0, 17, 1, 9 (two empty) */
    const int64_t sizes[NLIST] = {0, 5, 0, 17, 1, 9};
    int64_t ntotal = 0;
    for (int l = 0; l < NLIST; l++)
        ntotal += sizes[l];
    float *cent = malloc(sizeof(float) * NLIST * D);
    float *books = malloc(sizeof(float) * M * 256 * dsub);
    float *queries = malloc(sizeof(float) * NQ * D);
    uint8_t *codes = malloc((size_t)ntotal * M);
    int64_t *ids = malloc(sizeof(int64_t) * (size_t)ntotal);
    fill(cent, NLIST * D);
    fill(books, (size_t)M * 256 * dsub);
    fill(queries, NQ * D);
    for (int64_t i = 0; i < ntotal * M; i++)
        codes[i] = (uint8_t)(next_u64() & 255);
    for (int64_t i = 0; i < ntotal; i++)
        ids[i] = 1000 + 7 * i;

    /* coarse, both metrics, nprobe 1 .. nlist, and rejected nprobe */
    for (int np = 1; np <= NLIST; np++) {
        int32_t pr[NLIST];
        double dd[NLIST];
        CHECK(oracle_coarse(queries, cent, D, NLIST, np, pr, dd) == 0, "coarse");
        for (int i = 1; i < np; i++)
            CHECK(dd[i] >= dd[i - 1], "coarse sorted");
        CHECK(oracle_coarse_ip(queries, cent, D, NLIST, np, pr, dd) == 0, "coarse ip");
        for (int i = 1; i < np; i++)
            CHECK(dd[i] <= dd[i - 1], "coarse ip sorted");
        CHECK(oracle_coarse(queries, cent, D, NLIST, np, pr, NULL) == 0, "coarse no dists");
    }
    {
        int32_t pr[NLIST + 1];
        CHECK(oracle_coarse(queries, cent, D, NLIST, 0, pr, NULL) < 0, "coarse nprobe 0");
        CHECK(oracle_coarse(queries, cent, D, NLIST, NLIST + 1, pr, NULL) < 0, "coarse nprobe > nlist");
    }

    /* tables in every mode, and rejected shapes */
    {
        double *lut = malloc(sizeof(double) * M * 256);
        for (int mode = 0; mode < 2; mode++) {
            CHECK(oracle_lut(queries, cent, books, D, M, mode, lut) == 0, "lut");
            for (int i = 0; i < M * 256; i++)
                CHECK(lut[i] >= 0, "lut entries are squared distances");
        }
        CHECK(oracle_lut_ip(queries, books, D, M, lut) == 0, "lut ip");
        CHECK(oracle_lut(queries, cent, books, D, 3, 0, lut) < 0, "lut m not dividing d");
        CHECK(oracle_lut_ip(queries, books, D, 0, lut) < 0, "lut ip m 0");
        free(lut);
    }

    /* searches: every mode, nprobe = nlist, k above the candidates, threads */
    const int ks[3] = {1, 10, 64};
    for (int mode = 0; mode < 3; mode++)
        for (int np = 1; np <= NLIST; np += NLIST - 1)
            for (int ki = 0; ki < 3; ki++) {
                const int k = ks[ki];
                double *od = malloc(sizeof(double) * NQ * k);
                int64_t *oi = malloc(sizeof(int64_t) * NQ * k);
                int32_t *op = malloc(sizeof(int32_t) * NQ * np);
                for (int th = 1; th <= 3; th += 2) {
                    CHECK(oracle_search(cent, books, sizes, codes, ids, D, NLIST, M, queries, NQ,
                                        np, k, mode, NULL, od, oi, op, th) == 0,
                          "search");
                    check_rows(od, oi, NQ, k, mode == ORACLE_IP, np == NLIST ? ntotal : -1,
                               "search rows");
                }
                /* the distance of each returned entry is its entry distance */
                for (int q = 0; q < NQ; q++)
                    for (int j = 0; j < k && oi[(size_t)q * k + j] >= 0; j++) {
                        const int64_t pos = (oi[(size_t)q * k + j] - 1000) / 7;
                        int32_t list = 0;
                        int64_t acc = 0;
                        while (acc + sizes[list] <= pos)
                            acc += sizes[list++];
                        double e;
                        CHECK(oracle_entry_distances(queries + (size_t)q * D, cent, books, D, M, mode,
                                                     &list, codes + pos * M, 1, &e) == 0,
                              "entry distances");
                        CHECK(e == od[(size_t)q * k + j] || (mode == ORACLE_IP && -e == od[(size_t)q * k + j]),
                              "entry distance equals the search's");
                    }
                /* the same search with the probes given */
                CHECK(oracle_search(cent, books, sizes, codes, ids, D, NLIST, M, queries, NQ, np, k,
                                    mode, op, od, oi, NULL, 2) == 0,
                      "search with given probes");
                free(od);
                free(oi);
                free(op);
            }
    {
        double od[4];
        int64_t oi[4];
        CHECK(oracle_search(cent, books, sizes, codes, ids, D, NLIST, M, queries, 1, NLIST + 1, 4, 0,
                            NULL, od, oi, NULL, 1) < 0,
              "search nprobe > nlist");
        CHECK(oracle_search(cent, books, sizes, codes, ids, D, NLIST, M, queries, 1, 2, 0, 0, NULL,
                            od, oi, NULL, 1) < 0,
              "search k 0");
        CHECK(oracle_search(cent, books, sizes, codes, ids, D, NLIST, M, queries, 0, 2, 4, 0, NULL,
                            od, oi, NULL, 1) == 0,
              "search of no queries");
    }

    /* brute force over float and bfloat16 rows, k above n */
    {
        enum { N = 37, K = 50 };
        float *db = malloc(sizeof(float) * N * D);
        int64_t dbid[N];
        uint16_t *db16 = malloc(sizeof(uint16_t) * N * D);
        uint16_t *q16 = malloc(sizeof(uint16_t) * NQ * D);
        fill(db, (size_t)N * D);
        for (int i = 0; i < N; i++)
            dbid[i] = i;
        for (int i = 0; i < N * D; i++)
            db16[i] = (uint16_t)(next_u64() & 0x7F7F);
        for (int i = 0; i < NQ * D; i++)
            q16[i] = (uint16_t)(next_u64() & 0x7F7F);
        double od[NQ * K];
        int64_t oi[NQ * K];
        for (int th = 1; th <= 4; th += 3) {
            CHECK(oracle_bruteforce(db, dbid, N, D, queries, NQ, K, od, oi, th) == 0, "brute");
            check_rows(od, oi, NQ, K, 0, N, "brute rows");
            CHECK(oracle_bruteforce_bf16(db16, N, D, q16, NQ, K, od, oi, th) == 0, "brute bf16");
            check_rows(od, oi, NQ, K, 0, N, "brute bf16 rows");
        }
        free(db);
        free(db16);
        free(q16);
    }

#ifdef PLANT_OVERFLOW
    /* a read one past the id array: a build whose sanitizer works stops here */
    volatile int64_t past = ids[ntotal];
    (void)past;
#endif
    free(cent);
    free(books);
    free(queries);
    free(codes);
    free(ids);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
