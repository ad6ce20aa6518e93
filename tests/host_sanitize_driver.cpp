// Host-side paths of the library under AddressSanitizer and
// UndefinedBehaviorSanitizer: the index-file reader on crafted files (every
// way the header and body can be wrong: truncation at each boundary, a bad
// magic word, shapes out of range, list sizes that are negative or do not add
// up, trailing bytes, huge declared sizes in a small file), the host-array
// validation, the status strings, and the entry points' argument checks that
// return before any device work.  Built by the test with the library's host
// code instrumented (api.hip) and linked ahead of the built library, whose
// kernels it never launches: no GPU is needed or touched.
//
// The file layout is the one the library reads ("Support HNSW Search using
// GPUs": validate everything read from a file before it is used): a 32-byte
// header (magic "IVFPQ01\0", d, nlist, m, nbits as uint32, ntotal as uint64),
// then centroids [nlist][d] float32, codebooks [m][256][d/m] float32, list
// sizes [nlist] int64, codes [ntotal][m] uint8, ids [ntotal] int64.
//
// argv[1]: a scratch directory.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ivfpq.h"

static int failures = 0;
#define CHECK(cond, what)                                                      \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "FAIL %s (line %d): %s\n", what, __LINE__,    \
                         ivfpq_last_error());                                  \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

struct Shape {
    uint32_t d = 8, nlist = 3, m = 2, nbits = 8;
    uint64_t ntotal = 10;
    std::vector<int64_t> sizes{3, 0, 7};
};

static std::vector<unsigned char> image(const Shape &s, const char *magic = "IVFPQ01")
{
    std::vector<unsigned char> b(32, 0);
    std::memcpy(b.data(), magic, std::strlen(magic) < 8 ? std::strlen(magic) : 8);
    std::memcpy(b.data() + 8, &s.d, 4);
    std::memcpy(b.data() + 12, &s.nlist, 4);
    std::memcpy(b.data() + 16, &s.m, 4);
    std::memcpy(b.data() + 20, &s.nbits, 4);
    std::memcpy(b.data() + 24, &s.ntotal, 8);
    auto put = [&](size_t bytes, unsigned char fillv) { b.insert(b.end(), bytes, fillv); };
    const size_t dsub = s.m ? s.d / s.m : 0;
    put((size_t)s.nlist * s.d * 4, 0);           // centroids (zeros)
    put((size_t)s.m * 256 * dsub * 4, 0);        // codebooks
    for (size_t l = 0; l < s.nlist; ++l) {       // list sizes
        int64_t v = l < s.sizes.size() ? s.sizes[l] : 0;
        const unsigned char *p = reinterpret_cast<const unsigned char *>(&v);
        b.insert(b.end(), p, p + 8);
    }
    put((size_t)s.ntotal * s.m, 7);              // codes
    for (uint64_t i = 0; i < s.ntotal; ++i) {    // ids
        int64_t v = (int64_t)i;
        const unsigned char *p = reinterpret_cast<const unsigned char *>(&v);
        b.insert(b.end(), p, p + 8);
    }
    return b;
}

static std::string write_file(const std::string &dir, const std::string &name,
                              const unsigned char *data, size_t n)
{
    const std::string path = dir + "/" + name;
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f)
        return path;
    if (n)
        std::fwrite(data, 1, n, f);
    std::fclose(f);
    return path;
}

static ivfpq_status validate(const std::string &dir, const std::string &name,
                             const std::vector<unsigned char> &b, size_t n)
{
    return ivfpq_validate_index_file(write_file(dir, name, b.data(), n).c_str());
}

int main(int argc, char **argv)
{
    if (argc < 2) {
        std::fprintf(stderr, "usage: %s scratch-dir\n", argv[0]);
        return 2;
    }
    const std::string dir = argv[1];

    // --- index files --------------------------------------------------------
    const Shape good;
    const std::vector<unsigned char> ok = image(good);
    CHECK(validate(dir, "good", ok, ok.size()) == IVFPQ_OK, "valid file");
    // truncated at every length up to the full body (header boundary, each array)
    for (size_t n = 0; n < ok.size(); n += (n < 40 ? 1 : 13))
        CHECK(validate(dir, "trunc", ok, n) == IVFPQ_E_FORMAT, "truncated file");
    {
        std::vector<unsigned char> t = ok;
        t.push_back(0);
        CHECK(validate(dir, "trail", t, t.size()) == IVFPQ_E_FORMAT, "trailing byte");
    }
    {
        const std::vector<unsigned char> b = image(good, "IVFPQ02");
        CHECK(validate(dir, "magic", b, b.size()) == IVFPQ_E_FORMAT, "bad magic");
    }
    {
        Shape s;
        s.sizes = {3, 0, 6}; // sum 9 != ntotal 10
        const std::vector<unsigned char> b = image(s);
        CHECK(validate(dir, "sum", b, b.size()) == IVFPQ_E_FORMAT, "sizes not adding up");
        s.sizes = {-1, 4, 7}; // sum 10 with a negative size
        const std::vector<unsigned char> c = image(s);
        CHECK(validate(dir, "neg", c, c.size()) == IVFPQ_E_FORMAT, "negative list size");
        s.sizes = {INT64_MAX, INT64_MAX, 12}; // a sum that would overflow
        const std::vector<unsigned char> e = image(s);
        CHECK(validate(dir, "ovf", e, e.size()) == IVFPQ_E_FORMAT, "overflowing list sizes");
        // sizes whose sum wraps around to exactly ntotal (10 + 2 (2^63 - 1) + 2
        // = 10 modulo 2^64): each non-negative, the wrapped sum right
        s.nlist = 4;
        s.sizes = {10, INT64_MAX, INT64_MAX, 2};
        const std::vector<unsigned char> g2 = image(s);
        CHECK(validate(dir, "ovf2", g2, g2.size()) == IVFPQ_E_FORMAT, "sizes wrapping to ntotal");
    }
    {
        struct Bad {
            uint32_t d, nlist, m, nbits;
            uint64_t ntotal;
            const char *what;
        } bad[] = {
            {0, 3, 2, 8, 10, "d 0"},
            {2000, 3, 2, 8, 10, "d above 1024"},
            {8, 0, 2, 8, 10, "nlist 0"},
            {8, 3, 3, 8, 10, "m not dividing d"},
            {8, 3, 0, 8, 10, "m 0"},
            {8, 3, 2, 4, 10, "nbits 4"},
            {8, 3, 2, 8, 0xFFFFFFFFull, "ntotal 2^32 - 1"},
            {8, 3, 2, 8, 1ull << 40, "ntotal 2^40"},
        };
        for (const Bad &x : bad) {
            std::vector<unsigned char> b = ok; // header fields over a valid body
            std::memcpy(b.data() + 8, &x.d, 4);
            std::memcpy(b.data() + 12, &x.nlist, 4);
            std::memcpy(b.data() + 16, &x.m, 4);
            std::memcpy(b.data() + 20, &x.nbits, 4);
            std::memcpy(b.data() + 24, &x.ntotal, 8);
            CHECK(validate(dir, "shape", b, b.size()) == IVFPQ_E_FORMAT, x.what);
        }
        // huge but legal declared shapes in a small file: rejected by size
        std::vector<unsigned char> b = ok;
        const uint32_t big_nlist = 1u << 30, big_d = 1024;
        std::memcpy(b.data() + 8, &big_d, 4);
        std::memcpy(b.data() + 12, &big_nlist, 4);
        CHECK(validate(dir, "huge", b, b.size()) == IVFPQ_E_FORMAT, "huge declared shape");
        std::vector<unsigned char> c = ok;
        const uint64_t big_total = 0xFFFFFFFEull;
        std::memcpy(c.data() + 24, &big_total, 8);
        CHECK(validate(dir, "hugetotal", c, c.size()) == IVFPQ_E_FORMAT, "huge declared ntotal");
    }
    {
        Shape s; // an index with no entries: valid
        s.ntotal = 0;
        s.sizes = {0, 0, 0};
        const std::vector<unsigned char> b = image(s);
        CHECK(validate(dir, "empty", b, b.size()) == IVFPQ_OK, "index with no entries");
    }
    CHECK(ivfpq_validate_index_file(nullptr) == IVFPQ_E_INVALID_ARG, "NULL path");
    CHECK(ivfpq_validate_index_file((dir + "/does-not-exist").c_str()) == IVFPQ_E_IO,
          "missing file");
    CHECK(ivfpq_validate_index_file(dir.c_str()) != IVFPQ_OK, "a directory");
    {
        ivfpq_index *ix = reinterpret_cast<ivfpq_index *>(&failures); // must stay untouched on failure
        const std::vector<unsigned char> b = image(good, "XXXXXXX");
        const std::string p = write_file(dir, "badload", b.data(), b.size());
        CHECK(ivfpq_load_index(p.c_str(), 0, &ix) == IVFPQ_E_FORMAT && ix == nullptr,
              "load of a bad file");
        CHECK(ivfpq_load_index(p.c_str(), 0, nullptr) == IVFPQ_E_INVALID_ARG, "load with NULL out");
    }

    // --- host arrays ----------------------------------------------------------
    {
        std::vector<float> cent(8 * 3, 0.f), books(2 * 256 * 4, 0.f);
        std::vector<int64_t> sizes{3, 0, 7}, ids(10);
        std::vector<uint8_t> codes(10 * 2, 1);
        ivfpq_host_index h{8, 3, 2, 8, 10, cent.data(), books.data(), sizes.data(), codes.data(),
                           ids.data()};
        CHECK(ivfpq_validate_host_index(&h) == IVFPQ_OK, "valid host index");
        CHECK(ivfpq_validate_host_index(nullptr) == IVFPQ_E_INVALID_ARG, "NULL host index");
        ivfpq_host_index b = h;
        b.centroids = nullptr;
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_E_INVALID_ARG, "NULL centroids");
        b = h;
        b.codes = nullptr;
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_E_INVALID_ARG, "NULL codes");
        b = h;
        b.ntotal = 0;
        b.codes = nullptr;
        b.ids = nullptr;
        std::vector<int64_t> zero{0, 0, 0};
        b.list_sizes = zero.data();
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_OK, "empty host index without arrays");
        b = h;
        std::vector<int64_t> neg{-2, 5, 7};
        b.list_sizes = neg.data();
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_E_FORMAT, "negative host list size");
        b = h;
        b.m = 3;
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_E_FORMAT, "host m not dividing d");
        b = h;
        b.nbits = 16;
        CHECK(ivfpq_validate_host_index(&b) == IVFPQ_E_FORMAT, "host nbits 16");
        ivfpq_index *ix = nullptr;
        b = h;
        b.ids = nullptr;
        CHECK(ivfpq_load_index_host(&b, 0, &ix) == IVFPQ_E_INVALID_ARG && ix == nullptr,
              "load of bad host arrays");
        CHECK(ivfpq_load_index_host(&h, 0, nullptr) == IVFPQ_E_INVALID_ARG, "host load, NULL out");
    }

    // --- status strings and argument checks before device work -----------------
    for (int s = 0; s <= 7; ++s) {
        const char *t = ivfpq_status_string((ivfpq_status)s);
        CHECK(t != nullptr && t[0] != '\0', "status string");
    }
    CHECK(ivfpq_status_string((ivfpq_status)1234) != nullptr, "unknown status string");
    CHECK(ivfpq_last_error() != nullptr, "last error");
    ivfpq_info info;
    CHECK(ivfpq_index_info(nullptr, &info) == IVFPQ_E_INVALID_ARG, "info of NULL index");
    ivfpq_search_params p{8, 10, 0, 0, 0, 0};
    CHECK(ivfpq_search_ex(nullptr, &p, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
              IVFPQ_E_INVALID_ARG,
          "search of NULL index");
    CHECK(ivfpq_profile_begin(nullptr, 4) == IVFPQ_E_INVALID_ARG, "profile of NULL index");
    ivfpq_timings tm;
    CHECK(ivfpq_profile_end(nullptr, &tm) == IVFPQ_E_INVALID_ARG, "profile end of NULL index");
    ivfpq_flat_timings ftm;
    CHECK(ivfpq_flat_profile_end(nullptr, &ftm) == IVFPQ_E_INVALID_ARG, "flat profile of NULL");
    ivfpq_free_index(nullptr);
    ivfpq_flat_free(nullptr);
#ifdef PLANT_OVERFLOW
    // a read one past a heap array: a build whose sanitizer works stops here
    unsigned char *arr = new unsigned char[ok.size()];
    volatile unsigned char past = arr[ok.size()];
    (void)past;
    delete[] arr;
#endif

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host driver: all checks passed\n");
    return 0;
}
