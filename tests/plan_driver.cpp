// Host driver for the search work plan (csrc/plan.hpp): the same functions
// the device plan and scan kernels call, run on the CPU.  Reads cases from
// stdin, prints each query's plan and each item's pieces.
//
// input:  T, then per case: nlist nq nprobe kw target per_cu cus align,
//         list sizes [nlist], probes [nq * nprobe] (-1 or out of range: none)
// output: per case "case imax max_items grid", then per query
//         "query total chunk count" and per item "item start stop npieces
//         (list b e)*"
#include "plan.hpp"

#include <cstdio>
#include <vector>

int main()
{
    int T = 0;
    if (std::scanf("%d", &T) != 1)
        return 1;
    for (int t = 0; t < T; ++t) {
        long long nlist, nq, nprobe, kw, target, per_cu, cus, align;
        if (std::scanf("%lld %lld %lld %lld %lld %lld %lld %lld", &nlist, &nq, &nprobe, &kw,
                       &target, &per_cu, &cus, &align) != 8)
            return 1;
        std::vector<unsigned long long> sizes(nlist);
        for (auto &v : sizes)
            if (std::scanf("%llu", &v) != 1)
                return 1;
        std::vector<long long> probes(nq * nprobe);
        for (auto &v : probes)
            if (std::scanf("%lld", &v) != 1)
                return 1;
        const uint32_t imax = ivfpq::items_per_query(nq, (int)kw);
        const int64_t max_items = nq * (int64_t)imax;
        std::printf("case %u %lld %lld\n", imax, (long long)max_items,
                    (long long)ivfpq::scan_grid((int)per_cu, (int)cus, max_items));
        for (long long q = 0; q < nq; ++q) {
            uint64_t e = 0;
            for (long long p = 0; p < nprobe; ++p) {
                const long long l = probes[q * nprobe + p];
                if (l >= 0 && l < nlist)
                    e += sizes[l];
            }
            const uint32_t total = (uint32_t)e;
            const ivfpq::QueryPlan qp =
                ivfpq::plan_query(total, (uint32_t)target, imax, (uint32_t)align);
            std::printf("query %u %u %u\n", total, qp.chunk, qp.count);
            for (uint32_t i = 0; i < qp.count; ++i) {
                uint32_t start, stop;
                ivfpq::item_range(i, qp.chunk, total, &start, &stop);
                std::vector<long long> out;
                uint32_t acc = 0;
                for (long long p = 0; p < nprobe; ++p) {
                    const long long l = probes[q * nprobe + p];
                    const uint32_t sz = (l >= 0 && l < nlist) ? (uint32_t)sizes[l] : 0u;
                    uint32_t b, en;
                    if (ivfpq::piece_of(acc, acc + sz, start, stop, &b, &en)) {
                        out.push_back(l);
                        out.push_back(b);
                        out.push_back(en);
                    }
                    acc += sz;
                }
                std::printf("item %u %u %zu", start, stop, out.size() / 3);
                for (long long v : out)
                    std::printf(" %lld", v);
                std::printf("\n");
            }
        }
    }
    return 0;
}
