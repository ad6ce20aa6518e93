// Index building on the device: PQ encoding of database vectors.
//
// "Custom 8-bit floating point value format for reducing shared memory bank
// conflict in ANN search", IVFPQ section, index-building steps 2-3: the
// residual of a vector to the centroid of its cluster is cut into m
// sub-vectors of dsub consecutive dims and each one is quantized; with the
// product quantizer of "Billion-scale similarity search with GPUs" (IVFADC
// section: m quantizers of 256 reproduction values each on the residual of
// the coarse quantizer q1).  A quantizer returns its nearest reproduction
// value in squared L2; ties go to the smaller codeword.  The cluster (q1) is
// the coarse step's nearest list, computed before this kernel.
//
// A sub-quantizer's distance is evaluated exactly as the search evaluates a
// table entry F_j(v): r = x - c_l in float32, then sum_s (r_s - C_j[v][s])^2
// with fused multiply-adds over the dims in order.
#include "common.hpp"
#include "internal.hpp"

#include <hipcub/hipcub.hpp>

namespace ivfpq {

// Workgroup: 64 vectors (vector v0 + l in lane l of every wave); its four
// waves take the sub-quantizers j = wave, wave + 4, ...  For sub-quantizer j a
// lane scans the 256 codewords in order and keeps the first smallest
// distance.  The codeword being tested is the same for every lane of the wave,
// so its values arrive through scalar loads; the residual sub-vector stays in
// registers (DSUB > 0) or is re-formed per codeword from memory (DSUB == 0,
// any dsub).  Codes are staged in LDS and written as whole rows.
template <int DSUB>
__global__ __launch_bounds__(256) void encode_kernel(const float *__restrict__ x, int64_t n, int d,
                                                     int m, int dsub_rt,
                                                     const int32_t *__restrict__ lists, int nlist,
                                                     const float *__restrict__ centroids,
                                                     const float *__restrict__ codebooks,
                                                     uint8_t *__restrict__ codes)
{
    extern __shared__ uint8_t stage[]; // [64][m]
    const int dsub = DSUB > 0 ? DSUB : dsub_rt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t v0 = (int64_t)blockIdx.x * 64;
    const int64_t i = v0 + lane;
    const bool valid = i < n;
    int l = valid ? lists[i] : 0;
    // the coarse step returns lists in [0, nlist); anything else reads list 0
    // rather than memory outside the centroids
    l = (unsigned)l < (unsigned)nlist ? l : 0;
    const float *xi = x + (valid ? i : 0) * d;
    const float *cl = centroids + (size_t)l * d;

    for (int j = wave; j < m; j += 4) {
        const float *cb = codebooks + (size_t)j * 256 * dsub;
        float best = INFINITY;
        int arg = 0;
        if constexpr (DSUB > 0) {
            float r[DSUB];
#pragma unroll
            for (int s = 0; s < DSUB; ++s)
                r[s] = xi[j * DSUB + s] - cl[j * DSUB + s];
            for (int w = 0; w < 256; ++w) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < DSUB; ++s) {
                    const float df = r[s] - cb[w * DSUB + s];
                    acc = fmaf(df, df, acc);
                }
                if (acc < best) {
                    best = acc;
                    arg = w;
                }
            }
        } else {
            for (int w = 0; w < 256; ++w) {
                float acc = 0.f;
                for (int s = 0; s < dsub; ++s) {
                    const float df = (xi[j * dsub + s] - cl[j * dsub + s]) - cb[w * dsub + s];
                    acc = fmaf(df, df, acc);
                }
                if (acc < best) {
                    best = acc;
                    arg = w;
                }
            }
        }
        stage[lane * m + j] = (uint8_t)arg;
    }
    __syncthreads();
    const int64_t rows = n - v0 < 64 ? n - v0 : 64;
    for (int64_t b = threadIdx.x; b < rows * m; b += 256)
        codes[v0 * m + b] = stage[b];
}

template <int DSUB>
static hipError_t encode_variant(const DeviceIndex &ix, const float *x, int64_t n,
                                 const int32_t *lists, uint8_t *codes, hipStream_t stream)
{
    const int64_t blocks = (n + 63) / 64;
    const size_t lds = (size_t)64 * ix.m;
    hipLaunchKernelGGL(encode_kernel<DSUB>, dim3((unsigned)blocks), dim3(256), lds, stream, x, n,
                       ix.d, ix.m, ix.d / ix.m, lists, ix.nlist, ix.centroids, ix.codebooks, codes);
    return hipGetLastError();
}

hipError_t launch_encode(const DeviceIndex &ix, const float *x, int64_t n, const int32_t *lists,
                         uint8_t *codes, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    if ((n + 63) / 64 > 0x7FFFFFFF || (size_t)64 * ix.m > 64 * 1024)
        return hipErrorInvalidValue;
    switch (ix.d / ix.m) {
    case 2:
        return encode_variant<2>(ix, x, n, lists, codes, stream);
    case 3:
        return encode_variant<3>(ix, x, n, lists, codes, stream);
    case 4:
        return encode_variant<4>(ix, x, n, lists, codes, stream);
    case 8:
        return encode_variant<8>(ix, x, n, lists, codes, stream);
    case 12:
        return encode_variant<12>(ix, x, n, lists, codes, stream);
    case 16:
        return encode_variant<16>(ix, x, n, lists, codes, stream);
    default:
        return encode_variant<0>(ix, x, n, lists, codes, stream);
    }
}

// ---------------------------------------------------------------------------
// k-means (Lloyd's algorithm), the update step: each center becomes the mean
// of the vectors assigned to it; a center with no vector keeps its value.
// "Custom 8-bit floating point value format for reducing shared memory bank
// conflict in ANN search", IVFPQ section, index-building step 1 (clusters by
// k-means).  The assignment step is the coarse kernel with nprobe 1.
// ---------------------------------------------------------------------------

__global__ void kmeans_zero_kernel(double *__restrict__ sums, int64_t nsum,
                                   int32_t *__restrict__ counts, int k)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nsum)
        sums[i] = 0.0;
    if (i < k)
        counts[i] = 0;
}

// One wave per vector: its coordinates go into its center's sums with
// double-precision atomic adds (exact enough that the float32 mean is the
// same whatever the order of the adds, up to a rounding-boundary case).
__global__ __launch_bounds__(256) void kmeans_accumulate_kernel(
    const float *__restrict__ x, int64_t n, int d, const int32_t *__restrict__ assign, int k,
    double *__restrict__ sums, int32_t *__restrict__ counts)
{
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= n)
        return;
    const int a = assign[i];
    if ((unsigned)a >= (unsigned)k)
        return;
    const float *xi = x + i * d;
    double *s = sums + (size_t)a * d;
    for (int t = lane; t < d; t += 64)
        unsafeAtomicAdd(s + t, (double)xi[t]);
    if (lane == 0)
        atomicAdd(counts + a, 1);
}

__global__ void kmeans_finalize_kernel(float *__restrict__ centers, const double *__restrict__ sums,
                                       const int32_t *__restrict__ counts, int k, int d)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)k * d)
        return;
    const int cnt = counts[e / d];
    if (cnt > 0)
        centers[e] = (float)(sums[e] / (double)cnt);
}

hipError_t launch_kmeans_update(const float *x, int64_t n, int d, const int32_t *assign, int k,
                                double *sums, int32_t *counts, float *centers, hipStream_t stream)
{
    const int64_t nsum = (int64_t)k * d;
    const int64_t zn = nsum > k ? nsum : k;
    hipLaunchKernelGGL(kmeans_zero_kernel, dim3((unsigned)((zn + 255) / 256)), dim3(256), 0,
                       stream, sums, nsum, counts, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0)
        return e;
    hipLaunchKernelGGL(kmeans_accumulate_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0,
                       stream, x, n, d, assign, k, sums, counts);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(kmeans_finalize_kernel, dim3((unsigned)((nsum + 255) / 256)), dim3(256), 0,
                       stream, centers, sums, counts, k, d);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// list-major layout of encoded entries: "Custom 8-bit floating point value
// format for reducing shared memory bank conflict in ANN search", IVFPQ
// section, index-building step 4 (the codes are stored with their cluster
// membership); "Billion-scale similarity search with GPUs", IVFADC section
// (the codes of a list are stored contiguously).  Entries keep their input
// order inside a list (a stable sort by list number).
// ---------------------------------------------------------------------------

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

__global__ void iota_kernel(int32_t *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = (int32_t)i;
}

// Entries per list from the sorted list numbers: the distance between the
// first positions holding a number >= l and >= l + 1 (binary searches; one
// thread per list, no contended counters).
__global__ void list_count_sorted_kernel(const int32_t *__restrict__ keys, int64_t n, int nlist,
                                         uint32_t *__restrict__ counts)
{
    const int l = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (l >= nlist)
        return;
    auto first_at_least = [&](int v) {
        int64_t lo = 0, hi = n;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (keys[mid] < v)
                lo = mid + 1;
            else
                hi = mid;
        }
        return lo;
    };
    counts[l] = (uint32_t)(first_at_least(l + 1) - first_at_least(l));
}

// Position p of the layout takes entry perm[p]: its code row and its id (the
// row number when no ids are given).
__global__ void gather_entries_kernel(const int32_t *__restrict__ perm, int64_t n, int m,
                                      const uint8_t *__restrict__ codes_in,
                                      const int64_t *__restrict__ ids_in,
                                      uint8_t *__restrict__ codes_out,
                                      int64_t *__restrict__ ids_out)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n)
        return;
    const int64_t src = perm[p];
    for (int j = 0; j < m; ++j)
        codes_out[p * m + j] = codes_in[src * m + j];
    ids_out[p] = ids_in ? ids_in[src] : src;
}

hipError_t launch_list_layout(const int32_t *lists, int64_t n, int nlist, int m,
                              const uint8_t *codes_in, const int64_t *ids_in, uint32_t *counts,
                              int32_t *keys_out, int32_t *perm_in, int32_t *perm_out,
                              void *sort_tmp, size_t *sort_tmp_bytes, uint8_t *codes_out,
                              int64_t *ids_out, hipStream_t stream)
{
    int bits = 1;
    while (bits < 31 && (1ll << bits) < (int64_t)nlist)
        ++bits;
    if (!sort_tmp) // size query
        return hipcub::DeviceRadixSort::SortPairs(nullptr, *sort_tmp_bytes, lists, keys_out,
                                                  perm_in, perm_out, (int)n, 0, bits, stream);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    const unsigned cblocks = (unsigned)((nlist + 255) / 256);
    if (n == 0) {
        hipLaunchKernelGGL(zero_u32_kernel, dim3(cblocks), dim3(256), 0, stream, counts,
                           (int64_t)nlist);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(iota_kernel, dim3(blocks), dim3(256), 0, stream, perm_in, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    e = hipcub::DeviceRadixSort::SortPairs(sort_tmp, *sort_tmp_bytes, lists, keys_out, perm_in,
                                           perm_out, (int)n, 0, bits, stream);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(list_count_sorted_kernel, dim3(cblocks), dim3(256), 0, stream, keys_out, n,
                       nlist, counts);
    hipLaunchKernelGGL(gather_entries_kernel, dim3(blocks), dim3(256), 0, stream, perm_out, n, m,
                       codes_in, ids_in, codes_out, ids_out);
    return hipGetLastError();
}

} // namespace ivfpq
