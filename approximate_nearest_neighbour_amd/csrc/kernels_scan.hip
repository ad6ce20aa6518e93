// IVF-PQ kernels for gfx950: coarse top-nprobe, residual lookup tables in LDS,
// wave64 code scan with register top-k, cross-wave merge.
//
// Definitions ("Custom 8-bit floating point value format for reducing shared
// memory bank conflict in ANN search", IVFPQ section, search steps 1-5 and
// Eq. (1); "Billion-scale similarity search with GPUs", IVFADC section):
//   coarse   D[q,l] = |x_q - c_l|^2, the nprobe smallest are probed;
//   table    F_j(v) = sum_{t<dsub} (r[j dsub + t] - C_j[v][t])^2, r = x_q - c_l;
//   scan     R_i = sum_{j<m} F_j(code_i[j]) for every entry i of the list;
//   top-k    the k smallest R over all probed lists.
//
// Work decomposition: one workgroup of four waves per query.  For each
// probed list the workgroup writes the residual to LDS, builds the m x 256
// table in LDS (thread v computes codeword v of every sub-quantizer, in the
// difference form: a sum of squares, no cancellation), then the four waves
// scan the list with one entry per lane (the m code bytes of 64 consecutive
// entries are one contiguous 64*m-byte stretch: fully coalesced), each wave
// keeping its own register top-k.  The waves share a threshold through LDS
// (the smallest k-th value any wave holds).  At the end the four sorted
// top-k arrays are merged by bitonic merges and the ids gathered.
#include "internal.hpp"
#include "wave_select.hpp"

#include <hip/hip_fp16.h>

namespace ivfpq {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------

// Table for one (query, list): thread v (0..255) computes F_j(v) for every j.
template <bool F16>
__device__ __forceinline__ void build_table(const float *__restrict__ resid,
                                            const float *__restrict__ codebooks, int m, int dsub,
                                            void *lut)
{
    const int v = threadIdx.x;
    for (int j = 0; j < m; ++j) {
        const float *cw = codebooks + ((size_t)j * 256 + v) * dsub;
        const float *rj = resid + j * dsub;
        float acc = 0.f;
        for (int t = 0; t < dsub; ++t) {
            const float df = rj[t] - cw[t];
            acc = fmaf(df, df, acc);
        }
        if constexpr (F16)
            reinterpret_cast<__half *>(lut)[j * 256 + v] = __float2half_rn(acc);
        else
            reinterpret_cast<float *>(lut)[j * 256 + v] = acc;
    }
}

template <bool F16>
__device__ __forceinline__ float table_at(const void *lut, int idx)
{
    if constexpr (F16)
        return __half2float(reinterpret_cast<const __half *>(lut)[idx]);
    else
        return reinterpret_cast<const float *>(lut)[idx];
}

// R = sum_j F_j(code[j]), j ascending.  m % 4 == 0 reads the code row as
// 32-bit words; other m byte by byte.
template <bool F16>
__device__ __forceinline__ float adc_sum(const uint8_t *__restrict__ code, int m, const void *lut)
{
    float r = 0.f;
    if ((m & 3) == 0) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(code);
        for (int j4 = 0; j4 < (m >> 2); ++j4) {
            const uint32_t word = w[j4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                r += table_at<F16>(lut, (j4 * 4 + b) * 256 + ((word >> (8 * b)) & 255u));
        }
    } else {
        for (int j = 0; j < m; ++j)
            r += table_at<F16>(lut, j * 256 + code[j]);
    }
    return r;
}

__device__ __forceinline__ void publish_bound(uint32_t *word, float kth)
{
    if (kth < INFINITY && lane_id() == 0)
        atomicMin(word, float_order_key(kth));
}

__device__ __forceinline__ float read_bound(const uint32_t *word)
{
    return float_from_order_key(__atomic_load_n(word, __ATOMIC_RELAXED));
}

// Merge the top-k of the four waves (each sorted ascending in registers)
// through LDS scratch; wave 0 ends with the workgroup's top-k.
template <int NW>
__device__ __forceinline__ void merge_waves(WaveTopK<NW> &sel, float *mk, uint32_t *mv)
{
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if (wave > 0)
        sel.store(mk + (wave - 1) * 64 * NW, mv + (wave - 1) * 64 * NW);
    __syncthreads();
    if (wave == 0) {
#pragma unroll 1
        for (int w = 0; w < kWaves - 1; ++w)
            sel.merge_sorted(mk + w * 64 * NW, mv + w * 64 * NW);
    }
}

// ---------------------------------------------------------------------------
// coarse: |x - c_l|^2 for every list (direct differences, float32), top-nprobe
// ---------------------------------------------------------------------------

template <int NW>
__global__ __launch_bounds__(kBlock) void coarse_kernel(const float *__restrict__ queries, int d,
                                                        int nlist, int nprobe,
                                                        const float *__restrict__ centroids,
                                                        int32_t *__restrict__ probes,
                                                        float *__restrict__ probe_d)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int dpad = (d + 3) & ~3;
    float *x = reinterpret_cast<float *>(smem);
    uint32_t *bound = reinterpret_cast<uint32_t *>(x + dpad);
    float *mk = reinterpret_cast<float *>(bound + 4);
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kWaves - 1) * 64 * NW);

    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int t = tid; t < d; t += kBlock)
        x[t] = queries[q * d + t];
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();

    WaveTopK<NW> sel;
    sel.init(nprobe);
    int since = 0;
    for (int base = wave * 64; base < nlist; base += kBlock) {
        const int l = base + lane;
        float dist = INFINITY;
        if (l < nlist) {
            const float *c = centroids + (size_t)l * d;
            float acc = 0.f;
            if ((d & 3) == 0) {
                for (int t = 0; t < d; t += 4) {
                    const float4 cv = *reinterpret_cast<const float4 *>(c + t);
                    float df = x[t] - cv.x;
                    acc = fmaf(df, df, acc);
                    df = x[t + 1] - cv.y;
                    acc = fmaf(df, df, acc);
                    df = x[t + 2] - cv.z;
                    acc = fmaf(df, df, acc);
                    df = x[t + 3] - cv.w;
                    acc = fmaf(df, df, acc);
                }
            } else {
                for (int t = 0; t < d; ++t) {
                    const float df = x[t] - c[t];
                    acc = fmaf(df, df, acc);
                }
            }
            dist = acc;
        }
        sel.push(dist, (uint32_t)l);
        if (++since == 8) {
            since = 0;
            publish_bound(bound, sel.kth);
            sel.bound(read_bound(bound));
        }
    }
    sel.flush();
    merge_waves<NW>(sel, mk, mv);
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int e = r * 64 + lane;
            if (e < nprobe) {
                probes[q * nprobe + e] = (int32_t)sel.wv[r];
                if (probe_d)
                    probe_d[q * nprobe + e] = sel.wk[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// scan: per probed list, table in LDS + code scan + register top-k
// ---------------------------------------------------------------------------

template <int NW, bool F16, bool SCAN_ONLY>
__global__ __launch_bounds__(kBlock) void scan_kernel(
    const float *__restrict__ queries, int d, int m, int nlist, int nprobe, int k,
    const float *__restrict__ centroids, const float *__restrict__ codebooks,
    const uint32_t *__restrict__ list_off, const uint8_t *__restrict__ codes,
    const int64_t *__restrict__ ids, const int32_t *__restrict__ probes, float *__restrict__ out_d,
    int64_t *__restrict__ out_i)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int dpad = (d + 3) & ~3;
    float *resid = reinterpret_cast<float *>(smem);
    uint32_t *bound = reinterpret_cast<uint32_t *>(resid + dpad);
    void *lut = reinterpret_cast<void *>(bound + 4);
    float *mk = reinterpret_cast<float *>(lut); // reused after the last scan
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kWaves - 1) * 64 * NW);

    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int dsub = d / m;
    const float *x = queries + q * d;
    if (tid == 0)
        *bound = float_order_key(INFINITY);

    WaveTopK<NW> sel;
    sel.init(k);
    float sink = INFINITY;

    for (int p = 0; p < nprobe; ++p) {
        const int l = probes[q * nprobe + p];
        if ((unsigned)l >= (unsigned)nlist)
            continue; // block-uniform: an empty probe slot
        const uint32_t off = list_off[l];
        const uint32_t n = list_off[l + 1] - off;
        __syncthreads(); // everyone is done with the previous table
        for (int t = tid; t < d; t += kBlock)
            resid[t] = x[t] - centroids[(size_t)l * d + t];
        __syncthreads();
        build_table<F16>(resid, codebooks, m, dsub, lut);
        __syncthreads();
        if constexpr (!SCAN_ONLY)
            sel.bound(read_bound(bound));
        for (uint32_t base = wave * 64; base < n; base += kBlock) {
            const uint32_t i = base + lane;
            float r = INFINITY;
            if (i < n)
                r = adc_sum<F16>(codes + (size_t)(off + i) * m, m, lut);
            if constexpr (SCAN_ONLY)
                sink = fminf(sink, r);
            else
                sel.push(r, off + i);
        }
        if constexpr (!SCAN_ONLY)
            publish_bound(bound, sel.kth);
    }

    if constexpr (SCAN_ONLY) {
        // keep every distance live: the wave minimum goes to the output
        for (int s = 32; s >= 1; s >>= 1)
            sink = fminf(sink, __shfl_xor(sink, s));
        if (lane == 0 && wave < k)
            out_d[q * k + wave] = sink;
        return;
    } else {
        sel.flush();
        merge_waves<NW>(sel, mk, mv);
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < NW; ++r) {
                const int e = r * 64 + lane;
                if (e < k) {
                    out_d[q * k + e] = sel.wk[r];
                    out_i[q * k + e] = sel.wv[r] == kSentinel ? -1 : ids[sel.wv[r]];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// row-wise k-selection (the selection primitive on its own)
// ---------------------------------------------------------------------------

template <int NW>
__global__ __launch_bounds__(kBlock) void select_kernel(const float *__restrict__ keys, int64_t n,
                                                        int k, float *__restrict__ out_d,
                                                        int32_t *__restrict__ out_pos)
{
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *bound = reinterpret_cast<uint32_t *>(smem);
    float *mk = reinterpret_cast<float *>(bound + 4);
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kWaves - 1) * 64 * NW);
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();
    WaveTopK<NW> sel;
    sel.init(k);
    const float *rk = keys + row * n;
    int since = 0;
    for (int64_t base = wave * 64; base < n; base += kBlock) {
        const int64_t i = base + lane;
        sel.push(i < n ? rk[i] : INFINITY, (uint32_t)i);
        if (++since == 4) {
            since = 0;
            publish_bound(bound, sel.kth);
            sel.bound(read_bound(bound));
        }
    }
    sel.flush();
    merge_waves<NW>(sel, mk, mv);
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int e = r * 64 + lane;
            if (e < k) {
                out_d[row * k + e] = sel.wk[r];
                out_pos[row * k + e] = sel.wv[r] == kSentinel ? -1 : (int32_t)sel.wv[r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// tables to global memory (verification entry point)
// ---------------------------------------------------------------------------

template <bool F16>
__global__ __launch_bounds__(kBlock) void lut_kernel(const float *__restrict__ queries, int d,
                                                     int m, int nprobe,
                                                     const float *__restrict__ centroids,
                                                     const float *__restrict__ codebooks,
                                                     const int32_t *__restrict__ probes,
                                                     float *__restrict__ out)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int dpad = (d + 3) & ~3;
    float *resid = reinterpret_cast<float *>(smem);
    void *lut = reinterpret_cast<void *>(resid + dpad);
    const int64_t pair = blockIdx.x;
    const int64_t q = pair / nprobe;
    const int l = probes[pair];
    for (int t = threadIdx.x; t < d; t += kBlock)
        resid[t] = queries[q * d + t] - centroids[(size_t)l * d + t];
    __syncthreads();
    build_table<F16>(resid, codebooks, m, d / m, lut);
    __syncthreads();
    for (int e = threadIdx.x; e < m * 256; e += kBlock)
        out[pair * m * 256 + e] = table_at<F16>(lut, e);
}

__global__ void cnorm_kernel(const float *__restrict__ c, int d, int nlist, float *__restrict__ out)
{
    const int l = blockIdx.x * blockDim.x + threadIdx.x;
    if (l < nlist) {
        float s = 0.f;
        for (int t = 0; t < d; ++t)
            s = fmaf(c[(size_t)l * d + t], c[(size_t)l * d + t], s);
        out[l] = s;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int nw_for(int k)
{
    int nw = 1;
    while (nw * 64 < k)
        nw *= 2;
    return nw;
}

template <typename K>
static hipError_t set_lds(K kernel, size_t bytes)
{
    if (bytes > 64 * 1024)
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return hipSuccess;
}

template <int NW>
static hipError_t coarse_nw(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                            int32_t *probes, float *probe_d, hipStream_t stream)
{
    const size_t lds = (size_t)((ix.d + 3) & ~3) * 4 + 16 + (size_t)(kWaves - 1) * 64 * NW * 8;
    auto kern = coarse_kernel<NW>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nq), dim3(kBlock), lds, stream, queries, ix.d,
                       ix.nlist, nprobe, ix.centroids, probes, probe_d);
    return hipGetLastError();
}

hipError_t launch_coarse(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                         int32_t *probes, float *probe_d, hipStream_t stream)
{
    if (nq == 0)
        return hipSuccess;
    switch (nw_for(nprobe)) {
    case 1: return coarse_nw<1>(ix, queries, nq, nprobe, probes, probe_d, stream);
    case 2: return coarse_nw<2>(ix, queries, nq, nprobe, probes, probe_d, stream);
    case 4: return coarse_nw<4>(ix, queries, nq, nprobe, probes, probe_d, stream);
    case 8: return coarse_nw<8>(ix, queries, nq, nprobe, probes, probe_d, stream);
    default: return coarse_nw<16>(ix, queries, nq, nprobe, probes, probe_d, stream);
    }
}

template <int NW, bool F16, bool SO>
static hipError_t scan_variant(const DeviceIndex &ix, const SearchArgs &a, hipStream_t stream)
{
    const size_t table = (size_t)ix.m * 256 * (F16 ? 2 : 4);
    const size_t merge = (size_t)(kWaves - 1) * 64 * NW * 8;
    const size_t lds = (size_t)((ix.d + 3) & ~3) * 4 + 16 + (table > merge ? table : merge);
    auto kern = scan_kernel<NW, F16, SO>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)a.nq), dim3(kBlock), lds, stream, a.queries, ix.d,
                       ix.m, ix.nlist, a.nprobe, a.k, ix.centroids, ix.codebooks, ix.list_off, ix.codes,
                       ix.ids, a.probes, a.out_d, a.out_i);
    return hipGetLastError();
}

template <int NW>
static hipError_t scan_nw(const DeviceIndex &ix, const SearchArgs &a, hipStream_t stream)
{
    if (a.mode == 1)
        return a.lut ? scan_variant<NW, true, true>(ix, a, stream)
                     : scan_variant<NW, false, true>(ix, a, stream);
    return a.lut ? scan_variant<NW, true, false>(ix, a, stream)
                 : scan_variant<NW, false, false>(ix, a, stream);
}

hipError_t launch_scan(const DeviceIndex &ix, const SearchArgs &a, hipStream_t stream)
{
    if (a.nq == 0)
        return hipSuccess;
    switch (nw_for(a.k)) {
    case 1: return scan_nw<1>(ix, a, stream);
    case 2: return scan_nw<2>(ix, a, stream);
    case 4: return scan_nw<4>(ix, a, stream);
    case 8: return scan_nw<8>(ix, a, stream);
    default: return scan_nw<16>(ix, a, stream);
    }
}

hipError_t launch_luts(const DeviceIndex &ix, const float *queries, int64_t nq,
                       const int32_t *probes, int nprobe, int lut, float *out, hipStream_t stream)
{
    if (nq == 0)
        return hipSuccess;
    const size_t lds = (size_t)((ix.d + 3) & ~3) * 4 + (size_t)ix.m * 256 * 4;
    const unsigned grid = (unsigned)(nq * nprobe);
    if (lut) {
        hipError_t e = set_lds(lut_kernel<true>, lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(lut_kernel<true>, dim3(grid), dim3(kBlock), lds, stream, queries, ix.d,
                           ix.m, nprobe, ix.centroids, ix.codebooks, probes, out);
    } else {
        hipError_t e = set_lds(lut_kernel<false>, lds);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(lut_kernel<false>, dim3(grid), dim3(kBlock), lds, stream, queries,
                           ix.d, ix.m, nprobe, ix.centroids, ix.codebooks, probes, out);
    }
    return hipGetLastError();
}


template <int NW>
static hipError_t select_nw(const float *keys, int64_t rows, int64_t n, int k, float *out_d,
                            int32_t *out_pos, hipStream_t stream)
{
    const size_t lds = 16 + (size_t)(kWaves - 1) * 64 * NW * 8;
    hipLaunchKernelGGL(select_kernel<NW>, dim3((unsigned)rows), dim3(kBlock), lds, stream, keys, n,
                       k, out_d, out_pos);
    return hipGetLastError();
}

hipError_t launch_select(const float *keys, int64_t rows, int64_t n, int k, float *out_d,
                         int32_t *out_pos, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    switch (nw_for(k)) {
    case 1: return select_nw<1>(keys, rows, n, k, out_d, out_pos, stream);
    case 2: return select_nw<2>(keys, rows, n, k, out_d, out_pos, stream);
    case 4: return select_nw<4>(keys, rows, n, k, out_d, out_pos, stream);
    case 8: return select_nw<8>(keys, rows, n, k, out_d, out_pos, stream);
    default: return select_nw<16>(keys, rows, n, k, out_d, out_pos, stream);
    }
}

hipError_t launch_cnorms(const DeviceIndex &ix, hipStream_t stream)
{
    const int blocks = (ix.nlist + 255) / 256;
    hipLaunchKernelGGL(cnorm_kernel, dim3(blocks), dim3(256), 0, stream, ix.centroids, ix.d,
                       ix.nlist, ix.cnorms);
    return hipGetLastError();
}

} // namespace ivfpq
