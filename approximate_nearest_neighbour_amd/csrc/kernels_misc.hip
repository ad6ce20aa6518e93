// Auxiliary IVF-PQ kernels for gfx950: the coarse top-nprobe (float32
// direct differences), the row-wise k-selection on its own, the table
// writer used for verification.
//
// Coarse step on the vector ALUs ("Billion-scale similarity search with
// GPUs", IVFADC section; "Custom 8-bit floating point value format for
// reducing shared memory bank conflict in ANN search", IVFPQ search step 1):
// D[q,l] = |x_q - c_l|^2 for every list by direct differences, the nprobe
// smallest are probed.  Used where the matrix-core form does not apply
// (nprobe above 256 or very large d).  One workgroup of four waves per
// query; each wave streams a quarter of the centroids through a register
// top-k; the waves share a bound through LDS and end with a bitonic merge.
#include "common.hpp"
#include "internal.hpp"

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

// ---------------------------------------------------------------------------
// coarse: |x - c_l|^2 for every list (direct differences, float32), top-nprobe
// ---------------------------------------------------------------------------

template <int NW>
__global__ __launch_bounds__(kBlock) void coarse_kernel(const float *__restrict__ queries, int d,
                                                        int nlist, int nprobe,
                                                        const float *__restrict__ centroids,
                                                        int32_t *__restrict__ probes,
                                                        float *__restrict__ probe_d, int ip)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int dpad = (d + 3) & ~3;
    float *x = reinterpret_cast<float *>(smem);
    uint32_t *bound = reinterpret_cast<uint32_t *>(x + dpad);
    float *mk = reinterpret_cast<float *>(bound + 4);
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kWaves - 1) * 64 * NW);
    uint32_t *stage = mv + (kWaves - 1) * 64 * NW; // [kWaves][128]

    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    for (int t = tid; t < d; t += kBlock)
        x[t] = queries[q * d + t];
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();

    WaveTopK<NW> sel;
    sel.init(nprobe, stage + wave * 128);
    int since = 0;
    for (int base = wave * 64; base < nlist; base += kBlock) {
        const int l = base + lane;
        float dist = INFINITY;
        if (l < nlist) {
            const float *c = centroids + (size_t)l * d;
            float acc = 0.f;
            if (ip) {
                // inner-product metric: lists ranked by -<x, c_l>
                for (int t = 0; t < d; ++t)
                    acc = fmaf(x[t], c[t], acc);
                acc = -acc;
            } else if ((d & 3) == 0) {
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
    merge_waves<NW, kWaves>(sel, mk, mv);
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
    uint32_t *stage = mv + (kWaves - 1) * 64 * NW; // [kWaves][128]
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();
    WaveTopK<NW> sel;
    sel.init(k, stage + wave * 128);
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
    merge_waves<NW, kWaves>(sel, mk, mv);
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
                            int32_t *probes, float *probe_d, hipStream_t stream, bool ip)
{
    const size_t lds = (size_t)((ix.d + 3) & ~3) * 4 + 16 + (size_t)(kWaves - 1) * 64 * NW * 8 +
                       (size_t)kWaves * 512;
    auto kern = coarse_kernel<NW>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nq), dim3(kBlock), lds, stream, queries, ix.d,
                       ix.nlist, nprobe, ix.centroids, probes, probe_d, ip ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_coarse_valu(const DeviceIndex &ix, const float *queries, int64_t nq,
                              int nprobe, int32_t *probes, float *probe_d, hipStream_t stream,
                              bool ip)
{
    if (nq == 0)
        return hipSuccess;
    switch (nw_for(nprobe)) {
    case 1: return coarse_nw<1>(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
    case 2: return coarse_nw<2>(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
    case 4: return coarse_nw<4>(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
    case 8: return coarse_nw<8>(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
    default: return coarse_nw<16>(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
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
    const size_t lds = 16 + (size_t)(kWaves - 1) * 64 * NW * 8 + (size_t)kWaves * 512;
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
// ---------------------------------------------------------------------------
// reference streaming read (measurement support for the bandwidth roofline)
// ---------------------------------------------------------------------------

// Every 16-byte word of p is read once: a lane reads 64 contiguous bytes
// (four 16-byte loads) of each of two chunks per step, a grid-stride loop
// over 64-byte chunks, then the tail words.  The words are folded by XOR and
// a block writes its fold only when it equals a constant no data is expected
// to produce, so the loads stay live and next to nothing is written.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const size_t nchunk = n16 / 4;
    const size_t stride = (size_t)gridDim.x * 256;
    size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; c + stride < nchunk; c += 2 * stride) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = p[c * 4 + j];
            v[4 + j] = p[(c + stride) * 4 + j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; c < nchunk; c += stride)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 a = p[c * 4 + j];
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
    const size_t t = nchunk * 4 + (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t < n16) {
        const uint4 a = p[t];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u)
        sink[blockIdx.x] = acc;
}

hipError_t launch_stream_read(const void *data, size_t bytes, uint32_t *sink, int sink_words,
                              hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    int grid = cus * 8;
    grid = grid < sink_words ? grid : sink_words;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(data), n16, sink);
    return hipGetLastError();
}

} // namespace ivfpq
