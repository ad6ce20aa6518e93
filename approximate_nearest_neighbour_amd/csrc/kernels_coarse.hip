// Coarse quantizer on the matrix cores: D[q,l] = |x_q|^2 + |c_l|^2 - 2 x_q.c_l
// for every list, and the nprobe smallest per query ("Billion-scale
// similarity search with GPUs", IVFADC section: the coarse quantizer is a
// small brute-force matrix multiply; "Custom 8-bit floating point value
// format for reducing shared memory bank conflict in ANN search", IVFPQ
// search step 1).
//
// The dot products are v_mfma_f32_16x16x4_f32 (float32 products and sums).
// A workgroup of 4*RG waves takes TQ = 16*RG queries and sweeps a range of
// 64-centroid tiles: wave w computes the 16x16 block of query rows
// 16*(w/4).. and centroids 16*(w%4).. of a tile.  Its A operand (the query
// rows, all K-steps) stays in registers for the whole sweep; centroids were
// re-laid out at index load so that the B operand of one K-step of one
// 16-centroid block is 64 consecutive floats (one coalesced load per wave),
// and the next tile's B operand is loaded while the current tile is
// multiplied.  K-steps (KD) and blocks are padded with zeros at load, so the
// inner loop has no bounds tests.  The
// distance tile goes through LDS to the selection: each wave owns four
// queries, each with a register top-k (WaveTopK) fed 64 candidates per tile.
// More row groups per workgroup = fewer passes over the centroids.
//
// With `splits` > 1 the centroid tiles are divided among several workgroups
// per query tile; their sorted partial top-k are merged by a second kernel.
#include "common.hpp"
#include "internal.hpp"

namespace ivfpq {

typedef float v4f __attribute__((ext_vector_type(4)));

// Centroids in MFMA B-operand order: block b (16 centroids), K-step s (4
// dims), lane l -> c[16b + l%16][4s + l/16]; zero beyond nlist or d.  Norms
// padded with +inf so a padding centroid is never selected.
__global__ void centroid_blocks_kernel(const float *__restrict__ c, int d, int d4, int nlist,
                                       int nblk, float *__restrict__ cblk,
                                       float *__restrict__ cnorm_pad)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)nblk * d4 * 64;
    if (i < total) {
        const int lane = (int)(i & 63);
        const int64_t bs = i >> 6;
        const int s = (int)(bs % d4);
        const int64_t b = bs / d4;
        const int64_t row = 16 * b + (lane & 15);
        const int col = 4 * s + (lane >> 4);
        cblk[i] = (row < nlist && col < d) ? c[row * d + col] : 0.f;
    }
    if (i < (int64_t)nblk * 16) {
        float s = INFINITY;
        if (i < nlist) {
            s = 0.f;
            for (int t = 0; t < d; ++t)
                s = fmaf(c[i * d + t], c[i * d + t], s);
        }
        cnorm_pad[i] = s;
    }
}

constexpr int kQueriesPerWave = 4;

template <int NW, int RG, int KD>
__global__ __launch_bounds__(256 * RG) void coarse_mfma_kernel(
    const float *__restrict__ queries, int64_t nq, int d, int nblk, int nprobe,
    const float *__restrict__ cblk, const float *__restrict__ cnorm_pad, int splits,
    float *__restrict__ part_d, uint32_t *__restrict__ part_p, int32_t *__restrict__ probes,
    float *__restrict__ probe_d)
{
    constexpr int TQ = 16 * RG, THREADS = 256 * RG, QW = kQueriesPerWave, KW = 64 * NW;
    static_assert(TQ == QW * 4 * RG, "four queries per wave");
    extern __shared__ __align__(16) unsigned char smem[];
    const int xs = 4 * KD + 1; // odd stride: the 16 rows of an A read hit 16 banks
    float *xt = reinterpret_cast<float *>(smem);                      // [TQ][xs]
    float *xn = xt + TQ * xs;                                          // [TQ]
    float *dt = xn + TQ;                                               // [2][TQ][64]
    uint32_t *stage = reinterpret_cast<uint32_t *>(dt + 2 * TQ * 64); // [TQ][128]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    const int rg = wave >> 2, cbk = wave & 3;
    const int64_t q0 = (int64_t)blockIdx.x * TQ;
    const int split = blockIdx.y;
    const int ntile = (nblk + 3) / 4;
    const int t0 = (int)((int64_t)ntile * split / splits);
    const int t1 = (int)((int64_t)ntile * (split + 1) / splits);

    for (int i = tid; i < TQ * 4 * KD; i += THREADS) {
        const int row = i / (4 * KD), col = i % (4 * KD);
        const int64_t q = q0 + row;
        xt[row * xs + col] = (q < nq && col < d) ? queries[q * d + col] : 0.f;
    }
    __syncthreads();
    if (tid < TQ) {
        float s = 0.f;
        for (int c = 0; c < 4 * KD; ++c)
            s = fmaf(xt[tid * xs + c], xt[tid * xs + c], s);
        xn[tid] = s;
    }
    __syncthreads();

    WaveTopK<NW> sel[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i)
        sel[i].init(nprobe, stage + (wave * QW + i) * 128);

    // A layout of 16x16x4: lane l supplies row l%16, K-index l/16 of each step
    float a[KD];
    {
        const float *ap = xt + (rg * 16 + (lane & 15)) * xs + (lane >> 4);
#pragma unroll
        for (int s = 0; s < KD; ++s)
            a[s] = ap[4 * s];
    }
    float b0[KD], b1[KD];
    auto load_b = [&](int tile, float (&b)[KD]) {
        if (tile < t1) {
            const float *bp = cblk + (size_t)(tile * 4 + cbk) * KD * 64 + lane;
#pragma unroll
            for (int s = 0; s < KD; ++s)
                b[s] = bp[(size_t)s * 64];
        }
    };
    // one tile: prefetch the next tile's B into `bn`, multiply with `bc`,
    // distances through LDS buffer tile&1, then the four selections
    auto step = [&](int tile, const float (&bc)[KD], float (&bn)[KD]) {
        const int blk = tile * 4 + cbk, col = lane & 15;
        load_b(tile + 1, bn);
        const float cn = cnorm_pad[blk * 16 + col];
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KD; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], bc[s], acc, 0, 0, 0);
        // D layout of 16x16x4: lane l holds rows 4*(l/16) + r (r = 0..3) of column l%16
        float *dtile = dt + (tile & 1) * TQ * 64;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rg * 16 + 4 * (lane >> 4) + r;
            dtile[row * 64 + cbk * 16 + col] = xn[row] + cn - 2.f * acc[r];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < QW; ++i)
            sel[i].push(dtile[(wave * QW + i) * 64 + lane], (uint32_t)(tile * 64 + lane));
    };
    load_b(t0, b0);
    int tile = t0;
    for (; tile + 1 < t1; tile += 2) {
        step(tile, b0, b1);
        step(tile + 1, b1, b0);
    }
    if (tile < t1)
        step(tile, b0, b1);

#pragma unroll
    for (int i = 0; i < QW; ++i) {
        sel[i].flush();
        const int64_t q = q0 + wave * QW + i;
        if (q >= nq)
            continue;
        if (splits == 1) {
#pragma unroll
            for (int r = 0; r < NW; ++r) {
                const int e = r * 64 + lane;
                if (e < nprobe) {
                    probes[q * nprobe + e] = (int32_t)sel[i].wv[r];
                    if (probe_d)
                        probe_d[q * nprobe + e] = sel[i].wk[r];
                }
            }
        } else {
            const size_t base = ((size_t)q * splits + split) * KW;
#pragma unroll
            for (int r = 0; r < NW; ++r) {
                part_d[base + r * 64 + lane] = sel[i].wk[r];
                part_p[base + r * 64 + lane] = sel[i].wv[r];
            }
        }
    }
}

// Merge the `splits` sorted partial lists of each query (one wave per query).
template <int NW>
__global__ __launch_bounds__(64) void coarse_merge_kernel(const float *__restrict__ part_d,
                                                          const uint32_t *__restrict__ part_p,
                                                          int64_t nq, int splits, int nprobe,
                                                          int32_t *__restrict__ probes,
                                                          float *__restrict__ probe_d)
{
    constexpr int KW = 64 * NW;
    const int64_t q = blockIdx.x;
    const int lane = threadIdx.x;
    WaveTopK<NW> sel;
    sel.init(nprobe, nullptr);
    for (int s = 0; s < splits; ++s)
        sel.merge_sorted(part_d + ((size_t)q * splits + s) * KW,
                         part_p + ((size_t)q * splits + s) * KW);
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int coarse_cu_count()
{
    static int n = 0;
    if (!n) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
    }
    return n;
}

hipError_t launch_centroid_blocks(const DeviceIndex &ix, hipStream_t stream)
{
    const int64_t total = (int64_t)ix.nblk * ix.d4 * 64;
    const int64_t n = total > (int64_t)ix.nblk * 16 ? total : (int64_t)ix.nblk * 16;
    hipLaunchKernelGGL(centroid_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, ix.centroids, ix.d, ix.d4, ix.nlist, ix.nblk, ix.cblk,
                       ix.cnorm_pad);
    return hipGetLastError();
}

// Row groups per workgroup (16 queries each) and the centroid split: many
// centroids -> 4 row groups (fewer passes over the centroid array) when the
// registers allow it (1024 threads leave 128 per lane); the split keeps
// about 4 workgroup-waves per SIMD busy.
static void coarse_shape(int64_t nq, int nblk, int d4, int *rg, int *splits)
{
    *rg = nblk >= 1024 && d4 <= 24 ? 4 : 2;
    const int64_t wgs = (nq + 16 * *rg - 1) / (16 * *rg);
    const int ntile = (nblk + 3) / 4;
    const int64_t want = (int64_t)coarse_cu_count() * 16 / *rg; // ~4 waves per SIMD
    int s = (int)((want + wgs - 1) / wgs);
    s = s < 1 ? 1 : s;
    s = s > ntile ? ntile : s;
    s = s > 64 ? 64 : s;
    *splits = s;
}

size_t coarse_ws_bytes(const DeviceIndex &ix, int64_t nq, int nprobe)
{
    int nw = 1;
    while (nw * 64 < nprobe)
        nw *= 2;
    if (nw > 2 || ix.d4 > 32)
        return 0;
    int rg, splits;
    coarse_shape(nq, ix.nblk, ix.d4, &rg, &splits);
    return splits > 1 ? (size_t)nq * splits * 64 * nw * 8 : 0;
}

template <int NW, int RG, int KD>
static hipError_t coarse_mfma_variant(const DeviceIndex &ix, const float *queries, int64_t nq,
                                      int nprobe, int splits, void *ws, int32_t *probes,
                                      float *probe_d, hipStream_t stream)
{
    constexpr int TQ = 16 * RG;
    const size_t lds = (size_t)TQ * (4 * KD + 1) * 4 + TQ * 4 + 2 * TQ * 64 * 4 + TQ * 512;
    auto kern = coarse_mfma_kernel<NW, RG, KD>;
    if (lds > 160 * 1024)
        return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    float *part_d = static_cast<float *>(ws);
    uint32_t *part_p = reinterpret_cast<uint32_t *>(part_d + (size_t)nq * splits * 64 * NW);
    const dim3 grid((unsigned)((nq + TQ - 1) / TQ), (unsigned)splits);
    hipLaunchKernelGGL(kern, grid, dim3(256 * RG), lds, stream, queries, nq, ix.d, ix.nblk,
                       nprobe, ix.cblk, ix.cnorm_pad, splits, part_d, part_p, probes, probe_d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    hipLaunchKernelGGL(coarse_merge_kernel<NW>, dim3((unsigned)nq), dim3(64), 0, stream, part_d,
                       part_p, nq, splits, nprobe, probes, probe_d);
    return hipGetLastError();
}

template <int NW, int RG>
static hipError_t coarse_mfma_k(const DeviceIndex &ix, const float *queries, int64_t nq,
                                int nprobe, int splits, void *ws, int32_t *probes, float *probe_d,
                                hipStream_t stream)
{
    switch (ix.d4) {
    case 8:
        return coarse_mfma_variant<NW, RG, 8>(ix, queries, nq, nprobe, splits, ws, probes,
                                              probe_d, stream);
    case 16:
        return coarse_mfma_variant<NW, RG, 16>(ix, queries, nq, nprobe, splits, ws, probes,
                                               probe_d, stream);
    case 24:
        return coarse_mfma_variant<NW, RG, 24>(ix, queries, nq, nprobe, splits, ws, probes,
                                               probe_d, stream);
    case 32:
        if (RG == 2)
            return coarse_mfma_variant<NW, 2, 32>(ix, queries, nq, nprobe, splits, ws, probes,
                                                  probe_d, stream);
        return hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_coarse(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                         void *ws, int32_t *probes, float *probe_d, hipStream_t stream)
{
    if (nq == 0)
        return hipSuccess;
    int nw = 1;
    while (nw * 64 < nprobe)
        nw *= 2;
    // the matrix-core form keeps a tile's B operand in registers (d up to 128)
    // and four register top-k per wave (nprobe up to 128)
    if (nw > 2 || ix.d4 > 32)
        return launch_coarse_valu(ix, queries, nq, nprobe, probes, probe_d, stream);
    int rg, splits;
    coarse_shape(nq, ix.nblk, ix.d4, &rg, &splits);
    if (nw == 1)
        return rg == 4 ? coarse_mfma_k<1, 4>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                             stream)
                       : coarse_mfma_k<1, 2>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                             stream);
    return rg == 4 ? coarse_mfma_k<2, 4>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                         stream)
                   : coarse_mfma_k<2, 2>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                         stream);
}

} // namespace ivfpq
