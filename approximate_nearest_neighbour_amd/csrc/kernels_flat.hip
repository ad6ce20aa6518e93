// Exact k-nearest-neighbour search over a flat bfloat16 database
// ("Billion-scale similarity search with GPUs", exact search section: the
// squared L2 distance expands into |x|^2 + |y|^2 - 2 x.y, the x.y term is a
// matrix multiply, and a k-selection over each row of the distance matrix
// gives the result; here bf16 x bf16 products with float32 sums on the
// matrix cores, v_mfma_f32_16x16x32_bf16).
//
// The distance matrix is never stored.  Passes per batch of queries:
//
//  0. prep:    the A operand, each query times -2 in bfloat16 (exact),
//              padded to whole K-steps, and |x|^2 in float32.
//  1. minima:  the GEMM over every 64-row tile.  The accumulators start at
//              |y|^2 and the A operand holds -2x, so the matrix cores give
//              u = |y|^2 - 2 x.y itself; per query, each lane keeps the
//              running minimum of u over the rows it sees in a segment of G
//              tiles (16 rows per tile: its column c in each of the 4 column
//              blocks) and writes it out per segment: P = 16 * segments
//              "slot minima" per query, slot (segment, c) covering 4 G rows.
//  2. kth:     a value v with at least k slot minima <= v, close above the
//              k-th smallest (histogram of the minima).  Those k slot rows
//              are distinct rows with u <= v, so the k-th smallest distance is
//              at most |x|^2 + v (plus rounding).  tu = v + slack, slack =
//              2^-20 (|x|^2 + max |y|^2), covers the float32 rounding of the
//              distance |x|^2 + u.
//  3. collect: only slots whose minimum is <= tu can hold a row with
//              u <= tu.  Per segment, the queries are listed by hot slot and
//              the slot's rows multiplied again, 16 queries at a time, with
//              the same operands, start value and K order as in pass 1 (the
//              same u to the bit); rows with u <= tu (a superset of the true
//              top k, about k rows) are appended with their distance to the
//              query's candidate buffer (capacity C).  About k of a query's
//              P slots are hot, so this pass does a few percent of the
//              GEMM's work.  (A second full GEMM with the bound test, the
//              earlier form, remains behind a test switch for comparison.)
//  4. select:  exact top-k of each buffer (four-wave register selection).
//              A query whose candidates overflowed C (only when very many rows
//              tie) is redone by `fallback`, an exact streaming selection over
//              the whole database.
//
#include "common.hpp"
#include "internal.hpp"

#include <cstdlib>

namespace ivfpq {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// |v|^2 of a bf16 row in float32, terms added in index order.
__device__ __forceinline__ float bf16_row_norm(const uint16_t *v, int d)
{
    float s = 0.f;
    for (int t = 0; t < d; ++t) {
        const float x = bf16_to_float(v[t]);
        s = fmaf(x, x, s);
    }
    return s;
}

// The distance from the accumulated dot product: |x|^2 + |y|^2 - 2 x.y.
__device__ __forceinline__ float flat_distance(float xn, float yn, float dot)
{
    return fmaf(-2.f, dot, xn + yn);
}

// Device copy of the database: rows padded to dp = 32 * ks bf16 (zeros) and
// to a whole number of 64-row tiles (zero rows with norm +inf).
__global__ void flat_pack_kernel(const uint16_t *__restrict__ src, int64_t n, int d, int dp,
                                 int64_t npad, uint16_t *__restrict__ dst, float *__restrict__ norms)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < npad * dp) {
        const int64_t row = i / dp;
        const int col = (int)(i % dp);
        dst[i] = (row < n && col < d) ? src[row * d + col] : (uint16_t)0;
    }
    if (i < npad)
        norms[i] = i < n ? bf16_row_norm(src + i * d, d) : INFINITY;
}

// Pass 0: qs = -2 x in bfloat16, rows padded to dp with zeros, and
// qn = |x|^2 in float32.  -2 x is exact: x has at most 8 significant bits and
// the product only moves the exponent, so the top half of its float32 bits is
// the value.
__global__ void flat_query_prep_kernel(const uint16_t *__restrict__ q, int64_t nq, int d, int dp,
                                       uint16_t *__restrict__ qs, float *__restrict__ qn)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nq * dp) {
        const int64_t row = i / dp;
        const int col = (int)(i % dp);
        uint16_t v = 0;
        if (col < d)
            v = (uint16_t)(__float_as_uint(-2.f * bf16_to_float(q[row * d + col])) >> 16);
        qs[i] = v;
    }
    if (i < nq)
        qn[i] = bf16_row_norm(q + i * d, d);
}

// A operand of 16x16x32 from the padded -2x rows: lane l supplies row l%16,
// K-indices 8*(l/16)..+7 of each 32-wide K-step (the B operand uses the same
// K-split); rows past nq are zero.
template <int KS>
__device__ __forceinline__ void load_a(const uint16_t *__restrict__ qs, int64_t nq, int64_t row,
                                       int lane, bf16x8 (&a)[KS])
{
    constexpr int DP = 32 * KS;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (row < nq)
            v = *reinterpret_cast<const u16x8 *>(qs + row * DP + 32 * s + 8 * (lane >> 4));
        a[s] = __builtin_bit_cast(bf16x8, v);
    }
}

// u = |y|^2 - 2 x.y of a 16x16 block: the chain starts at |y|^2 of the
// block's column (yc, the same in the 4 values of a lane) and adds the
// products of -2x and y, K-steps in order.  Every pass computes u this way,
// so a row's u is the same value in all of them.
template <int KS>
__device__ __forceinline__ v4f mfma_u(const bf16x8 (&a)[KS], const bf16x8 (&b)[KS], float yc)
{
    v4f acc = v4f{yc, yc, yc, yc};
#pragma unroll
    for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

// Rounding allowance between |x|^2 + v and the float32 distances |x|^2 + u
// of rows with u <= v: 16 units of 2^-24 of |x|^2 + max |y|^2.
__device__ __forceinline__ float flat_slack(float xn, float ymax)
{
    return 0x1p-20f * (xn + ymax);
}

enum FlatPass { kPassMinima = 0, kPassCollect = 1 };

// Candidate counters one per 128-byte line: the appends of the many
// workgroups that share a block of queries would otherwise queue on the few
// lines that hold the block's counters.
constexpr int kCntStride = 32;

// Passes 1 and 3 (GEMM over every tile).  Workgroup: 4 waves, TQ = 64*RB
// queries (wave w: row blocks w*RB..), tiles [t0, t1) made of whole
// segments of `seg` tiles.  Tiles are staged in LDS (double buffer, one
// barrier per tile); each wave multiplies its RB row blocks by the tile's 4
// column blocks, one column block at a time (RB accumulators live).
// Collect-pass staging of candidates in LDS: entries per workgroup.
constexpr int kFlatStage = 1024;

// The collect pass keeps three waves per SIMD (its staging adds registers);
// the minima pass runs at two (four row blocks of A operands).
template <int KS, int RB, int PASS>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(PASS == kPassCollect ? 3 : 1))) void flat_gemm_kernel(
    const uint16_t *__restrict__ qs, const float *__restrict__ qn, int64_t nq,
    const uint16_t *__restrict__ db, const float *__restrict__ dbn, int64_t n, int64_t ntile,
    int seg, int64_t nseg, int splits, float *__restrict__ slots, int64_t nslot,
    const float *__restrict__ tuq, uint32_t cap, uint32_t *__restrict__ cnt,
    float *__restrict__ cand_d, uint32_t *__restrict__ cand_p)
{
    constexpr int DP = 32 * KS, TQ = 64 * RB, RS = DP + 8; // LDS row stride (bf16), +16 B
    constexpr int CHUNKS = 64 * DP / 8 / 256;              // 16-byte pieces per thread per tile
    extern __shared__ __align__(16) unsigned char smem[];
    float *xn = reinterpret_cast<float *>(smem);          // [TQ]
    float *tq = xn + TQ;                                   // [TQ]
    float *yn = tq + TQ;                                   // [2][64]
    uint16_t *bt = reinterpret_cast<uint16_t *>(yn + 128); // [2][64][RS]
    // collect pass: candidates staged in LDS (count, rows, distances, query
    // offsets) and appended to the query buffers in bulk, so that a wave does
    // not wait for a global atomic's return per candidate
    uint32_t *scount = reinterpret_cast<uint32_t *>(bt + 2 * 64 * RS);
    uint32_t *srow = scount + 4;
    float *sdist = reinterpret_cast<float *>(srow + kFlatStage);
    uint16_t *sq = reinterpret_cast<uint16_t *>(sdist + kFlatStage);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    const int64_t q0 = (int64_t)blockIdx.x * TQ;
    const int64_t s0 = nseg * blockIdx.y / splits, s1 = nseg * (blockIdx.y + 1) / splits;
    const int64_t t0 = s0 * seg, t1 = s1 * seg < ntile ? s1 * seg : ntile;

    if (PASS == kPassCollect) {
        for (int r = tid; r < TQ; r += 256) {
            const int64_t q = q0 + r;
            xn[r] = q < nq ? qn[q] : 0.f;
            tq[r] = q < nq ? tuq[q] : -INFINITY;
        }
        if (tid == 0)
            scount[0] = 0;
    }
    // one candidate into its query's buffer (the global append)
    auto append = [&](int64_t q, uint32_t row, float dist) {
        const uint32_t slot = atomicAdd(cnt + q * kCntStride, 1u);
        if (slot < cap) {
            cand_d[(size_t)q * cap + slot] = dist;
            cand_p[(size_t)q * cap + slot] = row;
        }
    };
    // all staged candidates to the global buffers (256 appends in flight at a
    // time), then the stage is empty; every thread calls it (barriers)
    auto drain = [&]() {
        const uint32_t sc = scount[0];
        const uint32_t m = sc < (uint32_t)kFlatStage ? sc : (uint32_t)kFlatStage;
        for (uint32_t i = tid; i < m; i += 256)
            append(q0 + sq[i], srow[i], sdist[i]);
        __syncthreads();
        if (tid == 0)
            scount[0] = 0;
        __syncthreads();
    };
    bf16x8 a[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        load_a<KS>(qs, nq, q0 + (wave * RB + rb) * 16 + (lane & 15), lane, a[rb]);

    u16x8 stg[CHUNKS];
    float ystg = INFINITY;
    auto fetch = [&](int64_t t) {
        if (t < t1) {
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c) {
                const int piece = c * 256 + tid; // 16-byte piece of the 64 x DP tile
                const int row = piece / (DP / 8), col = (piece % (DP / 8)) * 8;
                stg[c] = *reinterpret_cast<const u16x8 *>(db + (t * 64 + row) * DP + col);
            }
            if (tid < 64)
                ystg = dbn[t * 64 + tid];
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            const int piece = c * 256 + tid;
            const int row = piece / (DP / 8), col = (piece % (DP / 8)) * 8;
            *reinterpret_cast<u16x8 *>(bt + (buf * 64 + row) * RS + col) = stg[c];
        }
        if (tid < 64)
            yn[buf * 64 + tid] = ystg;
    };
    fetch(t0);
    stash(0);
    __syncthreads();
    // per lane: the 16 query rows it holds in the D layout (4*(lane/16) + r of
    // each row block)
    float xr[RB][4], tr[RB][4], mn[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (wave * RB + rb) * 16 + 4 * (lane >> 4) + r;
            if (PASS == kPassCollect) {
                xr[rb][r] = xn[row];
                tr[rb][r] = tq[row];
            }
            mn[rb][r] = INFINITY;
        }

    for (int64_t t = t0; t < t1; ++t) {
        const int buf = (int)(t - t0) & 1;
        fetch(t + 1);
        // u of this wave's row blocks and column block cb of the tile
        auto block_u = [&](int cb, v4f (&acc)[RB]) {
            bf16x8 b[KS];
            const uint16_t *bp = bt + (buf * 64 + cb * 16 + (lane & 15)) * RS + 8 * (lane >> 4);
#pragma unroll
            for (int s = 0; s < KS; ++s)
                b[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(bp + 32 * s));
            const float ycol = yn[buf * 64 + cb * 16 + (lane & 15)];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = mfma_u<KS>(a[rb], b, ycol);
        };
        if (PASS == kPassMinima) {
            // column blocks in pairs (one three-way minimum per two values),
            // each block's B operand read from LDS while the previous block
            // is multiplied
            auto load_b = [&](int cb, bf16x8 (&b)[KS], float &yc) {
                const uint16_t *bp =
                    bt + (buf * 64 + cb * 16 + (lane & 15)) * RS + 8 * (lane >> 4);
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    b[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(bp + 32 * s));
                yc = yn[buf * 64 + cb * 16 + (lane & 15)];
            };
            bf16x8 bA[KS], bB[KS];
            float yA, yB;
            load_b(0, bA, yA);
            load_b(1, bB, yB);
#pragma unroll
            for (int cb = 0; cb < 4; cb += 2) {
                v4f u0[RB], u1[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    u0[rb] = mfma_u<KS>(a[rb], bA, yA);
                if (cb + 2 < 4)
                    load_b(cb + 2, bA, yA);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    u1[rb] = mfma_u<KS>(a[rb], bB, yB);
                if (cb + 3 < 4)
                    load_b(cb + 3, bB, yB);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        mn[rb][r] = fminf(mn[rb][r], fminf(u0[rb][r], u1[rb][r]));
            }
        }
        // not unrolled: the compiler would keep all four blocks' operands live
#pragma unroll 1
        for (int cb = 0; cb < (PASS == kPassMinima ? 0 : 4); ++cb) {
            v4f acc[RB];
            block_u(cb, acc);
            {
                // rows under the bound are rare (about k of n per query): one
                // scalar test per row block (its 4 rows), then per row
                const int64_t row = t * 64 + cb * 16 + (lane & 15);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    bool pass[4];
                    bool any = false;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pass[r] = acc[rb][r] <= tr[rb][r];
                        any |= pass[r];
                    }
                    if (!__builtin_amdgcn_ballot_w64(any))
                        continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ql = (wave * RB + rb) * 16 + 4 * (lane >> 4) + r;
                        const int64_t q = q0 + ql;
                        const bool take = pass[r] && row < n && q < nq;
                        const uint64_t mask = __builtin_amdgcn_ballot_w64(take);
                        if (mask == 0)
                            continue;
                        // one LDS atomic per wave and row for all its lanes
                        uint32_t base = 0;
                        if (lane == 0)
                            base = atomicAdd(scount, (uint32_t)__popcll(mask));
                        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
                        if (take) {
                            const uint32_t at = base + mbcnt64(mask);
                            const float dist = xr[rb][r] + acc[rb][r];
                            if (at < (uint32_t)kFlatStage) {
                                srow[at] = (uint32_t)row;
                                sdist[at] = dist;
                                sq[at] = (uint16_t)ql;
                            } else {
                                append(q, (uint32_t)row, dist); // stage full
                            }
                        }
                    }
                }
            }
        }
        if (PASS == kPassMinima && ((t + 1) % seg == 0 || t + 1 == t1)) {
            const int64_t sg = t / seg;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t q = q0 + (wave * RB + rb) * 16 + 4 * (lane >> 4) + r;
                    if (q < nq)
                        slots[q * nslot + sg * 16 + (lane & 15)] = mn[rb][r];
                    mn[rb][r] = INFINITY;
                }
        }
        if (t + 1 < t1)
            stash(buf ^ 1);
        __syncthreads();
        if (PASS == kPassCollect) {
            // drain at half full (a tile rarely adds more than the rest)
            const uint32_t sc = (uint32_t)__builtin_amdgcn_readfirstlane((int)scount[0]);
            if (sc >= (uint32_t)kFlatStage / 2)
                drain();
        }
    }
    if (PASS == kPassCollect)
        drain();
}

// Block-wide (256 threads) reductions through LDS scratch red[8].
__device__ __forceinline__ float block_min(float v, float *red)
{
    for (int s = 32; s >= 1; s >>= 1)
        v = fminf(v, __shfl_xor(v, s));
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fminf(fminf(red[0], red[1]), fminf(red[2], red[3]));
}

__device__ __forceinline__ float block_max(float v, float *red)
{
    return -block_min(-v, red);
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *red)
{
    for (int s = 32; s >= 1; s >>= 1)
        v += (uint32_t)__shfl_xor((int)v, s);
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

constexpr int kKthBins = 2048; // 8 per thread
// slot minima per thread, held in registers: nslot <= 256 * kKthPer = 16,128
// (the plan keeps nslot <= 16,000)
constexpr int kKthPer = 63;

// Pass 2: per query an upper bound v of the k-th smallest of its nslot slot
// minima with at least k minima <= v: a 2048-bin histogram of the finite
// minima over [min, max]; v = the largest minimum in the bins up to the one
// that holds the k-th.  Then the collect threshold tu = v + slack (+inf when
// fewer than k minima are finite).  Each thread reads its minima once and
// keeps them in registers for the histogram and the final maximum.
__global__ __launch_bounds__(256) void flat_kth_kernel(const float *__restrict__ qn,
                                                       const float *__restrict__ slots,
                                                       int64_t nslot, int k, float ymax,
                                                       float *__restrict__ tuq)
{
    __shared__ uint32_t cnt[kKthBins];
    __shared__ float redf[8];
    __shared__ uint32_t redu[8];
    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x;
    const float *sq = slots + q * nslot;
    float vals[kKthPer];
    float lo = INFINITY, hi = -INFINITY;
    uint32_t fin = 0;
#pragma unroll
    for (int j = 0; j < kKthPer; ++j) {
        const int64_t i = tid + (int64_t)256 * j;
        const float v = i < nslot ? sq[i] : INFINITY;
        vals[j] = v;
        if (v < INFINITY) {
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
            ++fin;
        }
    }
    lo = block_min(lo, redf);
    hi = block_max(hi, redf);
    fin = block_sum(fin, redu);
    float v;
    if (fin < (uint32_t)k) {
        v = INFINITY;
    } else if (!(hi > lo)) {
        v = lo;
    } else {
        const float scale = kKthBins / (hi - lo);
        auto bin_of = [&](float x) {
            int b = (int)((x - lo) * scale);
            return b < 0 ? 0 : b >= kKthBins ? kKthBins - 1 : b;
        };
        for (int b = tid; b < kKthBins; b += 256)
            cnt[b] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kKthPer; ++j)
            if (vals[j] < INFINITY)
                atomicAdd(&cnt[bin_of(vals[j])], 1u);
        __syncthreads();
        // thread t owns bins 8t..8t+7: local sums, block prefix, find the bin
        uint32_t local = 0;
        for (int j = 0; j < 8; ++j)
            local += cnt[8 * tid + j];
        const int wave = tid >> 6, lane = tid & 63;
        uint32_t incl = wave_inclusive_sum(local);
        __syncthreads();
        if (lane == 63)
            redu[wave] = incl;
        __syncthreads();
        for (int w = 0; w < wave; ++w)
            incl += redu[w];
        uint32_t before = incl - local;
        int found = kKthBins;
        if (before < (uint32_t)k && incl >= (uint32_t)k) {
            for (int j = 0; j < 8; ++j) {
                before += cnt[8 * tid + j];
                if (before >= (uint32_t)k) {
                    found = 8 * tid + j;
                    break;
                }
            }
            redu[4] = (uint32_t)found;
        }
        __syncthreads();
        const int bsel = (int)redu[4];
        // largest finite minimum in bins 0..bsel
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kKthPer; ++j)
            if (vals[j] < INFINITY && bin_of(vals[j]) <= bsel)
                m = fmaxf(m, vals[j]);
        v = block_max(m, redf);
    }
    if (tid == 0)
        tuq[q] = v + flat_slack(qn[q], ymax);
}

// Wave-wide inclusive prefix sum in DPP (no LDS round trips): row_shr by 1, 2,
// 4, 8 inside each 16-lane row (lanes shifted in from outside read 0), then
// row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds lane 31's sum to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    return v;
}

// Pass 3 by recomputation.  Workgroup (segment sg, queries qb0 ..
// qb0 + kRecQB): a query is listed under column c when its minimum of slot
// (sg, c) is <= its bound tu; then each wave takes columns c = w, w + 4, ...
// and multiplies the listed queries, 16 at a time, by the rows of slot
// (sg, c): B block j holds the rows t*64 + 16 j + c of the segment's tiles t
// (tile tb + p in column p), so one slot is 4 blocks of 16 rows, kept in
// registers while its queries stream through.  Rows with u <= tu are staged
// in the wave's own LDS area (slots from a ballot, no atomics) and appended
// to the queries' candidate buffers when it fills and at the end: all of a
// lane's global atomics for a drain are issued before any is waited on.
constexpr int kRecQB = 2048;
constexpr int kRecStage = 384; // staged candidates per wave

template <int U>
__device__ __forceinline__ void rec_drain(uint32_t m, const uint16_t *sq, const uint32_t *srow,
                                          const float *sdist, int64_t qb0, uint32_t cap,
                                          uint32_t *__restrict__ cnt, float *__restrict__ cand_d,
                                          uint32_t *__restrict__ cand_p)
{
    const int lane = threadIdx.x & 63;
    uint32_t at[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = u * 64 + lane;
        at[u] = i < m ? atomicAdd(cnt + (qb0 + sq[i]) * kCntStride, 1u) : cap;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = u * 64 + lane;
        if (at[u] < cap) {
            const size_t base = (size_t)(qb0 + sq[i]) * cap + at[u];
            cand_d[base] = sdist[i];
            cand_p[base] = srow[i];
        }
    }
}

template <int KS>
__global__ __launch_bounds__(256) void flat_recompute_kernel(
    const uint16_t *__restrict__ qs, const float *__restrict__ qn, int64_t nq,
    const uint16_t *__restrict__ db, const float *__restrict__ dbn, int64_t n, int64_t ntile,
    int seg, const float *__restrict__ slots, int64_t nslot, const float *__restrict__ tuq,
    uint32_t cap, uint32_t *__restrict__ cnt, float *__restrict__ cand_d,
    uint32_t *__restrict__ cand_p)
{
    constexpr int DP = 32 * KS;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *count = reinterpret_cast<uint32_t *>(smem);         // [16]
    uint16_t *list = reinterpret_cast<uint16_t *>(count + 16);    // [16][kRecQB]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    // this wave's candidate stage: rows, distances, query (block index)
    uint32_t *srow = reinterpret_cast<uint32_t *>(list + 16 * kRecQB) + wave * kRecStage;
    float *sdist = reinterpret_cast<float *>(srow + (4 - wave) * kRecStage) + wave * kRecStage;
    uint16_t *sq = reinterpret_cast<uint16_t *>(sdist + (4 - wave) * kRecStage) + wave * kRecStage;
    uint32_t staged = 0; // wave-uniform
    const int64_t sg = blockIdx.x;
    const int64_t qb0 = (int64_t)blockIdx.y * kRecQB;
    const int64_t tb = sg * seg;
    const int64_t te = tb + seg < ntile ? tb + seg : ntile;
    if (tid < 16)
        count[tid] = 0;
    __syncthreads();
    // hot (query, column) pairs, listed per column (one LDS atomic per wave
    // and column for its 64 queries)
    for (int i0 = wave * 64; i0 < kRecQB; i0 += 256) {
        const int i = i0 + lane;
        const int64_t q = qb0 + i;
        const bool qv = q < nq;
        float m[16];
        float tq = -INFINITY;
        if (qv) {
            tq = tuq[q];
            const float4 *sp = reinterpret_cast<const float4 *>(slots + q * nslot + sg * 16);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 x = sp[v];
                m[4 * v] = x.x;
                m[4 * v + 1] = x.y;
                m[4 * v + 2] = x.z;
                m[4 * v + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 16; ++c)
                m[c] = INFINITY;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const bool hot = qv && m[c] <= tq;
            const uint64_t mask = __builtin_amdgcn_ballot_w64(hot);
            if (mask == 0)
                continue;
            uint32_t base = 0;
            if (lane == 0)
                base = atomicAdd(&count[c], (uint32_t)__popcll(mask));
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            if (hot)
                list[c * kRecQB + base + mbcnt64(mask)] = (uint16_t)i;
        }
    }
    __syncthreads();
    const int p = lane & 15, kq = lane >> 4;
    const int64_t t = tb + p;
    const bool tv = t < te;
    for (int c = wave; c < 16; c += 4) {
        const uint32_t nc = count[c];
        if (nc == 0)
            continue;
        const uint16_t *lc = list + c * kRecQB;
        // B operand of the slot: block j, column p = row (tb + p) * 64 + 16 j + c
        bf16x8 b[4][KS];
        float yc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t row = t * 64 + 16 * j + c;
            yc[j] = tv ? dbn[row] : INFINITY;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (tv)
                    v = *reinterpret_cast<const u16x8 *>(db + row * DP + 32 * s + 8 * kq);
                b[j][s] = __builtin_bit_cast(bf16x8, v);
            }
        }
        // the listed queries of a chunk: A operand (query base + p) and, per
        // D row (query base + 4 kq + r), its bound and |x|^2; the next
        // chunk's are loaded while this one is multiplied
        bf16x8 a[KS];
        int64_t qr[4];
        float tr[4], xr[4];
        auto fetch = [&](uint32_t base) {
            const uint32_t ia = base + p;
            load_a<KS>(qs, nq, ia < nc ? qb0 + lc[ia] : nq, lane, a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t ir = base + 4 * kq + r;
                qr[r] = ir < nc ? qb0 + lc[ir] : -1;
                tr[r] = qr[r] >= 0 ? tuq[qr[r]] : -INFINITY;
                xr[r] = qr[r] >= 0 ? qn[qr[r]] : 0.f;
            }
        };
        fetch(0);
        for (uint32_t base = 0; base < nc; base += 16) {
            v4f acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = mfma_u<KS>(a, b[j], yc[j]);
            const int64_t q_cur[4] = {qr[0], qr[1], qr[2], qr[3]};
            const float t_cur[4] = {tr[0], tr[1], tr[2], tr[3]};
            const float x_cur[4] = {xr[0], xr[1], xr[2], xr[3]};
            if (base + 16 < nc)
                fetch(base + 16);
            // rows t*64 + 16 j + c of this lane's column with u <= tu of D
            // row r: bit 4 j + r of `take`
            uint32_t take = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = t * 64 + 16 * j + c;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    take |= (q_cur[r] >= 0 && tv && row < n && acc[j][r] <= t_cur[r])
                                ? 1u << (4 * j + r)
                                : 0u;
            }
            if (!__builtin_amdgcn_ballot_w64(take != 0))
                continue;
            // each lane's takes go to consecutive stage entries: offsets from
            // a prefix sum over the wave
            const uint32_t mine = (uint32_t)__popc(take);
            const uint32_t incl = wave_scan_dpp(mine);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            if (staged + total > (uint32_t)kRecStage) {
                rec_drain<kRecStage / 64>(staged, sq, srow, sdist, qb0, cap, cnt, cand_d, cand_p);
                staged = 0;
            }
            uint32_t at = staged + incl - mine;
            while (take) {
                const int bit = __builtin_ctz(take);
                take &= take - 1;
                const int j = bit >> 2, r = bit & 3;
                float v = acc[0][0];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        v = (jj == j && rr == r) ? acc[jj][rr] : v;
                float xv = x_cur[0];
                int64_t qv = q_cur[0];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    xv = rr == r ? x_cur[rr] : xv;
                    qv = rr == r ? q_cur[rr] : qv;
                }
                srow[at] = (uint32_t)(t * 64 + 16 * j + c);
                sdist[at] = xv + v;
                sq[at] = (uint16_t)(qv - qb0);
                ++at;
            }
            staged += total;
        }
    }
    rec_drain<kRecStage / 64>(staged, sq, srow, sdist, qb0, cap, cnt, cand_d, cand_p);
}

constexpr int kFlatSelWaves = 4;

// Pass 3: exact top-k of each query's candidate buffer; an overflowed
// buffer marks the query for the fallback.
template <int NW>
__global__ __launch_bounds__(64 * kFlatSelWaves) void flat_select_kernel(
    const uint32_t *__restrict__ cnt, const float *__restrict__ cand_d,
    const uint32_t *__restrict__ cand_p, uint32_t cap, int64_t nq, int k, uint32_t *__restrict__ over,
    float *__restrict__ out_d, int64_t *__restrict__ out_i)
{
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *bound = reinterpret_cast<uint32_t *>(smem);
    float *mk = reinterpret_cast<float *>(bound + 4);
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kFlatSelWaves - 1) * 64 * NW);
    uint32_t *stage = mv + (kFlatSelWaves - 1) * 64 * NW;
    const int64_t q = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    const uint32_t c = cnt[q * kCntStride];
    if (c > cap) {
        if (tid == 0)
            over[q] = 1u;
        return;
    }
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();
    WaveTopK<NW> sel;
    sel.init(k, stage + wave * 128);
    const float *kd = cand_d + (size_t)q * cap;
    const uint32_t *kp = cand_p + (size_t)q * cap;
    int since = 0;
    for (uint32_t base = wave * 64; base < c; base += 64 * kFlatSelWaves) {
        const uint32_t i = base + lane;
        sel.push(i < c ? kd[i] : INFINITY, i < c ? kp[i] : kSentinel);
        if (++since == 4) {
            since = 0;
            publish_bound(bound, sel.kth);
            sel.bound(read_bound(bound));
        }
    }
    sel.flush();
    merge_waves<NW, kFlatSelWaves>(sel, mk, mv);
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int e = r * 64 + lane;
            if (e < k) {
                out_d[q * k + e] = sel.wk[r];
                out_i[q * k + e] = sel.wv[r] == kSentinel ? -1 : (int64_t)sel.wv[r];
            }
        }
    }
}

// Pass 4: exact streaming top-k over every row for the queries the select
// pass marked; the others return at once.  One lane per row, dot product in
// float32 over the padded row (the padding is zero).
template <int NW>
__global__ __launch_bounds__(64 * kFlatSelWaves) void flat_fallback_kernel(
    const uint16_t *__restrict__ queries, int d, const uint16_t *__restrict__ db, int dp,
    const float *__restrict__ dbn, int64_t n, int k, const uint32_t *__restrict__ over,
    float *__restrict__ out_d, int64_t *__restrict__ out_i)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int64_t q = blockIdx.x;
    if (!over[q])
        return;
    uint32_t *bound = reinterpret_cast<uint32_t *>(smem);
    float *xq = reinterpret_cast<float *>(bound + 4); // [dp]
    float *mk = xq + dp;
    uint32_t *mv = reinterpret_cast<uint32_t *>(mk + (kFlatSelWaves - 1) * 64 * NW);
    uint32_t *stage = mv + (kFlatSelWaves - 1) * 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    for (int t = tid; t < dp; t += 64 * kFlatSelWaves)
        xq[t] = t < d ? bf16_to_float(queries[q * d + t]) : 0.f;
    if (tid == 0)
        *bound = float_order_key(INFINITY);
    __syncthreads();
    const float xn = bf16_row_norm(queries + q * d, d);
    WaveTopK<NW> sel;
    sel.init(k, stage + wave * 128);
    int since = 0;
    for (int64_t base = wave * 64; base < n; base += 64 * kFlatSelWaves) {
        const int64_t row = base + lane;
        float dist = INFINITY;
        if (row < n) {
            const uint16_t *y = db + row * dp;
            float dot = 0.f;
            for (int t = 0; t < dp; ++t)
                dot = fmaf(xq[t], bf16_to_float(y[t]), dot);
            dist = flat_distance(xn, dbn[row], dot);
        }
        sel.push(dist, (uint32_t)row);
        if (++since == 4) {
            since = 0;
            publish_bound(bound, sel.kth);
            sel.bound(read_bound(bound));
        }
    }
    sel.flush();
    merge_waves<NW, kFlatSelWaves>(sel, mk, mv);
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < NW; ++r) {
            const int e = r * 64 + lane;
            if (e < k) {
                out_d[q * k + e] = sel.wk[r];
                out_i[q * k + e] = sel.wv[r] == kSentinel ? -1 : (int64_t)sel.wv[r];
            }
        }
    }
}

__global__ void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_flat_pack(const uint16_t *src, int64_t n, int d, int dp, int64_t npad,
                            uint16_t *dst, float *norms, hipStream_t stream)
{
    const int64_t total = npad * dp;
    if (total == 0)
        return hipSuccess;
    hipLaunchKernelGGL(flat_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, src, n, d, dp, npad, dst, norms);
    return hipGetLastError();
}

static int flat_cu_count()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

FlatPlan flat_plan(int64_t n, int k, int64_t nq, int dp)
{
    (void)nq;
    FlatPlan p;
    p.dp = dp;
    p.ntile = (n + 63) / 64;
    // at most 1000 segments (16000 slot minima per query): about 16 per
    // top-k row at k = 1024, so few top-k rows share a slot
    p.seg = (int)((p.ntile + 999) / 1000);
    p.seg = p.seg < 1 ? 1 : p.seg;
    p.nseg = (p.ntile + p.seg - 1) / p.seg;
    p.nslot = 16 * p.nseg;
    const int64_t c = 4 * (int64_t)k;
    p.cap = (uint32_t)(c < 4096 ? 4096 : c);
    return p;
}

// slot minima, bound, counter line, overflow flag, candidates, |x|^2 and the
// -2x rows (+ alignment)
size_t flat_ws_bytes(const FlatPlan &p, int64_t nq)
{
    return (size_t)nq * ((size_t)p.nslot * 4 + 12 + 4 * kCntStride + (size_t)p.cap * 8 +
                         (size_t)p.dp * 2) +
           640;
}

template <int KS, int RB, int PASS>
static hipError_t gemm_variant(const FlatDevice &fx, const uint16_t *qs, const float *qn,
                               int64_t nq, const FlatPlan &p, float *slots, const float *tuq,
                               uint32_t *cnt, float *cand_d, uint32_t *cand_p, hipStream_t stream)
{
    constexpr int TQ = 64 * RB, DP = 32 * KS;
    const size_t lds = (size_t)TQ * 8 + 128 * 4 + 2 * 64 * (DP + 8) * 2 +
                       (PASS == kPassCollect ? 16 + (size_t)kFlatStage * 10 : 0);
    auto kern = flat_gemm_kernel<KS, RB, PASS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    const int64_t qg = (nq + TQ - 1) / TQ;
    // about 10 workgroups per CU in all; a last round of workgroups that
    // fills only part of the chip costs as much as a full one, so among half
    // to twice that many segment splits the one with the fewest rounds x
    // segments per workgroup is taken (rounds from the resident workgroups
    // per CU the runtime reports; ties to fewer splits)
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t resident = (int64_t)per_cu * flat_cu_count();
    int64_t s0 = ((int64_t)flat_cu_count() * 10 + qg - 1) / qg;
    s0 = s0 < 1 ? 1 : s0 > p.nseg ? p.nseg : s0;
    auto cost = [&](int64_t sp) {
        return (double)((qg * sp + resident - 1) / resident) * (double)((p.nseg + sp - 1) / sp) *
               (1.0 + 0.002 * (double)sp);
    };
    int64_t splits = s0;
    double best = cost(s0);
    for (int64_t sp = s0 / 2 > 1 ? s0 / 2 : 1; sp <= 2 * s0 && sp <= p.nseg; ++sp) {
        const double c = cost(sp);
        if (c < best) {
            best = c;
            splits = sp;
        }
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)qg, (unsigned)splits), dim3(256), lds, stream, qs, qn,
                       nq, fx.vec, fx.norms, fx.n, p.ntile, p.seg, p.nseg, (int)splits, slots,
                       p.nslot, tuq, p.cap, cnt, cand_d, cand_p);
    return hipGetLastError();
}

template <int KS>
static hipError_t recompute_variant(const FlatDevice &fx, const uint16_t *qs, const float *qn,
                                    int64_t nq, const FlatPlan &p, const float *slots,
                                    const float *tuq, uint32_t *cnt, float *cand_d,
                                    uint32_t *cand_p, hipStream_t stream)
{
    const size_t lds = 64 + (size_t)16 * kRecQB * 2 + (size_t)4 * kRecStage * 10;
    auto kern = flat_recompute_kernel<KS>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    const dim3 grid((unsigned)p.nseg, (unsigned)((nq + kRecQB - 1) / kRecQB));
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, qs, qn, nq, fx.vec, fx.norms, fx.n,
                       p.ntile, p.seg, slots, p.nslot, tuq, p.cap, cnt, cand_d, cand_p);
    return hipGetLastError();
}

// Test switch: IVFPQ_TEST_FLAT_FULL_COLLECT=1 runs the collect pass as a
// second full GEMM with the bound test (read on every search).
static bool flat_full_collect()
{
    const char *e = std::getenv("IVFPQ_TEST_FLAT_FULL_COLLECT");
    return e && e[0] == '1';
}

template <int NW>
static hipError_t select_variant(const FlatDevice &fx, const uint16_t *q, int64_t nq, int k,
                                 const FlatPlan &p, const uint32_t *cnt, const float *cand_d,
                                 const uint32_t *cand_p, uint32_t *over, float *out_d,
                                 int64_t *out_i, hipStream_t stream, bool fallback)
{
    const size_t lds = 16 + (size_t)(kFlatSelWaves - 1) * 64 * NW * 8 + kFlatSelWaves * 512;
    if (!fallback) {
        hipLaunchKernelGGL(flat_select_kernel<NW>, dim3((unsigned)nq), dim3(64 * kFlatSelWaves),
                           lds, stream, cnt, cand_d, cand_p, p.cap, nq, k, over, out_d, out_i);
        return hipGetLastError();
    }
    const size_t lds_fb = lds + (size_t)fx.dp * 4;
    hipLaunchKernelGGL(flat_fallback_kernel<NW>, dim3((unsigned)nq), dim3(64 * kFlatSelWaves),
                       lds_fb, stream, q, fx.d, fx.vec, fx.dp, fx.norms, fx.n, k, over, out_d,
                       out_i);
    return hipGetLastError();
}

template <int KS>
static hipError_t gemm_pass(const FlatDevice &fx, const uint16_t *qs, const float *qn,
                            int64_t nq, const FlatPlan &p, float *slots, const float *tuq,
                            uint32_t *cnt, float *cand_d, uint32_t *cand_p, hipStream_t stream,
                            int pass)
{
    // minima pass: four row blocks per wave while the A operand fits the
    // registers (fewer B reads per product); full collect pass: two (its
    // append path needs the registers, and more waves hide its latency)
    constexpr int RBM = KS <= 4 ? 4 : 2;
    if (pass == kPassMinima)
        return gemm_variant<KS, RBM, kPassMinima>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d,
                                                  cand_p, stream);
    if (flat_full_collect())
        return gemm_variant<KS, 2, kPassCollect>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d,
                                                 cand_p, stream);
    return recompute_variant<KS>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream);
}

hipError_t launch_flat_stage(const FlatDevice &fx, const uint16_t *q, int64_t nq, int k,
                             const FlatPlan &p, void *ws, float *out_d, int64_t *out_i,
                             int stage, hipStream_t stream)
{
    if (nq == 0)
        return hipSuccess;
    float *slots = static_cast<float *>(ws);
    float *tuq = slots + (size_t)nq * p.nslot;
    uint32_t *cnt = reinterpret_cast<uint32_t *>(
        (reinterpret_cast<uintptr_t>(tuq + nq) + 127) & ~(uintptr_t)127); // [nq][kCntStride]
    uint32_t *over = cnt + (size_t)nq * kCntStride;
    float *cand_d = reinterpret_cast<float *>(over + nq);
    uint32_t *cand_p = reinterpret_cast<uint32_t *>(cand_d + (size_t)nq * p.cap);
    float *qn = reinterpret_cast<float *>(cand_p + (size_t)nq * p.cap);
    uint16_t *qs = reinterpret_cast<uint16_t *>(
        (reinterpret_cast<uintptr_t>(qn + nq) + 255) & ~(uintptr_t)255);
    if (fx.dp != p.dp)
        return hipErrorInvalidValue;
    switch (stage) {
    case 0:   // clear the counters, the A operand, slot minima
    case 2: { // collect
        if (stage == 0) {
            const int64_t nfill = nq * (kCntStride + 1); // counters and overflow flags
            hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((nfill + 255) / 256)), dim3(256),
                               0, stream, cnt, nfill, 0u);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            const int64_t total = nq * fx.dp;
            hipLaunchKernelGGL(flat_query_prep_kernel, dim3((unsigned)((total + 255) / 256)),
                               dim3(256), 0, stream, q, nq, fx.d, fx.dp, qs, qn);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        if (p.ntile == 0) // empty database: every row of the result is padding
            return hipSuccess;
        const int pass = stage == 0 ? kPassMinima : kPassCollect;
        switch (fx.dp / 32) {
        case 1: return gemm_pass<1>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 2: return gemm_pass<2>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 3: return gemm_pass<3>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 4: return gemm_pass<4>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 5: return gemm_pass<5>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 6: return gemm_pass<6>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 7: return gemm_pass<7>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        case 8: return gemm_pass<8>(fx, qs, qn, nq, p, slots, tuq, cnt, cand_d, cand_p, stream, pass);
        default: return hipErrorInvalidValue;
        }
    }
    case 1: { // k-th slot minimum -> collect threshold
        if (p.nslot > (int64_t)256 * kKthPer)
            return hipErrorInvalidValue;
        if (p.ntile == 0)
            return hipSuccess;
        hipLaunchKernelGGL(flat_kth_kernel, dim3((unsigned)nq), dim3(256), 0, stream, qn, slots,
                           p.nslot, k, fx.ymax, tuq);
        return hipGetLastError();
    }
    default: { // 3: select, 4: fallback
        const bool fb = stage == 4;
        int nw = 1;
        while (nw * 64 < k)
            nw *= 2;
        switch (nw) {
        case 1: return select_variant<1>(fx, q, nq, k, p, cnt, cand_d, cand_p, over, out_d, out_i, stream, fb);
        case 2: return select_variant<2>(fx, q, nq, k, p, cnt, cand_d, cand_p, over, out_d, out_i, stream, fb);
        case 4: return select_variant<4>(fx, q, nq, k, p, cnt, cand_d, cand_p, over, out_d, out_i, stream, fb);
        case 8: return select_variant<8>(fx, q, nq, k, p, cnt, cand_d, cand_p, over, out_d, out_i, stream, fb);
        default: return select_variant<16>(fx, q, nq, k, p, cnt, cand_d, cand_p, over, out_d, out_i, stream, fb);
        }
    }
    }
}

} // namespace ivfpq
