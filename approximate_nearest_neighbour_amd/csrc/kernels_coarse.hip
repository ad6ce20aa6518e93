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

#include <cstdlib>

namespace ivfpq {

typedef float v4f __attribute__((ext_vector_type(4)));

// Centroids in MFMA B-operand order: block b (16 centroids), K-step s (4
// dims), lane l -> c[16b + l%16][4s + l/16], stored as [b][s/4][l][s%4] so
// that one 16-byte load gives a lane four consecutive K-steps (a wave reads
// 1 KiB contiguous); zero beyond nlist or d.  Norms padded with +inf so a
// padding centroid is never selected.  d4 is a multiple of 8.
__global__ void centroid_blocks_kernel(const float *__restrict__ c, int d, int d4, int nlist,
                                       int nblk, float *__restrict__ cblk,
                                       float *__restrict__ cnorm_pad)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)nblk * d4 * 64;
    if (i < total) {
        const int j = (int)(i & 3);
        const int lane = (int)((i >> 2) & 63);
        const int64_t rest = i >> 8;
        const int s = 4 * (int)(rest % (d4 / 4)) + j;
        const int64_t b = rest / (d4 / 4);
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

// Distance tiles pass between the two roles of the coarse kernel through a
// ring of kRing buffers in LDS with two counters per buffer, instead of a
// workgroup barrier per tile: the roles take about as long per tile, and a
// barrier made each wait for the other's slower tiles.  Counters only grow:
// a matrix wave adds 1 to produced[b] once its part of a tile is in buffer b
// (8 parts per tile), a selection wave adds 1 to consumed[b] once it has
// read its rows (8 readers).  Waits are bounded: a wait that takes more than
// 2^22 polls sets `broken`, and from then on every wait returns at once (the
// kernel then ends with wrong probes instead of hanging; never expected).
constexpr int kRing = 4;

// Tiles (counted from the start of a split's range) after which the
// selection waves of both top-nprobe kernels exchange bounds: after tiles
// 1 and 3, every 4 tiles up to tile 31, every 16 up to tile 127, then every
// 128.  Early on the k-th values fall fastest and a split alone has seen few
// centroids, so the shared bounds are worth most there; later each exchange
// (some 4,000-6,000 cycles of the selection wave, measured: the lane
// selects, the global atomics and the loads of the shared values) costs more
// than the few candidates it removes.  At the 1B coarse
// shape (8 splits of 512 tiles, k 128) a stream model of the selection gives
// 429 candidates staged per query and split and 6.2 buffer merges from 18
// exchanges, against 553 and 8.8 from 64 with an exchange every 8 tiles
// (split-bfloat16 kernel alone, with the raised priority and the
// constant-mask selects below: 4.11 -> 3.52 ms).
__device__ __forceinline__ bool exchange_after(int x)
{
    return x == 1 || (x < 32 ? (x & 3) == 3 : x < 128 ? (x & 15) == 15 : (x & 127) == 127);
}

// Lane `i` (a compile-time constant) of `vec` replaced by the wave-uniform
// value `u`: a select under a constant lane mask, which the compiler
// rematerialises instead of keeping sixteen masks live in registers.
__device__ __forceinline__ float set_lane(float vec, int i, float u)
{
    return __builtin_amdgcn_inverse_ballot_w64(1ull << i) ? u : vec;
}

// The value of lane `i` (v_readlane).
__device__ __forceinline__ float lane_value(float vec, int i)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(vec), i));
}

__device__ __forceinline__ void ring_wait(const uint32_t *ctr, uint32_t target, uint32_t *broken)
{
    uint32_t n = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (__hip_atomic_load(broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
            break;
        if (++n > (1u << 22)) {
            __hip_atomic_store(broken, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // the buffer's LDS accesses stay after the wait
    __asm__ volatile("" ::: "memory");
}

// Count this wave's LDS writes (or reads) of a buffer once they are complete;
// the wait covers LDS operations only, so global loads in flight (the next
// tile's B operand) stay in flight.
__device__ __forceinline__ void ring_signal(uint32_t *ctr)
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup of 16 waves in two roles over the tiles of its range, meeting in
// the ring of distance tiles:
//  * 8 matrix waves: wave w computes column block w%4 of row groups
//    RPW*(w/4) .. +RPW of a tile (A operand of its rows in registers, the
//    next tile's B operand prefetched) and writes |x|^2 + |c|^2 - 2 x.c:
//    the accumulators start at |x|^2 + |c|^2 and the A operand holds -2 x,
//    so the products are added onto the norms and the result goes to LDS
//    as it is (inner product: they start at 0 and A holds -x, giving
//    -<x, c>);
//  * 8 selection waves: each owns QS = TQ/8 queries and pushes their 64
//    distances of a tile into its register top-k (WaveTopK).
// So the matrix cores and the selection run at the same time on every SIMD.
template <int NW, int RG, int RPW, int KD, bool IP>
__global__ __launch_bounds__(1024) void coarse_mfma_kernel(
    const float *__restrict__ queries, int64_t nq, int d, int nblk, int nprobe,
    const float *__restrict__ cblk, const float *__restrict__ cnorm_pad, int splits,
    float *__restrict__ part_d, uint32_t *__restrict__ part_p, uint32_t *__restrict__ qbound,
    uint32_t *__restrict__ pslot, int32_t *__restrict__ probes, float *__restrict__ probe_d)
{
    constexpr int TQ = 16 * RG, THREADS = 1024, MW = 8, QS = TQ / 8, KW = 64 * NW;
    static_assert(4 * RG / RPW == MW, "eight matrix waves");
    extern __shared__ __align__(16) unsigned char smem[];
    const int xs = 4 * KD + 1; // odd stride: the 16 rows of an A read hit 16 banks
    float *xt = reinterpret_cast<float *>(smem);                      // [TQ][xs]
    float *xn = xt + TQ * xs;                                          // [TQ]
    float *dt = xn + TQ;                                                   // [kRing][TQ][64]
    uint32_t *stage = reinterpret_cast<uint32_t *>(dt + kRing * TQ * 64); // [TQ][128]
    uint32_t *produced = stage + TQ * 128;                                 // [kRing]
    uint32_t *consumed = produced + kRing;                                 // [kRing]
    uint32_t *broken = consumed + kRing;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    const bool matrix = wave < MW;
    const int cbk = wave & 3, rg0 = RPW * ((wave & 7) >> 2);
    const int sw = wave - MW; // selection wave number
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
        float acc = 0.f;
        for (int c = 0; c < 4 * KD; ++c)
            acc = fmaf(xt[tid * xs + c], xt[tid * xs + c], acc);
        xn[tid] = acc;
    }
    if (tid < 2 * kRing + 1)
        produced[tid] = 0u; // produced, consumed, broken
    __syncthreads();

    // The two roles run separate loops, so each keeps only its own registers
    // live.
    if (matrix) {
        // A layout of 16x16x4: lane l supplies row l%16, K-index l/16 of each step
        // (scaled by -2, or -1 for the inner product: exact; the sign flip is
        // an integer operation, as a float negation here was folded into
        // the operands at the cost of a second copy of A)
        float a[RPW][KD];
#pragma unroll
        for (int g = 0; g < RPW; ++g) {
            const float *ap = xt + ((rg0 + g) * 16 + (lane & 15)) * xs + (lane >> 4);
#pragma unroll
            for (int s = 0; s < KD; ++s)
                a[g][s] = IP ? __int_as_float(__float_as_int(ap[4 * s]) ^ (int)0x80000000)
                             : -2.f * ap[4 * s];
        }
        // |x|^2 of the 4*RPW query rows this lane holds in the D layout
        float xr[RPW][4];
#pragma unroll
        for (int g = 0; g < RPW; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xr[g][r] = xn[(rg0 + g) * 16 + 4 * (lane >> 4) + r];
        // B operand and |c|^2 of a tile, loaded one tile ahead
        float b0[KD], b1[KD], c0 = INFINITY, c1 = INFINITY;
        // Unconditional (past the range it re-reads the last tile): a load
        // under a branch makes the compiler wait for it too early.
        auto load_b = [&](int tile, float (&b)[KD], float &cn) {
            tile = tile < t1 ? tile : t1 - 1;
            const float4 *bp =
                reinterpret_cast<const float4 *>(cblk) + (size_t)(tile * 4 + cbk) * (KD / 4) * 64 + lane;
#pragma unroll
            for (int s4 = 0; s4 < KD / 4; ++s4) {
                const float4 v = bp[(size_t)s4 * 64];
                b[4 * s4] = v.x;
                b[4 * s4 + 1] = v.y;
                b[4 * s4 + 2] = v.z;
                b[4 * s4 + 3] = v.w;
            }
            cn = cnorm_pad[(tile * 4 + cbk) * 16 + (lane & 15)];
        };
        // tile `tile` into its ring buffer, prefetching the next tile's B
        // operand; the buffer is taken once the selection waves have read
        // the tile that held it kRing tiles before
        auto multiply = [&](int tile, const float (&bc)[KD], float cc, float (&bn)[KD],
                            float &cnext) {
            const int col = lane & 15;
            load_b(tile + 1, bn, cnext);
            // keep the next tile's loads ahead of this tile's MFMAs (the
            // scheduler would otherwise sink them below)
            __builtin_amdgcn_sched_barrier(0);
            const int rb = (tile - t0) % kRing;
            const uint32_t visit = (uint32_t)((tile - t0) / kRing);
            if (visit > 0)
                ring_wait(&consumed[rb], 8u * visit, broken);
            float *dtile = dt + rb * TQ * 64;
            // inner product: a padding centroid (norm +inf) starts at +inf
            const float ic = cc == INFINITY ? INFINITY : 0.f;
#pragma unroll
            for (int g = 0; g < RPW; ++g) {
                v4f acc;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] = IP ? ic : xr[g][r] + cc;
#pragma unroll
                for (int s = 0; s < KD; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][s], bc[s], acc, 0, 0, 0);
                // D layout of 16x16x4: lane l holds rows 4*(l/16) + r of column l%16
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dtile[((rg0 + g) * 16 + 4 * (lane >> 4) + r) * 64 + cbk * 16 + col] = acc[r];
            }
            ring_signal(&produced[rb]);
        };
        if (t0 < t1)
            load_b(t0, b0, c0);
        int t = t0;
        for (; t + 1 < t1; t += 2) {
            multiply(t, b0, c0, b1, c1);
            multiply(t + 1, b1, c1, b0, c0);
        }
        if (t < t1)
            multiply(t, b0, c0, b1, c1);
        return;
    }

    // Splits of a query share two bounds on its k-th smallest distance:
    //  * each split's k-th value (its k values are at most that), the
    //    smallest over the splits kept by an atomic min per query;
    //  * each split's rk-th value, rk = ceil(k / splits), in a slot of its
    //    own: every split has rk values at most its slot, so the union of the
    //    splits has >= k values at most the largest slot (+inf until every
    //    split has published), a far tighter bound early in the sweep.
    // After the tiles exchange_after names a wave publishes its queries'
    // values and loads the shared ones, which it applies a tile later.
    // Values only decrease, so a stale load is a weaker bound, never a wrong
    // one.  Lane i of a selection wave handles query i for the k-th value;
    // the slots of query i, split s are loaded by lane i + 8 (s % 8), two
    // loads for up to 16 splits (more splits use the first bound only).
    // Selection waves issue first when both roles of a SIMD are ready.
    __builtin_amdgcn_s_setprio(3);
    const int rk = splits > 1 ? (nprobe + splits - 1) / splits : nprobe;
    WaveTopK<NW> sel[QS];
#pragma unroll
    for (int i = 0; i < QS; ++i)
        sel[i].init(nprobe, stage + (sw * QS + i) * 128, rk);
    int64_t ql = q0 + sw * QS + (lane < QS ? lane : 0);
    const bool qvalid = lane < QS && ql < nq;
    ql = ql < nq ? ql : nq - 1; // the loads stay unconditional
    const bool use_slots = splits > 1 && splits <= 16;
    const int64_t qs = q0 + sw * QS + (lane & 7);
    const bool slot_q = (lane & 7) < QS && qs < nq;
    const int s_lo = lane >> 3, s_hi = 8 + (lane >> 3);
    const uint32_t *ps_lo = pslot + (slot_q && s_lo < splits ? qs * splits + s_lo : 0);
    const uint32_t *ps_hi = pslot + (slot_q && s_hi < splits ? qs * splits + s_hi : 0);
    const bool lo_ok = slot_q && s_lo < splits, hi_ok = slot_q && s_hi < splits;
    uint32_t nb = float_order_key(INFINITY);
    uint32_t nu0 = 0u, nu1 = 0u; // order key 0 is below every float: neutral for max
    bool pending = false;
    for (int t = t0; t < t1; ++t) {
        if (pending) {
            uint32_t u = nu0 > nu1 ? nu0 : nu1;
            uint32_t o = xor_lane<8>(u);
            u = u > o ? u : o;
            o = xor_lane<16>(u);
            u = u > o ? u : o;
            o = xor_lane<32>(u);
            u = u > o ? u : o;
            u = use_slots ? u : float_order_key(INFINITY);
            const uint32_t b = nb < u ? nb : u;
            const float bf = float_from_order_key(b);
#pragma unroll
            for (int i = 0; i < QS; ++i)
                sel[i].bound(lane_value(bf, i));
            pending = false;
        }
        // all reads first (one LDS round trip), then the selections
        const int rb = (t - t0) % kRing;
        ring_wait(&produced[rb], 8u * (uint32_t)((t - t0) / kRing + 1), broken);
        const float *dtile = dt + rb * TQ * 64;
        float cand[QS];
#pragma unroll
        for (int i = 0; i < QS; ++i)
            cand[i] = dtile[(sw * QS + i) * 64 + lane];
        ring_signal(&consumed[rb]);
#pragma unroll
        for (int i = 0; i < QS; ++i)
            sel[i].push(cand[i], (uint32_t)(t * 64 + lane));
        if (splits > 1 && exchange_after(t - t0)) {
            // lane i: query i's values (one select under a constant mask each)
            float mine = INFINITY, mpart = INFINITY;
#pragma unroll
            for (int i = 0; i < QS; ++i) {
                mine = set_lane(mine, i, sel[i].kth);
                mpart = set_lane(mpart, i, sel[i].part);
            }
            if (qvalid && mine < INFINITY)
                atomicMin(qbound + ql, float_order_key(mine));
            if (use_slots && qvalid)
                __hip_atomic_store(pslot + ql * splits + split, float_order_key(mpart),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nb = __hip_atomic_load(qbound + ql, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (use_slots) {
                nu0 = __hip_atomic_load(ps_lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                nu1 = __hip_atomic_load(ps_hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                nu0 = lo_ok ? nu0 : 0u;
                nu1 = hi_ok ? nu1 : 0u;
            }
            pending = true;
        }
    }
#pragma unroll
    for (int i = 0; i < QS; ++i) {
        sel[i].flush();
        const int64_t q = q0 + sw * QS + i;
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

// ---------------------------------------------------------------------------
// Coarse distances as float32-exact products from bfloat16 matrix cores.
//
// Each operand is split into three bfloat16 parts, x = x0 + x1 + x2 (each part
// rounded to nearest from the remainder, so the sum is x itself for float32
// values of normal range), and x.c is the sum of the six products
// x2 c0, x0 c2, x1 c1, x1 c0, x0 c1, x0 c0 ("Leveraging the bfloat16 artificial
// intelligence datatype for higher-precision computations", Henry, Tang and
// Heinecke, 2019: the split and the dropped small terms).  Every product of
// two bfloat16 parts is exact in float32; the three dropped products are at
// most 2^-23 |x_i c_i| together.  v_mfma_f32_16x16x32_bf16 does 8x the K of
// the float32 16x16x4 instruction in half the cycles, so the six terms take
// 2.7x fewer matrix cycles than the float32 product.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// float32 -> bfloat16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_value(uint32_t b) { return __uint_as_float(b << 16); }

// x = p0 + p1 + p2, each a bfloat16 rounded from what the previous parts left
// (the remainders are exact in float32)
__device__ __forceinline__ void split_bf16x3(float x, uint16_t &p0, uint16_t &p1, uint16_t &p2)
{
    const uint32_t b0 = bf16_rne_bits(x);
    const float r1 = x - bf16_bits_value(b0);
    const uint32_t b1 = bf16_rne_bits(r1);
    const float r2 = r1 - bf16_bits_value(b1);
    p0 = (uint16_t)b0;
    p1 = (uint16_t)b1;
    p2 = (uint16_t)bf16_rne_bits(r2);
}

// Centroid parts in B-operand order of v_mfma_f32_16x16x32_bf16: for tile t
// (64 centroids), column block cb (16), K-block s (32 dims) and part p, lane l
// holds centroid 64 t + 16 cb + l%16, dims 32 s + 8 (l/16) .. +7; stored as
// [t][cb][s][p][l][8] so that a wave reads 1 KiB contiguous per (s, p).  Zero
// beyond nlist or d.
__global__ void centroid_x6_kernel(const float *__restrict__ c, int d, int nlist, int64_t ntile,
                                   int kb, uint16_t *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ntile * 4 * kb * 64)
        return;
    const int lane = (int)(i & 63);
    const int64_t rest = i >> 6;
    const int s = (int)(rest % kb);
    const int64_t tcb = rest / kb; // 4 t + cb
    const int64_t row = tcb * 16 + (lane & 15);
    const int col0 = 32 * s + 8 * (lane >> 4);
    u16x8_t v0, v1, v2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (row < nlist && col0 + e < d) ? c[row * d + col0 + e] : 0.f;
        uint16_t p0, p1, p2;
        split_bf16x3(x, p0, p1, p2);
        v0[e] = p0;
        v1[e] = p1;
        v2[e] = p2;
    }
    uint16_t *o = out + ((tcb * kb + s) * 3) * 512 + lane * 8;
    *reinterpret_cast<u16x8_t *>(o) = v0;
    *reinterpret_cast<u16x8_t *>(o + 512) = v1;
    *reinterpret_cast<u16x8_t *>(o + 1024) = v2;
}

// Workgroup of 8 waves, 64 queries, a range of 64-centroid tiles:
//  * 4 matrix waves: wave w computes column block w of every tile for all 64
//    queries (four row groups, four independent accumulator chains): the A
//    parts of the 64 queries stay in registers (3 parts x 4 row groups x KB
//    K-blocks), the B parts of a K-block are reloaded for the next tile right
//    after their last product here (one tile of latency, no second buffer);
//    accumulators start at |x|^2 + |c|^2 (0 for the inner product) and A holds
//    -2x (-x), so the chain's result is the distance;
//  * 4 selection waves: 16 queries each, a register top-k per query (WaveTopK).
// The roles meet in the ring of distance tiles (ring_wait / ring_signal) as
// in the float32 kernel, with 4 writers and 4 readers per tile.
template <int NW, int KB, bool IP>
__global__ __launch_bounds__(512) void coarse_x6_kernel(
    const float *__restrict__ queries, int64_t nq, int d, int nblk, int nprobe,
    const uint16_t *__restrict__ cx6, const float *__restrict__ cnorm_pad, int splits,
    float *__restrict__ part_d, uint32_t *__restrict__ part_p, uint32_t *__restrict__ qbound,
    uint32_t *__restrict__ pslot, int32_t *__restrict__ probes, float *__restrict__ probe_d)
{
    constexpr int TQ = 64, THREADS = 512, MW = 4, QS = 16, KW = 64 * NW;
    constexpr int XS = 32 * KB + 1; // odd stride
    extern __shared__ __align__(16) unsigned char smem[];
    float *xt = reinterpret_cast<float *>(smem);                            // [TQ][XS]
    float *xn = xt + TQ * XS;                                               // [TQ]
    float *dt = xn + TQ;                                                    // [kRing][TQ][64]
    uint32_t *stage = reinterpret_cast<uint32_t *>(dt + kRing * TQ * 64);  // [TQ][128]
    uint32_t *produced = stage + TQ * 128;                                  // [kRing]
    uint32_t *consumed = produced + kRing;                                  // [kRing]
    uint32_t *broken = consumed + kRing;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform in the wave
    const bool matrix = wave < MW;
    const int64_t q0 = (int64_t)blockIdx.x * TQ;
    const int split = blockIdx.y;
    const int ntile = (nblk + 3) / 4;
    const int t0 = (int)((int64_t)ntile * split / splits);
    const int t1 = (int)((int64_t)ntile * (split + 1) / splits);

    for (int i = tid; i < TQ * 32 * KB; i += THREADS) {
        const int row = i / (32 * KB), col = i % (32 * KB);
        const int64_t q = q0 + row;
        xt[row * XS + col] = (q < nq && col < d) ? queries[q * d + col] : 0.f;
    }
    if (tid < 2 * kRing + 1)
        produced[tid] = 0u; // produced, consumed, broken
    __syncthreads();
    if (tid < TQ) {
        // |x|^2 in index order over whole groups of 4 dims (the zero padding
        // adds nothing): the same value as the float32 kernel's
        float acc = 0.f;
        for (int c = 0; c < 32 * KB; ++c)
            acc = fmaf(xt[tid * XS + c], xt[tid * XS + c], acc);
        xn[tid] = acc;
    }
    __syncthreads();

    if (matrix) {
        const int cb = wave;
        // A parts: row group g, K-block s: lane l supplies row 16 g + l%16,
        // dims 32 s + 8 (l/16) .. +7, scaled by -2 (-1 for the inner product)
        bf16x8_t a0[4][KB], a1[4][KB], a2[4][KB];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                const float *ap = xt + (g * 16 + (lane & 15)) * XS + 32 * s + 8 * (lane >> 4);
                u16x8_t v0, v1, v2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = IP ? -ap[e] : -2.f * ap[e];
                    uint16_t p0, p1, p2;
                    split_bf16x3(x, p0, p1, p2);
                    v0[e] = p0;
                    v1[e] = p1;
                    v2[e] = p2;
                }
                a0[g][s] = __builtin_bit_cast(bf16x8_t, v0);
                a1[g][s] = __builtin_bit_cast(bf16x8_t, v1);
                a2[g][s] = __builtin_bit_cast(bf16x8_t, v2);
            }
        float xr[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xr[g][r] = xn[g * 16 + 4 * (lane >> 4) + r];
        // B parts of one K-block of a tile (past the range: the last tile again,
        // so the loads stay unconditional)
        auto b_ptr = [&](int tile, int s, int p) {
            tile = tile < t1 ? tile : t1 - 1;
            return reinterpret_cast<const u16x8_t *>(
                cx6 + ((((size_t)tile * 4 + cb) * KB + s) * 3 + p) * 512 + lane * 8);
        };
        bf16x8_t b[KB][3];
        float cc = INFINITY;
        if (t0 < t1) {
#pragma unroll
            for (int s = 0; s < KB; ++s)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    b[s][p] = __builtin_bit_cast(bf16x8_t, *b_ptr(t0, s, p));
            cc = cnorm_pad[((size_t)t0 * 4 + cb) * 16 + (lane & 15)];
        }
        for (int tile = t0; tile < t1; ++tile) {
            const int rb = (tile - t0) % kRing;
            const uint32_t visit = (uint32_t)((tile - t0) / kRing);
            v4f acc[4];
            const float ic = cc == INFINITY ? INFINITY : 0.f;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[g][r] = IP ? ic : xr[g][r] + cc;
            const int tn = tile + 1;
            const float cn = cnorm_pad[((size_t)(tn < t1 ? tn : t1 - 1) * 4 + cb) * 16 + (lane & 15)];
#pragma unroll
            for (int s = 0; s < KB; ++s) {
                // small terms first, the leading product last
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[g][s], b[s][0], acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[g][s], b[s][2], acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[g][s], b[s][1], acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[g][s], b[s][0], acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[g][s], b[s][1], acc[g], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[g][s], b[s][0], acc[g], 0, 0, 0);
                // this K-block's B parts are done: the next tile's
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    b[s][p] = __builtin_bit_cast(bf16x8_t, *b_ptr(tn, s, p));
                __builtin_amdgcn_sched_barrier(0);
            }
            cc = cn;
            if (visit > 0)
                ring_wait(&consumed[rb], 4u * visit, broken);
            float *dtile = dt + rb * TQ * 64;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dtile[(g * 16 + 4 * (lane >> 4) + r) * 64 + cb * 16 + (lane & 15)] = acc[g][r];
            ring_signal(&produced[rb]);
        }
        return;
    }

    const int sw = wave - MW; // selection wave: queries 16 sw .. 16 sw + 15
    // the selection is the slower role here: its waves issue first when both
    // roles of a SIMD are ready (the matrix waves' MFMA chains fill the gaps)
    __builtin_amdgcn_s_setprio(3);
    const int rk = splits > 1 ? (nprobe + splits - 1) / splits : nprobe;
    WaveTopK<NW> sel[QS];
#pragma unroll
    for (int i = 0; i < QS; ++i)
        sel[i].init(nprobe, stage + (sw * QS + i) * 128, rk);
    // shared bounds between the splits, as in the float32 kernel (exchanged
    // after the tiles exchange_after names): lane i
    // (< 16) publishes query i's k-th value and its slot value; the slots of
    // query i, split s, are loaded by lane i + 16 (s % 4), four loads for up
    // to 16 splits (more splits use the first bound only)
    int64_t ql = q0 + sw * QS + (lane < QS ? lane : 0);
    const bool qvalid = lane < QS && ql < nq;
    ql = ql < nq ? ql : nq - 1;
    const bool use_slots = splits > 1 && splits <= 16;
    const int64_t qs = q0 + sw * QS + (lane & 15);
    const bool slot_q = qs < nq;
    uint32_t nb = float_order_key(INFINITY);
    uint32_t nu[4] = {0u, 0u, 0u, 0u}; // order key 0 is below every float
    bool pending = false;
    for (int t = t0; t < t1; ++t) {
        if (pending) {
            uint32_t u = nu[0];
#pragma unroll
            for (int j = 1; j < 4; ++j)
                u = u > nu[j] ? u : nu[j];
            uint32_t o = xor_lane<16>(u);
            u = u > o ? u : o;
            o = xor_lane<32>(u);
            u = u > o ? u : o;
            u = use_slots ? u : float_order_key(INFINITY);
            const uint32_t bnd = nb < u ? nb : u;
            const float bf = float_from_order_key(bnd);
#pragma unroll
            for (int i = 0; i < QS; ++i)
                sel[i].bound(lane_value(bf, i));
            pending = false;
        }
        const int rb = (t - t0) % kRing;
        ring_wait(&produced[rb], 4u * (uint32_t)((t - t0) / kRing + 1), broken);
        const float *dtile = dt + rb * TQ * 64;
        float cand[QS];
#pragma unroll
        for (int i = 0; i < QS; ++i)
            cand[i] = dtile[(sw * QS + i) * 64 + lane];
        ring_signal(&consumed[rb]);
#pragma unroll
        for (int i = 0; i < QS; ++i)
            sel[i].push(cand[i], (uint32_t)(t * 64 + lane));
        if (splits > 1 && exchange_after(t - t0)) {
            // lane i: query i's values (one select under a constant mask each)
            float mine = INFINITY, mpart = INFINITY;
#pragma unroll
            for (int i = 0; i < QS; ++i) {
                mine = set_lane(mine, i, sel[i].kth);
                mpart = set_lane(mpart, i, sel[i].part);
            }
            if (qvalid && mine < INFINITY)
                atomicMin(qbound + ql, float_order_key(mine));
            if (use_slots && qvalid)
                __hip_atomic_store(pslot + ql * splits + split, float_order_key(mpart),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nb = __hip_atomic_load(qbound + ql, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (use_slots) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sj = (lane >> 4) + 4 * j;
                    const bool ok = slot_q && sj < splits;
                    const uint32_t *ps = pslot + (ok ? qs * splits + sj : 0);
                    const uint32_t v =
                        __hip_atomic_load(ps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    nu[j] = ok ? v : 0u;
                }
            }
            pending = true;
        }
    }
#pragma unroll
    for (int i = 0; i < QS; ++i) {
        sel[i].flush();
        const int64_t q = q0 + sw * QS + i;
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

// nprobe = 1 (the nearest list of every vector: assignment when an index
// is built, k-means): the same products and the same distance expression as
// above, but a lane keeps the smallest distance of each of its rows (its
// column of every tile) in registers, so there is no selection role, no
// distance tile in LDS and no barrier inside the sweep.  Eight matrix waves
// (4 column blocks x 2 row groups of RPW*16 rows), two workgroups per CU.
// Lane minima meet across the 16 columns of a block by shuffles, across the
// 4 blocks in LDS, across centroid splits in coarse_argmin_merge_kernel.
// Equal distances go to the smaller centroid number (a lane sweeps its
// centroids in increasing order and keeps the first; elsewhere the smaller
// number wins), so the result is the first minimum, as argmin defines it.
__device__ __forceinline__ void argmin_take(float &bv, int32_t &bi, float ov, int32_t oi)
{
    if (ov < bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

template <int RG, int RPW, int KD>
__global__ __launch_bounds__(256 * RG / RPW) __attribute__((amdgpu_waves_per_eu(4)))
void coarse_argmin_kernel(const float *__restrict__ queries, int64_t nq, int d, int nblk,
                          const float *__restrict__ cblk, const float *__restrict__ cnorm_pad,
                          int splits, float *__restrict__ part_d, int32_t *__restrict__ part_i,
                          int32_t *__restrict__ probes, float *__restrict__ probe_d, int ip)
{
    constexpr int TQ = 16 * RG, THREADS = 256 * RG / RPW;
    static_assert(THREADS == 512, "eight matrix waves");
    extern __shared__ __align__(16) unsigned char smem[];
    const int xs = 4 * KD + 1; // odd stride: the 16 rows of an A read hit 16 banks
    float *xt = reinterpret_cast<float *>(smem);            // [TQ][xs]
    float *xn = xt + TQ * xs;                                // [TQ]
    float *md = xn + TQ;                                     // [TQ][4] block minima
    int32_t *mi = reinterpret_cast<int32_t *>(md + TQ * 4);  // [TQ][4] their centroids

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cbk = wave & 3, rg0 = RPW * (wave >> 2);
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
        float acc = 0.f;
        for (int c = 0; c < 4 * KD; ++c)
            acc = fmaf(xt[tid * xs + c], xt[tid * xs + c], acc);
        xn[tid] = acc;
    }
    __syncthreads();

    float a[RPW][KD];
#pragma unroll
    for (int g = 0; g < RPW; ++g) {
        const float *ap = xt + ((rg0 + g) * 16 + (lane & 15)) * xs + (lane >> 4);
#pragma unroll
        for (int s = 0; s < KD; ++s)
            a[g][s] = ap[4 * s];
    }
    float xr[RPW][4];
#pragma unroll
    for (int g = 0; g < RPW; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            xr[g][r] = xn[(rg0 + g) * 16 + 4 * (lane >> 4) + r];
    float bv[RPW][4];
    int32_t bi[RPW][4];
#pragma unroll
    for (int g = 0; g < RPW; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bv[g][r] = INFINITY;
            bi[g][r] = INT32_MAX; // no centroid yet
        }

    // B operand and |c|^2 of a tile, loaded one tile ahead
    float b0[KD], b1[KD], c0 = INFINITY, c1 = INFINITY;
    auto load_b = [&](int tile, float (&b)[KD], float &cn) {
        tile = tile < t1 ? tile : t1 - 1;
        const float4 *bp =
            reinterpret_cast<const float4 *>(cblk) + (size_t)(tile * 4 + cbk) * (KD / 4) * 64 + lane;
#pragma unroll
        for (int s4 = 0; s4 < KD / 4; ++s4) {
            const float4 v = bp[(size_t)s4 * 64];
            b[4 * s4] = v.x;
            b[4 * s4 + 1] = v.y;
            b[4 * s4 + 2] = v.z;
            b[4 * s4 + 3] = v.w;
        }
        cn = cnorm_pad[(tile * 4 + cbk) * 16 + (lane & 15)];
    };
    // tile `tile` with operand bc, the next tile's operand loaded into bn
    auto step = [&](int tile, const float (&bc)[KD], float cc, float (&bn)[KD], float &cnext) {
        load_b(tile + 1, bn, cnext);
        __builtin_amdgcn_sched_barrier(0);
        const int32_t cid = (tile * 4 + cbk) * 16 + (lane & 15);
#pragma unroll
        for (int g = 0; g < RPW; ++g) {
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KD; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][s], bc[s], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float dist =
                    ip ? (cc == INFINITY ? INFINITY : -acc[r]) : xr[g][r] + cc - 2.f * acc[r];
                if (dist < bv[g][r]) {
                    bv[g][r] = dist;
                    bi[g][r] = cid;
                }
            }
        }
    };
    if (t0 < t1)
        load_b(t0, b0, c0);
    for (int t = t0; t < t1; t += 2) {
        step(t, b0, c0, b1, c1);
        if (t + 1 < t1)
            step(t + 1, b1, c1, b0, c0);
    }

    // the 16 columns of the block: lanes 16h .. 16h+15 hold the same rows
#pragma unroll
    for (int g = 0; g < RPW; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) {
                const float ov = __shfl_xor(bv[g][r], sh);
                const int32_t oi = __shfl_xor(bi[g][r], sh);
                argmin_take(bv[g][r], bi[g][r], ov, oi);
            }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int g = 0; g < RPW; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (rg0 + g) * 16 + 4 * (lane >> 4) + r;
                md[row * 4 + cbk] = bv[g][r];
                mi[row * 4 + cbk] = bi[g][r];
            }
    }
    __syncthreads();
    if (tid < TQ && q0 + tid < nq) {
        float v = md[tid * 4];
        int32_t i = mi[tid * 4];
#pragma unroll
        for (int c = 1; c < 4; ++c)
            argmin_take(v, i, md[tid * 4 + c], mi[tid * 4 + c]);
        const int64_t q = q0 + tid;
        if (splits == 1) {
            probes[q] = i == INT32_MAX ? 0 : i;
            if (probe_d)
                probe_d[q] = v;
        } else {
            part_d[q * splits + split] = v;
            part_i[q * splits + split] = i;
        }
    }
}

// The splits' minima of each query, in split order (one thread per query).
__global__ __launch_bounds__(256) void coarse_argmin_merge_kernel(
    const float *__restrict__ part_d, const int32_t *__restrict__ part_i, int64_t nq, int splits,
    int32_t *__restrict__ probes, float *__restrict__ probe_d)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= nq)
        return;
    float v = part_d[q * splits];
    int32_t i = part_i[q * splits];
    for (int s = 1; s < splits; ++s)
        argmin_take(v, i, part_d[q * splits + s], part_i[q * splits + s]);
    probes[q] = i == INT32_MAX ? 0 : i;
    if (probe_d)
        probe_d[q] = v;
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

__global__ void coarse_bound_init_kernel(uint32_t *__restrict__ qbound, int64_t n);

bool coarse_uses_x6(int d, int nlist) { return d <= 96 && nlist >= 16384; }

hipError_t launch_centroid_blocks(const DeviceIndex &ix, hipStream_t stream)
{
    const int64_t total = (int64_t)ix.nblk * ix.d4 * 64;
    const int64_t n = total > (int64_t)ix.nblk * 16 ? total : (int64_t)ix.nblk * 16;
    hipLaunchKernelGGL(centroid_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, ix.centroids, ix.d, ix.d4, ix.nlist, ix.nblk, ix.cblk,
                       ix.cnorm_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !ix.cx6)
        return e;
    const int64_t ntile = ix.nblk / 4;
    const int64_t nx = ntile * 4 * ix.x6_kb * 64;
    hipLaunchKernelGGL(centroid_x6_kernel, dim3((unsigned)((nx + 255) / 256)), dim3(256), 0,
                       stream, ix.centroids, ix.d, ix.nlist, ntile, ix.x6_kb, ix.cx6);
    return hipGetLastError();
}

// The bf16x6 kernel for one (NW, KB): the same workgroup grid, splits and
// workspace as the float32 kernel with four row groups.
template <int NW, int KB>
static hipError_t coarse_x6_variant(const DeviceIndex &ix, const float *queries, int64_t nq,
                                    int nprobe, int splits, void *ws, int32_t *probes,
                                    float *probe_d, hipStream_t stream, bool ip)
{
    constexpr int TQ = 64;
    const size_t lds = (size_t)TQ * (32 * KB + 1) * 4 + TQ * 4 + (size_t)kRing * TQ * 64 * 4 +
                       TQ * 512 + (2 * kRing + 1) * 4;
    auto kern = ip ? coarse_x6_kernel<NW, KB, true> : coarse_x6_kernel<NW, KB, false>;
    if (lds > 160 * 1024)
        return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    float *part_d = static_cast<float *>(ws);
    uint32_t *part_p = reinterpret_cast<uint32_t *>(part_d + (size_t)nq * splits * 64 * NW);
    uint32_t *qbound = part_p + (size_t)nq * splits * 64 * NW;
    uint32_t *pslot = qbound + nq;
    if (splits > 1) {
        const int64_t n = nq * (1 + (int64_t)splits);
        hipLaunchKernelGGL(coarse_bound_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, stream, qbound, n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const dim3 grid((unsigned)((nq + TQ - 1) / TQ), (unsigned)splits);
    hipLaunchKernelGGL(kern, grid, dim3(512), lds, stream, queries, nq, ix.d, ix.nblk, nprobe,
                       ix.cx6, ix.cnorm_pad, splits, part_d, part_p, qbound, pslot, probes,
                       probe_d);
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    hipLaunchKernelGGL(coarse_merge_kernel<NW>, dim3((unsigned)nq), dim3(64), 0, stream, part_d,
                       part_p, nq, splits, nprobe, probes, probe_d);
    return hipGetLastError();
}

template <int NW>
static hipError_t coarse_x6_k(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                              int splits, void *ws, int32_t *probes, float *probe_d,
                              hipStream_t stream, bool ip)
{
    switch (ix.x6_kb) {
    case 1:
        return coarse_x6_variant<NW, 1>(ix, queries, nq, nprobe, splits, ws, probes, probe_d, stream, ip);
    case 2:
        return coarse_x6_variant<NW, 2>(ix, queries, nq, nprobe, splits, ws, probes, probe_d, stream, ip);
    case 3:
        return coarse_x6_variant<NW, 3>(ix, queries, nq, nprobe, splits, ws, probes, probe_d, stream, ip);
    default:
        return hipErrorInvalidValue;
    }
}

// Test switch: IVFPQ_TEST_COARSE_FP32=1 runs the float32 kernel where the
// bf16x6 one would (read on every call).
static bool coarse_force_fp32()
{
    const char *e = std::getenv("IVFPQ_TEST_COARSE_FP32");
    return e && e[0] == '1';
}

// Row groups per workgroup (16 queries each) and the centroid split: many
// centroids -> 4 row groups (fewer passes over the centroid array) when the
// registers allow it (1024 threads leave 128 per lane).  The split starts
// from about four rounds of workgroups over the CUs (one 16-wave workgroup
// resident per CU); a last round that fills only part of the chip costs as
// much as a full one, so among s0 .. 2 s0 splits the one with the fewest
// rounds x tiles per workgroup is taken (1% per extra split against it: more
// splits mean more selection and merge work).
static void coarse_shape(int64_t nq, int nblk, int d4, int *rg, int *splits)
{
    *rg = nblk >= 1024 && d4 <= 24 ? 4 : 2;
    const int64_t wgs = (nq + 16 * *rg - 1) / (16 * *rg);
    const int ntile = (nblk + 3) / 4;
    const int64_t slots = coarse_cu_count();
    const int smax = ntile < 64 ? ntile : 64;
    int s0 = (int)((slots * 4 + wgs - 1) / wgs);
    s0 = s0 < 1 ? 1 : s0;
    s0 = s0 > smax ? smax : s0;
    auto cost = [&](int s) {
        const int64_t rounds = (wgs * s + slots - 1) / slots;
        return (double)rounds * ((ntile + s - 1) / s) * (1.0 + 0.01 * (s - s0));
    };
    int best = s0;
    double bc = cost(s0);
    for (int s = s0 + 1; s <= 2 * s0 && s <= smax; ++s) {
        const double c = cost(s);
        if (c < bc) {
            bc = c;
            best = s;
        }
    }
    *splits = best;
}

// Shared bounds of the splits: per query, then per (query, split) slot.
__global__ void coarse_bound_init_kernel(uint32_t *__restrict__ qbound, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        qbound[i] = float_order_key(INFINITY);
}

// nprobe = 1: 64 queries per workgroup (two row groups per wave) while the
// two A operands fit the registers (K-steps <= 16), else 32; the split keeps
// about four rounds of two resident workgroups per CU.
static void argmin_shape(int64_t nq, int nblk, int d4, int *rg, int *splits)
{
    *rg = d4 <= 16 ? 4 : 2;
    const int64_t wgs = (nq + 16 * *rg - 1) / (16 * *rg);
    const int ntile = (nblk + 3) / 4;
    const int64_t want = (int64_t)coarse_cu_count() * 8;
    int s = (int)((want + wgs - 1) / wgs);
    s = s < 1 ? 1 : s;
    s = s > ntile ? ntile : s;
    s = s > 64 ? 64 : s;
    *splits = s;
}

size_t coarse_ws_bytes(const DeviceIndex &ix, int64_t nq, int nprobe)
{
    if (nprobe == 1 && ix.d4 <= 32) {
        int rg, splits;
        argmin_shape(nq, ix.nblk, ix.d4, &rg, &splits);
        return splits > 1 ? (size_t)nq * splits * 8 : 0;
    }
    int nw = 1;
    while (nw * 64 < nprobe)
        nw *= 2;
    if (nw > 2 || ix.d4 > 32)
        return 0;
    int rg, splits;
    coarse_shape(nq, ix.nblk, ix.d4, &rg, &splits);
    // partial top-k of every split, the per-query bound, the per-split slots
    return splits > 1 ? (size_t)nq * splits * 64 * nw * 8 + (size_t)nq * 4 +
                            (size_t)nq * splits * 4
                      : 0;
}

template <int NW, int RG, int RPW, int KD>
static hipError_t coarse_mfma_variant(const DeviceIndex &ix, const float *queries, int64_t nq,
                                      int nprobe, int splits, void *ws, int32_t *probes,
                                      float *probe_d, hipStream_t stream, bool ip)
{
    constexpr int TQ = 16 * RG;
    const size_t lds = (size_t)TQ * (4 * KD + 1) * 4 + TQ * 4 + (size_t)kRing * TQ * 64 * 4 +
                       TQ * 512 + (2 * kRing + 1) * 4;
    auto kern = ip ? coarse_mfma_kernel<NW, RG, RPW, KD, true>
                   : coarse_mfma_kernel<NW, RG, RPW, KD, false>;
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
    uint32_t *qbound = part_p + (size_t)nq * splits * 64 * NW;
    uint32_t *pslot = qbound + nq;
    if (splits > 1) {
        const int64_t n = nq * (1 + (int64_t)splits); // qbound and pslot are contiguous
        hipLaunchKernelGGL(coarse_bound_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, stream, qbound, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const dim3 grid((unsigned)((nq + TQ - 1) / TQ), (unsigned)splits);
    hipLaunchKernelGGL(kern, grid, dim3(1024), lds, stream, queries, nq, ix.d, ix.nblk, nprobe,
                       ix.cblk, ix.cnorm_pad, splits, part_d, part_p, qbound, pslot, probes,
                       probe_d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    hipLaunchKernelGGL(coarse_merge_kernel<NW>, dim3((unsigned)nq), dim3(64), 0, stream, part_d,
                       part_p, nq, splits, nprobe, probes, probe_d);
    return hipGetLastError();
}

// 64 queries per workgroup (two row groups per matrix wave) while the two A
// operands fit the registers (K-steps <= 24), else 32.
template <int NW>
static hipError_t coarse_mfma_k(const DeviceIndex &ix, const float *queries, int64_t nq,
                                int nprobe, int rg, int splits, void *ws, int32_t *probes,
                                float *probe_d, hipStream_t stream, bool ip)
{
    switch (ix.d4) {
    case 8:
        return rg == 4 ? coarse_mfma_variant<NW, 4, 2, 8>(ix, queries, nq, nprobe, splits, ws,
                                                          probes, probe_d, stream, ip)
                       : coarse_mfma_variant<NW, 2, 1, 8>(ix, queries, nq, nprobe, splits, ws,
                                                          probes, probe_d, stream, ip);
    case 16:
        return rg == 4 ? coarse_mfma_variant<NW, 4, 2, 16>(ix, queries, nq, nprobe, splits, ws,
                                                           probes, probe_d, stream, ip)
                       : coarse_mfma_variant<NW, 2, 1, 16>(ix, queries, nq, nprobe, splits, ws,
                                                           probes, probe_d, stream, ip);
    case 24:
        return rg == 4 ? coarse_mfma_variant<NW, 4, 2, 24>(ix, queries, nq, nprobe, splits, ws,
                                                           probes, probe_d, stream, ip)
                       : coarse_mfma_variant<NW, 2, 1, 24>(ix, queries, nq, nprobe, splits, ws,
                                                           probes, probe_d, stream, ip);
    case 32:
        return coarse_mfma_variant<NW, 2, 1, 32>(ix, queries, nq, nprobe, splits, ws, probes,
                                                 probe_d, stream, ip);
    default:
        return hipErrorInvalidValue;
    }
}

template <int RG, int RPW, int KD>
static hipError_t coarse_argmin_variant(const DeviceIndex &ix, const float *queries, int64_t nq,
                                        int splits, void *ws, int32_t *probes, float *probe_d,
                                        hipStream_t stream, bool ip)
{
    constexpr int TQ = 16 * RG;
    const size_t lds = (size_t)TQ * (4 * KD + 1) * 4 + TQ * 4 + TQ * 4 * 8;
    float *part_d = static_cast<float *>(ws);
    int32_t *part_i = reinterpret_cast<int32_t *>(part_d + (size_t)nq * splits);
    const dim3 grid((unsigned)((nq + TQ - 1) / TQ), (unsigned)splits);
    hipLaunchKernelGGL((coarse_argmin_kernel<RG, RPW, KD>), grid, dim3(256 * RG / RPW), lds,
                       stream, queries, nq, ix.d, ix.nblk, ix.cblk, ix.cnorm_pad, splits, part_d,
                       part_i, probes, probe_d, ip ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    hipLaunchKernelGGL(coarse_argmin_merge_kernel, dim3((unsigned)((nq + 255) / 256)), dim3(256),
                       0, stream, part_d, part_i, nq, splits, probes, probe_d);
    return hipGetLastError();
}

static hipError_t launch_coarse_argmin(const DeviceIndex &ix, const float *queries, int64_t nq,
                                       void *ws, int32_t *probes, float *probe_d,
                                       hipStream_t stream, bool ip)
{
    int rg, splits;
    argmin_shape(nq, ix.nblk, ix.d4, &rg, &splits);
    switch (ix.d4) {
    case 8:
        return coarse_argmin_variant<4, 2, 8>(ix, queries, nq, splits, ws, probes, probe_d,
                                              stream, ip);
    case 16:
        return coarse_argmin_variant<4, 2, 16>(ix, queries, nq, splits, ws, probes, probe_d,
                                               stream, ip);
    case 24:
        return coarse_argmin_variant<2, 1, 24>(ix, queries, nq, splits, ws, probes, probe_d,
                                               stream, ip);
    case 32:
        return coarse_argmin_variant<2, 1, 32>(ix, queries, nq, splits, ws, probes, probe_d,
                                               stream, ip);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_coarse(const DeviceIndex &ix, const float *queries, int64_t nq, int nprobe,
                         void *ws, int32_t *probes, float *probe_d, hipStream_t stream,
                         bool ip)
{
    if (nq == 0)
        return hipSuccess;
    int nw = 1;
    while (nw * 64 < nprobe)
        nw *= 2;
    if (nprobe == 1 && ix.d4 <= 32)
        return launch_coarse_argmin(ix, queries, nq, ws, probes, probe_d, stream, ip);
    // the matrix-core form keeps a tile's B operand in registers (d up to 128)
    // and four register top-k per wave (nprobe up to 128)
    if (nw > 2 || ix.d4 > 32)
        return launch_coarse_valu(ix, queries, nq, nprobe, probes, probe_d, stream, ip);
    int rg, splits;
    coarse_shape(nq, ix.nblk, ix.d4, &rg, &splits);
    // many centroids of up to 96 dims: the bf16x6 kernel (its grid and
    // workspace are those of the four-row-group float32 kernel)
    if (ix.cx6 && rg == 4 && !coarse_force_fp32())
        return nw == 1 ? coarse_x6_k<1>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                        stream, ip)
                       : coarse_x6_k<2>(ix, queries, nq, nprobe, splits, ws, probes, probe_d,
                                        stream, ip);
    if (nw == 1)
        return coarse_mfma_k<1>(ix, queries, nq, nprobe, rg, splits, ws, probes, probe_d, stream,
                                ip);
    return coarse_mfma_k<2>(ix, queries, nq, nprobe, rg, splits, ws, probes, probe_d, stream, ip);
}

} // namespace ivfpq
