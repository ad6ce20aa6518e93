// Wave64 register primitives for gfx950: cross-lane exchange and
// data-independent sorting networks on lane-stride register arrays.
//
// Lane-stride array ("Billion-scale similarity search with GPUs", k-selection
// section, register-array preliminaries): element e of an array of 64*R
// elements lives in register e / 64 of lane e % 64.  The register index must
// be a compile-time constant, the lane may be a run-time value.  A
// compare-exchange between elements e and e ^ s happens inside one lane when
// s >= 64 (two registers of the same lane) and across lanes otherwise.
//
// Cross-lane exchange by distance, all in registers (no LDS round trip: the
// selection's sorts are latency-bound chains of these steps):
//   s = 1, 2 : DPP quad_perm
//   s = 4    : DPP row_half_mirror (l -> l ^ 7 inside 8 lanes) then quad_perm
//              [3,2,1,0] (l -> l ^ 3): together l ^ 4
//   s = 8    : DPP row_ror:8 (rotation by 8 inside a 16-lane row == xor 8)
//   s = 16   : v_permlane16_swap of the value with itself: one result holds
//              rows 0,0,2,2, the other rows 1,1,3,3; a lane of an odd row
//              takes the first, of an even row the second
//   s = 32   : v_permlane32_swap likewise (halves lo,lo and hi,hi)
// The networks are bitonic: sort of 2^n elements in n(n+1)/2 steps, merge of
// a bitonic sequence of 2^n elements in n steps; their step tables and lane
// masks are in network.hpp (shared with a host check of the same tables).
// Every lane executes the same instruction stream whatever the data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "network.hpp"

namespace ivfpq {

constexpr uint32_t kSentinel = 0xFFFFFFFFu;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v)
{
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "lane distance");
    if constexpr (S == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); // quad_perm 1,0,3,2
    } else if constexpr (S == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false); // quad_perm 2,3,0,1
    } else if constexpr (S == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); // row_ror:8
    } else if constexpr (S == 4) {
        const int h = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
        return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, false);    // quad_perm 3,2,1,0
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return __builtin_amdgcn_inverse_ballot_w64(0xFFFF0000FFFF0000ull) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return __builtin_amdgcn_inverse_ballot_w64(0xFFFFFFFF00000000ull) ? r[0] : r[1];
    }
}

template <int S>
__device__ __forceinline__ float xor_lane(float v)
{
    return __uint_as_float(xor_lane<S>(__float_as_uint(v)));
}

// The same exchange through the LDS crossbar at distances 4, 16 and 32
// (ds_swizzle in bit-mask mode, xor inside 32-lane halves; ds_bpermute for
// 32): a round trip through the LDS pipe but no VALU instruction.  Wide
// arrays take it: a merge step over many registers has that many independent
// exchanges in flight, so their latency hides and the VALU is the busy pipe.
template <int S>
__device__ __forceinline__ uint32_t xor_lane_lds(uint32_t v)
{
    if constexpr (S == 4 || S == 16)
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (S << 10));
    else if constexpr (S == 32)
        return (uint32_t)__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, (int)v);
    else
        return xor_lane<S>(v);
}

#ifndef IVFPQ_LDS_XCHG_MIN_R
#define IVFPQ_LDS_XCHG_MIN_R 8
#endif
#ifndef IVFPQ_LDS_XCHG_S4
#define IVFPQ_LDS_XCHG_S4 1
#endif
// Register count from which a step's lane exchanges go through the LDS.
constexpr int kLdsExchangeMinR = IVFPQ_LDS_XCHG_MIN_R;

// Compare-exchange of (k, v) with the partner lane at distance S, keep_min
// (this lane keeps the smaller key) given for all 64 lanes as a compile-time
// mask: the two comparisons become lane masks, the choice between them three
// scalar mask operations, and the exchange two selects.  Equal keys never
// move, so the two lanes of a pair always take consistent decisions.
//
// At distance 16 and 32 the row swap hands every lane both elements of its
// pair, [0] the one of the lane with bit S clear and [1] the other, so both
// lanes of a pair evaluate the same comparison and take the smaller or the
// larger element by their mask bit: one compare and two selects instead of
// two exchanges, two compares and two selects.  Equal keys then keep their
// places in ascending blocks and trade them in descending ones; either way
// the pair's (key, value) elements stay whole.
template <int S, uint64_t KEEP_MIN, bool LDS = false>
__device__ __forceinline__ void cx_lane_mask(float &k, uint32_t &v)
{
    constexpr bool VIA_LDS = LDS && (S == 16 || S == 32 || (S == 4 && IVFPQ_LDS_XCHG_S4));
    if constexpr (VIA_LDS) {
        const float pk = __uint_as_float(xor_lane_lds<S>(__float_as_uint(k)));
        const uint32_t pv = xor_lane_lds<S>(v);
        const uint64_t lt = __builtin_amdgcn_ballot_w64(pk < k);
        const uint64_t gt = __builtin_amdgcn_ballot_w64(pk > k);
        const bool take = __builtin_amdgcn_inverse_ballot_w64((lt & KEEP_MIN) | (gt & ~KEEP_MIN));
        k = take ? pk : k;
        v = take ? pv : v;
    } else if constexpr (S == 16 || S == 32) {
        const uint32_t ku = __float_as_uint(k);
        auto kk = S == 16 ? __builtin_amdgcn_permlane16_swap(ku, ku, false, false)
                          : __builtin_amdgcn_permlane32_swap(ku, ku, false, false);
        auto vv = S == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                          : __builtin_amdgcn_permlane32_swap(v, v, false, false);
        const float lo = __uint_as_float(kk[0]);
        const float hi = __uint_as_float(kk[1]);
        const uint64_t hl = __builtin_amdgcn_ballot_w64(hi < lo);
        const bool take_hi = __builtin_amdgcn_inverse_ballot_w64(~(hl ^ KEEP_MIN));
        k = take_hi ? hi : lo;
        v = take_hi ? vv[1] : vv[0];
    } else {
        const float pk = xor_lane<S>(k);
        const uint32_t pv = xor_lane<S>(v);
        const uint64_t lt = __builtin_amdgcn_ballot_w64(pk < k);
        const uint64_t gt = __builtin_amdgcn_ballot_w64(pk > k);
        const bool take = __builtin_amdgcn_inverse_ballot_w64((lt & KEEP_MIN) | (gt & ~KEEP_MIN));
        k = take ? pk : k;
        v = take ? pv : v;
    }
}

// The lane compare-exchanges of one bitonic step, register by register.
template <int S, int B, bool DESC, int R, int... RR>
__device__ __forceinline__ void cx_lanes(float (&k)[R], uint32_t (&v)[R],
                                         std::integer_sequence<int, RR...>)
{
    (cx_lane_mask<S, keep_min_mask(S, B, DESC, RR), (R >= kLdsExchangeMinR)>(k[RR], v[RR]), ...);
}

// In-lane compare-exchange between registers (a holds the lower element).
__device__ __forceinline__ void cx_reg(float &ka, uint32_t &va, float &kb, uint32_t &vb, bool up)
{
    bool swap = up ? (kb < ka) : (ka < kb);
    float tk = ka;
    uint32_t tv = va;
    ka = swap ? kb : ka;
    va = swap ? vb : va;
    kb = swap ? tk : kb;
    vb = swap ? tv : vb;
}

// One step of a bitonic network on an R-register lane-stride array: pairs
// (e, e ^ S) inside blocks of B elements; a block runs ascending when
// ((e & B) == 0) != DESC.  B == 0 means "the whole array ascending" (merge).
template <int R, int B, int S, bool DESC>
__device__ __forceinline__ void bitonic_step(float (&k)[R], uint32_t (&v)[R])
{
    if constexpr (S >= 64) {
        constexpr int RS = S / 64;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // the block bit B >= 2S >= 128 sits in the register index
            if ((r & RS) == 0)
                cx_reg(k[r], v[r], k[r | RS], v[r | RS], block_ascending(B, DESC, r));
        }
    } else {
        cx_lanes<S, B, DESC>(k, v, std::make_integer_sequence<int, R>{});
    }
}

// The steps of a schedule (network.hpp), in order.
template <int R, bool DESC, const auto &SCHED, size_t... I>
__device__ __forceinline__ void run_schedule(float (&k)[R], uint32_t (&v)[R],
                                             std::index_sequence<I...>)
{
    (bitonic_step<R, SCHED[I].B, SCHED[I].S, DESC>(k, v), ...);
}

// Bitonic merge (half-cleaner chain S = N/2 .. 1) of a bitonic sequence of
// N = 64 R elements into ascending order.
template <int R>
__device__ __forceinline__ void bitonic_merge_up(float (&k)[R], uint32_t (&v)[R])
{
    run_schedule<R, false, kMergeUp<R>>(k, v, std::make_index_sequence<kMergeUp<R>.size()>{});
}

// Full bitonic sort of a 64-element single-register array.
template <bool DESC>
__device__ __forceinline__ void sort64(float &key, uint32_t &val)
{
    float k[1] = {key};
    uint32_t v[1] = {val};
    run_schedule<1, DESC, kSort64>(k, v, std::make_index_sequence<kSort64.size()>{});
    key = k[0];
    val = v[0];
}

// Order-preserving map of a float to uint32 (for atomic min of thresholds).
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int mbcnt64(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

} // namespace ivfpq
