// Schedules of the bitonic networks that the register k-selection runs, and
// the lane masks of their steps.  Plain constexpr C++ (no HIP): the device
// code (wave_ops.hpp) runs exactly these tables, and a host program can run
// and check the same tables.
//
// "Billion-scale similarity search with GPUs", k-selection section (odd-size
// merging and sorting networks): a sort of 2^n elements is n(n+1)/2 steps of
// bitonic half-cleaners, a merge of a bitonic sequence of 2^n elements n
// steps.  Here the arrays are lane-stride (element e in register e / 64 of lane
// e % 64) and every size is a power of two (64 times the register count).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <array>

namespace ivfpq {

// One step: compare-exchange of the pairs (e, e ^ S) inside blocks of B
// elements; a block runs ascending when ((e & B) == 0) != desc.  B == 0 means
// one block, the whole array, ascending when !desc.
struct NetStep {
    int B;
    int S;
};

// Full bitonic sort of N elements (N a power of two): blocks B = 2, 4, ..., N
// (the last one the whole array, B = 0), in each the half-cleaners
// S = B / 2, ..., 1.
constexpr int sort_steps(int n)
{
    int lg = 0;
    while ((1 << lg) < n)
        ++lg;
    return lg * (lg + 1) / 2;
}

template <int N>
constexpr std::array<NetStep, sort_steps(N)> sort_schedule()
{
    std::array<NetStep, sort_steps(N)> a{};
    int i = 0;
    for (int B = 2; B <= N; B *= 2)
        for (int S = B / 2; S >= 1; S /= 2)
            a[i++] = NetStep{B == N ? 0 : B, S};
    return a;
}

// Bitonic merge of N elements (a bitonic sequence) into one order: S = N/2,
// ..., 1, one block.
constexpr int merge_steps(int n)
{
    int lg = 0;
    while ((1 << lg) < n)
        ++lg;
    return lg;
}

template <int N>
constexpr std::array<NetStep, merge_steps(N)> merge_schedule()
{
    std::array<NetStep, merge_steps(N)> a{};
    int i = 0;
    for (int S = N / 2; S >= 1; S /= 2)
        a[i++] = NetStep{0, S};
    return a;
}

// The schedules the selection uses: the 64-element sort of a staging buffer
// and the merge of a 64·R-element register array.
constexpr auto kSort64 = sort_schedule<64>();
template <int R>
constexpr auto kMergeUp = merge_schedule<64 * R>();

// Lanes of register r that keep the smaller key in a step with S < 64 (the
// pairs are lanes l and l ^ S of the same register): bit l set when element
// r*64 + l is the lower of its pair and its block runs ascending, or the upper
// and its block runs descending.
constexpr uint64_t keep_min_mask(int S, int B, bool DESC, int r)
{
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l) {
        const int e = r * 64 + l;
        const bool lower = (l & S) == 0;
        const bool up = B == 0 ? !DESC : (((e & B) == 0) != DESC);
        if (lower == up)
            m |= 1ull << l;
    }
    return m;
}

// For S >= 64 (pairs inside one lane, registers r and r | S/64): whether the
// block of register r runs ascending.
constexpr bool block_ascending(int B, bool DESC, int r)
{
    return B == 0 ? !DESC : (((r * 64) & B) == 0) != DESC;
}

} // namespace ivfpq
