// Device helpers shared by the IVF-PQ kernels.
#pragma once

#include "wave_select.hpp"

#include <hip/hip_fp16.h>

namespace ivfpq {

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations, not for its global loads, stores or atomics (a
// prefetch stays in flight across it, unlike __syncthreads' release fence).
// The memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier()
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Order-preserving float bound shared through memory with atomicMin.
__device__ __forceinline__ void publish_bound(uint32_t *word, float kth)
{
    if (kth < INFINITY && lane_id() == 0)
        atomicMin(word, float_order_key(kth));
}

__device__ __forceinline__ float read_bound(const uint32_t *word)
{
    return float_from_order_key(__atomic_load_n(word, __ATOMIC_RELAXED));
}

// Merge the top-k of WAVES waves (each sorted ascending in registers)
// through LDS scratch [WAVES-1][64*NW] keys + values; wave 0 ends with the
// workgroup's top-k.  Contains barriers: call from block-uniform code.
template <int NW, int WAVES>
__device__ __forceinline__ void merge_waves(WaveTopK<NW> &sel, float *mk, uint32_t *mv)
{
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    __syncthreads();
    if (wave > 0)
        sel.store(mk + (wave - 1) * 64 * NW, mv + (wave - 1) * 64 * NW);
    __syncthreads();
    if (wave == 0) {
#pragma unroll 1
        for (int w = 0; w < WAVES - 1; ++w)
            sel.merge_sorted(mk + w * 64 * NW, mv + w * 64 * NW);
    }
}

// Wave-wide inclusive prefix sum of a 32-bit value.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_ds_bpermute(((lane - s) & 63) << 2, (int)v);
        v += lane >= s ? o : 0u;
    }
    return v;
}

// Lookup-table storage: float32 or IEEE binary16 (round to nearest even).
template <bool F16>
struct Table {
    using T = typename std::conditional<F16, __half, float>::type;
    __device__ __forceinline__ static void put(void *lut, int idx, float v)
    {
        if constexpr (F16)
            reinterpret_cast<__half *>(lut)[idx] = __float2half_rn(v);
        else
            reinterpret_cast<float *>(lut)[idx] = v;
    }
    __device__ __forceinline__ static float get(const void *lut, int idx)
    {
        if constexpr (F16)
            return __half2float(reinterpret_cast<const __half *>(lut)[idx]);
        else
            return reinterpret_cast<const float *>(lut)[idx];
    }
};

} // namespace ivfpq
