// Wave64 primitives for gfx950 (CDNA4): lane masks, ranks, inclusive scans and
// reductions across the 64 lanes of one wavefront.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hspz {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of mask in lanes below this lane.
__device__ __forceinline__ int lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ int32_t wave_incl_sum(int32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int32_t o = __shfl_up(v, d, 64);
        if (l >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ int32_t wave_incl_max(int32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int32_t o = __shfl_up(v, d, 64);
        if (l >= d) v = max(v, o);
    }
    return v;
}

__device__ __forceinline__ int32_t wave_max(int32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ uint64_t wave_incl_sum_u64(uint64_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint64_t o = __shfl_up(v, d, 64);
        if (l >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d, 64);
        if (l >= d) v += o;
    }
    return v;
}

}  // namespace hspz
