// Wave64 primitives for gfx950 (CDNA4): lane masks, ranks, inclusive scans and
// reductions across the 64 lanes of one wavefront.
//
// The 32-bit scans use DPP: four row shifts (1, 2, 4, 8) scan each 16-lane row, then
// row_bcast:15 carries row 0's total into row 1 and row 2's into row 3, and
// row_bcast:31 carries the total of rows 0-1 into rows 2-3.  Lanes whose DPP source is
// outside the row read the operation's identity.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

namespace hspz {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of mask in lanes below this lane.
__device__ __forceinline__ int lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// DPP controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
#define HSPZ_DPP_SCAN(OP, IDENT, x)                                                         \
    do {                                                                                    \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x111, 0xF, 0xF, false));           \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x112, 0xF, 0xF, false));           \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x114, 0xF, 0xF, false));           \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x118, 0xF, 0xF, false));           \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x142, 0xA, 0xF, false));           \
        x = OP(x, __builtin_amdgcn_update_dpp(IDENT, x, 0x143, 0xC, 0xF, false));           \
    } while (0)

__device__ __forceinline__ int32_t op_add_i32(int32_t a, int32_t b) { return a + b; }
__device__ __forceinline__ int32_t op_max_i32(int32_t a, int32_t b) { return max(a, b); }

__device__ __forceinline__ int32_t wave_incl_sum(int32_t v) {
    HSPZ_DPP_SCAN(op_add_i32, 0, v);
    return v;
}

__device__ __forceinline__ int32_t wave_incl_max(int32_t v) {
    HSPZ_DPP_SCAN(op_max_i32, INT_MIN, v);
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t v) {
    return (uint32_t)wave_incl_sum((int32_t)v);
}

// Value of v in lane l (l wave-uniform).
__device__ __forceinline__ int32_t lane_value(int32_t v, int l) {
    return __builtin_amdgcn_readlane(v, l);
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

}  // namespace hspz
