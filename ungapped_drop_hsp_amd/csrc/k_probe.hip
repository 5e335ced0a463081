// Random-line probe: the rate at which the memory fabric serves 128-byte lines at
// random addresses, measured with the access pattern of the score gate's reference
// windows ("D. Score gate", D.2: each anchor reads a window of the reference at an
// address that nothing predicts; D.5 names reference-window locality as the lever on
// that cost).
//
// Every lane reads `in_flight` windows per iteration, each `window_dwords` dwords
// (1 = a single 4-byte gather, 16 = a 64-byte window in 16-byte loads, as the gate's
// 4-bit windows) at the start of a random 128-byte line of the region, issuing all of
// them before it uses any, so each lane keeps that many lines in flight.  Line indices
// come from a per-lane xorshift generator scaled into the region by a high multiply.
// The loaded words are folded into one value that is stored only if it equals a key
// the host never passes, which keeps every load live.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hspz_internal.h"

#define HSPZ_API extern "C" __attribute__((visibility("default")))

namespace hspz {

namespace {

constexpr int kProbeThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(16)));

__device__ __forceinline__ uint32_t xorshift32(uint32_t x) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

template <int K, int W>
__global__ __launch_bounds__(kProbeThreads) void k_line_probe(const uint32_t *__restrict__ base,
                                                              uint32_t n_lines, uint32_t iters,
                                                              uint32_t seed, uint32_t key,
                                                              uint32_t *__restrict__ sink) {
    const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t x = (gid + 1u) * 0x9E3779B9u ^ seed;
    x = xorshift32(x | 1u);
    uint32_t acc = 0;
    for (uint32_t it = 0; it < iters; it++) {
        uint32_t line[K];
#pragma unroll
        for (int k = 0; k < K; k++) {
            x = xorshift32(x);
            line[k] = __umulhi(x, n_lines);
        }
        if (W == 1) {
            uint32_t v[K];
#pragma unroll
            for (int k = 0; k < K; k++) v[k] = base[(uint64_t)line[k] * 32u];
#pragma unroll
            for (int k = 0; k < K; k++) acc ^= v[k];
        } else {
            u32x4 v[K][W / 4];
#pragma unroll
            for (int k = 0; k < K; k++) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(base + (uint64_t)line[k] * 32u);
#pragma unroll
                for (int j = 0; j < W / 4; j++) v[k][j] = p[j];
            }
#pragma unroll
            for (int k = 0; k < K; k++)
#pragma unroll
                for (int j = 0; j < W / 4; j++) acc ^= v[k][j].x ^ v[k][j].y ^ v[k][j].z ^ v[k][j].w;
        }
    }
    if (acc == key) sink[gid & 63u] = acc;
}

template <int W>
hipError_t launch_probe_w(int in_flight, dim3 grid, const uint32_t *base, uint32_t n_lines,
                          uint32_t iters, uint32_t seed, uint32_t key, uint32_t *sink,
                          hipStream_t s) {
    switch (in_flight) {
    case 1:
        hipLaunchKernelGGL((k_line_probe<1, W>), grid, dim3(kProbeThreads), 0, s, base, n_lines,
                           iters, seed, key, sink);
        break;
    case 2:
        hipLaunchKernelGGL((k_line_probe<2, W>), grid, dim3(kProbeThreads), 0, s, base, n_lines,
                           iters, seed, key, sink);
        break;
    case 4:
        hipLaunchKernelGGL((k_line_probe<4, W>), grid, dim3(kProbeThreads), 0, s, base, n_lines,
                           iters, seed, key, sink);
        break;
    default:
        hipLaunchKernelGGL((k_line_probe<8, W>), grid, dim3(kProbeThreads), 0, s, base, n_lines,
                           iters, seed, key, sink);
        break;
    }
    return hipGetLastError();
}

}  // namespace

}  // namespace hspz

// Test-only: launches the probe on stream (the caller times it with events on the same
// stream).  Reads window_dwords dwords at the start of each of lanes * iters * in_flight
// random 128-byte lines of d_region (region_bytes long, 128-byte aligned); writes d_sink
// (64 u32) only if the folded words equal key.
HSPZ_API int hspz_debug_line_probe(const uint32_t *d_region, uint64_t region_bytes,
                                   uint32_t window_dwords, uint32_t in_flight, uint32_t blocks,
                                   uint32_t iters, uint32_t seed, uint32_t key, uint32_t *d_sink,
                                   void *stream) {
    using namespace hspz;
    if (!d_region || !d_sink || region_bytes < 128 || region_bytes / 128 > 0xFFFFFFFFull ||
        (reinterpret_cast<uintptr_t>(d_region) & 127) != 0 || blocks == 0)
        return HSPZ_E_INVALID;
    if (!(window_dwords == 1 || window_dwords == 16) ||
        !(in_flight == 1 || in_flight == 2 || in_flight == 4 || in_flight == 8))
        return HSPZ_E_INVALID;
    const uint32_t n_lines = (uint32_t)(region_bytes / 128);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t st = window_dwords == 1
                        ? launch_probe_w<1>((int)in_flight, dim3(blocks), d_region, n_lines,
                                            iters, seed, key, d_sink, s)
                        : launch_probe_w<16>((int)in_flight, dim3(blocks), d_region, n_lines,
                                             iters, seed, key, d_sink, s);
    return st == hipSuccess ? HSPZ_OK : HSPZ_E_HIP;
}
