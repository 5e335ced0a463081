// Reference-locality buckets for the bucketed score gate ("D. Score gate", D.5): a stable
// counting sort of one call's anchors by the reference slice their reference end falls
// in (slice = r >> shift, the last slice taking everything beyond), each anchor carrying
// its raw index, so that the gate can read a slice's windows from one XCD's L2 and write
// its results back by raw index.
//
//   k_bucket_hist     per-workgroup slice counts, stored slice-major:
//                     hist[b * nblk + block]
//   (device scan)     inclusive scan of hist, so that the first anchor of slice b in
//                     workgroup `block` goes to incl[b * nblk + block] - hist[...]
//   k_bucket_scatter  stable scatter of (anchor, raw index): a workgroup takes its anchors
//                     in rounds of 256 in index order, ranks lanes per slice with eight
//                     ballots, ranks waves in order through LDS counts, and carries a
//                     running count per slice to the next round
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;                    // anchors per thread
constexpr int kBlock = kThreads * kItems;     // 4,096 anchors per workgroup

__device__ __forceinline__ uint32_t slice_of(uint64_t a, int shift, uint32_t nb) {
    return min((uint32_t)a >> shift, nb - 1u);
}

__global__ __launch_bounds__(kThreads) void k_bucket_hist(const uint64_t *__restrict__ a,
                                                          uint32_t n, int shift, uint32_t nb,
                                                          uint32_t nblk,
                                                          uint32_t *__restrict__ hist) {
    __shared__ uint32_t h[256];
    const int t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kBlock;
#pragma unroll
    for (int r = 0; r < kItems; r++) {
        const uint64_t i = base + (uint64_t)r * kThreads + t;
        if (i < n) atomicAdd(&h[slice_of(a[i], shift, nb)], 1u);
    }
    __syncthreads();
    if ((uint32_t)t < nb) hist[(uint64_t)t * nblk + blockIdx.x] = h[t];
}

__global__ __launch_bounds__(kThreads) void k_bucket_scatter(
    const uint64_t *__restrict__ a, uint32_t n, int shift, uint32_t nb, uint32_t nblk,
    const uint32_t *__restrict__ incl, const uint32_t *__restrict__ hist,
    uint64_t *__restrict__ sa, uint32_t *__restrict__ si) {
    __shared__ uint32_t running[256];
    __shared__ uint32_t wcnt[kThreads / 64][256];
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int lane = lane_id();
    if ((uint32_t)t < nb) {
        const uint64_t hi = (uint64_t)t * nblk + blockIdx.x;
        running[t] = incl[hi] - hist[hi];
    } else {
        running[t] = 0;
    }
#pragma unroll
    for (int v = 0; v < kThreads / 64; v++) wcnt[v][t] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kBlock;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < kItems; r++) {
        const uint64_t i = base + (uint64_t)r * kThreads + t;
        const bool ok = i < n;
        const uint64_t av = ok ? a[i] : 0ull;
        const uint32_t d = ok ? slice_of(av, shift, nb) : 0u;
        uint64_t m = __ballot(ok);
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const uint32_t rank = (uint32_t)__popcll(m & below);
        if (ok && rank == 0) wcnt[w][d] = (uint32_t)__popcll(m);
        __syncthreads();
        if (ok) {
            uint32_t dst = running[d] + rank;
            for (int v = 0; v < w; v++) dst += wcnt[v][d];
            sa[dst] = av;
            si[dst] = (uint32_t)i;
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int v = 0; v < kThreads / 64; v++) {
            add += wcnt[v][t];
            wcnt[v][t] = 0;
        }
        running[t] += add;
        __syncthreads();
    }
}

// Zero n bytes; each thread clears bytes t, t + stride, ... (stores coalesce per wave).
__global__ __launch_bounds__(kThreads) void k_zero_bytes(uint8_t *__restrict__ p, uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0;
}

}  // namespace

uint32_t bucket_blocks(uint32_t n) { return (uint32_t)(((uint64_t)n + kBlock - 1) / kBlock); }

hipError_t launch_bucket_hist(const uint64_t *anchors, uint32_t n, int shift, uint32_t nb,
                              uint32_t *hist, hipStream_t s) {
    const uint32_t nblk = bucket_blocks(n);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bucket_hist, dim3(nblk), dim3(kThreads), 0, s, anchors, n, shift, nb,
                       nblk, hist);
    return hipGetLastError();
}

hipError_t launch_bucket_scatter(const uint64_t *anchors, uint32_t n, int shift, uint32_t nb,
                                 const uint32_t *incl, const uint32_t *hist, uint64_t *sa,
                                 uint32_t *si, hipStream_t s) {
    const uint32_t nblk = bucket_blocks(n);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bucket_scatter, dim3(nblk), dim3(kThreads), 0, s, anchors, n, shift, nb,
                       nblk, incl, hist, sa, si);
    return hipGetLastError();
}

hipError_t launch_zero_bytes(uint8_t *p, uint64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t want = (n + kThreads * 16 - 1) / (kThreads * 16);
    hipLaunchKernelGGL(k_zero_bytes, dim3((uint32_t)std::min<uint64_t>(want, 1u << 16)),
                       dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace hspz
