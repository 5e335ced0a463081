// Diagnostics (not on the pass): the number of bases an exact decision of each anchor's
// gate flag has to score, summed over a launch.  The right walk scores bases until and
// including the first one that drops more than xdrop below its best, or until its best
// reaches T (the flag is then 1 whatever follows); the left walk is needed only when
// R* < T and stops the same way, at its drop or once R* + its best reaches T.  No walk
// scores a base past a sequence end.  This is the algorithmic work of the score gate,
// used to price a gate launch against the VALU roofline.
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;

// Bases scored by one walk in direction D; *best receives its best (the best so far when
// it stops at stop).
template <int D>
__device__ __forceinline__ uint32_t walk_len(const int32_t *tab, const uint8_t *rp,
                                             const uint8_t *qp, int32_t xdrop, int32_t stop,
                                             int32_t *best) {
    int32_t s = 0, b = 0;
    uint32_t k = 0;
    for (;;) {
        const int64_t off = D > 0 ? (int64_t)k : -1 - (int64_t)k;
        const uint8_t rb = rp[off], qb = qp[off];
        if (rb == (kCodeEdge << kRefShift) || qb == kCodeEdge) break;
        s += tab[rb | qb];
        k++;
        if (s > b) {
            b = s;
            if (b >= stop) break;
        } else if (b - s > xdrop) {
            break;
        }
    }
    *best = b;
    return k;
}

__global__ __launch_bounds__(kThreads) void k_walk_steps(const uint64_t *__restrict__ anchors,
                                                         uint32_t n,
                                                         const uint8_t *__restrict__ ref,
                                                         const uint8_t *__restrict__ qry,
                                                         ScoreParams sp,
                                                         uint64_t *__restrict__ partial) {
    __shared__ int32_t tab[kTabSize];
    __shared__ uint64_t wsum[kThreads / 64];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint64_t steps = 0;
    if (i < n) {
        const uint64_t a = anchors[i];
        const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
        if (r <= sp.n_ref && q <= sp.n_qry) {
            int32_t R = 0, L = 0;
            steps = walk_len<+1>(tab, ref + r, qry + q, sp.xdrop, sp.T, &R);
            if (R < sp.T) steps += walk_len<-1>(tab, ref + r, qry + q, sp.xdrop, sp.T - R, &L);
        }
    }
    const uint64_t tot = wave_incl_sum_u64(steps);
    if (lane_id() == 63) wsum[threadIdx.x >> 6] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < kThreads / 64; w++) t += wsum[w];
        partial[blockIdx.x] = t;
    }
}

}  // namespace

hipError_t launch_walk_steps(const uint64_t *anchors, uint32_t n, const uint8_t *ref,
                             const uint8_t *qry, const ScoreParams &sp, uint64_t *partial,
                             hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_walk_steps, dim3(blocks), dim3(kThreads), 0, s, anchors, n, ref, qry, sp,
                       partial);
    return hipGetLastError();
}

uint32_t walk_steps_blocks(uint32_t n) { return (n + kThreads - 1) / kThreads; }

}  // namespace hspz
