// Exact X-drop materialization ("E. X-drop materialization", E.1-E.5).
//
// One wave per survivor walks both sides with exact_walk_tiles over the 4-bit copies
// (512-base tiles, eight bases per lane, the next tile read ahead; earliest endpoints).  With the
// entropy-adjusted decision on, the wave then counts the record's reference bases
// (entropy_accept).  Lane 0 stores the 16-byte record and the status.
#include <climits>

#include "hspz_internal.h"
#include "walk.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kWaves = 1;  // one wave per workgroup: a finished walk frees its slot at once
constexpr int kThreads = 64 * kWaves;
constexpr int kTab4 = 96;  // pair indices r * 16 + q for codes up to 5
constexpr int kPer = 8;  // bases per lane: 512-base tiles (16 measured slower on long walks)

__device__ __forceinline__ double xlog2x(uint32_t c) {
#pragma clang fp contract(off)
    return c > 0 ? (double)c * log2((double)c) : 0.0;
}

// Entropy-adjusted decision (the pages name it without a formula; this is the engine's
// reading): with n_b the A/C/G/T counts of the reference interval rs..=rs+len (N
// excluded) and n their sum, H = (n log2 n - sum_b n_b log2 n_b) / n bits, summed A, C,
// G, T in that order in double precision without contraction; accept iff n > 0 and
// score * H >= 2K.  The whole wave counts the interval, 64 bases per step.
__device__ __forceinline__ bool entropy_accept(const uint8_t *__restrict__ ref, uint32_t rs,
                                               uint32_t len, int64_t score, int32_t K) {
#pragma clang fp contract(off)
    const int l = lane_id();
    uint32_t cnt[4] = {0, 0, 0, 0};
    for (uint64_t base = 0; base <= len; base += 64) {
        const uint64_t t = base + l;
        const uint32_t code = t <= len ? (uint32_t)(ref[rs + t] >> kRefShift) : 7u;
#pragma unroll
        for (int c = 0; c < 4; c++) cnt[c] += (uint32_t)__popcll(__ballot(code == (uint32_t)c));
    }
    const uint32_t n = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    if (n == 0) return false;
    double s = xlog2x(cnt[0]);
    s = s + xlog2x(cnt[1]);
    s = s + xlog2x(cnt[2]);
    s = s + xlog2x(cnt[3]);
    const double H = (xlog2x(n) - s) / (double)n;
    return (double)score * H >= 2.0 * (double)K;
}

__global__ __launch_bounds__(kThreads) void k_materialize(
    const uint64_t *__restrict__ anchors, const uint32_t *__restrict__ ids, uint32_t n_surv,
    hspz_segment_pair *__restrict__ hsp, uint8_t *__restrict__ status,
    const uint8_t *__restrict__ ref, const uint32_t *__restrict__ ref4,
    const uint32_t *__restrict__ qry4, ScoreParams sp) {
    // pair scores indexed by r * 16 + q (codes 0..5 of the 4-bit copies)
    __shared__ int32_t tab4[kTab4];
    for (int i = threadIdx.x; i < kTab4; i += kThreads) {
        const int r = i >> 4, q = i & 15;
        tab4[i] = (r <= kCodeEdge && q <= kCodeEdge) ? sp.tab[(r << kRefShift) | q] : 0;
    }
    __syncthreads();
    const uint32_t i = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (i >= n_surv) return;
    const uint64_t a = anchors[ids[i]];
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    const bool bad = r > sp.n_ref || q > sp.n_qry;  // outside the sequences: empty walks
    int32_t R, L;
    uint32_t k, m;
    exact_walk_tiles<+1, true, kPer, true>(tab4, ref4, qry4, kPad4 + (bad ? sp.n_ref : r),
                                     kPad4 + (bad ? sp.n_qry : q), sp.xdrop, INT32_MAX, R, k);
    exact_walk_tiles<-1, true, kPer, true>(tab4, ref4, qry4, kPad4 + (bad ? 0u : r),
                                     kPad4 + (bad ? 0u : q), sp.xdrop, INT32_MAX, L, m);
    const int64_t total = (int64_t)L + (int64_t)R;
    bool ok = total >= (int64_t)sp.T;  // wave-uniform
    if (ok && sp.entropy_mode == 1) ok = entropy_accept(ref, r - m, m + k - 1u, total, sp.K);
    if (lane_id() == 0) {
        hspz_segment_pair rec;
        rec.ref_start = r - m;
        rec.query_start = q - m;
        rec.len = m + k - 1u;
        rec.score = (int32_t)total;
        hsp[i] = rec;
        status[i] = ok ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_materialize(const uint64_t *anchors, const uint32_t *ids, uint32_t n_surv,
                              hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                              const uint32_t *ref4, const uint32_t *qry4, const ScoreParams &sp,
                              hipStream_t s) {
    if (n_surv == 0) return hipSuccess;
    const uint32_t blocks = (n_surv + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_materialize, dim3(blocks), dim3(kThreads), 0, s, anchors, ids, n_surv,
                       hsp, status, ref, ref4, qry4, sp);
    return hipGetLastError();
}

}  // namespace hspz
