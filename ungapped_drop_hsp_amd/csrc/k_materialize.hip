// Exact X-drop materialization ("E. X-drop materialization", E.1-E.5).
//
// One wave per survivor.  Each step scores a 64-base tile: lane i holds base
// base + i, an inclusive wave scan (DPP) gives the running score, a prefix maximum
// (seeded with the best so far) gives the running best, and a ballot of lanes whose
// drawdown exceeds xdrop marks the first drop.  The running best in the lane before the
// first drop is the tile's best; its extent is the lowest lane attaining it, so an equal
// later maximum never moves the endpoint.  Lane 0 stores the 16-byte record and the
// status.
#include <climits>

#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D>
__device__ __forceinline__ void exact_walk(const int32_t *tab, const uint8_t *rp,
                                           const uint8_t *qp, int32_t xdrop, int32_t &best_out,
                                           uint32_t &ext_out) {
    const int l = lane_id();
    int32_t best = 0, carry = 0;
    uint32_t ext = 0, base = 0;
    for (;;) {
        const int64_t off = D > 0 ? (int64_t)base + l : -(int64_t)base - 1 - l;
        const int32_t sg = tab[rp[off] | qp[off]];
        const int32_t s = wave_incl_sum(sg) + carry;
        // running best including every base up to this lane (and the tiles before)
        const int32_t run_best = max(wave_incl_max(s), best);
        const uint64_t dm = __ballot(run_best - s > xdrop);
        const int f = dm ? (int)__builtin_ctzll(dm) : 64;  // first dropping lane
        if (f > 0) {
            const int32_t tb = lane_value(run_best, f - 1);  // best before the drop
            if (tb > best) {
                const uint64_t at = __ballot(l < f && s == tb);
                ext = base + (uint32_t)__builtin_ctzll(at) + 1u;
                best = tb;
            }
        }
        if (dm) break;
        carry = lane_value(s, 63);
        base += 64;
    }
    best_out = best;
    ext_out = ext;
}

__global__ __launch_bounds__(kThreads) void k_materialize(
    const uint64_t *__restrict__ anchors, const uint32_t *__restrict__ ids, uint32_t n_surv,
    hspz_segment_pair *__restrict__ hsp, uint8_t *__restrict__ status,
    const uint8_t *__restrict__ ref, const uint8_t *__restrict__ qry, ScoreParams sp) {
    __shared__ int32_t tab[kTabSize];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();
    const uint32_t i = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (i >= n_surv) return;
    const uint64_t a = anchors[ids[i]];
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    const bool bad = r > sp.n_ref || q > sp.n_qry;  // outside the sequences: empty walks
    int32_t R, L;
    uint32_t k, m;
    exact_walk<+1>(tab, ref + (bad ? sp.n_ref : r), qry + (bad ? sp.n_qry : q), sp.xdrop, R, k);
    exact_walk<-1>(tab, ref + (bad ? 0u : r), qry + (bad ? 0u : q), sp.xdrop, L, m);
    if (lane_id() == 0) {
        const int64_t total = (int64_t)L + (int64_t)R;
        hspz_segment_pair rec;
        rec.ref_start = r - m;
        rec.query_start = q - m;
        rec.len = m + k - 1u;
        rec.score = (int32_t)total;
        hsp[i] = rec;
        status[i] = total >= (int64_t)sp.T ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_materialize(const uint64_t *anchors, const uint32_t *ids, uint32_t n_surv,
                              hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                              const uint8_t *qry, const ScoreParams &sp, hipStream_t s) {
    if (n_surv == 0) return hipSuccess;
    const uint32_t blocks = (n_surv + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_materialize, dim3(blocks), dim3(kThreads), 0, s, anchors, ids, n_surv,
                       hsp, status, ref, qry, sp);
    return hipGetLastError();
}

}  // namespace hspz
