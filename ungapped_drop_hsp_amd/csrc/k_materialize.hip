// Exact X-drop materialization ("E. X-drop materialization", E.1-E.5).
//
// Two ways to the same records:
//  - k_materialize: one wave per survivor walks both sides on its own, with
//    exact_walk_tiles over the 4-bit copies (512-base tiles, eight bases per lane, the
//    next tile read ahead; earliest endpoints).  With the entropy-adjusted decision on,
//    the wave then counts the record's reference bases (entropy_accept).  Lane 0 stores
//    the 16-byte record and the status.
//  - the diagonal-shared walks (k_mm_*), for calls with many survivors.  Survivors are
//    sorted stably by diagonal (after a sort by reference end, unless the caller knows
//    their query ends never decrease), so each one's neighbours on its diagonal sit next
//    to it, and k_mm_gather lays their anchors out in that order.  Each side's walk stops
//    at its drop, or at its first strictly new best at or past its neighbour's start:
//    from there the two walks are one (same later bases, same running best, same drop,
//    and every base scored before lies below that best), so it keeps only its running
//    score at the neighbour's start.  k_mm_lanes walks every side one lane each, for up
//    to 128 bases in eight-base blocks (the first 32 in every lane, the rest only in the
//    lanes of the walks still open, packed together), and lists the walks still open
//    after that; k_mm_list walks
//    those one wave each in 512-base tiles.  A side that merged takes the best of the
//    first walk along its chain that ran to its drop, plus the summed scores at the starts
//    in between, and that walk's extent plus the distance to it: one scan over both
//    sides (k_mm_scan_*) gives the sums and the ordered list of drop-ended walks, and
//    k_mm_finish forms every record.  On tandem repeats, where thousands of survivors
//    share a diagonal, this walks each stretch of a diagonal about once instead of once
//    per survivor.
#include <algorithm>
#include <climits>

#include "hspz_internal.h"
#include "mat_shared.h"
#include "walk.h"
#include "walk_merge.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kWaves = 1;  // one wave per workgroup: a finished walk frees its slot at once
constexpr int kThreads = 64 * kWaves;
constexpr int kTab4 = 96;  // pair indices r * 16 + q for codes up to 5
constexpr int kPer = 8;  // bases per lane: 512-base tiles (16 measured slower on long walks)
// Window of the shared walks' lane stage, in blocks of eight bases per side: about 0.3% of
// the walks on dense tandem repeats run past 128 bases.  Per 1.04 M-survivor chunk, lane
// stage + listed walks measured 183 + 51, 110 + 26, 84 + 17 and 93 + 15 us at 8, 12, 16
// and 24 blocks, with every lane held to its wave's longest walk.
constexpr int kLaneBlocks = 16;
constexpr int kLanePrefetch = 3;  // blocks each lane reads ahead
// Blocks of the lane stage's first phase, after which the open walks are packed: the lane
// stage measured 84 us per chunk unpacked and 67 us at 4; 2 to 6 are within noise.
constexpr int kLaneFirst = 4;
// Largest grid of the one-wave-per-survivor kernels (a launch holds fewer than 2^32
// threads); beyond it each workgroup strides over several survivors.
constexpr uint32_t kWaveGridMax = 1u << 22;

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
    // a wave per survivor; a grid capped at kWaveGridMax workgroups strides over the rest
    for (uint64_t i64 = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); i64 < n_surv;
         i64 += (uint64_t)gridDim.x * kWaves) {
        const uint32_t i = (uint32_t)i64;
        const uint64_t a = anchors[ids[i]];
        const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
        const bool bad = r > sp.n_ref || q > sp.n_qry;  // outside the sequences: empty walks
        int32_t R, L;
        uint32_t k, m;
        exact_walk_tiles<+1, true, kPer, true>(tab4, ref4, qry4, kPad4 + (bad ? sp.n_ref : r),
                                               kPad4 + (bad ? sp.n_qry : q), sp.xdrop,
                                               INT32_MAX, R, k);
        exact_walk_tiles<-1, true, kPer, true>(tab4, ref4, qry4, kPad4 + (bad ? 0u : r),
                                               kPad4 + (bad ? 0u : q), sp.xdrop, INT32_MAX, L,
                                               m);
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
}

// Sort keys: the reference end (first pass; skipped when the query ends already never
// decrease) and the diagonal r - q + n_qry (second pass, stable); an anchor outside the
// sequences gets the diagonal key n_ref + n_qry + 1 and never merges.  Also clears the
// lane stage's open-walk counts.
__global__ __launch_bounds__(256) void k_mm_keys(const uint64_t *__restrict__ anchors,
                                                 const uint32_t *__restrict__ ids, uint32_t n,
                                                 uint32_t n_ref, uint32_t n_qry,
                                                 uint32_t *__restrict__ key_r,
                                                 uint32_t *__restrict__ val,
                                                 uint32_t *__restrict__ lcnt) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < 2) lcnt[i] = 0;
    if (i >= n) return;
    const uint64_t a = anchors[ids[i]];
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    key_r[i] = (r > n_ref || q > n_qry) ? 0u : r;
    val[i] = i;
}

__device__ __forceinline__ uint32_t diag_key(uint64_t a, uint32_t n_ref, uint32_t n_qry) {
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    return (r > n_ref || q > n_qry) ? n_ref + n_qry + 1u : r - q + n_qry;
}

__global__ __launch_bounds__(256) void k_mm_diag(const uint64_t *__restrict__ anchors,
                                                 const uint32_t *__restrict__ ids,
                                                 const uint32_t *__restrict__ val, uint32_t n,
                                                 uint32_t n_ref, uint32_t n_qry,
                                                 uint32_t *__restrict__ key_d) {
    const uint32_t s = blockIdx.x * 256 + threadIdx.x;
    if (s >= n) return;
    key_d[s] = diag_key(anchors[ids[val[s]]], n_ref, n_qry);
}

// The anchors in sorted order, so that the walks read themselves and their neighbours
// with unit-stride loads instead of chains of dependent gathers.
__global__ __launch_bounds__(256) void k_mm_gather(const uint64_t *__restrict__ anchors,
                                                   const uint32_t *__restrict__ ids,
                                                   const uint32_t *__restrict__ val, uint32_t n,
                                                   uint64_t *__restrict__ sa) {
    const uint32_t s = blockIdx.x * 256 + threadIdx.x;
    if (s < n) sa[s] = anchors[ids[val[s]]];
}

// Sorted survivor s (sa: the anchors in sorted order): its anchor and the walk indices of
// its neighbours' starts on its diagonal (UINT32_MAX for none).  The right neighbour is
// the next survivor on the diagonal (its right walk starts at base rn, i.e. after walk
// index rn - 1 - r of this one); the left neighbour is the previous one (its left walk
// starts below base rp, walk index r - 1 - rp of this one).  A neighbour at the same
// reference end (a duplicate anchor) is none.
struct MmAnchor {
    uint32_t r, q, wr, wl;
    bool bad;  // outside the sequences: both walks are empty
};

__device__ __forceinline__ MmAnchor mm_anchor(const uint64_t *__restrict__ sa,
                                              const uint32_t *__restrict__ key_d, uint32_t n,
                                              uint32_t s, const ScoreParams &sp) {
    MmAnchor A;
    const uint64_t a = sa[s];
    A.r = (uint32_t)a;
    A.q = (uint32_t)(a >> 32);
    A.bad = A.r > sp.n_ref || A.q > sp.n_qry;
    A.wr = UINT32_MAX;
    A.wl = UINT32_MAX;
    // every load at once (the neighbours' indices clamped into the array), then the tests
    const uint32_t sn = s + 1 < n ? s + 1 : s, sp_ = s > 0 ? s - 1 : s;
    const uint64_t an = sa[sn], ap = sa[sp_];
    const uint32_t key = key_d[s], kn = key_d[sn], kp = key_d[sp_];
    if (!A.bad) {
        const uint32_t rn = (uint32_t)an, rp = (uint32_t)ap;
        if (sn != s && kn == key && rn > A.r) A.wr = rn - 1u - A.r;
        if (sp_ != s && kp == key && rp < A.r) A.wl = A.r - 1u - rp;
    }
    return A;
}

__device__ __forceinline__ void mm_store(const MatSide &m, uint32_t s, int32_t best, uint32_t ext,
                                         bool merged, int32_t ds) {
    m.best[s] = best;
    m.ext[s] = ext;
    m.term[s] = merged ? 0u : 1u;
    m.ds[s] = merged ? ds : 0;
}

// The merge walk of one lane, in blocks of eight bases read from the 4-bit copies, for at
// most NB blocks.  Block k holds walk positions 8k .. 8k + 7: a right walk's nibbles
// mr + 8k .. mr + 8k + 7 (mr the padded nibble index of the anchor's first base), a left
// walk's mr - 8 - 8k .. mr - 1 - 8k in reverse.  Each base updates the running score,
// the running best with its earliest extent, the largest drawdown, and at walk index wm
// the running score (ds) and the best before that base.  Every lane runs whole blocks:
// eight-base blocks are exact when 7 * (largest pair score) <= xdrop, since a walk that
// has dropped cannot climb back to its best inside the same block, so a block's final
// best and extent are those before its drop, and a block has a strict new best at or
// past wm (a merge) only if no drop came first.  At a block's end the walk merged if its
// best rose above the best before wm (or above the block's starting best once wm lies
// behind), and dropped if the drawdown passed xdrop; a merge takes precedence, being
// the earlier event.  Returns false if the walk did neither within the window; the
// caller then walks it again in full.  Each sequence's dwords are read PF blocks ahead
// of their use (a ring of PF + 2 dwords), so that a block's loads have the blocks before
// it to land.  Reads at most 8 * (NB + PF) + 16 nibbles from mr on either side, inside
// the edge padding.
// The running state of a lane walk between blocks: score, best, earliest extent of the
// best, and the score at walk index wm once the walk has passed it.
struct LaneWalk {
    int32_t s = 0, best = 0, ds = 0;
    uint32_t ext = 0;
};

// Blocks K0 .. K1 - 1 of the walk, from the state w after block K0 - 1 (w is updated to
// the state after the last block walked); a lane that is not active takes no part.
template <int D, int K0, int K1, int PF>
__device__ __forceinline__ bool lane_merge_walk(const int32_t *tab4,
                                                const uint32_t *__restrict__ ref4,
                                                const uint32_t *__restrict__ qry4, uint32_t mr,
                                                uint32_t mq, int32_t xdrop, uint32_t wm,
                                                bool active, LaneWalk &w, int32_t &best,
                                                uint32_t &ext, bool &merged, int32_t &ds) {
    static_assert(8 * (K1 + PF) + 16 <= kPad4, "the window must stay inside the edge padding");
    const uint32_t ar = D > 0 ? mr : mr - 8u, aq = D > 0 ? mq : mq - 8u;
    const uint32_t *__restrict__ pr = ref4 + (ar >> 3);
    const uint32_t *__restrict__ pq = qry4 + (aq >> 3);
    const uint32_t shr = (ar & 7u) * 4u, shq = (aq & 7u) * 4u;
    // block k's nibbles are the funnel of dwords p[k] (low) and p[k + 1] (high) for a right
    // walk, p[-k] (low) and p[1 - k] (high) for a left one; ring slot i holds dword
    // p[k + i] or p[1 - k - i], so block k reads slots 0 and 1
    auto at = [](const uint32_t *__restrict__ p, int i) { return D > 0 ? p[i] : p[1 - i]; };
    uint32_t rr[PF + 2], qq[PF + 2];
#pragma unroll
    for (int i = 0; i < PF + 2; i++) {
        rr[i] = at(pr, K0 + i);
        qq[i] = at(pq, K0 + i);
    }
    // The lanes run in step with no branch of their own: a lane that ends in a block keeps
    // its results from there and goes on scoring (its reads stay inside the window), and
    // the wave leaves once every lane has ended.  A branch per lane would make every value
    // of the ring cross a join, and copying a register that a load still writes waits for
    // the load; unrolled, the ring is register renaming.
    int32_t s = w.s, b_run = w.best, ds_run = w.ds;
    uint32_t e_run = w.ext;
    bool done = !active;
    best = 0;
    ext = 0;
    merged = false;
    ds = 0;
#pragma unroll
    for (int k = K0; k < K1; k++) {
        const uint32_t R = D > 0 ? __builtin_amdgcn_alignbit(rr[1], rr[0], shr)
                                 : __builtin_amdgcn_alignbit(rr[0], rr[1], shr);
        const uint32_t Q = D > 0 ? __builtin_amdgcn_alignbit(qq[1], qq[0], shq)
                                 : __builtin_amdgcn_alignbit(qq[0], qq[1], shq);
#pragma unroll
        for (int i = 0; i < PF + 1; i++) {
            rr[i] = rr[i + 1];
            qq[i] = qq[i + 1];
        }
        rr[PF + 1] = at(pr, k + PF + 2);  // block k + PF + 1's new dword
        qq[PF + 1] = at(pq, k + PF + 2);
        const uint32_t hi = 0xF0F0F0F0u;
        // pair indices r * 16 + q: nibble j's in byte j / 2 of c[j % 2]
        const uint32_t c[2] = {((R << 4) & hi) | (Q & ~hi), (R & hi) | ((Q >> 4) & ~hi)};
        const uint32_t b0 = 8u * (uint32_t)k;
        const int32_t best0 = b_run;
        int32_t bpre = b_run, dd = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int nib = D > 0 ? j : 7 - j;
            const int32_t sg = tab4[(c[nib & 1] >> (8 * (nib >> 1))) & 0xFFu];
            const uint32_t i = b0 + (uint32_t)j;
            s += sg;
            const bool at_wm = i == wm;
            bpre = at_wm ? b_run : bpre;
            ds_run = at_wm ? s : ds_run;
            e_run = s > b_run ? i + 1u : e_run;
            b_run = max(b_run, s);
            dd = max(dd, b_run - s);
        }
        const int32_t thr = wm < b0 ? best0 : (wm < b0 + 8u ? bpre : INT32_MAX);
        const bool mrg = b_run > thr;  // a merge is the earlier event
        const bool end = !done && (mrg || dd > xdrop);
        best = end ? b_run : best;
        ext = end ? e_run : ext;
        ds = end ? ds_run : ds;
        merged = end ? mrg : merged;
        done = done || end;
        if (__ballot(!done) == 0) {
            // the loads still in flight are used on this path too, so that the compiler
            // keeps each one where it is issued rather than sinking it to its first use
#pragma unroll
            for (int i = 0; i < PF + 2; i++) asm volatile("" ::"v"(rr[i]), "v"(qq[i]));
            break;
        }
    }
    w.s = s;
    w.best = b_run;
    w.ds = ds_run;
    w.ext = e_run;
    return done;
}

// Lane stage of the diagonal-shared walks, per side in two phases.  Every lane walks its
// survivor's first kLaneFirst blocks; the walks still running then go, with their state,
// through LDS to as few waves as they fill (about one in eight on dense tandem repeats),
// which walk them on to block NB.  A wave thus runs its first phase as long as its
// longest short walk and its second only for the long ones, instead of every lane
// waiting for the wave's longest walk.  Walks still running at block NB go to a list
// (right walks from list[0], left walks from list[n]; counts in lcnt) that k_mm_list
// walks in full, each wave reserving its share with one atomic.
template <int NB>
__global__ __launch_bounds__(256) void k_mm_lanes(
    const uint64_t *__restrict__ sa, const uint32_t *__restrict__ key_d, uint32_t n,
    const uint32_t *__restrict__ ref4, const uint32_t *__restrict__ qry4, ScoreParams sp,
    MatSide right, MatSide left, uint32_t *__restrict__ list, uint32_t *__restrict__ lcnt) {
    static_assert(kLaneFirst < NB, "the second phase needs blocks");
    __shared__ int32_t tab4[kTab4];
    // walks carried into the second phase: state, walk geometry and survivor index
    __shared__ int32_t c_s[256], c_best[256], c_ds[256];
    __shared__ uint32_t c_ext[256], c_wm[256], c_mr[256], c_mq[256], c_idx[256];
    __shared__ uint32_t c_n[2];  // per side, so that no wave still reads the one cleared
    if (threadIdx.x < 2) c_n[threadIdx.x] = 0;
    for (int i = threadIdx.x; i < kTab4; i += 256) {
        const int r = i >> 4, q = i & 15;
        tab4[i] = (r <= kCodeEdge && q <= kCodeEdge) ? sp.tab[(r << kRefShift) | q] : 0;
    }
    const uint32_t s = blockIdx.x * 256 + threadIdx.x;
    const bool live = s < n;
    MmAnchor A{};
    if (live) A = mm_anchor(sa, key_d, n, s, sp);
    const int w = threadIdx.x >> 6, lane = lane_id();
#pragma unroll
    for (int side = 0; side < 2; side++) {
        const MatSide &m = side == 0 ? right : left;
        __syncthreads();  // orders the table and counters above, and the last side's reads
        const uint32_t mr = kPad4 + (A.bad ? (side == 0 ? sp.n_ref : 0u) : A.r);
        const uint32_t mq = kPad4 + (A.bad ? (side == 0 ? sp.n_qry : 0u) : A.q);
        const uint32_t wm = side == 0 ? A.wr : A.wl;
        LaneWalk st;
        int32_t best, ds;
        uint32_t ext;
        bool merged, done;
        if (side == 0)
            done = lane_merge_walk<+1, 0, kLaneFirst, kLanePrefetch>(
                tab4, ref4, qry4, mr, mq, sp.xdrop, wm, live, st, best, ext, merged, ds);
        else
            done = lane_merge_walk<-1, 0, kLaneFirst, kLanePrefetch>(
                tab4, ref4, qry4, mr, mq, sp.xdrop, wm, live, st, best, ext, merged, ds);
        if (live && done) mm_store(m, s, best, ext, merged, ds);
        if (live && !done) {
            const uint32_t c = atomicAdd(&c_n[side], 1u);
            c_s[c] = st.s;
            c_best[c] = st.best;
            c_ds[c] = st.ds;
            c_ext[c] = st.ext;
            c_wm[c] = wm;
            c_mr[c] = mr;
            c_mq[c] = mq;
            c_idx[c] = s;
        }
        __syncthreads();
        const uint32_t cn = c_n[side];  // uniform
        if ((uint32_t)w * 64u < cn) {
            const uint32_t c = (uint32_t)w * 64u + (uint32_t)lane;
            const bool has = c < cn;
            LaneWalk ct;
            uint32_t cwm = UINT32_MAX, cmr = kPad4, cmq = kPad4, cidx = 0;
            if (has) {
                ct.s = c_s[c];
                ct.best = c_best[c];
                ct.ds = c_ds[c];
                ct.ext = c_ext[c];
                cwm = c_wm[c];
                cmr = c_mr[c];
                cmq = c_mq[c];
                cidx = c_idx[c];
            }
            bool cdone;
            if (side == 0)
                cdone = lane_merge_walk<+1, kLaneFirst, NB, kLanePrefetch>(
                    tab4, ref4, qry4, cmr, cmq, sp.xdrop, cwm, has, ct, best, ext, merged, ds);
            else
                cdone = lane_merge_walk<-1, kLaneFirst, NB, kLanePrefetch>(
                    tab4, ref4, qry4, cmr, cmq, sp.xdrop, cwm, has, ct, best, ext, merged, ds);
            if (has && cdone) mm_store(m, cidx, best, ext, merged, ds);
            const bool open = has && !cdone;
            const uint64_t om = __ballot(open);
            if (om) {
                uint32_t at = 0;
                if (lane == 0) at = atomicAdd(&lcnt[side], (uint32_t)__popcll(om));
                at = __shfl(at, 0, 64);
                if (open) list[(uint64_t)side * n + at + lane_rank(om)] = cidx;
            }
        }
    }
}

// One wave per sorted survivor: its right walk (neighbour: the next survivor on the
// diagonal) and its left walk (neighbour: the previous one), each a one-wave merge walk.
__global__ __launch_bounds__(64) void k_mm_walk(const uint64_t *__restrict__ sa,
                                                const uint32_t *__restrict__ key_d, uint32_t n,
                                                const uint8_t *__restrict__ ref,
                                                const uint8_t *__restrict__ qry, ScoreParams sp,
                                                MatSide right, MatSide left) {
    __shared__ int32_t tab[kTabSize];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();
    for (uint64_t s64 = blockIdx.x; s64 < n; s64 += gridDim.x) {
        const uint32_t s = (uint32_t)s64;
        const MmAnchor A = mm_anchor(sa, key_d, n, s, sp);
        const uint8_t *rr = ref + (A.bad ? sp.n_ref : A.r), *qr = qry + (A.bad ? sp.n_qry : A.q);
        const uint8_t *rl = ref + (A.bad ? 0u : A.r), *ql = qry + (A.bad ? 0u : A.q);
        int32_t R, L, dr, dlft;
        uint32_t k, m;
        bool mr, ml;
        exact_walk_merge<+1, true>(tab, rr, qr, sp.xdrop, A.wr, R, k, mr, dr);
        exact_walk_merge<-1, true>(tab, rl, ql, sp.xdrop, A.wl, L, m, ml, dlft);
        if (lane_id() == 0) {
            mm_store(right, s, R, k, mr, dr);
            mm_store(left, s, L, m, ml, dlft);
        }
    }
}

// The walks the lane stage left open: one wave per listed walk (right walks first), a
// fixed grid striding over the counts read on the device.  They include the chain ends
// that run thousands of bases, so they walk 512-base tiles from the 4-bit copies.
__global__ __launch_bounds__(256) void k_mm_list(const uint64_t *__restrict__ sa,
                                                 const uint32_t *__restrict__ key_d, uint32_t n,
                                                 const uint32_t *__restrict__ ref4,
                                                 const uint32_t *__restrict__ qry4,
                                                 ScoreParams sp, MatSide right, MatSide left,
                                                 const uint32_t *__restrict__ list,
                                                 const uint32_t *__restrict__ lcnt) {
    __shared__ int32_t tab4[kTab4];
    for (int i = threadIdx.x; i < kTab4; i += 256) {
        const int r = i >> 4, q = i & 15;
        tab4[i] = (r <= kCodeEdge && q <= kCodeEdge) ? sp.tab[(r << kRefShift) | q] : 0;
    }
    __syncthreads();
    const uint32_t cr = lcnt[0];
    const uint64_t total = (uint64_t)cr + lcnt[1];
    const uint64_t nw = (uint64_t)gridDim.x * 4;
    for (uint64_t t = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < total; t += nw) {
        const bool rt = t < cr;
        const uint32_t s = rt ? list[t] : list[(uint64_t)n + (t - cr)];
        const MmAnchor A = mm_anchor(sa, key_d, n, s, sp);
        int32_t best, ds;
        uint32_t ext;
        bool merged;
        if (rt)
            exact_walk_tiles_merge<+1>(tab4, ref4, qry4, kPad4 + (A.bad ? sp.n_ref : A.r),
                                       kPad4 + (A.bad ? sp.n_qry : A.q), sp.xdrop, A.wr, best,
                                       ext, merged, ds);
        else
            exact_walk_tiles_merge<-1>(tab4, ref4, qry4, kPad4 + (A.bad ? 0u : A.r),
                                       kPad4 + (A.bad ? 0u : A.q), sp.xdrop, A.wl, best, ext,
                                       merged, ds);
        if (lane_id() == 0) mm_store(rt ? right : left, s, best, ext, merged, ds);
    }
}

// The chain bookkeeping of both sides in one scan: inclusive sums (modulo 2^32) of four
// streams, the right and left end flags (term) and scores at the neighbour's start (ds),
// into cnt and sum; the last pass also lists each side's drop-ended walks in order
// (pos[cnt[s] - 1] = s for a walk s that ran to its drop).  Three launches: block-local
// scans with block totals, one workgroup scanning the totals, and the offsets.
constexpr int kMsPer = 4;                 // survivors per thread
constexpr int kMsBlock = 256 * kMsPer;    // survivors per block

__device__ __forceinline__ uint32_t op_add_u32(uint32_t a, uint32_t b) { return a + b; }

// Inclusive wave scan in wrapping unsigned arithmetic (the DPP steps of wave_incl_sum).
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
    HSPZ_DPP_SCAN(op_add_u32, 0, v);
    return v;
}

__device__ __forceinline__ uint32_t *ms_stream(const MatSide &r, const MatSide &l, int st,
                                               bool out) {
    const MatSide &m = st < 2 ? r : l;
    if (st & 1) return out ? m.sum : reinterpret_cast<uint32_t *>(m.ds);
    return out ? m.cnt : m.term;
}

__global__ __launch_bounds__(256) void k_mm_scan_local(MatSide right, MatSide left, uint32_t n,
                                                       uint32_t *__restrict__ blk) {
    __shared__ uint32_t wtot[4][4];  // [wave][stream]
    const int t = threadIdx.x, w = t >> 6;
    const uint64_t i0 = (uint64_t)blockIdx.x * kMsBlock + (uint64_t)t * kMsPer;
    uint32_t v[4][kMsPer];
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const uint32_t *in = ms_stream(right, left, st, false);
        if (i0 + kMsPer <= n) {  // 16-byte aligned: the arrays are, and i0 % 4 == 0
            const uint4 x = *reinterpret_cast<const uint4 *>(in + i0);
            v[st][0] = x.x;
            v[st][1] = x.y;
            v[st][2] = x.z;
            v[st][3] = x.w;
        } else {
#pragma unroll
            for (int j = 0; j < kMsPer; j++) v[st][j] = i0 + j < n ? in[i0 + j] : 0u;
        }
#pragma unroll
        for (int j = 1; j < kMsPer; j++) v[st][j] += v[st][j - 1];
    }
    uint32_t excl[4];
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const uint32_t tot = v[st][kMsPer - 1];
        const uint32_t incl = wave_scan_u32(tot);
        excl[st] = incl - tot;
        if (lane_id() == 63) wtot[w][st] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; st++) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            before += u < w ? wtot[u][st] : 0u;
            all += wtot[u][st];
        }
        excl[st] += before;
        uint32_t *out = ms_stream(right, left, st, true);
        if (i0 + kMsPer <= n) {
            *reinterpret_cast<uint4 *>(out + i0) =
                make_uint4(v[st][0] + excl[st], v[st][1] + excl[st], v[st][2] + excl[st],
                           v[st][3] + excl[st]);
        } else {
#pragma unroll
            for (int j = 0; j < kMsPer; j++)
                if (i0 + j < n) out[i0 + j] = v[st][j] + excl[st];
        }
        if (t == 0) blk[4ull * blockIdx.x + st] = all;
    }
}

// One workgroup: the exclusive scan of nb block totals per stream, in place.
__global__ __launch_bounds__(1024) void k_mm_scan_blocks(uint32_t *__restrict__ blk, uint32_t nb) {
    __shared__ uint32_t wtot[16][4];
    const int t = threadIdx.x, w = t >> 6;
    uint32_t carry[4] = {0, 0, 0, 0};
    for (uint32_t b0 = 0; b0 < nb; b0 += 1024) {
        const uint32_t b = b0 + (uint32_t)t;
        uint32_t x[4], excl[4];
#pragma unroll
        for (int st = 0; st < 4; st++) {
            x[st] = b < nb ? blk[4ull * b + st] : 0u;
            const uint32_t incl = wave_scan_u32(x[st]);
            excl[st] = incl - x[st];
            if (lane_id() == 63) wtot[w][st] = incl;
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 4; st++) {
            uint32_t before = 0, all = 0;
            for (int u = 0; u < 16; u++) {
                before += u < w ? wtot[u][st] : 0u;
                all += wtot[u][st];
            }
            if (b < nb) blk[4ull * b + st] = carry[st] + before + excl[st];
            carry[st] += all;
        }
        __syncthreads();  // wtot is rewritten by the next round
    }
}

__global__ __launch_bounds__(256) void k_mm_scan_add(MatSide right, MatSide left, uint32_t n,
                                                     const uint32_t *__restrict__ blk) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const uint32_t b = i / kMsBlock;
    const uint4 off = *reinterpret_cast<const uint4 *>(blk + 4ull * b);
    const uint32_t cr = right.cnt[i] + off.x, cl = left.cnt[i] + off.z;
    right.cnt[i] = cr;
    right.sum[i] += off.y;
    left.cnt[i] = cl;
    left.sum[i] += off.w;
    if (right.term[i]) right.pos[cr - 1u] = i;
    if (left.term[i]) left.pos[cl - 1u] = i;
}

// One thread per sorted survivor: each side's best and extent through its chain, then the
// record and status at the survivor's own index.  A right chain runs to the first
// drop-ended walk t >= s (its bests add the scores at the starts s .. t - 1); a left chain
// to the last drop-ended walk t <= s (scores at starts t + 1 .. s).
__global__ __launch_bounds__(256) void k_mm_finish(
    const uint64_t *__restrict__ sa, const uint32_t *__restrict__ val, uint32_t n,
    MatSide right, MatSide left, hspz_segment_pair *__restrict__ hsp,
    uint8_t *__restrict__ status, int32_t T) {
    const uint32_t s = blockIdx.x * 256 + threadIdx.x;
    if (s >= n) return;
    const uint32_t j = val[s];
    const uint64_t a = sa[s];
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    int32_t R = right.best[s], L = left.best[s];
    uint32_t k = right.ext[s], m = left.ext[s];
    // Every chain ends at a drop-ended walk (a diagonal's last survivor has no right
    // neighbour, its first none on the left); the index checks only keep a broken chain
    // inside the lists.
    const uint32_t nr = right.cnt[n - 1], nl = left.cnt[n - 1];
    if (!right.term[s] && right.cnt[s] < nr) {
        const uint32_t t = right.pos[right.cnt[s]];  // first drop-ended walk after s
        const uint32_t rt = (uint32_t)sa[t];
        // sum of the scores at the starts s .. t - 1: exclusive prefix at t minus at s
        const uint32_t ex_t = right.sum[t] - (uint32_t)right.ds[t];
        const uint32_t ex_s = right.sum[s] - (uint32_t)right.ds[s];
        R = right.best[t] + (int32_t)(ex_t - ex_s);
        k = right.ext[t] + (rt - r);
    }
    if (!left.term[s] && left.cnt[s] >= 1u && left.cnt[s] <= nl) {
        const uint32_t t = left.pos[left.cnt[s] - 1u];  // last drop-ended walk before s
        const uint32_t rt = (uint32_t)sa[t];
        L = left.best[t] + (int32_t)(left.sum[s] - left.sum[t]);
        m = left.ext[t] + (r - rt);
    }
    const int64_t total = (int64_t)L + (int64_t)R;
    hspz_segment_pair rec;
    rec.ref_start = r - m;
    rec.query_start = q - m;
    rec.len = m + k - 1u;
    rec.score = (int32_t)total;
    hsp[j] = rec;
    status[j] = total >= (int64_t)T ? 1 : 0;
}

// The entropy-adjusted decision for the records that reach T: one wave per survivor.
__global__ __launch_bounds__(64) void k_mm_entropy(const hspz_segment_pair *__restrict__ hsp,
                                                   uint8_t *__restrict__ status, uint32_t n,
                                                   const uint8_t *__restrict__ ref,
                                                   ScoreParams sp) {
    for (uint64_t i64 = blockIdx.x; i64 < n; i64 += gridDim.x) {
        const uint32_t i = (uint32_t)i64;
        if (status[i] == 0) continue;  // uniform
        const hspz_segment_pair rec = hsp[i];
        const bool ok = entropy_accept(ref, rec.ref_start, rec.len, rec.score, sp.K);
        if (lane_id() == 0) status[i] = ok ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_mm_keys(const uint64_t *anchors, const uint32_t *ids, uint32_t n,
                          uint32_t n_ref, uint32_t n_qry, uint32_t *key_r, uint32_t *val,
                          uint32_t *lcnt, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mm_keys, dim3((n + 255) / 256), dim3(256), 0, s, anchors, ids, n, n_ref,
                       n_qry, key_r, val, lcnt);
    return hipGetLastError();
}

hipError_t launch_mm_diag(const uint64_t *anchors, const uint32_t *ids, const uint32_t *val,
                          uint32_t n, uint32_t n_ref, uint32_t n_qry, uint32_t *key_d,
                          hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mm_diag, dim3((n + 255) / 256), dim3(256), 0, s, anchors, ids, val, n,
                       n_ref, n_qry, key_d);
    return hipGetLastError();
}

hipError_t launch_mm_gather(const uint64_t *anchors, const uint32_t *ids, const uint32_t *val,
                            uint32_t n, uint64_t *sa, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mm_gather, dim3((n + 255) / 256), dim3(256), 0, s, anchors, ids, val, n,
                       sa);
    return hipGetLastError();
}

hipError_t launch_mm_walk(const uint64_t *sa, const uint32_t *key_d, uint32_t n,
                          const uint8_t *ref, const uint8_t *qry, const uint32_t *ref4,
                          const uint32_t *qry4,
                          const ScoreParams &sp, const MatSide &right, const MatSide &left,
                          bool lanes, uint32_t *list, uint32_t *lcnt, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (!lanes) {
        hipLaunchKernelGGL(k_mm_walk, dim3(std::min(n, kWaveGridMax)), dim3(64), 0, s, sa, key_d,
                           n, ref, qry, sp, right, left);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_mm_lanes<kLaneBlocks>, dim3((n + 255) / 256), dim3(256), 0, s, sa, key_d,
                       n, ref4, qry4, sp, right, left, list, lcnt);
    const uint64_t grid = std::min<uint64_t>((2ull * n + 3) / 4, 2048);
    hipLaunchKernelGGL(k_mm_list, dim3((uint32_t)grid), dim3(256), 0, s, sa, key_d, n, ref4, qry4,
                       sp, right, left, list, lcnt);
    return hipGetLastError();
}

uint32_t mm_scan_blocks(uint32_t n) { return (n + kMsBlock - 1) / kMsBlock; }

hipError_t launch_mm_scan(const MatSide &right, const MatSide &left, uint32_t n, uint32_t *blk,
                          hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint32_t nb = mm_scan_blocks(n);
    hipLaunchKernelGGL(k_mm_scan_local, dim3(nb), dim3(256), 0, s, right, left, n, blk);
    hipLaunchKernelGGL(k_mm_scan_blocks, dim3(1), dim3(1024), 0, s, blk, nb);
    hipLaunchKernelGGL(k_mm_scan_add, dim3((n + 255) / 256), dim3(256), 0, s, right, left, n, blk);
    return hipGetLastError();
}

hipError_t launch_mm_finish(const uint64_t *sa, const uint32_t *val,
                            uint32_t n, const MatSide &right, const MatSide &left,
                            hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                            const ScoreParams &sp, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_mm_finish, dim3((n + 255) / 256), dim3(256), 0, s, sa, val, n,
                       right, left, hsp, status, sp.T);
    if (sp.entropy_mode == 1)
        hipLaunchKernelGGL(k_mm_entropy, dim3(std::min(n, kWaveGridMax)), dim3(64), 0, s, hsp,
                           status, n, ref, sp);
    return hipGetLastError();
}

hipError_t launch_materialize(const uint64_t *anchors, const uint32_t *ids, uint32_t n_surv,
                              hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                              const uint32_t *ref4, const uint32_t *qry4, const ScoreParams &sp,
                              hipStream_t s) {
    if (n_surv == 0) return hipSuccess;
    const uint32_t blocks = std::min((n_surv + kWaves - 1) / kWaves, kWaveGridMax);
    hipLaunchKernelGGL(k_materialize, dim3(blocks), dim3(kThreads), 0, s, anchors, ids, n_surv,
                       hsp, status, ref, ref4, qry4, sp);
    return hipGetLastError();
}

}  // namespace hspz
