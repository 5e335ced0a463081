// Score-only X-drop gate ("D. Score gate", D.1-D.3).
//
// Every kernel here keeps, per walk and per block of B bases, only the drawdown
// d = best - score (d' = max(d - sigma, 0)), its running maximum and the score.  The
// drawdown is held as its complement g = INT32_MAX - d: then d' = max(d - sigma, 0) is
// the signed saturating add g' = sat(g + sigma) (the clamp at INT32_MAX is the clamp of
// d at 0), one instruction per base, and the running maximum of d is the running
// minimum of g.  The score is carried plus INT32_MAX (mod 2^32), so the best so far,
// score + d, is one subtraction of g.  d never exceeds xdrop + B * (xdrop + 1), far from
// the lower limit.  A drop
// inside a block shows as max(d) > xdrop at the block's end.  B satisfies
// (B - 1) * max(sigma) <= xdrop, so after a drop the score cannot climb back above the
// best inside the same block: best = score + d at the block's end is exactly the
// maximum before the first drop, with no per-base branch.  Bases outside a sequence are
// edge codes scoring -(xdrop + 1), which forces that drop where the sequence ends.
//
// Two paths decide the same flag:
//
//  window (k_gate_window): one lane per anchor, 64 anchors per wave step (consecutive
//    raw ids; in the key-grouped stage, consecutive positions of k-mer runs).  Each lane
//    loads a window of both sequences around its anchor once
//    (4-bit codes, 16-byte loads, kept in registers): by default 72 bases before the
//    anchor and 48 from it.  The right walk then scores up to six blocks of eight bases
//    and the left walk up to nine, all lanes in step, so every block's window word has a
//    compile-time register index.  Pair scores come from a 16-bit LDS
//    table indexed by (ref code << 4) | query code, formed for four bases at once with
//    byte-wise bit selects.  A lane stops at its walk's first drop, or once R* (right)
//    or R* + best so far (left) reaches T, when the flag is 1 whatever follows.  Where
//    survivors are rare the reach test decides almost nothing; where most anchors
//    survive (tandem repeats) it decides them inside the first window instead of
//    sending nearly all of them on to the later stages.  Walks still running at the
//    window's end are appended to a deferred list: each wave collects them in LDS and
//    the workgroup reserves its share of the global list with one atomic.  The stages
//    that form their own anchors put each deferred anchor in a second list beside its
//    slot, which the next stage reads in order.  The key-grouped stage instead keeps its
//    deferred anchors in LDS and its workgroups run the wider second window and then the
//    exact walk on them at their end (stage2_pool); only what overflows LDS goes to the
//    lists.
//
//  exact, all anchors (k_gate): one lane per anchor walking base blocks straight from
//    the byte-per-base sequences, refilling finished lanes from the wave's tile of
//    anchors (ranks from a ballot).  Used when the window path's preconditions do not
//    hold.
//
//  exact, listed anchors (k_gate_list_wave, and exact_flag inside stage2_pool): one wave
//    per anchor the window stages left, walking 64-base tiles with wave scans (walk.h),
//    since those walks are long.
#include <algorithm>
#include <type_traits>

#include "hspz_internal.h"
#include "walk.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPerLane = 8;
constexpr int kTile = 64 * kPerLane;  // anchors per wave tile (exact path)

// ------------------------------------------------------------------ exact path

// Eight consecutive bytes starting at p, any alignment: three aligned dwords and two
// byte funnels.  Reads [p - 3, p + 12).
__device__ __forceinline__ void load8(const uint8_t *p, uint32_t &lo, uint32_t &hi) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t *w = reinterpret_cast<const uint32_t *>(a & ~uintptr_t(3));
    const uint32_t sh = (uint32_t)(a & 3);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    lo = __builtin_amdgcn_alignbyte(w1, w0, sh);
    hi = __builtin_amdgcn_alignbyte(w2, w1, sh);
}

constexpr int32_t kG0 = INT32_MAX;  // g of a zero drawdown

// Sets an anchor's flag to 1 where the flags were cleared beforehand: a byte per anchor,
// or with Bits a bit per anchor (bit slot % 32 of 32-bit word slot / 32), set atomically
// since the words are shared.
template <bool Bits>
__device__ __forceinline__ void set_flag(uint8_t *__restrict__ flags, uint32_t slot) {
    if (Bits)
        atomicOr(reinterpret_cast<uint32_t *>(flags) + (slot >> 5), 1u << (slot & 31u));
    else
        flags[slot] = 1;
}

// One base: g = INT32_MAX - d becomes INT32_MAX - max(d - sg, 0).
__device__ __forceinline__ int32_t dd_step(int32_t g, int32_t sg) {
    return __builtin_elementwise_add_sat(g, sg);
}

// Score B bases in walk direction D starting at (rp, qp) (right: rp[0..B), left:
// rp[-1] down to rp[-B]).  g and gmin are the complemented drawdown and its minimum.
template <int D, int B>
__device__ __forceinline__ void block_step(const int32_t *tab, const uint8_t *rp,
                                           const uint8_t *qp, int32_t &g, int32_t &gmin,
                                           int32_t &s) {
    uint32_t rl, rh, ql, qh;
    load8(D > 0 ? rp : rp - B, rl, rh);
    load8(D > 0 ? qp : qp - B, ql, qh);
    const uint32_t pl = rl | ql, ph = rh | qh;
#pragma unroll
    for (int i = 0; i < B; i++) {
        const int bi = D > 0 ? i : B - 1 - i;
        const uint32_t idx = (bi < 4 ? (pl >> (8 * bi)) : (ph >> (8 * (bi - 4)))) & 0xFFu;
        const int32_t sg = tab[idx];
        g = dd_step(g, sg);
        gmin = min(gmin, g);
        s += sg;
    }
}

// Walk every anchor of a tile (an[0..cnt), LDS or global) in direction D.  D > 0 parks
// R* in rstar[]; D < 0 decides the flag into fl8[].
template <int D, int B>
__device__ __forceinline__ void walk_phase(const uint64_t *an, int cnt, const int32_t *tab,
                                           const uint8_t *__restrict__ ref,
                                           const uint8_t *__restrict__ qry,
                                           const ScoreParams &sp, int32_t *rstar,
                                           uint8_t *fl8) {
    const int lane = lane_id();
    int next = 64;
    int cur = lane < cnt ? lane : -1;
    const uint8_t *rp = ref, *qp = qry;  // next base to score (right) or one past it (left)
    int32_t g = kG0, gmin = kG0, s = 0, other = 0;
    const int32_t glim = kG0 - sp.xdrop;  // a drop once gmin < glim

    auto start = [&](int i) {
        const uint64_t a = an[i];
        uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
        if (r > sp.n_ref || q > sp.n_qry) {  // outside the sequences: both sides score 0
            r = D > 0 ? sp.n_ref : 0;
            q = D > 0 ? sp.n_qry : 0;
        }
        rp = ref + r;
        qp = qry + q;
        g = kG0;
        gmin = kG0;
        s = 0;
        other = D > 0 ? 0 : rstar[i];
    };
    if (cur >= 0) start(cur);

    for (;;) {
        if (__ballot(cur >= 0) == 0) break;
        bool done = false;
        if (cur >= 0) {
            block_step<D, B>(tab, rp, qp, g, gmin, s);
            rp += D * B;
            qp += D * B;
            const int32_t best = s + (kG0 - g);
            const bool keep = (int64_t)other + best >= (int64_t)sp.T;
            done = gmin < glim || keep;
            if (done) {
                if (D > 0) rstar[cur] = keep ? sp.T : best;  // R* >= T already decides
                else fl8[cur] = keep ? 1 : 0;
            }
        }
        const uint64_t dm = __ballot(done);
        if (dm) {
            if (done) {
                cur = next + lane_rank(dm);
                if (cur < cnt) start(cur);
                else cur = -1;
            }
            next += __popcll(dm);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <int B>
__global__ __launch_bounds__(kThreads) void k_gate(const uint64_t *__restrict__ anchors,
                                                   uint32_t n, uint8_t *__restrict__ flags,
                                                   const uint8_t *__restrict__ ref,
                                                   const uint8_t *__restrict__ qry,
                                                   ScoreParams sp, int aligned8) {
    __shared__ int32_t tab[kTabSize];
    __shared__ int32_t rstar[kWaves][kTile];
    __shared__ uint32_t flg[kWaves][kTile / 4];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();

    const int w = threadIdx.x >> 6;
    const int lane = lane_id();
    const uint64_t tile0 = ((uint64_t)blockIdx.x * kWaves + w) * kTile;
    if (tile0 >= n) return;
    const int cnt = (int)min<uint64_t>((uint64_t)kTile, (uint64_t)n - tile0);
    const uint64_t *an = anchors + tile0;
    uint8_t *fl8 = reinterpret_cast<uint8_t *>(flg[w]);

    walk_phase<+1, B>(an, cnt, tab, ref, qry, sp, rstar[w], fl8);
    walk_phase<-1, B>(an, cnt, tab, ref, qry, sp, rstar[w], fl8);

    if (cnt == kTile && aligned8) {
        const uint2 v = reinterpret_cast<const uint2 *>(flg[w])[lane];
        reinterpret_cast<uint2 *>(flags + tile0)[lane] = v;
    } else {
        for (int i = lane; i < cnt; i += 64) flags[tile0 + i] = fl8[i];
    }
}

// The exact flag of anchor a, decided by the whole wave: the right walk, then the left one
// unless R* alone reaches T; each stops as soon as the flag is known.  An anchor outside
// the sequences scores 0 on both sides.
__device__ __forceinline__ bool exact_flag(const int32_t *tab, const uint8_t *__restrict__ ref,
                                           const uint8_t *__restrict__ qry, uint64_t a,
                                           const ScoreParams &sp) {
    const uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
    if (r > sp.n_ref || q > sp.n_qry) return false;
    int32_t R, L;
    uint32_t ext;
    exact_walk<+1, false, false>(tab, ref + r, qry + q, sp.xdrop, sp.T, R, ext);
    if (R >= sp.T) return true;
    exact_walk<-1, false, false>(tab, ref + r, qry + q, sp.xdrop, sp.T - R, L, ext);
    return (int64_t)R + L >= (int64_t)sp.T;
}

// The exact decision for the anchors the window stages could not finish (*count of them,
// listed by index, read on the device).  Their walks are long (homologous stretches), so
// each gets one wave that walks 64-base tiles (exact_walk) and stops as soon as the flag
// is known: at the drop, or once R* (right) or R* + best so far (left) reaches T.
__global__ __launch_bounds__(kThreads) void k_gate_list_wave(const uint64_t *__restrict__ anchors,
                                                             const uint32_t *__restrict__ list,
                                                             const uint32_t *__restrict__ count,
                                                             uint8_t *__restrict__ flags,
                                                             const uint8_t *__restrict__ ref,
                                                             const uint8_t *__restrict__ qry,
                                                             ScoreParams sp, int bits) {
    __shared__ int32_t tab[kTabSize];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();
    const uint64_t total = *count;
    const uint64_t nw = (uint64_t)gridDim.x * kWaves;
    for (uint64_t t = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); t < total; t += nw) {
        const uint32_t i = list[t];
        const bool keep = exact_flag(tab, ref, qry, anchors[i], sp);
        if (lane_id() == 0) {
            if (bits) {
                if (keep) set_flag<true>(flags, i);
            } else {
                flags[i] = keep ? 1 : 0;
            }
        }
    }
}

// ------------------------------------------------------------------ window path

// 64-anchor steps per wave of the first window stage: at most kSteps, and fewer for
// calls too small to give every SIMD several waves that way (kFillWaves waves in all).
constexpr int kSteps = 32;
constexpr uint64_t kFillWaves = 8192;
// Window sizes, in blocks of eight bases (right of the anchor, left of it).  The first
// stage sees every anchor: (6, 9) decides about 98.4% of random anchors on the 50 Mb
// workload; the narrower (4, 7) about 86%, with fewer block steps but more leftovers.
// A second stage of (8, 12) takes the first stage's leftovers and passes on about 0.15%
// of all anchors to the exact walk.
constexpr int kWideRight = 6, kWideLeft = 9;
constexpr int kNarrowRight = 4, kNarrowLeft = 7;
constexpr int kStage2Right = 8, kStage2Left = 12;
constexpr int kSeg = 512;   // LDS slots per wave for deferred anchor indices
constexpr int kSegKg = 256;  // the same with anchors, in the raw-order fused stage
// LDS entries per wave for the key-grouped stage's deferred anchors (seed, occurrence and
// anchor, 16 bytes), sized so that seven of its workgroups still fit a CU's LDS
constexpr int kSegPool = 208;
constexpr int kXPool = 128;  // anchors per workgroup for its own exact walks

typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));

// W dwords of a 4-bit copy from dword m on (8 * W consecutive codes), read from the copy
// or from its twin (alt dwords further on), whichever keeps a window of up to 16 dwords
// inside one 128-byte line.  Longer windows cross a line in either.
template <int W>
__device__ __forceinline__ void load_window(const uint32_t *__restrict__ base, uint32_t alt,
                                            uint32_t m, uint32_t (&Wd)[W]) {
    static_assert(W % 4 == 0, "whole 16-byte loads");
    const uint32_t off = (m & 31u) > (uint32_t)kTwinShift ? alt + m - kTwinShift : m;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(base + off);
#pragma unroll
    for (int j = 0; j < W / 4; j++) {
        const u32x4 v = p[j];
        Wd[4 * j + 0] = v.x;
        Wd[4 * j + 1] = v.y;
        Wd[4 * j + 2] = v.z;
        Wd[4 * j + 3] = v.w;
    }
}

// The same window read from the 4-bit copy alone (it may span two lines).
template <int W>
__device__ __forceinline__ void load_plain(const uint32_t *__restrict__ base, uint32_t m,
                                           uint32_t (&Wd)[W]) {
    static_assert(W % 4 == 0, "whole 16-byte loads");
    const u32x4 *p = reinterpret_cast<const u32x4 *>(base + m);
#pragma unroll
    for (int j = 0; j < W / 4; j++) {
        const u32x4 v = p[j];
        Wd[4 * j + 0] = v.x;
        Wd[4 * j + 1] = v.y;
        Wd[4 * j + 2] = v.z;
        Wd[4 * j + 3] = v.w;
    }
}

// Eight bases: R and Q hold codes of bases 0..7 in nibbles 0..7.  Even bases' table
// indices (r << 4 | q) land in the bytes of ie, odd bases' in the bytes of io.
template <bool Right>
__device__ __forceinline__ void block8(const int16_t *tab, uint32_t R, uint32_t Q, int32_t &g,
                                       int32_t &gmin, uint32_t &s) {
    const uint32_t hi = 0xF0F0F0F0u;
    uint32_t ie = ((R << 4) & hi) | (Q & ~hi);
    uint32_t io = (R & hi) | ((Q >> 4) & ~hi);
    // keep ie and io whole: each table address is then one byte-select shift of them
    asm volatile("" : "+v"(ie), "+v"(io));
#pragma unroll
    for (int t = 0; t < 8; t++) {
        const int i = Right ? t : 7 - t;
        const uint32_t w = (i & 1) ? io : ie;
        const int32_t sg = tab[(w >> (8 * (i >> 1))) & 0xFFu];
        g = dd_step(g, sg);
        gmin = min(gmin, g);
        s += (uint32_t)sg;
    }
}

// Calls f(integral_constant<int, K>) for K = 0, 1, ... while f returns true, unrolled at
// compile time, so register arrays indexed by K stay in registers.
template <int K, int N>
struct Unrolled {
    template <class F>
    __device__ __forceinline__ static void run(F &&f) {
        if (f(std::integral_constant<int, K>())) Unrolled<K + 1, N>::run(f);
    }
};
template <int N>
struct Unrolled<N, N> {
    template <class F>
    __device__ __forceinline__ static void run(F &&) {}
};

// The windows of one anchor per lane: 8 * LB bases before the anchor and 8 * RB from it
// (plus one dword for the funnel shift), 4-bit codes of both sequences.  load() only
// issues the reads, so a wave can fetch the next step's windows while it scores this
// step's.  decide() is called by all lanes of the wave together and returns the flag
// (0 or 1), or 2 when a walk is still running at the window's end.  With EarlyKeep a walk
// also stops once the flag is 1 whatever follows (R*, or R* + best so far, reaches T; on
// the right tested every other block).
template <int RB, int LB, bool EarlyKeep, bool RefTwin = true>
struct Win {
    static constexpr int W = (LB + RB + 1 + 3) / 4 * 4;
    static_assert(8 * LB + 8 <= kPad4, "left window stays inside the edge padding");
    uint32_t R[W], Q[W];
    uint32_t shr, shq;
    bool inrange;

    __device__ __forceinline__ void load(bool in, uint32_t r, uint32_t q,
                                         const uint32_t *__restrict__ ref4,
                                         const uint32_t *__restrict__ qry4,
                                         const WindowParams &wp) {
        inrange = in;
        const uint32_t wr = (in ? r : 0u) + (uint32_t)(kPad4 - 8 * LB);
        const uint32_t wq = (in ? q : 0u) + (uint32_t)(kPad4 - 8 * LB);
        if (RefTwin)
            load_window<W>(ref4, wp.ref4_alt, wr >> 3, R);
        else
            load_plain<W>(ref4, wr >> 3, R);
        load_window<W>(qry4, wp.qry4_alt, wq >> 3, Q);
        shr = (wr & 7u) * 4u;
        shq = (wq & 7u) * 4u;
    }

    __device__ __forceinline__ int decide(const int16_t *tab, const WindowParams &wp) const {
        // Every lane scores every block the wave runs (a lane that has finished only
        // scores its own registers again) and its results are taken at its first drop.
        // The lane states are wave-uniform 64-bit masks, so the loops need no divergent
        // regions and their bookkeeping stays in scalar registers.
        const int32_t glim = kG0 - wp.xdrop;  // a drop once gmin < glim
        const uint64_t live = __builtin_amdgcn_ballot_w64(inrange);
        uint64_t keep = 0;
        int32_t rstar = 0;
        // right: bases r + 8k .. r + 8k + 7 are window dword LB + k onward.  s carries the
        // running score plus kG0 (mod 2^32), so the best so far, score + drawdown, is
        // s - g in one subtraction (it fits int32).
        uint64_t act = live;
        int32_t g = kG0, gmin = kG0;
        uint32_t s = (uint32_t)kG0;
        Unrolled<0, RB>::run([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if (act == 0) return false;
            const uint32_t Rb = __builtin_amdgcn_alignbit(R[LB + k + 1], R[LB + k], shr);
            const uint32_t Qb = __builtin_amdgcn_alignbit(Q[LB + k + 1], Q[LB + k], shq);
            block8<true>(tab, Rb, Qb, g, gmin, s);
            const int32_t best = (int32_t)(s - (uint32_t)g);
            const uint64_t drop = __builtin_amdgcn_ballot_w64(gmin < glim) & act;
            rstar = __builtin_amdgcn_inverse_ballot_w64(drop) ? best : rstar;
            act &= ~drop;
            // the early keep is tested on every other block and the last: a walk whose best
            // has reached T stays exact if it runs on (its R* only grows), and the test's
            // instructions cost more than the block it can save (1.2% of the stage on the
            // 50 Mb workload)
            if (EarlyKeep && (k % 2 == 1 || k == RB - 1)) {
                const uint64_t hit = __builtin_amdgcn_ballot_w64(best >= wp.T) & act;
                keep |= hit;
                act &= ~hit;
            }
            return true;
        });
        uint64_t undecided = act;
        // left: bases r - 8k - 8 .. r - 8k - 1 are window dword LB - 1 - k onward
        act = live & ~keep & ~undecided;
        g = kG0;
        gmin = kG0;
        s = (uint32_t)kG0;
        const int32_t need = wp.T - rstar;  // the left best that makes the flag 1
        Unrolled<0, LB>::run([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if (act == 0) return false;
            const uint32_t Rb = __builtin_amdgcn_alignbit(R[LB - k], R[LB - 1 - k], shr);
            const uint32_t Qb = __builtin_amdgcn_alignbit(Q[LB - k], Q[LB - 1 - k], shq);
            block8<false>(tab, Rb, Qb, g, gmin, s);
            const uint64_t reach = __builtin_amdgcn_ballot_w64((int32_t)(s - (uint32_t)g) >= need);
            const uint64_t drop = __builtin_amdgcn_ballot_w64(gmin < glim) & act;
            const uint64_t done = EarlyKeep ? (drop | (reach & act)) : drop;
            keep |= done & reach;
            act &= ~done;
            return true;
        });
        undecided |= act;
        return __builtin_amdgcn_inverse_ballot_w64(undecided)
                   ? 2
                   : (__builtin_amdgcn_inverse_ballot_w64(keep) ? 1 : 0);
    }
};

// An anchor outside the sequences scores 0 on both sides: flag 0 without a walk.
__device__ __forceinline__ bool in_range(bool valid, uint64_t a, const WindowParams &wp) {
    return valid && (uint32_t)a <= wp.n_ref && (uint32_t)(a >> 32) <= wp.n_qry;
}

// Deferred indices are gathered per wave in LDS (S slots) and reserved in the global list
// once per workgroup (a full wave segment is flushed on its own).  With P each index
// carries its anchor into a parallel list (sega in LDS, defer_a in the global list).
template <int S, bool P>
__device__ __forceinline__ void defer_push_g(uint32_t *seg, uint64_t *sega, uint32_t &nseg,
                                             bool dfr, uint32_t i, uint64_t a,
                                             uint32_t *__restrict__ defer,
                                             uint64_t *__restrict__ defer_a,
                                             uint32_t *__restrict__ defer_cnt) {
    const int lane = lane_id();
    const uint64_t m = __ballot(dfr);
    if (!m) return;
    const uint32_t c = (uint32_t)__popcll(m);
    if (nseg + c > (uint32_t)S) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(defer_cnt, nseg);
        base = __shfl(base, 0, 64);
        for (uint32_t j = lane; j < nseg; j += 64) {
            defer[base + j] = seg[j];
            if (P) defer_a[base + j] = sega[j];
        }
        nseg = 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (dfr) {
        const uint32_t k = nseg + lane_rank(m);
        seg[k] = i;
        if (P) sega[k] = a;
    }
    nseg += c;
}

// The key-grouped stage's deferral.  A deferred anchor's slot needs its seed's prefix, a
// random read that would hold the whole wave for one lane, so each entry keeps the seed
// (relative to the batch), the occurrence and the anchor, and the slot is formed where the
// entries are consumed: for a segment that fills, here with up to 64 reads in flight.
template <int S>
__device__ __forceinline__ void defer_push_kg(uint32_t *segs, uint32_t *sego, uint64_t *sega,
                                              uint32_t &nseg, bool dfr, uint32_t sr,
                                              uint32_t occ, uint64_t a, const PrefixView &prefix,
                                              uint32_t hit_lo, uint32_t *__restrict__ defer,
                                              uint64_t *__restrict__ defer_a,
                                              uint32_t *__restrict__ defer_cnt) {
    const int lane = lane_id();
    const uint64_t m = __ballot(dfr);
    if (!m) return;
    const uint32_t c = (uint32_t)__popcll(m);
    if (nseg + c > (uint32_t)S) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(defer_cnt, nseg);
        base = __shfl(base, 0, 64);
        for (uint32_t j = lane; j < nseg; j += 64) {
            defer[base + j] = prefix.at(segs[j]) - 1u - hit_lo - sego[j];
            defer_a[base + j] = sega[j];
        }
        nseg = 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (dfr) {
        const uint32_t k = nseg + lane_rank(m);
        segs[k] = sr;
        sego[k] = occ;
        sega[k] = a;
    }
    nseg += c;
}

// All waves of the block call this once at the end.
template <int S, bool P>
__device__ __forceinline__ void defer_flush_block_g(uint32_t (*seg)[S], uint64_t (*sega)[S],
                                                    uint32_t *seg_n, uint32_t *blk_base,
                                                    uint32_t nseg, uint32_t *__restrict__ defer,
                                                    uint64_t *__restrict__ defer_a,
                                                    uint32_t *__restrict__ defer_cnt) {
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    if (lane == 0) seg_n[w] = nseg;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int v = 0; v < kWaves; v++) tot += seg_n[v];
        *blk_base = tot ? atomicAdd(defer_cnt, tot) : 0u;
    }
    __syncthreads();
    uint32_t base = *blk_base;
    for (int v = 0; v < w; v++) base += seg_n[v];
    for (uint32_t j = lane; j < nseg; j += 64) {
        defer[base + j] = seg[w][j];
        if (P) defer_a[base + j] = sega[w][j];
    }
}

__device__ __forceinline__ void defer_push(uint32_t *seg, uint32_t &nseg, bool dfr, uint32_t i,
                                           uint32_t *__restrict__ defer,
                                           uint32_t *__restrict__ defer_cnt) {
    defer_push_g<kSeg, false>(seg, nullptr, nseg, dfr, i, 0, defer, nullptr, defer_cnt);
}

__device__ __forceinline__ void defer_flush_block(uint32_t (*seg)[kSeg], uint32_t *seg_n,
                                                  uint32_t *blk_base, uint32_t nseg,
                                                  uint32_t *__restrict__ defer,
                                                  uint32_t *__restrict__ defer_cnt) {
    defer_flush_block_g<kSeg, false>(seg, nullptr, seg_n, blk_base, nseg, defer, nullptr,
                                     defer_cnt);
}

// The second window stage run by the workgroup of the key-grouped first stage, once all
// four waves are done with their steps: the deferred entries still in the waves' LDS
// segments are taken 64 at a time, each wave a step in turn, with the wider windows.  The
// lines of a step's windows are read while the other waves on the SIMD score their
// blocks, instead of in a separate launch whose one step per wave waits on them.  An
// entry's slot (its seed's prefix, less hit_lo and the occurrence, the slot rule of
// "C. Hit discovery", C.5) is read only once the wider window leaves its flag open or 1.
// A deferred slot's anchor is stored unless its flag is 0 (the exact walk reads it
// there); the flags were cleared, so only 1s are written (Bits: set_flag).  Segments a
// wave flushed to the global list on the way are left to the separate second stage.  The
// anchors the wider windows leave go on, up to kXPool of them, to the exact walk the
// workgroup then runs itself (one wave per anchor, as the exact list does), the rest to
// the exact list.  cnt[1] counts the exact list, cnt[2] the anchors pooled here, cnt[3]
// the exact walks pooled here.  (The raw-order first stage, whose calls are often small,
// leaves both stages to their own launches: run inside its few workgroups, they slowed
// the 5 Mb dense-repeat workload's chunks from 0.080 to 0.10-0.15 ms.)
struct ExactPool {
    uint32_t slot[kXPool];
    uint64_t a[kXPool];
    uint32_t n;  // reserved entries (may exceed kXPool: those went to the exact list)
};

template <int S, bool Bits>
__device__ __forceinline__ void stage2_pool(const uint32_t (*segs)[S], const uint32_t (*sego)[S],
                                            const uint64_t (*sega)[S], const PrefixView &prefix,
                                            uint32_t hit_lo, uint32_t *seg_n, uint32_t nseg,
                                            const int16_t *tab,
                                            uint64_t *__restrict__ anchors,
                                            uint8_t *__restrict__ flags,
                                            const uint32_t *__restrict__ ref4,
                                            const uint32_t *__restrict__ qry4,
                                            const WindowParams &wp, uint32_t *__restrict__ list2,
                                            uint32_t *__restrict__ cnt, ExactPool &xp,
                                            const int32_t *tab32, const uint8_t *__restrict__ ref8,
                                            const uint8_t *__restrict__ qry8,
                                            const ScoreParams &sp) {
    static_assert(kWaves == 4, "four wave segments");
    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    if (lane == 0) seg_n[w] = nseg;
    __syncthreads();
    const uint32_t n0 = seg_n[0], n1 = seg_n[1], n2 = seg_n[2];
    const uint32_t total = n0 + n1 + n2 + seg_n[3];
    if (threadIdx.x == 0 && total) atomicAdd(cnt + 2, total);  // the pooled count
    for (uint32_t e0 = (uint32_t)w * 64; e0 < total; e0 += kWaves * 64) {  // uniform
        const uint32_t e = e0 + lane;
        const bool valid = e < total;
        uint32_t sr = 0, occ = 0;
        uint64_t a = 0;
        if (valid) {
            uint32_t v = 0, j = e;
            if (j >= n0) {
                j -= n0;
                v = 1;
                if (j >= n1) {
                    j -= n1;
                    v = 2;
                    if (j >= n2) {
                        j -= n2;
                        v = 3;
                    }
                }
            }
            sr = segs[v][j];
            occ = sego[v][j];
            a = sega[v][j];
        }
        Win<kStage2Right, kStage2Left, true> win;
        win.load(in_range(valid, a, wp), (uint32_t)a, (uint32_t)(a >> 32), ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        uint32_t slot = 0;
        if (valid && res != 0) {
            slot = prefix.at(sr) - 1u - hit_lo - occ;
            anchors[slot] = a;
        }
        if (valid && res == 1) set_flag<Bits>(flags, slot);
        const uint64_t m = __ballot(valid && res == 2);
        if (m) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&xp.n, (uint32_t)__popcll(m));
            base = __shfl(base, 0, 64);
            const uint32_t k = base + (uint32_t)lane_rank(m);
            const bool pooled = k < (uint32_t)kXPool;
            if (valid && res == 2 && pooled) {
                xp.slot[k] = slot;
                xp.a[k] = a;
            }
            const uint64_t m2 = __ballot(valid && res == 2 && !pooled);
            if (m2) {
                uint32_t b2 = 0;
                if (lane == 0) b2 = atomicAdd(cnt + 1, (uint32_t)__popcll(m2));
                b2 = __shfl(b2, 0, 64);
                if (valid && res == 2 && !pooled) list2[b2 + lane_rank(m2)] = slot;
            }
        }
    }
    __syncthreads();
    const uint32_t nx = min(xp.n, (uint32_t)kXPool);
    if (threadIdx.x == 0 && nx) atomicAdd(cnt + 3, nx);  // the pooled exact walks
    for (uint32_t e = (uint32_t)w; e < nx; e += kWaves) {  // uniform
        const bool keep = exact_flag(tab32, ref8, qry8, xp.a[e], sp);
        if (lane == 0 && keep) set_flag<Bits>(flags, xp.slot[e]);
    }
}

// First stage: every anchor, consecutive 64-anchor steps per wave.
template <int RB, int LB>
__global__ __launch_bounds__(kThreads) void k_gate_window(
    const uint64_t *__restrict__ anchors, uint32_t n, uint32_t steps,
    uint8_t *__restrict__ flags, const uint32_t *__restrict__ ref4,
    const uint32_t *__restrict__ qry4, WindowParams wp, uint32_t *__restrict__ defer,
    uint32_t *__restrict__ defer_cnt) {
    __shared__ int16_t tab[kWinTab];
    __shared__ uint32_t seg[kWaves][kSeg];
    __shared__ uint32_t seg_n[kWaves];
    __shared__ uint32_t blk_base;
    if (threadIdx.x < kWinTab) tab[threadIdx.x] = wp.tab[threadIdx.x];
    __syncthreads();

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t nseg = 0;
    const uint64_t first = ((uint64_t)blockIdx.x * kWaves + w) * (64ull * steps);
    for (uint32_t step = 0; step < steps; step++) {
        const uint64_t i0 = first + (uint64_t)step * 64;
        if (i0 >= n) break;  // uniform
        const uint64_t i = i0 + lane;
        const bool valid = i < n;
        const uint64_t a = valid ? anchors[i] : 0ull;
        Win<RB, LB, true> win;
        win.load(in_range(valid, a, wp), (uint32_t)a, (uint32_t)(a >> 32), ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        if (valid && res != 2) flags[i] = (uint8_t)res;
        defer_push(seg[w], nseg, valid && res == 2, (uint32_t)i, defer, defer_cnt);
    }
    defer_flush_block(seg, seg_n, &blk_base, nseg, defer, defer_cnt);
}

// Directory of the fused first stage: the seed that owns the first slot of each wave's
// range, i.e. the first seed whose prefix - hit_lo exceeds that slot.  One wave per entry
// searches 64 ways: each round its lanes read the last prefix of 64 equal segments of the
// range and a ballot picks the first segment past the slot, so a search costs about
// log64(seeds) dependent reads where a per-thread binary search costs log2(seeds) (a
// chunk's prefixes are few enough to stay in L2, so the extra reads are cheap).  The
// first wave also clears the four deferred-list counters the stages append to.
__global__ __launch_bounds__(kThreads) void k_slot_dir(ChunkSeeds cs, uint32_t n_waves,
                                                       uint32_t steps,
                                                       uint32_t *__restrict__ cnt) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t w = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (w == 0 && lane < 4) cnt[lane] = 0;
    if (w >= n_waves) return;  // uniform
    const uint32_t t = w * (64u * steps);
    // the answer lies in [lo, hi], and the chunk's last seed is past every wave's first slot
    // (t < n), so the ballot over the probes always holds lane 63's bit
    uint32_t lo = 0, hi = cs.n_seeds - 1;
    while (hi - lo >= 64) {  // uniform
        const uint64_t step = ((uint64_t)hi - lo + 64) / 64;
        const uint32_t idx = (uint32_t)min((uint64_t)lo + (lane + 1) * step - 1, (uint64_t)hi);
        const uint64_t m = __ballot(cs.prefix.at(idx) - cs.hit_lo > t);
        const uint32_t f = (uint32_t)__builtin_ctzll(m);
        hi = (uint32_t)min((uint64_t)lo + (f + 1) * step - 1, (uint64_t)hi);
        lo = (uint32_t)(lo + f * step);
    }
    const uint32_t idx = min(lo + lane, hi);
    const uint64_t m = __ballot(lo + lane <= hi && cs.prefix.at(idx) - cs.hit_lo > t);
    if (lane == 0) cs.dir[w] = lo + (uint32_t)__builtin_ctzll(m);
}

// First stage fused with the backward expansion ("C. Hit discovery", C.5): a wave walks
// the same 64-slot steps as k_gate_window, but builds each slot's anchor from the seed
// that owns it.  The wave keeps a window of 64 consecutive seeds in LDS (prefix - hit_lo,
// bucket start and query end, read once, coalesced), starting at the owner of its first
// slot; lanes binary-search it for their slot, and the window slides on by 64 seeds when
// a slot lies past it (seeds with no hits can take several slides).  Occurrence
// j = prefix[s] - 1 - hit_lo - slot of seed s is the bucket entry pos[first[s] + j].  The
// anchor is stored only when the slot is deferred or kept.
template <int RB, int LB>
__global__ __launch_bounds__(kThreads) void k_gate_window_fused(
    ChunkSeeds cs, uint32_t n, uint32_t steps, uint64_t *__restrict__ anchors,
    uint8_t *__restrict__ flags,
    const uint32_t *__restrict__ ref4, const uint32_t *__restrict__ qry4, WindowParams wp,
    uint32_t *__restrict__ defer, uint64_t *__restrict__ defer_a,
    uint32_t *__restrict__ defer_cnt) {
    __shared__ int16_t tab[kWinTab];
    __shared__ uint32_t seg[kWaves][kSegKg];
    __shared__ uint64_t sega[kWaves][kSegKg];
    __shared__ uint32_t seg_n[kWaves];
    __shared__ uint32_t blk_base;
    __shared__ uint32_t rel[kWaves][64];  // prefix - hit_lo of the window's seeds
    __shared__ uint32_t fst[kWaves][64];  // their bucket starts
    __shared__ uint32_t qen[kWaves][64];  // their query ends
    if (threadIdx.x < kWinTab) tab[threadIdx.x] = wp.tab[threadIdx.x];
    __syncthreads();

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t nseg = 0;
    const uint64_t wave = (uint64_t)blockIdx.x * kWaves + w;
    const uint64_t first = wave * (64ull * steps);
    uint32_t wb = first < n ? cs.dir[wave] : 0u;  // window: seeds wb .. wb + 63
    bool loaded = false;                          // uniform
    for (uint32_t step = 0; step < steps; step++) {
        const uint64_t i0 = first + (uint64_t)step * 64;
        if (i0 >= n) break;  // uniform
        const uint32_t t = (uint32_t)(i0 + lane);
        const bool valid = t < n;
        uint32_t top = 0, bstart = 0, qend = 0;  // of the slot's owner
        bool found = !valid;
        for (;;) {  // uniform: ends once every slot has its owner
            if (!loaded) {
                // the three reads are issued together (a seed past the end reads the
                // last seed, of which there is at least one, and is then masked)
                const uint32_t sj = wb + lane;
                const bool in = sj < cs.n_seeds;
                const uint32_t sr = in ? sj : cs.n_seeds - 1u;
                const uint32_t pr = cs.prefix.at(sr), fs = cs.first[sr], qe = cs.q_end[sr];
                rel[w][lane] = in ? pr - cs.hit_lo : 0xFFFFFFFFu;
                fst[w][lane] = in ? fs : 0u;
                qen[w][lane] = in ? qe : 0u;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                loaded = true;
            }
            if (!found && t < rel[w][63]) {
                int L = 0;  // number of the window's seeds whose prefix - hit_lo is <= t
#pragma unroll
                for (int k = 32; k >= 1; k >>= 1)
                    if (rel[w][L + k - 1] <= t) L += k;
                top = rel[w][L];
                bstart = fst[w][L];
                qend = qen[w][L];
                found = true;
            }
            if (__ballot(!found) == 0) break;
            // a slot lies past the window: every lane is done reading it, slide it on
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            wb += 64;
            loaded = false;
        }
        uint64_t a = 0;
        if (valid) a = (uint64_t)cs.pos[bstart + (top - 1u - t)] | ((uint64_t)qend << 32);
        Win<RB, LB, true> win;
        win.load(in_range(valid, a, wp), (uint32_t)a, (uint32_t)(a >> 32), ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        if (valid && res != 2) flags[t] = (uint8_t)res;
        if (valid && res == 1) anchors[t] = a;
        // a deferred slot's anchor travels in the list; the next stage stores it if kept
        defer_push_g<kSegKg, true>(seg[w], sega[w], nseg, valid && res == 2, t, a, defer,
                                   defer_a, defer_cnt);
    }
    defer_flush_block_g<kSegKg, true>(seg, sega, seg_n, &blk_base, nseg, defer, defer_a,
                                      defer_cnt);
}

// ------------------------------------------------------------------ key-grouped first stage
//
// A range of seeds' anchors (one chunk, or a whole batch of chunks) in another order: run
// by run of the strand's seeds grouped by k-mer, the range's seeds of the k-mer (m of
// them, a contiguous stretch of the run) times the k-mer's bucket (c reference ends).  Within a run the anchors go bucket entry
// by bucket entry, the m seeds of each entry next to each other, so the lanes of a wave
// that share a bucket entry read the same reference window and the lanes that share a
// seed the same query window: a run's c + m windows serve its c * m anchors.  Flags are
// decided per anchor exactly as in the fused stage; a kept or deferred anchor's raw slot
// (its seed's inclusive prefix - 1 - hit_lo - its occurrence) is formed only for it.

// Index in the sorted stretch qs[lo, hi) of the first seed >= x (seeds ascend).  Short
// stretches (most runs hold a few seeds) are counted with independent loads.
__device__ __forceinline__ uint32_t kg_lower(const uint32_t *__restrict__ qs, uint32_t lo,
                                             uint32_t hi, uint32_t x) {
    if (hi - lo <= 8) {
        if (hi == lo) return lo;
        uint32_t v[8];  // all eight reads first, so none waits for another
#pragma unroll
        for (uint32_t k = 0; k < 8; k++) v[k] = qs[min(lo + k, hi - 1)];
        uint32_t below = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8; k++) below += (lo + k < hi && v[k] < x) ? 1u : 0u;
        return lo + below;
    }
    while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (qs[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Per run: the range's seeds of its k-mer (index of the first in qs, and how many) and
// the anchors they make with the k-mer's bucket; then the inclusive prefix of those
// anchor counts within each workgroup's kScanBlock runs (one run per thread, so that
// the runs' searches overlap), and each workgroup's total (the offsets of the
// workgroups come from launch_scan_blocks; consumers add them).
constexpr int kKgThreads = kScanBlock;
__global__ __launch_bounds__(kKgThreads) void k_kg_groups(KeyGroups kg, uint32_t seed_lo,
                                                          uint32_t seed_hi, KgScratch ks) {
    __shared__ uint64_t wave_tot[kKgThreads / 64];
    const int t = threadIdx.x;
    const uint64_t r = (uint64_t)blockIdx.x * kKgThreads + t;
    uint32_t cnt = 0;
    if (r < kg.n_runs) {
        const uint32_t c = kg.run_c[r];
        const uint4 sp = kg.run_span[r];  // issued with run_c: one round of loads
        const uint32_t A = sp.x, B = sp.y;
        uint32_t a = 0, b = 0;
        if (c == 0 || sp.w < seed_lo || sp.z > seed_hi) {
            // no anchors, or no seed in the range: nothing to search
        } else if (sp.z >= seed_lo && sp.w <= seed_hi) {
            a = A;  // the whole run lies in the range
            b = B;
        } else if (B - A <= 8) {
            // both bounds from one round of loads (a run is never empty)
            uint32_t v[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; k++) v[k] = kg.qs[min(A + k, B - 1)];
            a = b = A;
#pragma unroll
            for (uint32_t k = 0; k < 8; k++) {
                const bool in = A + k < B;
                a += (in && v[k] < seed_lo) ? 1u : 0u;
                b += (in && v[k] <= seed_hi) ? 1u : 0u;
            }
        } else {
            a = kg_lower(kg.qs, A, B, seed_lo);
            b = seed_hi + 1u == 0u ? B : kg_lower(kg.qs, a, B, seed_hi + 1u);
        }
        ks.a[r] = a;
        ks.m[r] = b - a;
        // at most the range's hits, which fit 32 bits
        cnt = (uint32_t)((uint64_t)c * (b - a));
    }
    const uint64_t incl = wave_incl_sum_u64(cnt);
    if (lane_id() == 63) wave_tot[t >> 6] = incl;
    __syncthreads();
    uint64_t run = incl;
    for (int w = 0; w < (t >> 6); w++) run += wave_tot[w];
    if (r < kg.n_runs) ks.G[r] = (uint32_t)run;
    if (t == kKgThreads - 1) ks.blksum[blockIdx.x] = run;
}

// Inclusive prefix of run r's anchors over the range: its workgroup's offset plus the
// workgroup-local prefix.
__device__ __forceinline__ uint32_t kg_prefix(const KgScratch &ks, uint32_t r) {
    return ks.G[r] + ks.blkoff[r / kScanBlock];
}

// Per wave of the key-grouped stage: the run owning its first slot (the first run whose
// inclusive prefix exceeds it).  The first thread also clears the deferred-list counters.
__global__ __launch_bounds__(kThreads) void k_kg_dir(KgScratch ks, uint32_t n_runs,
                                                     uint32_t n_waves, uint32_t steps,
                                                     uint32_t *__restrict__ cnt) {
    const uint32_t w = blockIdx.x * kThreads + threadIdx.x;
    if (w == 0) {
        cnt[0] = 0;
        cnt[1] = 0;
        cnt[2] = 0;
        cnt[3] = 0;
    }
    if (w >= n_waves) return;
    const uint32_t t = w * (64u * steps);
    uint32_t lo = 0, hi = n_runs;
    while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (kg_prefix(ks, mid) > t) hi = mid;
        else lo = mid + 1;
    }
    ks.dir[w] = lo;
}

// A run as the key-grouped stage's window holds it: inclusive and exclusive prefix of its
// anchors in the call (rs above rel for an entry past the last run), bucket start, first
// seed in qs, the smaller of its bucket entries and its seeds in the range (bit 31 set
// when that is the bucket entries) and the hardware reciprocal of that count.
struct KgRun {
    uint32_t rel, rs, f, a, m;
    float q;
};

// The first window stage over the key-grouped order (see above).  As k_gate_window_fused,
// a wave keeps a window of 64 runs in LDS (prefix end, bucket size and start, first seed
// in qs, seeds); each step's lanes find the run owning their position from the marks the
// runs leave at their first positions in the step, by a max-scan across the wave.
template <int RB, int LB, bool Bits>
__global__ __launch_bounds__(kThreads) void k_gate_window_kg(
    KeyGroups kg, KgScratch ks, PrefixView prefix, uint32_t batch_lo,
    uint32_t hit_lo, uint32_t n, uint32_t steps, const uint32_t *__restrict__ pos,
    uint64_t *__restrict__ anchors, uint8_t *__restrict__ flags,
    const uint32_t *__restrict__ ref4, const uint32_t *__restrict__ qry4, WindowParams wp,
    uint32_t *__restrict__ defer, uint64_t *__restrict__ defer_a,
    uint32_t *__restrict__ defer_cnt, uint32_t *__restrict__ list2, ScoreParams sp,
    const uint8_t *__restrict__ ref8, const uint8_t *__restrict__ qry8) {
    __shared__ int16_t tab[kWinTab];
    __shared__ int32_t tab32[kTabSize];  // the exact walks' table
    __shared__ ExactPool xp;
    __shared__ uint32_t segs[kWaves][kSegPool];  // deferred: seed - batch_lo
    __shared__ uint32_t sego[kWaves][kSegPool];  // occurrence
    __shared__ uint64_t sega[kWaves][kSegPool];  // anchor
    __shared__ uint32_t seg_n[kWaves];
    __shared__ KgRun run[kWaves][64];    // the wave's window of runs
    __shared__ uint32_t mk[kWaves][64];  // marks of the step's positions (run index)
    if (threadIdx.x < kWinTab) tab[threadIdx.x] = wp.tab[threadIdx.x];
    if (threadIdx.x < kTabSize) tab32[threadIdx.x] = sp.tab[threadIdx.x];
    if (threadIdx.x == 0) xp.n = 0;
    __syncthreads();

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t nseg = 0;
    const uint64_t wave = (uint64_t)blockIdx.x * kWaves + w;
    const uint64_t first = wave * (64ull * steps);
    uint32_t wb = first < n ? ks.dir[wave] : 0u;  // window: runs wb .. wb + 63
    bool loaded = false;                          // uniform
    bool small = true;  // uniform: every run of the window has under 2^22 anchors
    for (uint32_t step = 0; step < steps; step++) {
        const uint64_t i0 = first + (uint64_t)step * 64;
        if (i0 >= n) break;  // uniform
        const uint32_t t = (uint32_t)(i0 + lane);
        const bool valid = t < n;
        uint32_t start = 0, bfirst = 0, sa = 0, m = 1;  // of the position's run
        float rcp = 1.f;
        bool found = !valid;
        bool step_small = small;  // uniform: over every window this step reads
        for (;;) {  // uniform: ends once every position has its run
            if (!loaded) {
                // the six reads are issued together (a run past the end reads the last
                // run, of which there is at least one, and is then masked)
                const uint32_t r = wb + lane;
                const bool in = r < kg.n_runs;
                const uint32_t rr = in ? r : kg.n_runs - 1u;
                const uint32_t g = ks.G[rr], off = ks.blkoff[rr / kScanBlock];
                const uint32_t c = kg.run_c[rr], f = kg.run_first[rr];
                const uint32_t sa0 = ks.a[rr], m0 = ks.m[rr];
                const uint32_t cm = c * m0;  // the run's anchors in this call
                KgRun &q = run[w][lane];
                q.rel = in ? g + off : 0xFFFFFFFFu;
                q.rs = in ? g + off - cm : 0xFFFFFFFFu;  // above rel: holds no position
                q.f = in ? f : 0u;
                q.a = in ? sa0 : 0u;
                // the smaller of c and m runs fastest (bit 31: c, the bucket entries)
                const uint32_t x = !in ? 1u : (c < m0 ? c : m0);
                q.m = x | (in && c < m0 ? 0x80000000u : 0u);
                q.q = __builtin_amdgcn_rcpf((float)x);
                small = __ballot(in && cm >= (1u << 22)) == 0;
                step_small = step_small && small;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                loaded = true;
            }
            // positions past the window's last run wait for the next window
            const uint32_t lim = run[w][63].rel;
            const bool look = !found && t < lim;
            if (__ballot(look)) {  // uniform
                // Each run of the window holding positions of this step marks the first of
                // them (its start, or the step's first position) with its index.  Runs
                // start in order, so a position holds one mark at most, and the largest
                // mark at or below a position, an inclusive max-scan over the lanes, is
                // the run that holds it (-1: no mark).
                mk[w][lane] = 0xFFFFFFFFu;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                const uint32_t t0 = (uint32_t)i0;
                const uint32_t re = run[w][lane].rel, rb = run[w][lane].rs;
                const uint32_t pm = rb > t0 ? rb - t0 : 0u;
                if (re > rb && re > t0 && pm < 64u) mk[w][pm] = (uint32_t)lane;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                const int32_t o = wave_incl_max((int32_t)mk[w][lane]);
                if (look) {  // o >= 0: the run holding t is in the window and marks <= t
                    const KgRun q = run[w][(uint32_t)o & 63u];
                    start = q.rs;
                    bfirst = q.f;
                    sa = q.a;
                    m = q.m;
                    rcp = q.q;
                    found = true;
                }
            }
            if (__ballot(!found) == 0) break;
            // a position lies past the window: every lane is done reading it, slide it on
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            wb += 64;
            loaded = false;
        }
        // position u of the run's c * m anchors: with x the smaller of c and m, the one
        // that runs fastest (a run cut by a step boundary then has its x windows read in
        // both steps, not its m query windows), u / x indexes the other and u % x this
        // one.  When every run the step reads has under 2^22 anchors, the quotient comes
        // from the float reciprocal: u and x are exact in float, the hardware reciprocal
        // is within one unit in the last place and the product rounds once, so the
        // estimate is within one of u / x (exact for x = 1) and the remainder's sign
        // corrects it; 24-bit multiplies suffice, since u, x and the quotient stay under
        // 2^22.
        uint32_t occ = 0, seed = 0;
        uint64_t a = 0;
        if (valid) {
            const uint32_t u = t - start;
            const bool sw = (m >> 31) != 0u;
            const uint32_t x = m & 0x7FFFFFFFu;
            uint32_t qq, r;
            if (step_small) {
                qq = (uint32_t)((float)u * rcp);
                r = u - __umul24(qq, x);
                if ((int32_t)r < 0) {
                    qq -= 1u;
                    r += x;
                } else if (r >= x) {
                    qq += 1u;
                    r -= x;
                }
            } else {
                qq = u / x;
                r = u - qq * x;
            }
            occ = sw ? r : qq;
            const uint32_t js = sa + (sw ? qq : r);
            a = (uint64_t)pos[bfirst + occ] | ((uint64_t)kg.qe[js] << 32);
            seed = kg.qs[js];  // read with the anchor: a kept or deferred slot needs it
        }
        Win<RB, LB, true> win;
        win.load(in_range(valid, a, wp), (uint32_t)a, (uint32_t)(a >> 32), ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        if (valid && res == 1) {
            const uint32_t slot = prefix.at(seed - batch_lo) - 1u - hit_lo - occ;
            anchors[slot] = a;
            set_flag<Bits>(flags, slot);
        }
        // a deferred anchor travels with its seed and occurrence (its slot is formed where
        // it is consumed); the next stage stores it if kept
        defer_push_kg<kSegPool>(segs[w], sego[w], sega[w], nseg, valid && res == 2,
                                seed - batch_lo, occ, a, prefix, hit_lo, defer, defer_a,
                                defer_cnt);
    }
    stage2_pool<kSegPool, Bits>(segs, sego, sega, prefix, hit_lo, seg_n, nseg, tab, anchors,
                                flags, ref4, qry4, wp, list2, defer_cnt, xp, tab32, ref8, qry8,
                                sp);
}

// First stage over anchors sorted by reference slice (bucketed gate, "D. Score gate",
// D.5).  The sorted array is cut into eight equal contiguous parts, one per XCD, and
// workgroup b scores tile b / 8 of part b % 8: workgroups are dispatched in index order
// and placed on the eight XCDs in turn, so each XCD walks its part of the reference from
// start to end and holds about one slice of it (read without its twin) in its L2 at a
// time.  The mapping only places work; every tile is scored exactly once wherever it
// runs.  Results go back by raw index: the flag of a kept anchor is set to 1 (the caller
// zeroed all flags), a deferred anchor's raw index joins the list for the second stage.
template <int RB, int LB>
__global__ __launch_bounds__(kThreads) void k_gate_window_bucketed(
    const uint64_t *__restrict__ sa, const uint32_t *__restrict__ si, uint32_t n,
    uint32_t part, uint32_t steps, uint8_t *__restrict__ flags,
    const uint32_t *__restrict__ ref4,
    const uint32_t *__restrict__ qry4, WindowParams wp, uint32_t *__restrict__ defer,
    uint32_t *__restrict__ defer_cnt) {
    __shared__ int16_t tab[kWinTab];
    __shared__ uint32_t seg[kWaves][kSeg];
    __shared__ uint32_t seg_n[kWaves];
    __shared__ uint32_t blk_base;
    if (threadIdx.x < kWinTab) tab[threadIdx.x] = wp.tab[threadIdx.x];
    __syncthreads();

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t nseg = 0;
    const uint64_t lo = (uint64_t)(blockIdx.x & 7u) * part;
    const uint64_t hi = std::min<uint64_t>(lo + part, n);
    const uint64_t first = lo + ((uint64_t)(blockIdx.x >> 3) * kWaves + w) * (64ull * steps);
    for (uint32_t step = 0; step < steps; step++) {
        const uint64_t j0 = first + (uint64_t)step * 64;
        if (j0 >= hi) break;  // uniform
        const uint64_t j = j0 + lane;
        const bool valid = j < hi;
        uint64_t a = 0;
        uint32_t raw = 0;
        if (valid) {
            a = sa[j];
            raw = si[j];
        }
        Win<RB, LB, true, false> win;
        win.load(in_range(valid, a, wp), (uint32_t)a, (uint32_t)(a >> 32), ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        if (valid && res == 1) flags[raw] = 1;
        defer_push(seg[w], nseg, valid && res == 2, raw, defer, defer_cnt);
    }
    defer_flush_block(seg, seg_n, &blk_base, nseg, defer, defer_cnt);
}

// Later stage: the anchors listed by the previous stage (*count of them), wider windows.
template <int RB, int LB>
__global__ __launch_bounds__(kThreads) void k_gate_window_list(
    const uint64_t *anchors, const uint32_t *__restrict__ list,
    const uint64_t *__restrict__ list_a, uint64_t *anchors_out,
    const uint32_t *__restrict__ count, uint8_t *__restrict__ flags,
    const uint32_t *__restrict__ ref4, const uint32_t *__restrict__ qry4, WindowParams wp,
    uint32_t *__restrict__ defer, uint32_t *__restrict__ defer_cnt, int bits) {
    __shared__ int16_t tab[kWinTab];
    __shared__ uint32_t seg[kWaves][kSeg];
    __shared__ uint32_t seg_n[kWaves];
    __shared__ uint32_t blk_base;
    if (threadIdx.x < kWinTab) tab[threadIdx.x] = wp.tab[threadIdx.x];
    __syncthreads();

    const int lane = lane_id();
    const int w = threadIdx.x >> 6;
    uint32_t nseg = 0;
    const uint32_t total = *count;
    const uint64_t stride = (uint64_t)gridDim.x * kWaves * 64;
    for (uint64_t t0 = ((uint64_t)blockIdx.x * kWaves + w) * 64; t0 < total; t0 += stride) {
        const uint64_t t = t0 + lane;
        const bool valid = t < total;
        uint32_t i = 0, r = 0, q = 0;
        uint64_t a = 0;
        if (valid) {
            i = list[t];
            a = list_a ? list_a[t] : anchors[i];  // uniform choice
            r = (uint32_t)a;
            q = (uint32_t)(a >> 32);
        }
        Win<RB, LB, true> win;
        win.load(valid && r <= wp.n_ref && q <= wp.n_qry, r, q, ref4, qry4, wp);
        const int res = win.decide(tab, wp);
        if (bits) {  // cleared beforehand: only 1s are written
            if (valid && res == 1) set_flag<true>(flags, i);
        } else if (valid && res != 2) {
            flags[i] = (uint8_t)res;
        }
        // anchors that came in the list are stored where they are kept or go on
        if (list_a && valid && res != 0) anchors_out[i] = a;
        defer_push(seg[w], nseg, valid && res == 2, i, defer, defer_cnt);
    }
    defer_flush_block(seg, seg_n, &blk_base, nseg, defer, defer_cnt);
}

// Clears the deferred-list counters: second stage, exact list, pooled second stage,
// pooled exact walks.
__global__ void k_zero_counts(uint32_t *p) {
    p[0] = 0;
    p[1] = 0;
    p[2] = 0;
    p[3] = 0;
}



}  // namespace

hipError_t launch_gate(int block_bases, const uint64_t *anchors, uint32_t n, uint8_t *flags,
                       const uint8_t *ref, const uint8_t *qry, const ScoreParams &sp,
                       hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint32_t per_block = kWaves * kTile;
    const uint32_t blocks = (uint32_t)(((uint64_t)n + per_block - 1) / per_block);
    const int aligned8 = ((reinterpret_cast<uintptr_t>(flags) & 7) == 0) ? 1 : 0;
    switch (block_bases) {
    case 8:
        hipLaunchKernelGGL(k_gate<8>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    case 4:
        hipLaunchKernelGGL(k_gate<4>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    case 2:
        hipLaunchKernelGGL(k_gate<2>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    default:
        hipLaunchKernelGGL(k_gate<1>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_gate_list_wave(const uint64_t *anchors, const uint32_t *list,
                                 const uint32_t *count, uint32_t max_count, uint8_t *flags,
                                 const uint8_t *ref, const uint8_t *qry, const ScoreParams &sp,
                                 hipStream_t s, bool bits) {
    if (max_count == 0) return hipSuccess;
    const uint32_t blocks =
        (uint32_t)std::min<uint64_t>(((uint64_t)max_count + kWaves - 1) / kWaves, 4096);
    hipLaunchKernelGGL(k_gate_list_wave, dim3(blocks), dim3(kThreads), 0, s, anchors, list, count,
                       flags, ref, qry, sp, bits ? 1 : 0);
    return hipGetLastError();
}

// The second stage strides over whatever the first left, up to all n anchors.
// list1_a: the anchors of list1's entries, or NULL when they are read from anchors[];
// with list1_a, the anchors the stage keeps or defers are stored into anchors_out.
static void launch_stage2(bool narrow, bool pooled, const uint64_t *anchors, uint32_t n,
                          uint8_t *flags, const uint32_t *ref4, const uint32_t *qry4,
                          const WindowParams &wp, uint32_t *list1, const uint64_t *list1_a,
                          uint64_t *anchors_out, uint32_t *list2, uint32_t *cnt, hipStream_t s,
                          bool bits = false) {
    // enough waves for one 64-anchor step each when an eighth of the anchors is listed
    // (about one step per wave on the 50 Mb workload: 7% faster than three).  After a
    // first stage that runs the second stage on its own deferred anchors, the list holds
    // only the segments its waves flushed on the way (none on random sequence), and a
    // smaller grid strides over them.
    const uint32_t cap2 = narrow ? n : n / 8 + 1;
    const uint32_t blocks2 = (uint32_t)std::min<uint64_t>(
        ((uint64_t)cap2 + kWaves * 64 - 1) / (kWaves * 64), pooled ? 2048 : 16384);
    hipLaunchKernelGGL((k_gate_window_list<kStage2Right, kStage2Left>), dim3(blocks2),
                       dim3(kThreads), 0, s, anchors, list1, list1_a, anchors_out, cnt, flags, ref4,
                       qry4, wp, list2, cnt + 1, bits ? 1 : 0);
}

hipError_t launch_gate_window(bool narrow, const uint64_t *anchors, uint32_t n, uint8_t *flags,
                              const uint32_t *ref4, const uint32_t *qry4, const WindowParams &wp,
                              uint32_t *list1, uint32_t *list2, uint32_t *cnt, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(1), 0, s, cnt);
    if (n == 0) return hipGetLastError();
    const uint32_t steps = gate_window_steps(n);
    const uint64_t per_block = (uint64_t)kWaves * 64 * steps;
    const uint32_t blocks = (uint32_t)(((uint64_t)n + per_block - 1) / per_block);
    if (narrow)
        hipLaunchKernelGGL((k_gate_window<kNarrowRight, kNarrowLeft>), dim3(blocks),
                           dim3(kThreads), 0, s, anchors, n, steps, flags, ref4, qry4, wp,
                           list1, cnt);
    else
        hipLaunchKernelGGL((k_gate_window<kWideRight, kWideLeft>), dim3(blocks), dim3(kThreads),
                           0, s, anchors, n, steps, flags, ref4, qry4, wp, list1, cnt);
    launch_stage2(narrow, false, anchors, n, flags, ref4, qry4, wp, list1, nullptr, nullptr,
                  list2, cnt, s);
    return hipGetLastError();
}

uint32_t gate_window_steps(uint64_t n) {
    const uint64_t want = (n + 64 * kFillWaves - 1) / (64 * kFillWaves);
    return (uint32_t)std::min<uint64_t>(std::max<uint64_t>(want, 1), kSteps);
}

uint64_t gate_window_waves(uint64_t n) {
    const uint64_t slots = 64ull * gate_window_steps(n);
    return (n + slots - 1) / slots;
}

hipError_t launch_gate_window_fused(bool narrow, const ChunkSeeds &cs, uint32_t n,
                                    uint64_t *anchors, uint8_t *flags, const uint32_t *ref4,
                                    const uint32_t *qry4, const WindowParams &wp,
                                    uint32_t *list1, uint64_t *list1_a, uint32_t *list2,
                                    uint32_t *cnt, hipStream_t s) {
    if (n == 0) {
        hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(1), 0, s, cnt);
        return hipGetLastError();
    }
    const uint32_t steps = gate_window_steps(n);
    const uint32_t n_waves = (uint32_t)gate_window_waves(n);
    hipLaunchKernelGGL(k_slot_dir, dim3((n_waves + kWaves - 1) / kWaves), dim3(kThreads), 0,
                       s, cs, n_waves, steps, cnt);
    const uint32_t blocks = (n_waves + kWaves - 1) / kWaves;
    if (narrow)
        hipLaunchKernelGGL((k_gate_window_fused<kNarrowRight, kNarrowLeft>), dim3(blocks),
                           dim3(kThreads), 0, s, cs, n, steps, anchors, flags, ref4, qry4, wp,
                           list1, list1_a, cnt);
    else
        hipLaunchKernelGGL((k_gate_window_fused<kWideRight, kWideLeft>), dim3(blocks),
                           dim3(kThreads), 0, s, cs, n, steps, anchors, flags, ref4, qry4, wp,
                           list1, list1_a, cnt);
    // its second stage is a launch of its own: small calls (many chunks of about 2^20
    // anchors, often with long walks) leave the first stage too few waves to run it in
    launch_stage2(narrow, false, anchors, n, flags, ref4, qry4, wp, list1, list1_a, anchors,
                  list2, cnt, s);
    return hipGetLastError();
}

hipError_t launch_kg_groups(const KeyGroups &kg, const KgScratch &ks, uint32_t seed_lo,
                            uint32_t seed_hi, hipStream_t s) {
    if (kg.n_runs == 0) return hipSuccess;
    const uint32_t nblk = (kg.n_runs + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(k_kg_groups, dim3(nblk), dim3(kKgThreads), 0, s, kg, seed_lo, seed_hi, ks);
    return launch_scan_blocks(ks.blksum, nblk, ks.blkoff, ks.info, s);
}

hipError_t launch_gate_window_kg(const KeyGroups &kg, const KgScratch &ks,
                                 PrefixView prefix, uint32_t batch_lo, uint32_t seed_lo,
                                 uint32_t seed_hi, uint32_t hit_lo, uint32_t n,
                                 const uint32_t *pos, uint64_t *anchors, uint8_t *flags,
                                 const uint32_t *ref4, const uint32_t *qry4,
                                 const WindowParams &wp, uint32_t *list1, uint64_t *list1_a,
                                 uint32_t *list2, uint32_t *cnt, const ScoreParams &sp,
                                 const uint8_t *ref8, const uint8_t *qry8, bool groups_ready,
                                 bool bits, hipStream_t s) {
    if (n == 0 || kg.n_runs == 0) {
        hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(1), 0, s, cnt);
        return hipGetLastError();
    }
    const uint32_t nr = kg.n_runs;
    hipError_t st;
    if (!groups_ready && (st = launch_kg_groups(kg, ks, seed_lo, seed_hi, s)) != hipSuccess)
        return st;
    const uint32_t steps = gate_window_steps(n);
    const uint32_t n_waves = (uint32_t)gate_window_waves(n);
    hipLaunchKernelGGL(k_kg_dir, dim3((n_waves + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                       ks, nr, n_waves, steps, cnt);
    const uint64_t flag_bytes = bits ? ((uint64_t)n + 31) / 32 * 4 : (uint64_t)n;
    if ((st = launch_zero_bytes(flags, flag_bytes, s)) != hipSuccess) return st;
    const uint32_t blocks = (n_waves + kWaves - 1) / kWaves;
    if (bits)
        hipLaunchKernelGGL((k_gate_window_kg<kWideRight, kWideLeft, true>), dim3(blocks),
                           dim3(kThreads), 0, s, kg, ks, prefix, batch_lo, hit_lo, n, steps, pos,
                           anchors, flags, ref4, qry4, wp, list1, list1_a, cnt, list2, sp, ref8,
                           qry8);
    else
        hipLaunchKernelGGL((k_gate_window_kg<kWideRight, kWideLeft, false>), dim3(blocks),
                           dim3(kThreads), 0, s, kg, ks, prefix, batch_lo, hit_lo, n, steps, pos,
                           anchors, flags, ref4, qry4, wp, list1, list1_a, cnt, list2, sp, ref8,
                           qry8);
    launch_stage2(false, true, anchors, n, flags, ref4, qry4, wp, list1, list1_a, anchors,
                  list2, cnt, s, bits);
    return hipGetLastError();
}

hipError_t launch_gate_window_bucketed(const uint64_t *anchors, uint32_t n, const uint64_t *sa,
                                       const uint32_t *si, uint8_t *flags, const uint32_t *ref4,
                                       const uint32_t *qry4, const WindowParams &wp,
                                       uint32_t *list1, uint32_t *list2, uint32_t *cnt,
                                       hipStream_t s) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(1), 0, s, cnt);
    if (n == 0) return hipGetLastError();
    hipError_t st = launch_zero_bytes(flags, n, s);
    if (st != hipSuccess) return st;
    const uint32_t part = (uint32_t)(((uint64_t)n + 7) / 8);
    const uint32_t steps = gate_window_steps(n);
    const uint64_t per_block = (uint64_t)kWaves * 64 * steps;
    const uint32_t blocks = 8u * (uint32_t)(((uint64_t)part + per_block - 1) / per_block);
    hipLaunchKernelGGL((k_gate_window_bucketed<kWideRight, kWideLeft>), dim3(blocks),
                       dim3(kThreads), 0, s, sa, si, n, part, steps, flags, ref4, qry4, wp,
                       list1, cnt);
    launch_stage2(false, false, anchors, n, flags, ref4, qry4, wp, list1, nullptr, nullptr,
                  list2, cnt, s);
    return hipGetLastError();
}

}  // namespace hspz
