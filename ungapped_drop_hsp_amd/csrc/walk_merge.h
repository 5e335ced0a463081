// The one-wave walk that may merge into a neighbour's, for the diagonal-shared
// materialization ("E. X-drop materialization", E.2-E.3): exact_walk's scan and drop
// test, plus a stop at the first strict new best at or past the neighbour's start.
#pragma once

#include <climits>

#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

// The one-wave walk of exact_walk (64-base tiles, one base per lane) for a walk that may
// merge into a neighbour's: survivors on one diagonal are walked each from its own anchor,
// and wm is the walk index of the neighbour's start (the base just before a right
// neighbour's first base, or the last base before a left neighbour's first base; pass
// UINT32_MAX for no neighbour).  If the walk sets a strictly new best at an index >= wm
// before it drops, it is the neighbour's walk from there on: same later bases, same running
// best, same drop, same earliest best (every base the walk had scored before lies strictly
// below that best).  The walk then stops with merged = true and ds = its running score at
// index wm (0 when wm is past its start already); the caller adds ds to the neighbour's
// best and the anchors' distance to the neighbour's extent.  Otherwise it runs to its drop
// like exact_walk with Ext (merged = false; best and ext are its own).  With ReadAhead
// the next tile's scores are read while a tile is scored; the walk reads at most 127
// bases past the first edge base, inside the padding.
template <int D, bool ReadAhead>
__device__ __forceinline__ void exact_walk_merge(const int32_t *tab, const uint8_t *rp,
                                                 const uint8_t *qp, int32_t xdrop, uint32_t wm,
                                                 int32_t &best_out, uint32_t &ext_out,
                                                 bool &merged, int32_t &ds) {
    const int l = lane_id();
    int32_t best = 0, carry = 0;
    uint32_t ext = 0, base = 0;
    merged = false;
    ds = 0;
    auto score = [&](uint32_t b) {
        const int64_t off = D > 0 ? (int64_t)b + l : -(int64_t)b - 1 - l;
        return tab[rp[off] | qp[off]];
    };
    int32_t sg = score(0);
    for (;;) {
        const int32_t sg_next = ReadAhead ? score(base + 64) : 0;
        const int32_t s = wave_incl_sum(sg) + carry;
        const int32_t run_best = max(wave_incl_max(s), best);
        int32_t prev = __shfl_up(run_best, 1, 64);  // running best before this lane's base
        if (l == 0) prev = best;
        if (wm >= base && wm < base + 64u) ds = lane_value(s, (int)(wm - base));
        const uint64_t dm = __ballot(run_best - s > xdrop);
        const uint64_t mm = __ballot(s > prev && base + (uint32_t)l >= wm);  // strict new best
        const int f = dm ? (int)__builtin_ctzll(dm) : 64;  // first dropping lane
        const int g = mm ? (int)__builtin_ctzll(mm) : 64;  // first merging lane
        if (g < f) {
            merged = true;
            break;
        }
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
        sg = ReadAhead ? sg_next : score(base);
    }
    best_out = best;
    ext_out = ext;
}

// The merge walk over 512-base tiles (eight bases per lane) read from the 4-bit copies,
// with exact_walk_tiles' scan, drop test and deferred extent search, for walks that run
// long (thousands of bases along a tandem array).  Lane l of a tile holds walk positions
// p0 = base + 8l .. p0 + 7.  The walk merges at the first strict new best at a position
// >= wm; such a best exists in a lane iff the largest running score the lane reaches at
// positions >= wm exceeds both the running best before the lane and every running score
// the lane reaches below wm.  In a tile entirely past wm that is simply the lane's
// largest running score against the running best before it.  The walk stops at the
// first lane that merges or drops.  If one lane does both, the lane re-walks its bases
// (as the drop does anyway) and the earlier event wins.  A merged walk returns ds, its
// running score at wm, and no best or extent; otherwise best and ext are exactly
// exact_walk_tiles'.  mr, mq: padded nibble indices of the anchor's first base (right
// walk) or of the base just above its first (left walk).  The next tile is read ahead:
// at most 1,032 nibbles past the first edge base, inside the padding.
template <int D>
__device__ __forceinline__ void exact_walk_tiles_merge(const int32_t *tab4,
                                                       const uint32_t *__restrict__ ref4,
                                                       const uint32_t *__restrict__ qry4,
                                                       uint32_t mr, uint32_t mq, int32_t xdrop,
                                                       uint32_t wm, int32_t &best_out,
                                                       uint32_t &ext_out, bool &merged,
                                                       int32_t &ds) {
    constexpr int PER = 8;
    constexpr uint32_t kTileBases = 64u * PER;
    static_assert(2 * 64 * PER + 8 <= kPad4, "a tile and the one read ahead fit the padding");
    constexpr int32_t kLow = INT32_MIN / 2;  // below every running score
    const int l = lane_id();
    const int32_t glim = INT32_MAX - xdrop;
    int32_t best = 0, carry = 0;
    uint32_t base = 0;
    uint32_t e_base = 0, e_lim = 0;
    int32_t e_carry = 0;
    merged = false;
    ds = 0;
    const uint32_t ar = D > 0 ? mr + PER * l : mr - PER * l - PER;
    const uint32_t aq = D > 0 ? mq + PER * l : mq - PER * l - PER;
    const uint32_t *__restrict__ pr = ref4 + (ar >> 3);
    const uint32_t *__restrict__ pq = qry4 + (aq >> 3);
    const uint32_t shr = (ar & 7u) * 4u, shq = (aq & 7u) * 4u;
    // pair indices r * 16 + q of the lane's eight bases of tile b: nibble k's in byte
    // k / 2 of code[k % 2] (nibbles in address order)
    auto load = [&](uint32_t b, uint32_t (&code)[2]) {
        const uint32_t *wr = D > 0 ? pr + (b >> 3) : pr - (b >> 3);
        const uint32_t *wq = D > 0 ? pq + (b >> 3) : pq - (b >> 3);
        const uint32_t R = __builtin_amdgcn_alignbit(wr[1], wr[0], shr);
        const uint32_t Q = __builtin_amdgcn_alignbit(wq[1], wq[0], shq);
        const uint32_t hi = 0xF0F0F0F0u;
        code[0] = ((R << 4) & hi) | (Q & ~hi);
        code[1] = (R & hi) | ((Q >> 4) & ~hi);
    };
    auto scores = [&](const uint32_t (&code)[2], int32_t (&sg)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const int k = D > 0 ? j : PER - 1 - j;  // the nibble of walk position j
            sg[j] = tab4[(code[k & 1] >> (8 * (k >> 1))) & 0xFFu];
        }
    };
    uint32_t cur[2];
    load(0, cur);
    for (;;) {
        uint32_t nxt[2];
        load(base + kTileBases, nxt);
        int32_t sg[PER];
        scores(cur, sg);
        int32_t acc = 0, mx = kLow;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            acc += sg[j];
            mx = max(mx, acc);
        }
        const int32_t incl = wave_incl_sum(acc);
        const int32_t C = carry + incl - acc;  // running score before this lane
        const int32_t run_max = wave_incl_max(C + mx);
        int32_t prev_max = __shfl_up(run_max, 1, 64);
        if (l == 0) prev_max = kLow;
        const int32_t before = max(best, prev_max);  // running best before this lane
        int32_t g = INT32_MAX - (before - C), gmin = g;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            g = __builtin_elementwise_add_sat(g, sg[j]);
            gmin = min(gmin, g);
        }
        const uint64_t dl = __ballot(gmin < glim);
        // lanes holding a strict new best at a position >= wm
        const uint32_t p0 = base + (uint32_t)(PER * l);
        bool mlane;
        if (wm < base) {
            mlane = C + mx > before;
        } else if (wm < base + kTileBases) {  // the tile of wm (uniform)
            int32_t sc = C, pre = before, post = kLow, dsv = 0;
#pragma unroll
            for (int j = 0; j < PER; j++) {
                sc += sg[j];
                const uint32_t p = p0 + (uint32_t)j;
                if (p < wm) pre = max(pre, sc);
                else post = max(post, sc);
                dsv = p == wm ? sc : dsv;
            }
            mlane = post > pre;
            ds = lane_value(dsv, (int)((wm - base) / PER));
        } else {
            mlane = false;
        }
        const uint64_t mm = __ballot(mlane);
        const int f = dl ? (int)__builtin_ctzll(dl) : 64;  // first dropping lane
        const int gm = mm ? (int)__builtin_ctzll(mm) : 64;  // first merging lane
        int32_t tb;
        uint32_t lim = kTileBases;
        if (dl || mm) {
            // every lane re-walks its bases: the first drop, the running best before it,
            // and the first strict new best at a position >= wm
            int32_t sc = C, rbv = before, tbl = before;
            int fj = PER, mj = PER;
#pragma unroll
            for (int j = 0; j < PER; j++) {
                sc += sg[j];
                const bool nb = sc > rbv && p0 + (uint32_t)j >= wm;
                mj = (mj == PER && nb) ? j : mj;
                rbv = max(rbv, sc);
                const bool first = fj == PER && rbv - sc > xdrop;
                fj = first ? j : fj;
                tbl = first ? rbv : tbl;
            }
            if (gm < f || (gm == f && lane_value(mj, gm) < lane_value(fj, f))) {
                merged = true;
                break;
            }
            lim = (uint32_t)(PER * f + lane_value(fj, f));
            tb = lane_value(tbl, f);
        } else {
            tb = max(best, lane_value(run_max, 63));
        }
        if (tb > best) {
            best = tb;
            e_base = base;
            e_carry = carry;
            e_lim = lim;
        }
        if (dl) break;
        carry += lane_value(incl, 63);
        base += kTileBases;
        cur[0] = nxt[0];
        cur[1] = nxt[1];
    }
    uint32_t ext = 0;
    if (!merged && best > 0) {
        // the first base of the noted tile, before its drop, whose running score is best
        uint32_t code[2];
        load(e_base, code);
        int32_t sg[PER];
        scores(code, sg);
        int32_t acc = 0;
#pragma unroll
        for (int j = 0; j < PER; j++) acc += sg[j];
        const int32_t C = e_carry + wave_incl_sum(acc) - acc;
        int32_t sc = C;
        int gj = PER;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            sc += sg[j];
            gj = (gj == PER && sc == best && (uint32_t)(PER * l + j) < e_lim) ? j : gj;
        }
        const uint64_t hit = __ballot(gj < PER);
        const int gl = (int)__builtin_ctzll(hit);
        ext = e_base + (uint32_t)(PER * gl + lane_value(gj, gl)) + 1u;
    }
    best_out = merged ? 0 : best;
    ext_out = ext;
}

}  // namespace hspz
