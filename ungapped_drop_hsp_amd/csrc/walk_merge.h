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
// like exact_walk with Ext (merged = false; best and ext are its own).  The scores of
// the next Ahead tiles are read while a tile is scored, so that a long walk does not wait
// on memory at every tile; the walk reads at most 64 * (Ahead + 1) + 63 bases past the
// first edge base, inside the padding.
template <int D, int Ahead>
__device__ __forceinline__ void exact_walk_merge(const int32_t *tab, const uint8_t *rp,
                                                 const uint8_t *qp, int32_t xdrop, uint32_t wm,
                                                 int32_t &best_out, uint32_t &ext_out,
                                                 bool &merged, int32_t &ds) {
    static_assert(Ahead >= 0 && 64 * (Ahead + 1) + 64 <= kPad,
                  "the tiles read ahead must stay inside the edge padding");
    const int l = lane_id();
    int32_t best = 0, carry = 0;
    uint32_t ext = 0, base = 0;
    merged = false;
    ds = 0;
    auto score = [&](uint32_t b) {
        const int64_t off = D > 0 ? (int64_t)b + l : -(int64_t)b - 1 - l;
        return tab[rp[off] | qp[off]];
    };
    int32_t ring[Ahead + 1];  // ring[a]: the scores of tile base + 64 a
#pragma unroll
    for (int a = 0; a <= Ahead; a++) ring[a] = score(64u * (uint32_t)a);
    for (;;) {
        const int32_t sg = ring[0];
#pragma unroll
        for (int a = 0; a < Ahead; a++) ring[a] = ring[a + 1];
        if (Ahead > 0) ring[Ahead] = score(base + 64u * (uint32_t)(Ahead + 1));
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
        if (Ahead == 0) ring[0] = score(base);
    }
    best_out = best;
    ext_out = ext;
}

}  // namespace hspz
