// One-wave exact X-drop walk over 64-base tiles ("E. X-drop materialization", E.2-E.3;
// the same walk decides the score gate's longest cases, "D. Score gate", D.1-D.2).
//
// Lane i scores base base + i of the tile; an inclusive wave scan (DPP) gives the running
// score, a prefix maximum seeded with the best so far gives the running best, and a
// ballot of lanes whose drawdown exceeds xdrop marks the first drop.  The running best in
// the lane before the first drop is the tile's best; with Ext its extent is the lowest
// lane attaining it, so an equal later maximum never moves the endpoint.  The walk also
// ends once best >= stop (the caller's decision is then known; pass INT32_MAX to walk to
// the drop).  Bases outside a sequence are edge codes scoring -(xdrop + 1), so a walk
// ends within the first tile that reaches an edge; the padding (kPad bytes) holds that
// tile and the one read ahead of it.
#pragma once

#include <climits>

#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

template <int D, bool Ext, bool ReadAhead>
__device__ __forceinline__ void exact_walk(const int32_t *tab, const uint8_t *rp,
                                           const uint8_t *qp, int32_t xdrop, int32_t stop,
                                           int32_t &best_out, uint32_t &ext_out) {
    const int l = lane_id();
    int32_t best = 0, carry = 0;
    uint32_t ext = 0, base = 0;
    auto score = [&](uint32_t b) {
        const int64_t off = D > 0 ? (int64_t)b + l : -(int64_t)b - 1 - l;
        return tab[rp[off] | qp[off]];
    };
    int32_t sg = score(0);
    for (;;) {
        // with ReadAhead the next tile's scores are read while this one is scored (long
        // walks); a walk reaching an edge drops inside the tile that holds it, so this
        // reads at most 127 bases past the first edge base, inside the padding
        const int32_t sg_next = ReadAhead ? score(base + 64) : 0;
        const int32_t s = wave_incl_sum(sg) + carry;
        // running best including every base up to this lane (and the tiles before)
        const int32_t run_best = max(wave_incl_max(s), best);
        const uint64_t dm = __ballot(run_best - s > xdrop);
        const int f = dm ? (int)__builtin_ctzll(dm) : 64;  // first dropping lane
        if (f > 0) {
            const int32_t tb = lane_value(run_best, f - 1);  // best before the drop
            if (tb > best) {
                if (Ext) {
                    const uint64_t at = __ballot(l < f && s == tb);
                    ext = base + (uint32_t)__builtin_ctzll(at) + 1u;
                }
                best = tb;
            }
        }
        if (dm || best >= stop) break;
        carry = lane_value(s, 63);
        base += 64;
        sg = ReadAhead ? sg_next : score(base);
    }
    best_out = best;
    ext_out = ext;
}

}  // namespace hspz
