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

// The same walk with PER bases per lane (64 * PER-base tiles): lane l scores walk
// positions base + PER*l .. base + PER*l + PER - 1.  Each lane forms its bases' local
// prefix sums and prefix maxima; wave scans of the lane totals and of the lane maxima
// (relative to the tile) give every base its running score and running best, so a base
// drops when its running best exceeds its score by more than xdrop.  The first drop is
// the lowest (lane, base) that drops; the best before it is the running best of the base
// just before it, and with Ext its extent is the first base of the tile whose score equals
// that best (a later base of the tile, past the drop, never counts).  With ReadAhead the
// next tile's bases are read while this one is scored.  The walk reads at most
// 64 * PER * (ReadAhead ? 2 : 1) - 1 bases past the first edge base, inside the padding.
template <int D, bool Ext, int PER, bool ReadAhead>
__device__ __forceinline__ void exact_walk_tiles(const int32_t *tab, const uint8_t *rp,
                                                 const uint8_t *qp, int32_t xdrop, int32_t stop,
                                                 int32_t &best_out, uint32_t &ext_out) {
    static_assert(PER >= 1 && 64 * PER * (ReadAhead ? 2 : 1) <= kPad,
                  "a tile (and the one read ahead) must fit the edge padding");
    constexpr int32_t kLow = INT32_MIN / 2;  // below every running best (bests are >= 0)
    const int l = lane_id();
    int32_t best = 0, carry = 0;
    uint32_t ext = 0, base = 0;
    auto load = [&](uint32_t b, uint32_t (&code)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const int64_t w = (int64_t)b + PER * l + j;  // walk position
            const int64_t off = D > 0 ? w : -w - 1;
            code[j] = rp[off] | qp[off];
        }
    };
    uint32_t cur[PER];
    load(0, cur);
    for (;;) {
        uint32_t nxt[PER];
        if (ReadAhead) load(base + 64u * PER, nxt);
        int32_t p[PER], m[PER];
        int32_t acc = 0, mx = kLow;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            acc += tab[cur[j]];
            p[j] = acc;
            mx = max(mx, acc);
            m[j] = mx;
        }
        const int32_t incl = wave_incl_sum(acc);  // tile score through this lane
        const int32_t S = incl - acc;             // tile score before this lane
        const int32_t lane_max = wave_incl_max(S + m[PER - 1]);
        int32_t prev_max = __shfl_up(lane_max, 1, 64);  // best of the tile's earlier lanes
        if (l == 0) prev_max = kLow;
        const int32_t before = max(best, carry + prev_max);  // running best before this lane
        int32_t sj[PER], rb[PER];
        int fj = PER;  // this lane's first dropping base (PER: none)
#pragma unroll
        for (int j = PER - 1; j >= 0; j--) {
            sj[j] = carry + S + p[j];
            rb[j] = max(before, carry + S + m[j]);
            if (rb[j] - sj[j] > xdrop) fj = j;
        }
        const uint64_t dl = __ballot(fj < PER);
        int32_t tb;        // running best before the first drop, or at the tile's end
        uint32_t limit;    // positions of the tile that count: [0, limit)
        if (dl) {
            const int f = (int)__builtin_ctzll(dl);
            const int ff = lane_value(fj, f);
            // running best of the base before the drop: in lane f, or lane f - 1's last
            int32_t rb_prev = rb[PER - 1];
#pragma unroll
            for (int j = 1; j < PER; j++)
                if (fj == j) rb_prev = rb[j - 1];
            if (ff > 0) tb = lane_value(rb_prev, f);
            else if (f > 0) tb = lane_value(rb[PER - 1], f - 1);
            else tb = best;
            limit = (uint32_t)(PER * f + ff);
        } else {
            tb = max(best, carry + lane_value(lane_max, 63));
            limit = 64u * PER;
        }
        if (tb > best) {
            if (Ext) {
                int gj = PER;  // this lane's first base reaching tb inside the limit
#pragma unroll
                for (int j = PER - 1; j >= 0; j--)
                    if (sj[j] == tb && (uint32_t)(PER * l + j) < limit) gj = j;
                const uint64_t gl = __ballot(gj < PER);
                const int g = (int)__builtin_ctzll(gl);
                ext = base + (uint32_t)(PER * g + lane_value(gj, g)) + 1u;
            }
            best = tb;
        }
        if (dl || best >= stop) break;
        carry += lane_value(incl, 63);
        base += 64u * PER;
        if (ReadAhead) {
#pragma unroll
            for (int j = 0; j < PER; j++) cur[j] = nxt[j];
        } else {
            load(base, cur);
        }
    }
    best_out = best;
    ext_out = ext;
}

}  // namespace hspz
