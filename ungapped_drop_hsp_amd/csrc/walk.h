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

// The same walk with PER (8 or 16) bases per lane (64 * PER-base tiles), read from the
// 4-bit copies: lane l scores walk positions base + PER*l .. base + PER*l + PER - 1, PER / 8
// funnel-shifted dwords of each sequence (a right walk takes its nibbles in address
// order, a left walk in reverse), and looks each pair up in tab4[r * 16 + q].
//  - Each lane sums its bases' pair scores (kept in registers) and takes the maximum of
//    its local prefix sums; wave scans of the lane sums and of the lane maxima (offset by
//    the sums before the lane) give each lane its running score and running best at its
//    first base.
//  - A lane holds a drop iff its running drawdown, started from (running best - running
//    score) at its first base, exceeds xdrop at one of its bases.  The drawdown is carried
//    complemented, g = INT32_MAX - d, so that max(d - sigma, 0) is one saturating add.
//  - Only in the tile of the first drop, the lowest dropping lane re-walks its bases to
//    find the dropping base and the running best just before it (a dropping base never
//    raises the best, since its score lies more than xdrop below it).
//  - With Ext the extent is the first base whose running score equals the final best.
//    Every earlier tile's scores stay below that best, so the base lies in the last tile
//    that raised the best, before that tile's drop if it has one: the walk notes that
//    tile, and after the walk reads it again and searches it once.
// mr and mq are the padded nibble indices of the anchor's bases (reference end r at
// kPad4 + r): a right walk starts there, a left walk just below.  With ReadAhead the next
// tile's bases are read while this one is scored.  The walk reads at most
// 64 * PER * (ReadAhead ? 2 : 1) + 7 bases past the first edge base, inside the padding.
template <int D, bool Ext, int PER, bool ReadAhead>
__device__ __forceinline__ void exact_walk_tiles(const int32_t *tab4,
                                                 const uint32_t *__restrict__ ref4,
                                                 const uint32_t *__restrict__ qry4, uint32_t mr,
                                                 uint32_t mq, int32_t xdrop, int32_t stop,
                                                 int32_t &best_out, uint32_t &ext_out) {
    static_assert(PER == 8 || PER == 16, "whole dwords of nibbles per lane");
    constexpr int NW = PER / 8;  // dwords of each sequence per lane
    static_assert(64 * PER * (ReadAhead ? 2 : 1) + 8 <= kPad4,
                  "a tile (and the one read ahead) must fit the edge padding");
    constexpr int32_t kLow = INT32_MIN / 2;  // below every running best (bests are >= 0)
    const int l = lane_id();
    const int32_t glim = INT32_MAX - xdrop;  // a drop once the complemented drawdown < glim
    int32_t best = 0, carry = 0;
    uint32_t base = 0;
    // the last tile that raised the best: its first walk position, the running score before
    // it, and the positions of it that count (those before its drop)
    uint32_t e_base = 0, e_lim = 0;
    int32_t e_carry = 0;
    // The lane's PER nibbles of one sequence in tile b, dword i holding nibbles 8i .. 8i + 7:
    // their lowest padded nibble index is a0 + b for a right walk and a0 - b for a left one,
    // with a0 = m + PER*l or m - PER*l - PER.  Tiles are whole dwords apart, so the funnel
    // shift (a0 % 8 nibbles) and the lane's first dword are set once per walk.
    const uint32_t ar = D > 0 ? mr + PER * l : mr - PER * l - PER;
    const uint32_t aq = D > 0 ? mq + PER * l : mq - PER * l - PER;
    const uint32_t *__restrict__ pr = ref4 + (ar >> 3);
    const uint32_t *__restrict__ pq = qry4 + (aq >> 3);
    const uint32_t shr = (ar & 7u) * 4u, shq = (aq & 7u) * 4u;
    auto nibs = [&](const uint32_t *__restrict__ p0, uint32_t sh, uint32_t b, uint32_t (&v)[NW]) {
        const uint32_t *w = D > 0 ? p0 + (b >> 3) : p0 - (b >> 3);
        uint32_t x[NW + 1];
#pragma unroll
        for (int i = 0; i <= NW; i++) x[i] = w[i];
#pragma unroll
        for (int i = 0; i < NW; i++) v[i] = __builtin_amdgcn_alignbit(x[i + 1], x[i], sh);
    };
    // pair indices r * 16 + q of the lane's nibbles: nibble k's in byte (k % 8) / 2 of
    // code[2 * (k / 8) + k % 2]
    auto load = [&](uint32_t b, uint32_t (&code)[2 * NW]) {
        uint32_t R[NW], Q[NW];
        nibs(pr, shr, b, R);
        nibs(pq, shq, b, Q);
        const uint32_t hi = 0xF0F0F0F0u;
#pragma unroll
        for (int i = 0; i < NW; i++) {
            code[2 * i] = ((R[i] << 4) & hi) | (Q[i] & ~hi);
            code[2 * i + 1] = (R[i] & hi) | ((Q[i] >> 4) & ~hi);
        }
    };
    // the pair scores of the lane's bases in walk order
    auto scores = [&](uint32_t (&code)[2 * NW], int32_t (&sg)[PER]) {
        // keep the index words whole: each table address is one byte-select shift of them
#pragma unroll
        for (int i = 0; i < 2 * NW; i++) asm volatile("" : "+v"(code[i]));
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const int k = D > 0 ? j : PER - 1 - j;  // the nibble of walk position j
            const uint32_t word = code[2 * (k >> 3) + (k & 1)];
            sg[j] = tab4[(word >> (8 * ((k & 7) >> 1))) & 0xFFu];
        }
    };
    uint32_t cur[2 * NW];
    load(0, cur);
    for (;;) {
        uint32_t nxt[2 * NW];
        if (ReadAhead) load(base + 64u * PER, nxt);
        int32_t sg[PER];
        scores(cur, sg);
        int32_t acc = 0, mx = kLow;  // local sum, and maximum of the local prefix sums
#pragma unroll
        for (int j = 0; j < PER; j++) {
            acc += sg[j];
            mx = max(mx, acc);
        }
        const int32_t incl = wave_incl_sum(acc);  // tile score through this lane
        const int32_t C = carry + incl - acc;     // running score before this lane
        const int32_t run_max = wave_incl_max(C + mx);
        int32_t prev_max = __shfl_up(run_max, 1, 64);  // best of the tile's earlier lanes
        if (l == 0) prev_max = kLow;
        const int32_t before = max(best, prev_max);  // running best before this lane
        // the drawdown walk of this lane's bases, from before - C
        int32_t g = INT32_MAX - (before - C), gmin = g;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            g = __builtin_elementwise_add_sat(g, sg[j]);
            gmin = min(gmin, g);
        }
        const uint64_t dl = __ballot(gmin < glim);
        int32_t tb;              // running best before the first drop, or at the tile's end
        uint32_t lim = 64u * PER;  // positions of the tile before its drop
        if (dl) {
            const int f = (int)__builtin_ctzll(dl);
            // every lane re-walks its bases; the dropping lane's results are taken
            int32_t sc = C, rbv = before, tbl = before;
            int fj = PER;
#pragma unroll
            for (int j = 0; j < PER; j++) {
                sc += sg[j];
                rbv = max(rbv, sc);
                const bool first = fj == PER && rbv - sc > xdrop;
                fj = first ? j : fj;
                tbl = first ? rbv : tbl;
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
        if (dl || best >= stop) break;
        carry += lane_value(incl, 63);
        base += 64u * PER;
        if (ReadAhead) {
#pragma unroll
            for (int i = 0; i < 2 * NW; i++) cur[i] = nxt[i];
        } else {
            load(base, cur);
        }
    }
    uint32_t ext = 0;
    if (Ext && best > 0) {
        // the first base of the noted tile, before its drop, whose running score is best
        uint32_t code[2 * NW];
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
    best_out = best;
    ext_out = ext;
}

}  // namespace hspz
