// Diagonal-shared materialization ("E. X-drop materialization", E.1-E.5): the kernels in
// k_materialize.hip, sequenced by the engine (sort keys, a stable radix sort by reference
// end then by diagonal, the walks, scans of their results, the records), and the
// engine's scratch for them.  Per-side walk results live in sorted order.
#pragma once

#include "hspz_internal.h"

namespace hspz {

// Scratch for cap survivors: sort keys and values (ping-pong), radix digit counts and
// their scan, both sides' results (carved out of one allocation), the block sums and
// offsets of its scans, and the lane stage's list of open walks.
struct MatScratch {
    uint32_t *ka = nullptr, *va = nullptr, *kb = nullptr, *vb = nullptr;
    uint32_t *hist = nullptr, *incl = nullptr;
    uint32_t *side = nullptr;
    uint64_t *sum = nullptr;
    uint32_t *off = nullptr;
    PlanInfo *info = nullptr;
    uint32_t *list = nullptr;  // walks the lane stage left open (2 * cap)
    uint32_t *lcnt = nullptr;  // their counts, right and left
    uint64_t *sa = nullptr;    // the anchors in sorted order
    uint32_t *sblk = nullptr;  // the side scan's block totals (4 per block)
    uint64_t cap = 0;
};

struct MatSide {
    int32_t *best;
    uint32_t *ext;
    uint32_t *term;   // 1: the walk ran to its drop; 0: it merged into its neighbour's
    int32_t *ds;      // its running score at the neighbour's start (0 if it ran to its drop)
    uint32_t *cnt;    // inclusive scan of term
    uint32_t *sum;    // inclusive scan of ds, modulo 2^32
    uint32_t *pos;    // sorted positions of the walks that ran to their drops
};
hipError_t launch_mm_keys(const uint64_t *anchors, const uint32_t *ids, uint32_t n,
                          uint32_t n_ref, uint32_t n_qry, uint32_t *key_r, uint32_t *val,
                          uint32_t *lcnt, hipStream_t s);
hipError_t launch_mm_diag(const uint64_t *anchors, const uint32_t *ids, const uint32_t *val,
                          uint32_t n, uint32_t n_ref, uint32_t n_qry, uint32_t *key_d,
                          hipStream_t s);
// The walks: with lanes, a lane stage over eight-base blocks (exact only when
// 7 * (largest pair score) <= xdrop) plus one wave per walk it left open, listed in list
// (2 * n entries) with counts in lcnt (cleared by launch_mm_keys); else one wave per
// survivor.
// sa[s] = anchors[ids[val[s]]]: the anchors in sorted order, for the walks and records.
hipError_t launch_mm_gather(const uint64_t *anchors, const uint32_t *ids, const uint32_t *val,
                            uint32_t n, uint64_t *sa, hipStream_t s);
hipError_t launch_mm_walk(const uint64_t *sa, const uint32_t *key_d, uint32_t n,
                          const uint8_t *ref,
                          const uint8_t *qry, const uint32_t *ref4, const uint32_t *qry4,
                          const ScoreParams &sp, const MatSide &right, const MatSide &left,
                          bool lanes, uint32_t *list, uint32_t *lcnt, hipStream_t s);
// Both sides' cnt, sum and pos from term and ds in one scan; blk holds
// 4 * mm_scan_blocks(n) words.  Every array of a side must be 16-byte aligned.
uint32_t mm_scan_blocks(uint32_t n);
hipError_t launch_mm_scan(const MatSide &right, const MatSide &left, uint32_t n, uint32_t *blk,
                          hipStream_t s);
hipError_t launch_mm_finish(const uint64_t *sa, const uint32_t *val,
                            uint32_t n, const MatSide &right, const MatSide &left,
                            hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                            const ScoreParams &sp, hipStream_t s);

}  // namespace hspz
