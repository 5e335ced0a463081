// Internal declarations of libhspz: device data layout, score constants and the kernel
// launchers (the engine's state is in engine.h).  Nothing here is part of the C ABI
// (include/hspz.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "hspz.h"

namespace hspz {

// ---- device layout -----------------------------------------------------------------
// Sequences live on the device one byte per base, padded on both sides with kPad
// "edge" bytes (more than the byte-reading walks, the gate's exact ones and the walk-step
// count, read past a sequence end: a 64-base tile and the one read ahead).  A reference byte holds code*8 and a query byte holds code, so
// OR-ing a reference byte with a query byte gives the pair index ref*8 + query (0..45)
// into the score table.  Codes: A,C,G,T = 0..3, N = 4, edge (outside the sequence) = 5.
constexpr int kPad = 1024;
constexpr uint8_t kCodeN = 4;
constexpr uint8_t kCodeEdge = 5;
constexpr int kRefShift = 3;
constexpr int kTabSize = 64;

// 4-bit copy of each sequence for the windowed score gate: eight bases per dword, the
// base at padded nibble index m in dword m / 8, bits 4 * (m % 8).  Base b sits at padded
// nibble b + kPad4; kPad4 edge nibbles precede and follow the sequence.  Codes are the
// unshifted ones above on both sequences (A,C,G,T = 0..3, N = 4, edge = 5).  Each copy
// is followed, at the next 128-byte boundary, by its twin: twin dword j holds copy dword
// j + kTwinShift.  A window of at most 16 dwords starting at copy dword m lies inside one
// 128-byte line of the copy when m % 32 <= 16, and of the twin otherwise.  The padding
// also holds the materializer's tile of 512 bases, the one it reads ahead and the dword
// its funnel shift reads past them.
constexpr int kPad4 = 1152;
constexpr int kTwinShift = 16;

// Seeds per block of the device prefix scan.
constexpr int kScanBlock = 1024;
// Flag bytes per block of the compaction kernels.
constexpr int kCompactBlock = 8192;

// Score table and gate constants, passed by value to the X-drop kernels.  tab[ref*8 +
// query] is the substitution score; any pair with N scores n_score; any pair with an
// edge byte scores -(xdrop + 1), which ends a walk exactly where the sequence ends.
struct ScoreParams {
    int32_t tab[kTabSize];
    int32_t xdrop;
    int32_t T;
    uint32_t n_ref;
    uint32_t n_qry;
    int32_t K;             // hsp_threshold, for the entropy-adjusted decision
    int32_t entropy_mode;  // 0 = accept iff score >= T; 1 = also score * H >= 2K
};

// Constants of the windowed gate.  tab[r * 16 + q] is the 16-bit pair score for codes
// r, q in 0..5 (edge pairs score -(xdrop + 1)); the window path is used only when every
// entry fits 16 bits and blocks of eight bases are exact (7 * max score <= xdrop).
constexpr int kWinTab = 96;
struct WindowParams {
    int16_t tab[kWinTab];
    int32_t xdrop;
    int32_t T;
    uint32_t n_ref;
    uint32_t n_qry;
    // dword offset of each 4-bit copy's line-split twin (the same codes 64 bytes earlier)
    uint32_t ref4_alt;
    uint32_t qry4_alt;
};

// Spaced seed: care offsets within the window (first care position most significant).
struct SeedShape {
    int32_t care[16];
    int32_t weight;
};

// ---- launchers (kernels in k_*.hip) --------------------------------------------------
// Device seeder and indexer (k_seed.hip).
hipError_t launch_encode(const uint8_t *ascii, uint64_t n, int strand, uint8_t *bytes, int shift,
                         uint32_t *nibbles, uint64_t nibble_words, hipStream_t s);
hipError_t launch_window_keys(const uint8_t *codes, int shift, uint64_t nw, const SeedShape &sh,
                              uint8_t *valid, uint32_t *key, hipStream_t s);
hipError_t launch_gather_pairs(const uint32_t *pos, uint32_t count, const uint32_t *key,
                               uint32_t span, uint32_t *key_out, uint32_t *end_out,
                               hipStream_t s);
hipError_t launch_key_hist(const uint32_t *key, uint32_t n, uint32_t *cnt, hipStream_t s);
hipError_t launch_set_u32(uint32_t *p, uint32_t v, hipStream_t s);
uint32_t radix_blocks(uint32_t n);
hipError_t launch_radix_hist(const uint32_t *key, uint32_t n, int shift, uint32_t *hist,
                             hipStream_t s);
hipError_t launch_radix_scatter(const uint32_t *key_in, const uint32_t *val_in, uint32_t n,
                                int shift, const uint32_t *incl, const uint32_t *hist,
                                uint32_t *key_out, uint32_t *val_out, hipStream_t s);

// Packed count table: 32-byte records (two uint4) of kCountTableKeys consecutive keys, the
// first key's bucket start then one count byte per key; records with a count over 254 are
// marked and their keys read from the full table.  count_table_records(nb) records cover
// keys 0 .. nb - 1; launch_count_table builds them from the cumulative ends end_tbl[0..nb].
constexpr uint32_t kCountTableKeys = 28;
uint32_t count_table_records(uint64_t nb);
hipError_t launch_count_table(const uint32_t *end_tbl, uint64_t nb, uint4 *ctab, hipStream_t s);
// 4-bit count table: count_nibble_words(nb) dwords, key k's count (capped at 15) in bits
// 4 (k % 8) .. of dword k / 8; launch_count_nibbles builds it from end_tbl[0..nb].
uint64_t count_nibble_words(uint64_t nb);
hipError_t launch_count_nibbles(const uint32_t *end_tbl, uint64_t nb, uint32_t *cnib,
                                hipStream_t s);
// Per seed: hit count, bucket start (first, when kmer is given) and block-local
// inclusive prefix; one 64-bit sum per kScanBlock seeds into blksum.  With kmer, counts
// and starts come from ctab (the packed table) when it is given, else from end_tbl.
// count, first, prefix and blksum may each be null: that output is not written.
hipError_t launch_count_scan(const uint32_t *kmer, const uint32_t *counts_in, uint64_t n,
                             const uint32_t *end_tbl, const uint4 *ctab, uint32_t *count,
                             uint32_t *first, uint32_t *prefix, uint64_t *blksum,
                             hipStream_t s);
// The plan's form of it: block-local inclusive prefix and block sums only, each seed's
// count read from the 4-bit table (end_tbl for counts of 15 or more).
hipError_t launch_count_prefix(const uint32_t *kmer, uint64_t n, const uint32_t *end_tbl,
                               const uint32_t *cnib, uint32_t *prefix, uint64_t *blksum,
                               hipStream_t s);
hipError_t launch_add_offsets(uint32_t *prefix, uint64_t n, const uint32_t *blkoff,
                              hipStream_t s);

// Plan results the device writes for one copy back: the batch total (64 bits, so a
// total over 2^32 - 1 is seen and refused) and the MAX_HITS chunk list.
constexpr uint32_t kChunkCap = 1024;
struct PlanInfo {
    uint64_t total;
    uint32_t n_chunks;  // kChunkCap + 1: the list did not fit (the host walks instead)
    uint32_t pad;
};
struct PlanBuf {
    PlanInfo info;
    hspz_chunk chunks[kChunkCap];
};
// Exclusive 64-bit scan of nblk block sums in one workgroup: blkoff[b] (32 bits, the
// offset to add to block b) and info->total.
hipError_t launch_scan_blocks(const uint64_t *blksum, uint64_t nblk, uint32_t *blkoff,
                              PlanInfo *info, hipStream_t s);
// The batch's inclusive prefix as the plan leaves it: block-local inclusive prefixes of
// kScanBlock seeds (count_scan) and each block's exclusive offset (launch_scan_blocks),
// added where a prefix is read instead of in a pass over the whole prefix.  at(i) is the
// global inclusive prefix of seed base + i of the batch, for p = the local prefixes from
// seed base on.
struct PrefixView {
    const uint32_t *p;
    const uint32_t *blkoff;
    uint32_t base;
    __device__ __forceinline__ uint32_t at(uint64_t i) const {
        return p[i] + blkoff[((uint64_t)base + i) / kScanBlock];
    }
};
// Greedy MAX_HITS walk over the inclusive prefix P[0..n) ("C. Hit discovery", C.3) by one
// wave; chunk seed indices are offset by batch_lo.  Reads info->total and writes
// buf->info.n_chunks and up to kChunkCap chunks.
hipError_t launch_chunk_walk(PrefixView P, uint64_t n, uint64_t max_hits, uint64_t batch_lo,
                             PlanBuf *buf, hipStream_t s);
// Expand the seeds of one chunk (count, first, prefix and q_end of its seeds).
hipError_t launch_expand(bool dense, const uint32_t *count, const uint32_t *first,
                         const uint32_t *q_end, PrefixView prefix, uint64_t n_seeds,
                         const uint32_t *pos, uint32_t hit_lo, uint64_t *anchors,
                         hipStream_t s);
hipError_t launch_gate(int block_bases, const uint64_t *anchors, uint32_t n, uint8_t *flags,
                       const uint8_t *ref, const uint8_t *qry, const ScoreParams &sp,
                       hipStream_t s);
// Windowed gate in two stages.  Stage 1 decides every anchor whose walks end within its
// window (48 bases right of the anchor and 72 left, or 32 and 56 when narrow) and lists
// the others in list1; stage 2 decides those with 64 and 96 bases and lists the rest in
// list2 (counts cnt[0], cnt[1]; the launcher clears both first).  launch_gate_list_wave
// then decides list2 exactly, one wave per listed anchor.
hipError_t launch_gate_window(bool narrow, const uint64_t *anchors, uint32_t n, uint8_t *flags,
                              const uint32_t *ref4, const uint32_t *qry4, const WindowParams &wp,
                              uint32_t *list1, uint32_t *list2, uint32_t *cnt, hipStream_t s);
// The seeds of one chunk, for the first gate stage fused with the expansion: their
// inclusive prefix (batch numbering, so prefix - hit_lo runs from 0 to the chunk's hits),
// bucket starts and query ends, the index bucket array, and the directory of the seed
// that owns the first slot of each wave's range (filled by the launcher).
struct ChunkSeeds {
    PrefixView prefix;
    const uint32_t *first;
    const uint32_t *q_end;
    const uint32_t *pos;
    uint32_t *dir;
    uint32_t n_seeds;
    uint32_t hit_lo;
};
// 64-slot steps per wave of the first window stage for a call of n anchors (fewer for
// small calls, so that the grid still fills the GPU), and the number of waves that gives
// (the entries of the fused stage's directory).
uint32_t gate_window_steps(uint64_t n);
uint64_t gate_window_waves(uint64_t n);
// As launch_gate_window, but the first stage builds each anchor from the chunk's seeds
// (occurrence j of seed s at slot prefix[s] - 1 - hit_lo - j, "C. Hit discovery", C.5)
// instead of reading it.  A deferred slot's anchor goes into list1_a (list1's capacity)
// beside its index in list1, and the second stage reads it there; anchors[i] receives the
// anchor of every slot whose flag is 1 and of every slot listed in list2 (what the exact
// list and the materializer read).  cs.dir holds gate_window_waves(n) entries.
hipError_t launch_gate_window_fused(bool narrow, const ChunkSeeds &cs, uint32_t n,
                                    uint64_t *anchors, uint8_t *flags, const uint32_t *ref4,
                                    const uint32_t *qry4, const WindowParams &wp,
                                    uint32_t *list1, uint64_t *list1_a, uint32_t *list2,
                                    uint32_t *cnt, hipStream_t s);
// Key-grouped first stage (gate_mode 5, and gate_mode 0 for ranges of seeds holding a
// large share of the strand's seeds).  The query strand's seeds are kept grouped by k-mer (built when
// the query is uploaded): qs lists the seed indices ordered by k-mer and, within a k-mer,
// ascending; qe their query ends; run_span each k-mer run's range in qs and its first and
// last seed; run_c and run_first the k-mer's reference bucket (size and start), set once
// a reference is there.
// A range's anchors (a chunk, or a whole batch) are then enumerated run by run: the
// range's seeds of a k-mer (a contiguous stretch of its run) times the k-mer's bucket, so
// the reference window of each bucket entry and the query window of each seed are read
// once per group instead of once per anchor.  Every anchor still gets its own flag at its
// raw slot.
struct KeyGroups {
    const uint32_t *qs;
    const uint32_t *qe;
    const uint32_t *run_c;
    const uint32_t *run_first;
    const uint4 *run_span;  // each run: its qs range [x, y) and its first and last seed
    uint32_t n_runs;
};
// Per-call scratch of the key-grouped stage, n_runs entries each (dir: one per wave).
struct KgScratch {
    uint32_t *G;       // inclusive prefix of the runs' anchors in the range, within each
                       // kScanBlock runs (plus blkoff[r / kScanBlock] for the range's)
    uint32_t *a;       // index in qs of the run's first seed in the range
    uint32_t *m;       // the run's seeds in the range
    uint32_t *dir;     // per wave: the run owning the wave's first slot
    uint64_t *blksum;  // per kScanBlock runs: their anchors
    uint32_t *blkoff;  // and the exclusive prefix of those
    PlanInfo *info;
};
// Upload side (k_seed.hip): identity values, run-start flags of a sorted key list, the
// query ends in grouped order, and each run's bucket size and start from end_tbl.
hipError_t launch_iota(uint32_t *v, uint32_t n, hipStream_t s);
hipError_t launch_kg_run_flags(const uint32_t *qk, uint32_t n, uint8_t *flag, hipStream_t s);
hipError_t launch_kg_gather(const uint32_t *qs, uint32_t n, const uint32_t *q_end, uint32_t *qe,
                            hipStream_t s);
hipError_t launch_kg_run_info(const uint32_t *qk, const uint32_t *runs, uint32_t n_runs,
                              const uint32_t *end_tbl, uint32_t *run_c, uint32_t *run_first,
                              hipStream_t s);
hipError_t launch_kg_run_span(const uint32_t *qs, uint32_t n, const uint32_t *runs,
                              uint32_t n_runs, uint4 *run_span, hipStream_t s);
// The first window stage of a range of the batch's seeds (seed_lo .. seed_hi, strand
// numbering; its first slot hit_lo; n anchors: a chunk, or the whole batch with hit_lo
// 0), key-grouped, then the second stage as launch_gate_window_fused: flags receives the
// range's flags (zeroed first, then 1 for the anchors kept), list1/list2
// the deferred slots, and list1_a (list1's capacity) the anchors of list1's slots, which
// the second stage reads there instead of at their scattered slots.  anchors receives the
// anchor of every slot whose flag is 1 and of every slot listed in list2 (what the exact
// list and the materializer read).  prefix is the batch's inclusive prefix (batch_lo = its
// first seed).
hipError_t launch_gate_window_kg(const KeyGroups &kg, const KgScratch &ks,
                                 PrefixView prefix, uint32_t batch_lo, uint32_t seed_lo,
                                 uint32_t seed_hi, uint32_t hit_lo, uint32_t n,
                                 const uint32_t *pos, uint64_t *anchors, uint8_t *flags,
                                 const uint32_t *ref4, const uint32_t *qry4,
                                 const WindowParams &wp, uint32_t *list1, uint64_t *list1_a,
                                 uint32_t *list2, uint32_t *cnt, const ScoreParams &sp,
                                 const uint8_t *ref8, const uint8_t *qry8, bool groups_ready,
                                 bool bits, hipStream_t s);
// The grouping pass of launch_gate_window_kg alone (k_kg_groups and the scan of its block
// sums), for seeds seed_lo .. seed_hi; launch_gate_window_kg with groups_ready set then
// starts after it.
hipError_t launch_kg_groups(const KeyGroups &kg, const KgScratch &ks, uint32_t seed_lo,
                            uint32_t seed_hi, hipStream_t s);
// Bucketed gate ("D. Score gate", D.5): stable sort of anchors by reference slice
// (k_bucket.hip) and the first window stage over the sorted anchors (k_gate.hip).
uint32_t bucket_blocks(uint32_t n);  // workgroups of the slice histogram and scatter
hipError_t launch_bucket_hist(const uint64_t *anchors, uint32_t n, int shift, uint32_t nb,
                              uint32_t *hist, hipStream_t s);
hipError_t launch_bucket_scatter(const uint64_t *anchors, uint32_t n, int shift, uint32_t nb,
                                 const uint32_t *incl, const uint32_t *hist, uint64_t *sa,
                                 uint32_t *si, hipStream_t s);
hipError_t launch_zero_bytes(uint8_t *p, uint64_t n, hipStream_t s);
hipError_t launch_gate_window_bucketed(const uint64_t *anchors, uint32_t n, const uint64_t *sa,
                                       const uint32_t *si, uint8_t *flags, const uint32_t *ref4,
                                       const uint32_t *qry4, const WindowParams &wp,
                                       uint32_t *list1, uint32_t *list2, uint32_t *cnt,
                                       hipStream_t s);
hipError_t launch_gate_list_wave(const uint64_t *anchors, const uint32_t *list,
                                 const uint32_t *count, uint32_t max_count, uint8_t *flags,
                                 const uint8_t *ref, const uint8_t *qry, const ScoreParams &sp,
                                 hipStream_t s, bool bits = false);
// ref: the padded byte reference past its padding (base 0), for the entropy decision;
// ref4, qry4: the 4-bit copies (base b at padded nibble kPad4 + b), for the walks.
hipError_t launch_materialize(const uint64_t *anchors, const uint32_t *ids, uint32_t n_surv,
                              hspz_segment_pair *hsp, uint8_t *status, const uint8_t *ref,
                              const uint32_t *ref4, const uint32_t *qry4, const ScoreParams &sp,
                              hipStream_t s);
// Stable compaction: count non-zero bytes per block, scan block counts on the device
// (total -> *d_total), then emit either the indices (ids != nullptr) or the selected
// 16-byte records (rec_in/rec_out).
// launch_compact for flags held one bit per element (bit i % 32 of word i / 32; bits past
// n clear), listing the set ones' indices in ids.
hipError_t launch_compact_bits(const uint32_t *bits, uint32_t n, uint32_t *blk,
                               uint32_t *d_total, uint32_t *ids, uint32_t cap, hipStream_t s);
hipError_t launch_compact(const uint8_t *flags, uint32_t n, uint32_t *blk, uint32_t *d_total,
                          uint32_t *ids, const hspz_segment_pair *rec_in,
                          hspz_segment_pair *rec_out, uint32_t cap, hipStream_t s);

hipError_t launch_walk_steps(const uint64_t *anchors, uint32_t n, const uint8_t *ref,
                             const uint8_t *qry, const ScoreParams &sp, uint64_t *partial,
                             hipStream_t s);
uint32_t walk_steps_blocks(uint32_t n);

}  // namespace hspz
