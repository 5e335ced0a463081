// The engine's state: one reference, one query strand, the plan of one batch, and the
// scratch of every call (host side only; kernels never see it).
#pragma once

#include <string>
#include <vector>

#include "hspz_internal.h"

namespace hspz {

struct MatScratch;

struct Engine {
    hspz_params params{};
    std::string pattern;
    std::vector<int32_t> care;
    int span = 0, weight = 0;
    int device = 0;
    int32_t T = 0;
    int block_bases = 8;
    ScoreParams sp{};
    WindowParams wp{};
    bool window_ok = false;  // the windowed gate is exact for these parameters
    std::string err;

    // reference
    bool has_ref = false;
    uint64_t n_ref = 0;
    uint32_t *d_end = nullptr;   // 4^w + 1 cumulative bucket ends, leading 0
    uint4 *d_ctab = nullptr;     // the same in packed records (launch_count_table)
    uint32_t *d_cnib = nullptr;  // each key's count in 4 bits (launch_count_nibbles)
    uint32_t *d_pos = nullptr;   // reference end coordinate of every valid window
    uint64_t n_index = 0;        // entries of d_pos
    uint8_t *d_ref = nullptr;    // padded encoded reference (kPad edge bytes each side)
    uint32_t *d_ref4 = nullptr;  // 4-bit packed reference (kPad4 edge nibbles each side),
                                 // then its line-split twin at wp.ref4_alt

    // query strand
    bool has_qry = false;
    uint64_t n_qry = 0;
    int strand = 0;
    uint8_t *d_qry = nullptr;
    uint32_t *d_qry4 = nullptr;  // the same layout as d_ref4 (twin at wp.qry4_alt)
    uint32_t *d_kmer = nullptr;
    uint32_t *d_qend = nullptr;
    uint64_t n_seeds = 0;
    std::vector<uint32_t> h_seed_start;  // window start of every seed (ascending)
    // the strand's seeds grouped by k-mer, for the key-grouped first gate stage
    // (KeyGroups in hspz_internal.h): built with the seeds when that stage may run;
    // kg_ready once the runs' buckets are known (a reference is there too)
    bool kg_built = false, kg_ready = false;
    uint32_t *d_kg_qk = nullptr, *d_kg_qs = nullptr, *d_kg_qe = nullptr;
    uint32_t *d_kg_runs = nullptr, *d_kg_run_c = nullptr, *d_kg_run_first = nullptr;
    uint4 *d_kg_run_span = nullptr;
    uint32_t kg_n_runs = 0;
    // its per-chunk scratch (KgScratch), for cap_kg runs and cap_kg_dir waves
    uint32_t *d_kg_G = nullptr, *d_kg_a = nullptr, *d_kg_m = nullptr;
    uint32_t *d_kg_dir = nullptr;
    uint64_t *d_kg_blksum = nullptr;
    uint32_t *d_kg_blkoff = nullptr;
    PlanInfo *d_kg_info = nullptr;
    uint64_t cap_kg = 0, cap_kg_dir = 0;

    // plan of one batch
    bool has_plan = false;
    bool plan_expandable = false;
    uint64_t batch_lo = 0, batch_n = 0, total = 0;
    uint32_t *d_count = nullptr, *d_prefix = nullptr;
    uint32_t *d_first = nullptr;  // bucket start of every seed of the batch
    // d_count and d_first hold this plan's values (the plan writes only the prefix; they
    // are filled on first use, ensure_plan_aux)
    bool plan_aux = false;
    uint64_t *d_blksum = nullptr;
    uint32_t *d_blkoff = nullptr;
    uint64_t cap_batch = 0;
    std::vector<hspz_chunk> chunks;

    // gate scratch: anchor indices left by each window stage, and their two counts
    uint32_t *d_defer = nullptr;  // 2 * cap_defer entries: stage-1 list, then stage-2 list
    uint64_t cap_defer = 0;
    uint64_t *d_defer_a = nullptr;  // the key-grouped stage's anchors of the stage-1 list
    uint64_t cap_defer_a = 0;
    uint32_t *d_defer_cnt = nullptr;
    bool gate_deferred_valid = false;

    // bucketed gate (gate_mode 4): reference slices of 2^slice_shift bases, and per-call
    // scratch for cap_bucket anchors: sorted anchors and raw indices, the slice-major
    // histogram and its scan
    int slice_shift = 22;
    uint32_t n_slices = 1;
    uint64_t *d_bsa = nullptr;
    uint32_t *d_bsi = nullptr;
    uint32_t *d_bhist = nullptr, *d_bincl = nullptr;
    uint64_t *d_bsum = nullptr;
    uint32_t *d_boff = nullptr;
    PlanInfo *d_binfo = nullptr;
    uint64_t cap_bucket = 0;

    // diagonal-shared materialization scratch (mat_shared.h), made on first use
    MatScratch *mat = nullptr;

    // compaction scratch
    uint32_t *d_cblk = nullptr;
    uint32_t *d_ctotal = nullptr;
    uint64_t cap_cblk = 0;
    uint32_t *h_pinned = nullptr;  // small pinned staging buffer (64 u32)
    PlanBuf *d_plan = nullptr;     // device plan results
    uint32_t *d_dir = nullptr;     // fused first stage: owner seed of each wave's range
    uint64_t cap_dir = 0;
    PlanBuf *h_plan = nullptr;     // pinned copy

    // whole-batch driver (hspz_run_batch): two sets of chunk buffers (chunk c uses set
    // c & 1, so the next chunk's gate can be queued before this chunk's materialization),
    // survivor buffers, record staging, and a pair of gate events per set
    uint64_t *rb_anchors[2] = {nullptr, nullptr};
    uint8_t *rb_flags[2] = {nullptr, nullptr};
    uint32_t *rb_ids[2] = {nullptr, nullptr};
    uint64_t rb_cap_a = 0;
    hspz_segment_pair *rb_hsp = nullptr;
    hspz_segment_pair *rb_out[2] = {nullptr, nullptr};  // accepted records, by chunk parity
    uint8_t *rb_status = nullptr;
    uint64_t rb_cap_s = 0;
    // the whole-batch gate of hspz_run_batch: the batch's flags (a bit per anchor, 32-bit
    // words), kept anchors and survivor ids
    uint8_t *bb_flags = nullptr;
    uint64_t *bb_anchors = nullptr;
    uint32_t *bb_ids = nullptr;
    uint64_t bb_cap = 0;
    hspz_segment_pair *h_rec = nullptr;  // pinned: accepted records of the last batch
    uint64_t h_rec_cap = 0, h_rec_n = 0;
    hipEvent_t gate_ev[4] = {nullptr, nullptr, nullptr, nullptr};
    hipEvent_t count_ev[2] = {nullptr, nullptr};  // survivor and record counts landed
    hipEvent_t plan_ev = nullptr;                  // the plan's copy to the host landed
    // the records' copies to the host run on their own stream (default priority) and
    // overlap the next chunks; copied_ev[b] marks the copy out of rb_out[b]
    hipStream_t copy_s = nullptr;
    hipEvent_t copied_ev[2] = {nullptr, nullptr};
    bool copy_pending[2] = {false, false};

    ~Engine();
    void free_plan();
};

}  // namespace hspz
