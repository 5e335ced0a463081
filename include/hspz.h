/*
 * hspz.h -- C ABI of libhspz, the MI355X (gfx950) seed-and-extend hot path described
 * by the hspZ documentation pages "C. Hit discovery", "D. Score gate" and
 * "E. X-drop materialization".
 *
 * One engine holds one reference (its spaced-seed index and encoded bases) and one
 * query strand (its encoded bases and seeds) in device memory.  A pass over one batch
 * of query seeds is:
 *
 *   hspz_plan         counts, global prefix, MAX_HITS chunk list     (C.1 - C.3)
 *   per chunk:
 *     hspz_find_hits  packed anchors in raw (backward) order        (C.4 - C.5)
 *     hspz_score_gate one survivor byte per anchor                  (D.1 - D.3)
 *     hspz_compact    increasing survivor ids                       (D.4)
 *     hspz_materialize exact X-drop SegmentPair + status per id     (E.1 - E.5)
 *     hspz_compact_hsps accepted SegmentPairs in survivor order     (E.5)
 *
 * hspz_find_hits_gate runs a chunk's expansion and gate as one call (the anchors are
 * formed inside the gate), and hspz_run_batch runs the whole pass over a batch inside
 * the library, leaving the accepted records in host memory (hspz_get_batch_records).
 * hspz_dedup_records removes repeated accepted records on the host.
 *
 * Conventions
 *  - Every function returns HSPZ_OK (0) or a negative HSPZ_E_* code; no exception or
 *    signal crosses the ABI.  On error, outputs are unspecified, every *n_out is set to
 *    0 and hspz_last_error(engine) describes the failure.
 *  - Pointers named d_* are device pointers on the engine's device, owned by the
 *    caller; the library never frees them.  h_* pointers are host memory.
 *  - stream is a hipStream_t (NULL = the default stream).  Calls that return a count
 *    (hspz_plan, hspz_compact, hspz_compact_hsps) synchronise that stream; every other
 *    kernel-launching call is asynchronous on it.
 *  - An engine is not thread-safe: use one engine per host thread.  Its calls share the
 *    engine's device scratch (the gate's deferred lists, compaction blocks, the bucketed
 *    gate's sorted copy, the shared walks' sort and per-side arrays), so calls of one
 *    engine on different streams must not overlap: give an engine one stream, or
 *    synchronise between streams.
 *  - Coordinates are 0-based.  Sequences are ASCII; A/C/G/T in either case are bases,
 *    every other byte is N.
 */
#ifndef HSPZ_H
#define HSPZ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSPZ_OK 0
#define HSPZ_E_INVALID (-1)  /* bad parameter, malformed seed pattern, out-of-range arg */
#define HSPZ_E_OVERFLOW (-2) /* batch total exceeds the 32-bit hit index (refused)      */
#define HSPZ_E_CAPACITY (-3) /* caller buffer too small                                 */
#define HSPZ_E_NOMEM (-4)    /* host or device allocation failed                        */
#define HSPZ_E_HIP (-5)      /* a HIP runtime call failed                               */
#define HSPZ_E_STATE (-6)    /* call out of order (e.g. find_hits before plan)          */

typedef struct hspz_engine hspz_engine;

/* One ungapped high-scoring segment pair ("E. X-drop materialization", E.4): the
 * closed interval ref_start..=ref_start+len on the reference and
 * query_start..=query_start+len on the query; len is an extent (the number of bases
 * covered minus one).  score is the X-drop total L* + R*.  16 bytes, little-endian,
 * this field order. */
typedef struct {
    uint32_t ref_start;
    uint32_t query_start;
    uint32_t len;
    int32_t score;
} hspz_segment_pair;

/* One MAX_HITS chunk ("C. Hit discovery", C.3): seeds seed_lo..=seed_hi (indices into
 * the current strand's seed list) whose anchors occupy hits hit_lo..hit_lo+n_hits-1 of
 * the batch's global prefix.  A chunk's anchors are numbered 0..n_hits-1 locally. */
typedef struct {
    uint64_t seed_lo;
    uint64_t seed_hi;
    uint64_t hit_lo;
    uint64_t n_hits;
} hspz_chunk;

/* Engine parameters.
 *  seed_pattern  spaced seed, '1' = care position; must start and end with '1',
 *                weight 1..14, span <= 64 ("C. Hit discovery", C.1 packed k-mer).
 *  sub           substitution scores, row = reference base, column = query base, order
 *                A,C,G,T, row-major; each |entry| <= 10000.
 *  n_score       score of any pair involving N; |n_score| <= 10000.
 *  xdrop         X-drop, 0 <= xdrop <= 1000000 ("D. Score gate", D.2).
 *  hsp_threshold K in 1 .. 2^30; the keep threshold T is derived from it once per engine.
 *  max_hits      MAX_HITS chunk cap, 0 = unlimited ("C. Hit discovery", C.3).
 *  expand_mode   0 = density rule (>= 16 hits per seed -> group per seed), 1 = always
 *                thread per seed, 2 = always group per seed ("C. Hit discovery", C.4).
 *  chunk_walk    0 = locate boundaries through block sums, copying one prefix block per
 *                boundary; 1 = copy the whole prefix and walk it.  Same chunks.
 *  device        HIP device ordinal the engine lives on.
 *  gate_mode     0 = windowed score gate when it is exact for these parameters (eight-base
 *                blocks, 16-bit pair scores), else the exact per-base walk; 1 = always the
 *                per-base walk; 2 = always windowed; 3 = always windowed with a narrower
 *                first window; 4 = the reference-locality bucketed gate ("D. Score gate",
 *                D.5): the call's anchors are sorted stably by reference slice (2^22
 *                bases or more, at most 256 slices) with their raw indices, each XCD's
 *                waves score the windows of about one slice at a time, and results go
 *                back by raw index; 5 = windowed, with hspz_find_hits_gate taking every
 *                chunk in key-grouped order: the chunk's seeds of each k-mer times that
 *                k-mer's bucket, so that same-k-mer seeds share the reads of the bucket's
 *                reference windows (mode 0 does this for chunks holding at least half as
 *                many seeds as the strand has distinct k-mers; the grouping is built by
 *                hspz_upload_query and hspz_upload_seeds in modes 0 and 5).  2 to 5 fail
 *                with HSPZ_E_INVALID if the window gate is not exact.  Every mode writes
 *                the same flags ("D. Score gate", D.2).
 *  entropy_mode  the accept decision of hspz_materialize ("E. X-drop materialization",
 *                E.5, which names an entropy-adjusted decision without a formula):
 *                0 = accept iff score >= T; 1 = also require score * H >= 2 * K, where H
 *                is the Shannon entropy in bits of the A/C/G/T composition of the
 *                record's reference interval (N excluded), computed in double precision
 *                as (n log2 n - sum_b n_b log2 n_b) / n; no A/C/G/T in the interval
 *                rejects.
 *  ref_buckets   reference slices of the bucketed gate (gate_mode 4; the pages' engine
 *                switch for reference-locality bucketing, "D. Score gate", D.5): 0 =
 *                automatic, slices of 2^22 bases (2 MiB of 4-bit codes, inside one XCD's
 *                L2), widened to keep at most 256; n in 1..256 = at most n slices, each
 *                of the smallest power-of-two width that allows it.  Ignored by the
 *                other gate modes; never changes any output.
 *  materialize_mode  how hspz_materialize walks ("E. X-drop materialization", E.1-E.3):
 *                1 = one wave per survivor, each walk on its own; 2 = diagonal-shared
 *                walks: survivors are sorted by diagonal, and a walk that reaches a
 *                strictly new best at or past its neighbour's start takes the rest from
 *                the neighbour (the walks coincide from there), so a stretch of a
 *                diagonal shared by many survivors is walked about once; 0 = 2 for calls
 *                of at least 131,072 survivors, else 1.  Mode 2 needs
 *                n_ref + n_qry + 2 < 2^32 (32-bit diagonal keys) and takes mode 1
 *                otherwise.  Every mode writes the same records and status.
 */
typedef struct {
    const char *seed_pattern;
    int32_t sub[16];
    int32_t n_score;
    int32_t xdrop;
    int32_t hsp_threshold;
    int32_t expand_mode;
    uint64_t max_hits;
    int32_t chunk_walk;
    int32_t device;
    int32_t gate_mode;
    int32_t entropy_mode;
    int32_t ref_buckets;
    int32_t materialize_mode;
} hspz_params;

/* Create an engine on params->device and compute the keep threshold T once: the least
 * int32 t with (float)t >= (float)K ("D. Score gate", D.2 invariant), so that the
 * gate's integer compare total >= T keeps exactly what the single-precision comparison
 * keeps.  *out receives the engine (caller frees it with hspz_engine_destroy).
 * Errors: HSPZ_E_INVALID (parameters), HSPZ_E_NOMEM, HSPZ_E_HIP. */
int hspz_engine_create(const hspz_params *params, hspz_engine **out);

/* Free the engine and every device buffer it owns.  NULL is accepted. */
int hspz_engine_destroy(hspz_engine *engine);

/* The keep threshold T computed at creation. */
int32_t hspz_keep_threshold(const hspz_engine *engine);

/* Last error message of this engine ("" if none); owned by the engine, valid until
 * the next call on it.  A NULL engine returns the message of the last failed create. */
const char *hspz_last_error(const hspz_engine *engine);

/* Copy the reference to the device, encode it there and build its spaced-seed index
 * there ("C. Hit discovery", C.1: a cumulative bucket-end table, one entry per packed
 * k-mer plus a leading 0, and the concatenated buckets of reference end coordinates,
 * ascending within a bucket; the buckets come from a stable radix sort of (k-mer, end)
 * pairs listed in position order).  h_ascii (len bytes, host) is not retained; bytes
 * other than A/C/G/T (either case) encode as N.  len < 2^32 - 1025.  Temporary device
 * memory during the call: about len + 26 bytes per reference window plus 8 * 4^weight
 * bytes.  Replaces any previous reference and invalidates a plan.  Synchronises stream.
 * Errors: HSPZ_E_INVALID, HSPZ_E_NOMEM, HSPZ_E_HIP. */
int hspz_upload_reference(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                          void *stream);

/* Encode one query strand on the device and list its seeds there: every window whose
 * care positions are all A/C/G/T, in ascending window position, each with its packed
 * k-mer and its query end coordinate (window start + span).  strand 0 = the sequence
 * as given, 1 = its reverse complement, in the reverse complement's own coordinates.
 * In gate_mode 0 and 5, when the window gate is exact, the call also groups the seeds by
 * k-mer for the key-grouped first gate stage (a stable radix sort of (k-mer, seed)
 * pairs, then the runs of equal k-mers); the engine then holds 16 more bytes per seed
 * and 36 per distinct k-mer, and each run's bucket is looked up again whenever a
 * reference is uploaded.  Replaces the previous query and invalidates a plan.
 * Synchronises stream.  Errors as above. */
int hspz_upload_query(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                      int32_t strand, void *stream);

/* Replace the current strand's seeds with the caller's ("C. Hit discovery", C.1: a seed
 * is a packed k-mer and the query end of its window), in place of the device seeder's:
 * h_kmer[i] < 4^w (w = the pattern's care positions) and h_q_end[i] in [span, query
 * length], the window starting at h_q_end[i] - span.  The query ends must not decrease
 * (the order hspz_upload_query produces, on which hspz_seed_range and the batch driver
 * rely).  The k-mers need not match the query's bases; the uploaded strand stays, since
 * the walks read it.  The key grouping of hspz_upload_query is rebuilt for these seeds.
 * Host arrays, copied; invalidates a plan; synchronises stream.
 * Errors: HSPZ_E_STATE (no query strand uploaded), HSPZ_E_INVALID (NULL arrays, a value
 * out of range, decreasing query ends; the seeds are left as they were), HSPZ_E_NOMEM,
 * HSPZ_E_HIP. */
int hspz_upload_seeds(hspz_engine *engine, const uint32_t *h_kmer, const uint32_t *h_q_end,
                      uint64_t n, void *stream);

/* Number of seeds of the current query strand. */
uint64_t hspz_num_seeds(const hspz_engine *engine);

/* Seed-index range [*seed_lo, *seed_hi) of the seeds whose window starts in
 * [pos_lo, pos_hi) -- a contiguous query batch.  Errors: HSPZ_E_STATE (no query). */
int hspz_seed_range(const hspz_engine *engine, uint64_t pos_lo, uint64_t pos_hi,
                    uint64_t *seed_lo, uint64_t *seed_hi);

/* Plan one batch, seeds [seed_lo, seed_hi) ("C. Hit discovery", C.1-C.3): count each
 * seed's hits, scan blocks of counts on the device, exclusive-scan the block sums in
 * 64 bits on the device (the global inclusive prefix is a block's local prefix plus its
 * offset; the library adds the offset wherever it reads a prefix), and cut MAX_HITS
 * chunks with the lower-bound walk (a seed is never split), also on the device; one copy
 * brings back the total and the chunk list.  Only the prefix stays on the device: the
 * per-seed counts and bucket starts are looked up again, once per plan, by the first call
 * that reads them (hspz_find_hits, a raw-order hspz_find_hits_gate, hspz_get_plan_arrays).
 * A batch whose total exceeds 2^32 - 1 is refused with HSPZ_E_OVERFLOW and leaves no
 * plan.
 * *total_hits and *n_chunks receive the totals (0 chunks when the total is 0).
 * Synchronises stream.  Errors: HSPZ_E_STATE (no reference/query), HSPZ_E_INVALID,
 * HSPZ_E_OVERFLOW, HSPZ_E_NOMEM, HSPZ_E_HIP. */
int hspz_plan(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi, void *stream,
              uint64_t *total_hits, uint32_t *n_chunks);

/* Chunk i of the current plan.  Errors: HSPZ_E_STATE (no plan), HSPZ_E_INVALID. */
int hspz_get_chunk(const hspz_engine *engine, uint32_t i, hspz_chunk *out);

/* Expand chunk i into packed anchors ("C. Hit discovery", C.4-C.5): occurrence j of
 * seed s is written to d_anchors[P[s] - 1 - hit_lo - j] as
 * (reference end) | (query end) << 32, so each bucket lands backwards from the seed's
 * inclusive prefix.  d_anchors holds cap u64 entries (device); cap must be at least the
 * chunk's n_hits.  The choice between thread-per-seed and group-per-seed expansion
 * changes memory traffic only, never the bytes.  Errors: HSPZ_E_STATE, HSPZ_E_INVALID,
 * HSPZ_E_CAPACITY, HSPZ_E_HIP. */
int hspz_find_hits(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors, uint64_t cap,
                   void *stream);

/* Score-only X-drop gate over n packed anchors ("D. Score gate", D.1-D.3).  For each
 * anchor (r, q) the right walk scores (r+i, q+i) and the left walk (r-1-i, q-1-i); each
 * stops at the first base whose running score is more than xdrop below its best so far,
 * or at a sequence end, and contributes that best (0 for an empty walk).  d_flags[i]
 * becomes 1 if the two bests sum to at least T, else 0; all n bytes are written.
 * d_anchors must hold coordinates within the uploaded sequences.  n < 2^32.
 * Errors: HSPZ_E_STATE, HSPZ_E_INVALID, HSPZ_E_HIP. */
int hspz_score_gate(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                    uint8_t *d_flags, void *stream);

/* hspz_score_gate for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and the
 * same d_flags bytes as hspz_score_gate, but the window gate's deferred-anchor lists and
 * counters live in a static device array of the library (64 MiB + 64 B on every GPU the
 * library runs on, held until the process ends), so the call allocates nothing and
 * synchronises nothing.  n is at most 2^23 (8,388,608); split longer anchor arrays into
 * several calls.  Every call on one GPU shares that array, from every engine: calls that
 * overlap on one GPU (other streams, other host threads) race, so serialise them.
 * Errors: as hspz_score_gate; HSPZ_E_CAPACITY when n exceeds 2^23, HSPZ_E_INVALID with
 * the bucketed gate (gate_mode 4), whose sort needs scratch proportional to n. */
int hspz_score_gate_noalloc(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                            uint8_t *d_flags, void *stream);

/* hspz_find_hits and hspz_score_gate for chunk i in one call ("C. Hit discovery", C.5;
 * "D. Score gate", D.1-D.3): the gate's first window stage builds each anchor from the
 * chunk's seeds as it scores it, so the anchors are not written out and read back.
 * d_flags receives the chunk's n_hits flags exactly as hspz_score_gate writes them;
 * afterwards d_anchors (cap >= n_hits u64 entries) holds the anchor of every slot whose
 * flag is 1, which is what hspz_materialize reads, and its other entries are
 * unspecified.  When the window gate does not apply (gate_mode 1, or scores or xdrop
 * outside its bounds), and with the bucketed gate (gate_mode 4, which sorts the written
 * anchors), the call is hspz_find_hits followed by hspz_score_gate, and every entry is
 * written.  Errors: as hspz_find_hits; HSPZ_E_INVALID for NULL buffers. */
int hspz_find_hits_gate(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors, uint64_t cap,
                        uint8_t *d_flags, void *stream);

/* Stable compaction of n flag bytes ("D. Score gate", D.4): d_ids receives, in
 * increasing order, the index of every non-zero byte.  *n_out receives their number;
 * if it exceeds cap (the capacity of d_ids, u32 entries) the call fails with
 * HSPZ_E_CAPACITY and *n_out = 0.  n < 2^32.  Synchronises stream. */
int hspz_compact(hspz_engine *engine, const uint8_t *d_flags, uint64_t n, uint32_t *d_ids,
                 uint64_t cap, uint64_t *n_out, void *stream);

/* Exact materialization of n_surv survivors ("E. X-drop materialization", E.1-E.5).
 * For each i the anchor d_anchors[d_ids[i]] is extended to both sides by the same
 * X-drop rule as the gate, keeping the earliest base that attains each side's best.
 * With left extent m and right extent k the record is
 * {r - m, q - m, m + k - 1, L* + R*}.  d_status[i] = 1 if the record is accepted
 * (score >= T, and with entropy_mode 1 also score * H >= 2K, see hspz_params), else 0;
 * d_hsp[i] is written in either case and is meaningful only when accepted.  The
 * diagonal-shared walks (materialize_mode) allocate their scratch in the engine on first
 * use and keep it.  Scores are summed in 32-bit integers on the device: a record is exact
 * while its two extents together stay below (2^31 - 1) / (largest pair score) - 1024
 * bases (21,473,812 with HOXD70), which keeps the score and every running score of both
 * walks, including the bases of their last 512-base tiles, inside int32.  Longer walks
 * are outside the supported range and their records are unspecified (the CPU oracle
 * refuses a record whose score does not fit int32).  Errors: HSPZ_E_STATE (no reference
 * or query uploaded), HSPZ_E_INVALID (n_surv >= 2^32, NULL buffers), HSPZ_E_NOMEM (the
 * shared walks' scratch), HSPZ_E_HIP. */
int hspz_materialize(hspz_engine *engine, const uint64_t *d_anchors, const uint32_t *d_ids,
                     uint64_t n_surv, hspz_segment_pair *d_hsp, uint8_t *d_status,
                     void *stream);

/* Stable compaction of the accepted records ("E. X-drop materialization", E.5): the
 * d_hsp[i] with d_status[i] != 0, in order, into d_out (cap records).  *n_out receives
 * their number; HSPZ_E_CAPACITY if it exceeds cap.  Synchronises stream. */
int hspz_compact_hsps(hspz_engine *engine, const hspz_segment_pair *d_hsp,
                      const uint8_t *d_status, uint64_t n, hspz_segment_pair *d_out,
                      uint64_t cap, uint64_t *n_out, void *stream);

/* ---- whole batch ------------------------------------------------------------------ */

/* Counts of the last hspz_run_batch call. */
typedef struct {
    uint64_t n_anchors;    /* raw anchors (the plan's total hits)                       */
    uint64_t n_chunks;     /* MAX_HITS chunks                                           */
    uint64_t n_survivors;  /* anchors the gate kept                                     */
    uint64_t n_accepted;   /* accepted records                                          */
    uint64_t gate_calls;   /* expansion-and-gate calls timed (time_gate != 0), else 0  */
    double gate_ms;        /* their summed durations from HIP events on the stream      */
    uint64_t whole_batch_gate; /* 1: one gate call covered every chunk, else 0          */
} hspz_batch_stats;

/* The whole pass for query seeds [seed_lo, seed_hi) of the current strand, in one call:
 * hspz_plan, then for every chunk hspz_find_hits_gate, hspz_compact, hspz_materialize
 * and hspz_compact_hsps in the pages' order ("C. Hit discovery" to
 * "E. X-drop materialization"), with the same kernels and the same records.  The chunk
 * buffers are the engine's own (grown as needed); the accepted records of every chunk,
 * in chunk order, are copied to pinned host memory the engine owns, from where
 * hspz_get_batch_records reads them.  Those copies run on a second stream that the
 * engine creates (default priority), ordered behind each chunk's records by events, so
 * that they overlap the next chunks' kernels; the call returns once every copy has
 * landed, also on error.  Where the key-grouped first gate stage serves the whole batch
 * (gate_mode 0 or 5, see hspz_params) and the batch has more than one chunk, at most
 * 2^30 anchors and at least 2^22 per chunk on average, the whole batch goes at once:
 * one gate call over every chunk's slots, one compaction of the batch's flags (survivor
 * ids are batch slots, so the chunks' survivors come one chunk after another), one
 * materialization of them all (their anchors are in query order) and one copy of the
 * accepted records.  The records are the chunks' records in chunk order, as chunk by
 * chunk (stats->whole_batch_gate = 1).  Its engine buffers take about 12 bytes per
 * anchor (a flag bit, kept anchors, survivor ids) and the gate's deferred lists 20 more;
 * where the device cannot hold them the batch goes chunk by chunk.  The accepted records
 * are compacted straight into the pinned host staging that hspz_get_batch_records reads.
 * With time_gate != 0 each expansion-and-gate call is
 * bracketed by HIP events on stream and *stats reports their number and summed duration.
 * The plan stays current afterwards.  Synchronises stream.  Errors: as hspz_plan,
 * hspz_find_hits and the calls above; HSPZ_E_INVALID for a NULL stats pointer. */
int hspz_run_batch(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi, int32_t time_gate,
                   hspz_batch_stats *stats, void *stream);

/* Copy the accepted records of the last hspz_run_batch (host to host): *n receives their
 * number and up to cap records go to h_out (h_out NULL with cap 0 only reports *n).
 * Errors: HSPZ_E_CAPACITY (cap < *n; the first cap records are still copied),
 * HSPZ_E_INVALID (NULL n, or NULL h_out with cap > 0). */
int hspz_get_batch_records(const hspz_engine *engine, hspz_segment_pair *h_out, uint64_t cap,
                           uint64_t *n);

/* Exact-duplicate removal of accepted records: the host dedup that follows acceptance in
 * the pages' funnel ("D. Score gate", introduction; the raw order it depends on is fixed
 * in "C. Hit discovery", C.5).  The pages give no rule.  This library's reading: two
 * records are duplicates when all four fields are equal, and the first of them in the
 * order of h_in is kept.  The kept records go to h_out in their input order and *n_out
 * receives their number.  The scope is the array passed: one chunk, one batch (the
 * records of hspz_run_batch, in chunk order) or a whole strand.  Host memory only; h_out
 * may equal h_in (in place), otherwise the two must not overlap.  Needs no engine and no
 * GPU.  Errors: HSPZ_E_INVALID (NULL n_out, or NULL h_in / h_out with n > 0),
 * HSPZ_E_CAPACITY (cap < *n_out; nothing is written to h_out), HSPZ_E_NOMEM;
 * hspz_last_error(NULL) describes the failure. */
int hspz_dedup_records(const hspz_segment_pair *h_in, uint64_t n, hspz_segment_pair *h_out,
                       uint64_t cap, uint64_t *n_out);

/* ---- inspection (tests and tools) -------------------------------------------------- */

/* Copy seeds [lo, hi) of the current strand to the host: packed k-mers and query end
 * coordinates (either pointer may be NULL).  Synchronous. */
int hspz_get_seeds(const hspz_engine *engine, uint64_t lo, uint64_t hi, uint32_t *h_kmer,
                   uint32_t *h_q_end);

/* The reference index built by hspz_upload_reference ("C. Hit discovery", C.1):
 * *n_buckets = 4^weight, *n_pos = the number of indexed reference windows; h_end, if
 * not NULL, receives the n_buckets + 1 cumulative bucket ends (u32, leading 0) and
 * h_pos, if not NULL, the n_pos reference end coordinates grouped by k-mer.  Call with
 * NULL arrays first to learn the sizes.  Synchronous.  Errors: HSPZ_E_STATE without a
 * reference, HSPZ_E_INVALID for a NULL size pointer. */
int hspz_get_index(const hspz_engine *engine, uint32_t *h_end, uint32_t *h_pos,
                   uint64_t *n_buckets, uint64_t *n_pos);

/* Copy the planned batch's per-seed hit counts and global inclusive prefix (u32 each,
 * one per seed of the batch) to the host (either pointer may be NULL).  The counts are
 * looked up first (on the null stream, from the uploaded k-mers and index alone) if no
 * call has needed them since the plan.  Synchronous. */
int hspz_get_plan_arrays(const hspz_engine *engine, uint32_t *h_counts, uint32_t *h_prefix);

/* Run the prefix and chunk steps ("C. Hit discovery", C.2-C.3) on n injected per-seed
 * counts (host array) instead of index lookups, leaving a plan whose chunks and prefix
 * can be read back but not expanded.  Synchronises stream.  Errors as hspz_plan. */
int hspz_debug_plan_counts(hspz_engine *engine, const uint32_t *h_counts, uint64_t n,
                           void *stream, uint64_t *total_hits, uint32_t *n_chunks);

/* Exact algorithmic work of the score gate over n anchors, summed into *total_steps: the
 * bases an exact decision of each flag scores.  The right walk runs up to and including
 * its first dropping base, or until its best reaches T; the left walk, needed only when
 * R* < T, runs up to its first dropping base or until R* + its best reaches T.  No walk
 * scores a base past a sequence end.  Allocates a small temporary device buffer;
 * synchronises stream.  Not part of a pass. */
int hspz_debug_walk_steps(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                          uint64_t *total_steps, void *stream);

/* How the last hspz_score_gate or hspz_find_hits_gate call split its anchors when it
 * took the window path: *n_stage2 walked past the first window (48 bases right of the
 * anchor and 72 left, or 32 and 56 with gate_mode 3) and went to the second (64 and 96);
 * *n_exact walked past that too and were decided by the exact per-base walk.
 * Synchronises stream.  Errors: HSPZ_E_STATE if that call did not take the window
 * path. */
int hspz_debug_gate_deferred(hspz_engine *engine, uint64_t *n_stage2, uint64_t *n_exact,
                             void *stream);

/* Test-only: the random-line probe, a ceiling for kernels whose traffic is one random
 * 128-byte line per unit of work -- the score gate's reference windows ("D. Score gate",
 * D.2: each anchor reads a window of the reference at an unpredictable address; D.5
 * names the locality of those windows as the lever on their cost).  Each of the
 * blocks * 256 lanes reads, iters times, in_flight windows of window_dwords (1 or 16)
 * dwords, each at the start of a random 128-byte line of d_region (region_bytes long,
 * 128-byte aligned, device memory), issuing all of them before it uses any.  Lines read
 * = blocks * 256 * iters * in_flight; the caller times the launch on stream with its own
 * events.  in_flight is 1, 2, 4 or 8.  d_sink (64 u32, device) is written only if the
 * folded words equal key.  Asynchronous; no engine.  Errors: HSPZ_E_INVALID (bad sizes,
 * alignment or counts), HSPZ_E_HIP (launch failure). */
int hspz_debug_line_probe(const uint32_t *d_region, uint64_t region_bytes,
                          uint32_t window_dwords, uint32_t in_flight, uint32_t blocks,
                          uint32_t iters, uint32_t seed, uint32_t key, uint32_t *d_sink,
                          void *stream);

#ifdef __cplusplus
}
#endif
#endif /* HSPZ_H */
