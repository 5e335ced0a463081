/*
 * CPU oracle for the hspZ seed-and-extend path: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct restatement of what the hspZ documentation pages
 * ("C. Hit discovery", "D. Score gate", "E. X-drop materialization") say the path
 * computes.  It exists so the HIP library can be checked byte for byte.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never does.  It shares no code, header, table or constant with the HIP library.
 *
 * Everything is integer arithmetic except the keep-threshold search, which evaluates
 * the single-precision comparison the score-gate page says the integer threshold must
 * reproduce.
 *
 * Readings where the pages leave a step open are marked "reading:" at the function
 * that takes them.  Parity-unpinned readings (no page value or closed form fixes them):
 * the window-validity rule, the exclusive-end anchor coordinate, the within-bucket
 * occurrence order, the lower-bound chunk cut against KegAlign, the N score constant,
 * the strictness of the X-drop test, the inclusive-extent len convention, strands and
 * batches, and the entropy-adjusted decision (orc_entropy_bits), whose formula the pages
 * never give.
 */
#ifndef HSPZ_ORACLE_H
#define HSPZ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    uint32_t ref_start, query_start, len;
    int32_t score;
} orc_segment_pair;

void orc_encode(const uint8_t *ascii, int64_t n, uint8_t *codes);
void orc_revcomp_codes(const uint8_t *codes, int64_t n, uint8_t *out);
int orc_pattern(const char *pattern, int32_t *care, int32_t *span);
int orc_window_key(const uint8_t *codes, int64_t n, int64_t p, const int32_t *care,
                   int weight, int span, uint32_t *key);
int64_t orc_query_seeds(const uint8_t *codes, int64_t n, const char *pattern,
                        uint32_t *kmer, uint32_t *q_end, int64_t *pos);
int64_t orc_ref_index(const uint8_t *codes, int64_t n, const char *pattern,
                      uint32_t *keys, uint32_t *ends);
void orc_counts_indexed(const uint32_t *keys, const uint32_t *ends, int64_t n_win,
                        const uint32_t *kmer, int64_t n_seeds, uint32_t *count,
                        int64_t *first);
void orc_counts_brute(const uint8_t *rcodes, int64_t nr, const char *pattern,
                      const uint32_t *kmer, int64_t n_seeds, uint32_t *count);
int orc_prefix(const uint32_t *count, int64_t n, uint64_t *P);
int64_t orc_chunks(const uint64_t *P, int64_t n, uint64_t max_hits, int64_t *seed_lo,
                   int64_t *seed_hi, uint64_t *hit_lo, uint64_t *n_hits);
void orc_anchors(const uint64_t *P, const uint32_t *count, const int64_t *first,
                 const uint32_t *ends, const uint32_t *q_end, int64_t seed_lo,
                 int64_t seed_hi, uint64_t hit_lo, uint64_t *anchors);
void orc_anchors_brute(const uint8_t *rcodes, int64_t nr, const char *pattern,
                       const uint64_t *P, const uint32_t *kmer, const uint32_t *q_end,
                       int64_t seed_lo, int64_t seed_hi, uint64_t hit_lo,
                       uint64_t *anchors);
int32_t orc_keep_threshold(int32_t K);
void orc_xdrop(const uint8_t *rc, int64_t nr, const uint8_t *qc, int64_t nq, int64_t r,
               int64_t q, int dir, const int32_t *sub, int32_t n_score, int32_t xdrop,
               int64_t *best, int64_t *ext);
void orc_gate(const uint64_t *anchors, int64_t n, const uint8_t *rc, int64_t nr,
              const uint8_t *qc, int64_t nq, const int32_t *sub, int32_t n_score,
              int32_t xdrop, int32_t T, uint8_t *flags);
void orc_gate_totals(const uint64_t *anchors, int64_t n, const uint8_t *rc, int64_t nr,
                     const uint8_t *qc, int64_t nq, const int32_t *sub, int32_t n_score,
                     int32_t xdrop, int64_t *totals, int64_t *steps);
int64_t orc_compact(const uint8_t *flags, int64_t n, uint32_t *ids);
double orc_entropy_bits(const uint8_t *rc, int64_t nr, int64_t rs, int64_t len);
int orc_materialize(const uint64_t *anchors, const uint32_t *ids, int64_t n_surv,
                    const uint8_t *rc, int64_t nr, const uint8_t *qc, int64_t nq,
                    const int32_t *sub, int32_t n_score, int32_t xdrop, int32_t T,
                    int32_t K, int32_t entropy_mode, orc_segment_pair *hsp,
                    uint8_t *status);
int64_t orc_compact_hsps(const orc_segment_pair *hsp, const uint8_t *status, int64_t n,
                         orc_segment_pair *out);

#ifdef __cplusplus
}
#endif
#endif
