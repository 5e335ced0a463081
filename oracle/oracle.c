/*
 * CPU oracle for the hspZ seed-and-extend path: TEST INFRASTRUCTURE ONLY.
 * See oracle.h for scope.  Plain C99, single-threaded, no blocking or fusion beyond
 * what the pages' definitions state.  Citations name the hspZ documentation page and
 * its step ("C. Hit discovery, C.5" etc.).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ encoding */

/* reading: A,C,G,T (either case) are codes 0..3; every other byte is N (code 4).  The
 * pages only say the sequences are "encoded" (D. Score gate, D.2). */
void orc_encode(const uint8_t *ascii, int64_t n, uint8_t *codes) {
    for (int64_t i = 0; i < n; i++) {
        switch (ascii[i]) {
        case 'A': case 'a': codes[i] = 0; break;
        case 'C': case 'c': codes[i] = 1; break;
        case 'G': case 'g': codes[i] = 2; break;
        case 'T': case 't': codes[i] = 3; break;
        default: codes[i] = 4; break;
        }
    }
}

/* reading: the reverse strand is the reverse complement (A<->T, C<->G, N->N) in its
 * own 0-based coordinates. */
void orc_revcomp_codes(const uint8_t *codes, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) {
        uint8_t c = codes[n - 1 - i];
        out[i] = (c < 4) ? (uint8_t)(3 - c) : 4;
    }
}

/* ------------------------------------------------------------------ seeds */

/* Spaced seed pattern: '1' marks a care position.  Returns the weight (number of care
 * positions) or -1 for a malformed pattern. */
int orc_pattern(const char *pattern, int32_t *care, int32_t *span) {
    int w = 0, n = (int)strlen(pattern);
    if (n == 0 || n > 64) return -1;
    for (int i = 0; i < n; i++) {
        if (pattern[i] == '1') care[w++] = i;
        else if (pattern[i] != '0') return -1;
    }
    if (w == 0 || w > 16 || pattern[0] != '1' || pattern[n - 1] != '1') return -1;
    *span = n;
    return w;
}

/* reading: a window starting at p is valid when it fits and every care position holds
 * A/C/G/T; its key packs the care codes two bits each, first care position most
 * significant.  ("C. Hit discovery, C.1": one packed k-mer per seed.) */
int orc_window_key(const uint8_t *codes, int64_t n, int64_t p, const int32_t *care,
                   int weight, int span, uint32_t *key) {
    if (p < 0 || p + span > n) return 0;
    uint32_t k = 0;
    for (int i = 0; i < weight; i++) {
        uint8_t c = codes[p + care[i]];
        if (c > 3) return 0;
        k = (k << 2) | c;
    }
    *key = k;
    return 1;
}

/* reading: the seeds of a query are all its valid windows in ascending position; the
 * seed's query coordinate is the exclusive window end p + span (the anchor is a
 * "(reference-end, query-end)" pair, D. Score gate, D.1). */
int64_t orc_query_seeds(const uint8_t *codes, int64_t n, const char *pattern,
                        uint32_t *kmer, uint32_t *q_end, int64_t *pos) {
    int32_t care[64], span;
    int w = orc_pattern(pattern, care, &span);
    if (w < 0) return -1;
    int64_t m = 0;
    for (int64_t p = 0; p + span <= n; p++) {
        uint32_t key;
        if (orc_window_key(codes, n, p, care, w, span, &key)) {
            if (kmer) kmer[m] = key;
            if (q_end) q_end[m] = (uint32_t)(p + span);
            if (pos) pos[m] = p;
            m++;
        }
    }
    return m;
}

/* ------------------------------------------------------------------ reference index */

typedef struct { uint32_t key, end; } orc_win;

static int orc_win_cmp(const void *a, const void *b) {
    const orc_win *x = (const orc_win *)a, *y = (const orc_win *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->end != y->end) return x->end < y->end ? -1 : 1;
    return 0;
}

/* The reference index as a list of (key, reference-end) pairs sorted by key and, within
 * a key, by ascending reference end.  reading: occurrence j of a bucket is its j-th
 * smallest reference end ("C. Hit discovery, C.5" names "occurrence j" without an
 * order).  Returns the number of valid windows. */
int64_t orc_ref_index(const uint8_t *codes, int64_t n, const char *pattern,
                      uint32_t *keys, uint32_t *ends) {
    int32_t care[64], span;
    int w = orc_pattern(pattern, care, &span);
    if (w < 0) return -1;
    int64_t m = 0;
    for (int64_t p = 0; p + span <= n; p++) {
        uint32_t key;
        if (orc_window_key(codes, n, p, care, w, span, &key)) m++;
    }
    orc_win *list = (orc_win *)malloc((size_t)(m > 0 ? m : 1) * sizeof(orc_win));
    if (!list) return -2;
    m = 0;
    for (int64_t p = 0; p + span <= n; p++) {
        uint32_t key;
        if (orc_window_key(codes, n, p, care, w, span, &key)) {
            list[m].key = key;
            list[m].end = (uint32_t)(p + span);
            m++;
        }
    }
    qsort(list, (size_t)m, sizeof(orc_win), orc_win_cmp);
    for (int64_t i = 0; i < m; i++) {
        keys[i] = list[i].key;
        ends[i] = list[i].end;
    }
    free(list);
    return m;
}

/* First index in the sorted key list whose key is >= k (upper = 0) or > k (upper = 1). */
static int64_t orc_bound_key(const uint32_t *keys, int64_t n, uint32_t k, int upper) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (keys[mid] < k || (upper && keys[mid] == k)) lo = mid + 1; else hi = mid;
    }
    return lo;
}

/* "C. Hit discovery, C.1": a seed's hit count is the size of its key's bucket (the
 * difference of adjacent cumulative bucket ends); empty buckets give 0.  Also returns
 * where the bucket starts in the sorted list. */
void orc_counts_indexed(const uint32_t *keys, const uint32_t *ends, int64_t n_win,
                        const uint32_t *kmer, int64_t n_seeds, uint32_t *count,
                        int64_t *first) {
    (void)ends;
    for (int64_t s = 0; s < n_seeds; s++) {
        int64_t lo = orc_bound_key(keys, n_win, kmer[s], 0);
        int64_t hi = orc_bound_key(keys, n_win, kmer[s], 1);
        count[s] = (uint32_t)(hi - lo);
        if (first) first[s] = lo;
    }
}

/* Brute force: count every reference window with the seed's key. */
void orc_counts_brute(const uint8_t *rcodes, int64_t nr, const char *pattern,
                      const uint32_t *kmer, int64_t n_seeds, uint32_t *count) {
    int32_t care[64], span;
    int w = orc_pattern(pattern, care, &span);
    for (int64_t s = 0; s < n_seeds; s++) {
        uint32_t c = 0;
        for (int64_t p = 0; w > 0 && p + span <= nr; p++) {
            uint32_t key;
            if (orc_window_key(rcodes, nr, p, care, w, span, &key) && key == kmer[s]) c++;
        }
        count[s] = c;
    }
}

/* ------------------------------------------------------------------ prefix and chunks */

/* "C. Hit discovery, C.2": the global inclusive prefix of the counts; a batch whose
 * total exceeds the 32-bit hit index is refused (returns -1), never wrapped. */
int orc_prefix(const uint32_t *count, int64_t n, uint64_t *P) {
    uint64_t acc = 0;
    for (int64_t s = 0; s < n; s++) {
        acc += count[s];
        P[s] = acc;
    }
    return acc > 0xFFFFFFFFull ? -1 : 0;
}

/* "C. Hit discovery, C.3": cut the seeds into contiguous ranges of about MAX_HITS hits
 * by a lower-bound walk over the seed prefixes; a seed is never split, so a chunk may
 * exceed the cap by one seed bucket.
 * reading: greedy from the first uncut seed s0 with base H = P[s0-1] (0 at s0 = 0): if
 * the remaining total fits in MAX the rest is one chunk, otherwise the chunk ends at the
 * first seed e >= s0 whose prefix reaches H + MAX.  A zero total gives no chunks; MAX 0
 * means unlimited.  Returns the number of chunks. */
int64_t orc_chunks(const uint64_t *P, int64_t n, uint64_t max_hits, int64_t *seed_lo,
                   int64_t *seed_hi, uint64_t *hit_lo, uint64_t *n_hits) {
    if (n == 0 || P[n - 1] == 0) return 0;
    int64_t c = 0, s0 = 0;
    while (s0 < n) {
        uint64_t H = s0 > 0 ? P[s0 - 1] : 0;
        int64_t e;
        if (max_hits == 0 || P[n - 1] - H <= max_hits) {
            e = n - 1;
        } else {
            e = s0;
            while (P[e] < H + max_hits) e++; /* first prefix >= H + MAX (lower bound) */
        }
        seed_lo[c] = s0;
        seed_hi[c] = e;
        hit_lo[c] = H;
        n_hits[c] = P[e] - H;
        c++;
        s0 = e + 1;
    }
    return c;
}

/* ------------------------------------------------------------------ anchors */

/* "C. Hit discovery, C.5": occurrence j of seed s in a chunk with hit base H goes to
 * slot P[s] - 1 - H - j, so each bucket is written backwards from the seed's (inclusive)
 * prefix.  reading: the anchor packs reference end in the low 32 bits and query end in
 * the high 32 bits. */
void orc_anchors(const uint64_t *P, const uint32_t *count, const int64_t *first,
                 const uint32_t *ends, const uint32_t *q_end, int64_t seed_lo,
                 int64_t seed_hi, uint64_t hit_lo, uint64_t *anchors) {
    for (int64_t s = seed_lo; s <= seed_hi; s++) {
        for (uint32_t j = 0; j < count[s]; j++) {
            uint64_t slot = P[s] - 1 - hit_lo - j;
            anchors[slot] = (uint64_t)ends[first[s] + j] | ((uint64_t)q_end[s] << 32);
        }
    }
}

/* Brute force: the same destinations, with the occurrences found by scanning every
 * reference window in ascending position. */
void orc_anchors_brute(const uint8_t *rcodes, int64_t nr, const char *pattern,
                       const uint64_t *P, const uint32_t *kmer, const uint32_t *q_end,
                       int64_t seed_lo, int64_t seed_hi, uint64_t hit_lo,
                       uint64_t *anchors) {
    int32_t care[64], span;
    int w = orc_pattern(pattern, care, &span);
    for (int64_t s = seed_lo; s <= seed_hi; s++) {
        uint64_t j = 0;
        for (int64_t p = 0; w > 0 && p + span <= nr; p++) {
            uint32_t key;
            if (orc_window_key(rcodes, nr, p, care, w, span, &key) && key == kmer[s]) {
                anchors[P[s] - 1 - hit_lo - j] =
                    (uint64_t)(p + span) | ((uint64_t)q_end[s] << 32);
                j++;
            }
        }
    }
}

/* ------------------------------------------------------------------ keep threshold */

/* "D. Score gate, D.2": the host computes once the least integer total that the
 * single-precision comparison keeps.  reading: that comparison is
 * (float)total >= (float)K; the least such int32 is found by bisection, which is valid
 * because int -> float conversion is monotone. */
int32_t orc_keep_threshold(int32_t K) {
    volatile float fk = (float)K;
    int64_t lo = INT32_MIN, hi = INT32_MAX; /* (float)INT32_MAX >= fk for every K */
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        volatile float fm = (float)(int32_t)mid;
        if (fm >= fk) hi = mid; else lo = mid + 1;
    }
    return (int32_t)lo;
}

/* ------------------------------------------------------------------ X-drop */

/* reading: a pair involving N scores n_score; otherwise the substitution matrix entry
 * sub[ref][query]. */
static int32_t orc_sigma(uint8_t r, uint8_t q, const int32_t *sub, int32_t n_score) {
    if (r > 3 || q > 3) return n_score;
    return sub[r * 4 + q];
}

/* One ungapped X-drop extension ("E. X-drop materialization", E.2 and E.3).
 * dir = +1: right, scoring (r+i, q+i) for i = 0, 1, ...  dir = -1: left, scoring
 * (r-1-i, q-1-i) -- the bases before the anchor.  The walk stops at the first base
 * whose running score falls more than xdrop below the best so far (reading: strict
 * '>') or at either sequence end.  best starts at 0 with extent 0 and only a strict
 * improvement moves it, so an equal later maximum never replaces the earliest
 * endpoint.  Returns the best score and its extent (number of bases); *scored, when
 * given, receives how many bases the walk scored. */
static void orc_walk(const uint8_t *rc, int64_t nr, const uint8_t *qc, int64_t nq,
                     int64_t r, int64_t q, int dir, const int32_t *sub, int32_t n_score,
                     int32_t xdrop, int64_t *best, int64_t *ext, int64_t *scored) {
    int64_t s = 0, b = 0, e = 0, n = 0;
    for (;;) {
        int64_t rp = dir > 0 ? r + n : r - 1 - n;
        int64_t qp = dir > 0 ? q + n : q - 1 - n;
        if (rp < 0 || qp < 0 || rp >= nr || qp >= nq) break;
        s += orc_sigma(rc[rp], qc[qp], sub, n_score);
        n += 1;
        if (s > b) {
            b = s;
            e = n;
        } else if (b - s > xdrop) {
            break;
        }
    }
    *best = b;
    *ext = e;
    if (scored) *scored = n;
}

void orc_xdrop(const uint8_t *rc, int64_t nr, const uint8_t *qc, int64_t nq, int64_t r,
               int64_t q, int dir, const int32_t *sub, int32_t n_score, int32_t xdrop,
               int64_t *best, int64_t *ext) {
    orc_walk(rc, nr, qc, nq, r, q, dir, sub, n_score, xdrop, best, ext, 0);
}

/* "D. Score gate, D.2-D.3": per anchor the right and left maxima before the first drop
 * are summed and the anchor is kept (flag 1) iff the total reaches the integer
 * threshold T; otherwise flag 0. */
void orc_gate(const uint64_t *anchors, int64_t n, const uint8_t *rc, int64_t nr,
              const uint8_t *qc, int64_t nq, const int32_t *sub, int32_t n_score,
              int32_t xdrop, int32_t T, uint8_t *flags) {
    for (int64_t i = 0; i < n; i++) {
        int64_t r = (int64_t)(anchors[i] & 0xFFFFFFFFull);
        int64_t q = (int64_t)(anchors[i] >> 32);
        int64_t R, k, L, m;
        orc_xdrop(rc, nr, qc, nq, r, q, +1, sub, n_score, xdrop, &R, &k);
        orc_xdrop(rc, nr, qc, nq, r, q, -1, sub, n_score, xdrop, &L, &m);
        flags[i] = (L + R >= (int64_t)T) ? 1 : 0;
    }
}

/* Diagnostics for tests and workload statistics: the exact L* + R* per anchor and, if
 * steps is given, the number of bases the two walks scored. */
void orc_gate_totals(const uint64_t *anchors, int64_t n, const uint8_t *rc, int64_t nr,
                     const uint8_t *qc, int64_t nq, const int32_t *sub, int32_t n_score,
                     int32_t xdrop, int64_t *totals, int64_t *steps) {
    for (int64_t i = 0; i < n; i++) {
        int64_t r = (int64_t)(anchors[i] & 0xFFFFFFFFull);
        int64_t q = (int64_t)(anchors[i] >> 32);
        int64_t R, k, L, m, nR, nL;
        orc_walk(rc, nr, qc, nq, r, q, +1, sub, n_score, xdrop, &R, &k, &nR);
        orc_walk(rc, nr, qc, nq, r, q, -1, sub, n_score, xdrop, &L, &m, &nL);
        totals[i] = L + R;
        if (steps) steps[i] = nR + nL;
    }
}

/* ------------------------------------------------------------------ compaction */

/* "D. Score gate, D.4": the survivors are the indices of the kept flags in ascending
 * (raw hit) order.  Returns their number. */
int64_t orc_compact(const uint8_t *flags, int64_t n, uint32_t *ids) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; i++)
        if (flags[i]) ids[m++] = (uint32_t)i;
    return m;
}

static double orc_xlog2x(int64_t c) {
    return c > 0 ? (double)c * log2((double)c) : 0.0;
}

/* reading of the "entropy-adjusted decision" ("E. X-drop materialization", E.5), which
 * the pages name without defining: the Shannon entropy, in bits, of the A/C/G/T counts
 * n_b of the reference interval rs..=rs+len (N excluded), n = the sum of the counts:
 * H = (n log2 n - (nA log2 nA + nC log2 nC + nG log2 nG + nT log2 nT)) / n, summed in
 * that order in double precision.  Returns -1 when the interval holds no A/C/G/T. */
double orc_entropy_bits(const uint8_t *rc, int64_t nr, int64_t rs, int64_t len) {
    int64_t cnt[4] = {0, 0, 0, 0};
    for (int64_t t = 0; t <= len; t++) {
        int64_t p = rs + t;
        if (p >= 0 && p < nr && rc[p] < 4) cnt[rc[p]]++;
    }
    int64_t n = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    if (n == 0) return -1.0;
    double s = orc_xlog2x(cnt[0]);
    s = s + orc_xlog2x(cnt[1]);
    s = s + orc_xlog2x(cnt[2]);
    s = s + orc_xlog2x(cnt[3]);
    return (orc_xlog2x(n) - s) / (double)n;
}

/* "E. X-drop materialization", E.1-E.5: each survivor's anchor is extended exactly to
 * both sides; the left extent m shifts both starts, the record's len is the inclusive
 * extent m + k - 1 so the interval is start..=start+len, the score is L* + R*.
 * The decision (reading): entropy_mode 0 accepts iff the score reaches T; entropy_mode 1
 * also requires score * H >= 2 K with H the interval's entropy in bits (orc_entropy_bits;
 * an interval without A/C/G/T is rejected), i.e. the score scaled by H / 2 -- the
 * fraction of the 2-bit maximum -- must still reach K.  Status 1 = accepted, 0 =
 * rejected.  The record is written either way; only accepted slots are output.
 * reading (score width; the pages name no width): a record's score is a 32-bit signed
 * integer.  The walks sum in 64 bits here, and a call in which any record's L* + R* does
 * not fit in int32 is refused: it returns -1 (the arrays are then unspecified) instead
 * of storing a wrapped score.  Returns 0 otherwise. */
int orc_materialize(const uint64_t *anchors, const uint32_t *ids, int64_t n_surv,
                    const uint8_t *rc, int64_t nr, const uint8_t *qc, int64_t nq,
                    const int32_t *sub, int32_t n_score, int32_t xdrop, int32_t T,
                    int32_t K, int32_t entropy_mode, orc_segment_pair *hsp,
                    uint8_t *status) {
    for (int64_t i = 0; i < n_surv; i++) {
        uint64_t a = anchors[ids[i]];
        int64_t r = (int64_t)(a & 0xFFFFFFFFull);
        int64_t q = (int64_t)(a >> 32);
        int64_t R, k, L, m;
        orc_xdrop(rc, nr, qc, nq, r, q, +1, sub, n_score, xdrop, &R, &k);
        orc_xdrop(rc, nr, qc, nq, r, q, -1, sub, n_score, xdrop, &L, &m);
        if (L + R > (int64_t)INT32_MAX || L + R < (int64_t)INT32_MIN) return -1;
        hsp[i].ref_start = (uint32_t)(r - m);
        hsp[i].query_start = (uint32_t)(q - m);
        hsp[i].len = (uint32_t)(m + k - 1);
        hsp[i].score = (int32_t)(L + R);
        int ok = L + R >= (int64_t)T;
        if (ok && entropy_mode == 1) {
            double H = orc_entropy_bits(rc, nr, r - m, m + k - 1);
            ok = H >= 0.0 && (double)(L + R) * H >= 2.0 * (double)K;
        }
        status[i] = ok ? 1 : 0;
    }
    return 0;
}

/* "E. X-drop materialization", E.5: the accepted records in survivor order. */
int64_t orc_compact_hsps(const orc_segment_pair *hsp, const uint8_t *status, int64_t n,
                         orc_segment_pair *out) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; i++)
        if (status[i]) out[m++] = hsp[i];
    return m;
}
