// Host side of libhspz: parameter validation, the keep threshold, reference index and
// query seed construction, the plan (prefix and MAX_HITS chunk walk) and the C ABI.
#include <algorithm>
#include <functional>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "engine.h"
#include "hspz_internal.h"
#include "mat_shared.h"

#define HSPZ_API extern "C" __attribute__((visibility("default")))

namespace hspz {

namespace {

thread_local std::string g_create_error;

int fail(Engine *e, int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (e) e->err = buf;
    else g_create_error = buf;
    return code;
}

#define HIP_TRY(e, call)                                                              \
    do {                                                                              \
        hipError_t _st = (call);                                                      \
        if (_st != hipSuccess)                                                        \
            return fail((e), HSPZ_E_HIP, "%s failed: %s", #call, hipGetErrorString(_st)); \
    } while (0)

template <class T>
void dfree(T *&p) {
    if (p) (void)hipFree(p);
    p = nullptr;
}

template <class T>
int dalloc(Engine *e, T *&p, uint64_t count) {
    dfree(p);
    const size_t bytes = (size_t)std::max<uint64_t>(count, 1) * sizeof(T);
    hipError_t st = hipMalloc(reinterpret_cast<void **>(&p), bytes);
    if (st != hipSuccess) {
        p = nullptr;
        return fail(e, HSPZ_E_NOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(st));
    }
    return HSPZ_OK;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Least int32 t with (float)t >= (float)K: the integer form of the single-precision keep
// comparison.  Searched from K downward and upward; float rounding moves it by at most
// one ulp of K, so the loops are short.
int32_t keep_threshold(int32_t K) {
    const float fk = (float)K;
    int64_t t = K;
    while (t > INT32_MIN && (float)(int32_t)(t - 1) >= fk) t--;
    while ((float)(int32_t)t < fk) t++;
    return (int32_t)t;
}

int ensure_compact(Engine *e, uint64_t n);

// Device buffer freed when it goes out of scope (upload temporaries).
template <class T>
struct DevBuf {
    T *p = nullptr;
    DevBuf() = default;
    DevBuf(const DevBuf &) = delete;
    DevBuf &operator=(const DevBuf &) = delete;
    ~DevBuf() {
        if (p) (void)hipFree(p);
    }
    T *release() {
        T *q = p;
        p = nullptr;
        return q;
    }
};

// Inclusive scan of n u32 counts on the device into prefix: block scans, the block-sum
// scan and the add-back, all on the device (the upload's counts total the indexed
// windows, below 2^32).  Uses the plan buffer's total field; synchronises s before the
// temporaries are freed.
int device_scan(Engine *e, uint32_t *counts, uint64_t n, uint32_t *prefix, hipStream_t s) {
    if (n == 0) return HSPZ_OK;
    const uint64_t nblk = (n + kScanBlock - 1) / kScanBlock;
    DevBuf<uint64_t> bs;
    DevBuf<uint32_t> bo;
    int rc;
    if ((rc = dalloc(e, bs.p, nblk)) || (rc = dalloc(e, bo.p, nblk))) return rc;
    HIP_TRY(e, launch_count_scan(nullptr, counts, n, nullptr, nullptr, counts, nullptr, prefix,
                                 bs.p, s));
    HIP_TRY(e, launch_scan_blocks(bs.p, nblk, bo.p, &e->d_plan->info, s));
    HIP_TRY(e, launch_add_offsets(prefix, n, bo.p, s));
    HIP_TRY(e, hipStreamSynchronize(s));
    return HSPZ_OK;
}

// Device seeder front half, shared by both uploads: copy the ASCII sequence to the
// device, encode the strand into the padded byte array (codes << shift) and the padded
// 4-bit array, compute every window's key and validity, and list the valid windows'
// start positions in ascending order (stable compaction).  *count = valid windows.
int seed_windows(Engine *e, const uint8_t *h_ascii, uint64_t len, int strand, int shift,
                 uint8_t *&bytes, uint32_t *&nibbles, uint32_t *alt, DevBuf<uint32_t> &key,
                 DevBuf<uint32_t> &pos, uint32_t *count, hipStream_t s) {
    *count = 0;
    int rc;
    DevBuf<uint8_t> ascii, valid;
    if ((rc = dalloc(e, ascii.p, len))) return rc;
    if (len)
        HIP_TRY(e, hipMemcpyAsync(ascii.p, h_ascii, len, hipMemcpyHostToDevice, s));
    // 4-bit copy, then at the next 128-byte boundary its twin: the same dwords shifted
    // down by 64 bytes, so any window of at most 64 bytes lies inside one 128-byte line
    // of one of the two
    const uint64_t nib = len + 2 * (uint64_t)kPad4;
    const uint64_t words = (nib + 31) / 32 * 4;
    const uint64_t twin = (words + 31) / 32 * 32;
    if (twin + words > 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "sequence too long");
    if ((rc = dalloc(e, bytes, len + 2 * (uint64_t)kPad))) return rc;
    if ((rc = dalloc(e, nibbles, twin + words))) return rc;
    HIP_TRY(e, launch_encode(ascii.p, len, strand, bytes, shift, nibbles, words, s));
    HIP_TRY(e, hipMemcpyAsync(nibbles + twin, nibbles + kTwinShift,
                              (words - kTwinShift) * sizeof(uint32_t), hipMemcpyDeviceToDevice,
                              s));
    HIP_TRY(e, hipMemsetAsync(nibbles + twin + words - kTwinShift, 0x55,
                              kTwinShift * sizeof(uint32_t), s));
    *alt = (uint32_t)twin;
    const uint64_t nw = len >= (uint64_t)e->span ? len - e->span + 1 : 0;
    if ((rc = dalloc(e, key.p, nw)) || (rc = dalloc(e, pos.p, nw)) ||
        (rc = dalloc(e, valid.p, nw)))
        return rc;
    SeedShape sh{};
    for (int i = 0; i < e->weight; i++) sh.care[i] = e->care[i];
    sh.weight = e->weight;
    HIP_TRY(e, launch_window_keys(bytes + kPad, shift, nw, sh, valid.p, key.p, s));
    if ((rc = ensure_compact(e, nw))) return rc;
    HIP_TRY(e, launch_compact(valid.p, (uint32_t)nw, e->d_cblk, e->d_ctotal, pos.p, nullptr,
                              nullptr, (uint32_t)nw, s));
    HIP_TRY(e, hipMemcpyAsync(e->h_pinned, e->d_ctotal, sizeof(uint32_t), hipMemcpyDeviceToHost,
                              s));
    HIP_TRY(e, hipStreamSynchronize(s));
    *count = e->h_pinned[0];
    return HSPZ_OK;
}

// Host half of the MAX_HITS walk ("C. Hit discovery", C.3), for chunk_walk = 1 and for
// plans with more than kChunkCap chunks.  incl holds the inclusive block sums; the
// device holds block-local prefixes, to which the host adds the block offsets.  With
// chunk_walk = 1 the whole prefix is copied back; otherwise one 1,024-entry prefix block is
// copied per boundary.
int host_walk(Engine *e, uint64_t n, uint64_t total, const std::vector<uint64_t> &incl,
              hipStream_t s) {
    const uint64_t MAX = e->params.max_hits;
    std::vector<uint32_t> full;  // whole prefix (chunk_walk = 1)
    if (e->params.chunk_walk == 1 && total > 0 && MAX != 0 && total > MAX) {
        full.resize(n);
        HIP_TRY(e, hipMemcpyAsync(full.data(), e->d_prefix, n * sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, s));
    }
    HIP_TRY(e, hipStreamSynchronize(s));
    for (uint64_t i = 0; i < full.size(); i++) {
        const uint64_t b = i / kScanBlock;
        full[i] += (uint32_t)(b ? incl[b - 1] : 0);
    }
    std::vector<uint32_t> blkvals(kScanBlock);
    uint64_t s0 = 0, H = 0;
    while (total > 0 && s0 < n) {
        hspz_chunk c{};
        c.seed_lo = e->batch_lo + s0;
        c.hit_lo = H;
        if (MAX == 0 || total - H <= MAX) {
            c.seed_hi = e->batch_lo + n - 1;
            c.n_hits = total - H;
            e->chunks.push_back(c);
            break;
        }
        const uint64_t target = H + MAX;  // first prefix >= target ends the chunk
        uint64_t eidx;
        if (!full.empty()) {
            eidx = (uint64_t)(std::lower_bound(full.begin() + s0, full.end(), target) -
                              full.begin());
        } else {
            const uint64_t b =
                (uint64_t)(std::lower_bound(incl.begin(), incl.end(), target) - incl.begin());
            const uint64_t lo = b * kScanBlock, cnt = std::min<uint64_t>(kScanBlock, n - lo);
            HIP_TRY(e, hipMemcpy(blkvals.data(), e->d_prefix + lo, cnt * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
            for (uint64_t j = 0; j < cnt; j++) blkvals[j] += (uint32_t)(b ? incl[b - 1] : 0);
            eidx = lo + (uint64_t)(std::lower_bound(blkvals.begin(), blkvals.begin() + cnt,
                                                    target) - blkvals.begin());
        }
        if (eidx >= n || eidx < s0)
            return fail(e, HSPZ_E_HIP, "chunk walk lost its boundary (internal error)");
        const uint64_t Pe = !full.empty() ? full[eidx] : blkvals[eidx % kScanBlock];
        c.seed_hi = e->batch_lo + eidx;
        c.n_hits = Pe - H;
        e->chunks.push_back(c);
        H = Pe;
        s0 = eidx + 1;
    }
    return HSPZ_OK;
}

// Shared by hspz_plan and hspz_debug_plan_counts once counts and block-local prefixes
// are on the device.  chunk_walk = 0: the 64-bit block-sum scan, the add-back and the
// chunk walk run on the device, and one copy brings back the total and the chunk list.
// chunk_walk = 1: the host scans the block sums and walks the whole prefix.  A total
// over 2^32 - 1 is refused either way.
// queued is called, when not null, once the plan's copy to the host is queued and before
// the host waits for it: work it queues runs while the host waits.
int finish_plan(Engine *e, uint64_t n, hipStream_t s, uint64_t *total_hits, uint32_t *n_chunks,
                const std::function<int()> &queued) {
    const uint64_t nblk = (n + kScanBlock - 1) / kScanBlock;
    e->chunks.clear();
    std::vector<uint64_t> incl;  // inclusive block sums, for the host walk
    uint64_t total = 0;
    bool walked = false;
    auto refuse = [&](uint64_t t) {
        e->has_plan = false;
        return fail(e, HSPZ_E_OVERFLOW,
                    "batch total exceeds the 32-bit hit index (%llu hits or more); refused",
                    (unsigned long long)t);
    };
    auto host_incl = [&]() -> int {
        std::vector<uint64_t> blk(nblk);
        if (nblk) {
            HIP_TRY(e, hipMemcpyAsync(blk.data(), e->d_blksum, nblk * sizeof(uint64_t),
                                      hipMemcpyDeviceToHost, s));
            HIP_TRY(e, hipStreamSynchronize(s));
        }
        incl.resize(nblk);
        uint64_t acc = 0;
        for (uint64_t b = 0; b < nblk; b++) incl[b] = acc += blk[b];
        return HSPZ_OK;
    };
    int rc;
    if (e->params.chunk_walk == 0) {
        HIP_TRY(e, launch_scan_blocks(e->d_blksum, nblk, e->d_blkoff, &e->d_plan->info, s));
        HIP_TRY(e, launch_chunk_walk(PrefixView{e->d_prefix, e->d_blkoff, 0}, n,
                                     e->params.max_hits, e->batch_lo, e->d_plan, s));
        HIP_TRY(e, hipMemcpyAsync(e->h_plan, e->d_plan, sizeof(PlanBuf), hipMemcpyDeviceToHost,
                                  s));
        if (!e->plan_ev) HIP_TRY(e, hipEventCreateWithFlags(&e->plan_ev, hipEventDisableTiming));
        HIP_TRY(e, hipEventRecord(e->plan_ev, s));
        if (queued && (rc = queued())) return rc;
        HIP_TRY(e, hipEventSynchronize(e->plan_ev));
        total = e->h_plan->info.total;
        if (total > 0xFFFFFFFFull) return refuse(total);
        const uint32_t nc = e->h_plan->info.n_chunks;
        if (nc <= kChunkCap) {
            e->chunks.assign(e->h_plan->chunks, e->h_plan->chunks + nc);
            walked = true;
        } else if ((rc = host_incl())) {
            return rc;
        }
    } else {
        if ((rc = host_incl())) return rc;
        total = nblk ? incl.back() : 0;
        if (total > 0xFFFFFFFFull) return refuse(total);
        std::vector<uint32_t> off(nblk);  // exclusive block offsets
        for (uint64_t b = 0; b < nblk; b++) off[b] = (uint32_t)(b ? incl[b - 1] : 0);
        if (nblk) {
            HIP_TRY(e, hipMemcpyAsync(e->d_blkoff, off.data(), nblk * sizeof(uint32_t),
                                      hipMemcpyHostToDevice, s));
        }
    }
    if (!walked && (rc = host_walk(e, n, total, incl, s))) return rc;
    if (e->params.chunk_walk != 0 && queued && (rc = queued())) return rc;
    e->total = total;
    e->has_plan = true;
    *total_hits = total;
    *n_chunks = (uint32_t)e->chunks.size();
    return HSPZ_OK;
}

// Per-batch and per-chunk scratch grows by at least a quarter at a time, so batches and
// chunks a few seeds or anchors apart do not reallocate (and synchronise) pass after pass.
int ensure_batch(Engine *e, uint64_t n) {
    if (n <= e->cap_batch && e->d_count) return HSPZ_OK;
    const uint64_t cap = std::max<uint64_t>({n, 1, e->cap_batch + e->cap_batch / 4});
    const uint64_t nblk = (cap + kScanBlock - 1) / kScanBlock;
    int rc;
    if ((rc = dalloc(e, e->d_count, cap))) return rc;
    if ((rc = dalloc(e, e->d_first, cap))) return rc;
    if ((rc = dalloc(e, e->d_prefix, cap))) return rc;
    if ((rc = dalloc(e, e->d_blksum, nblk))) return rc;
    if ((rc = dalloc(e, e->d_blkoff, nblk))) return rc;
    e->cap_batch = cap;
    return HSPZ_OK;
}

int ensure_compact(Engine *e, uint64_t n) {
    const uint64_t need = (n + kCompactBlock - 1) / kCompactBlock + 1;
    if (need <= e->cap_cblk && e->d_cblk) return HSPZ_OK;
    const uint64_t nblk = std::max<uint64_t>(need, e->cap_cblk + e->cap_cblk / 4);
    int rc = dalloc(e, e->d_cblk, nblk);
    if (rc) return rc;
    e->cap_cblk = nblk;
    return HSPZ_OK;
}

int set_device(Engine *e) {
    HIP_TRY(e, hipSetDevice(e->device));
    return HSPZ_OK;
}

// Whether the key-grouped first stage can serve this engine at all (gate_mode 0 or 5 with
// the window gate's preconditions).
bool kg_wanted(const Engine *e) {
    return e->window_ok && (e->params.gate_mode == 0 || e->params.gate_mode == 5);
}

// Each run's bucket size and start, once both the grouping and a reference are there.
int kg_run_info(Engine *e, hipStream_t s) {
    e->kg_ready = false;
    if (!e->kg_built || !e->has_ref) return HSPZ_OK;
    int rc;
    if ((rc = dalloc(e, e->d_kg_run_c, e->kg_n_runs)) ||
        (rc = dalloc(e, e->d_kg_run_first, e->kg_n_runs)))
        return rc;
    HIP_TRY(e, launch_kg_run_info(e->d_kg_qk, e->d_kg_runs, e->kg_n_runs, e->d_end,
                                  e->d_kg_run_c, e->d_kg_run_first, s));
    HIP_TRY(e, hipStreamSynchronize(s));
    e->kg_ready = true;
    return HSPZ_OK;
}

// The strand's seeds grouped by k-mer (the key-grouped first stage): a stable radix sort
// of (k-mer, seed) pairs, the query ends in that order, and the start of each k-mer's run.
int kg_build(Engine *e, hipStream_t s) {
    e->kg_built = e->kg_ready = false;
    e->kg_n_runs = 0;
    if (!kg_wanted(e) || e->n_seeds == 0) return HSPZ_OK;
    const uint32_t n = (uint32_t)e->n_seeds;
    int rc;
    DevBuf<uint32_t> kb, vb;
    if ((rc = dalloc(e, e->d_kg_qk, n)) || (rc = dalloc(e, e->d_kg_qs, n)) ||
        (rc = dalloc(e, kb.p, n)) || (rc = dalloc(e, vb.p, n)))
        return rc;
    HIP_TRY(e, hipMemcpyAsync(e->d_kg_qk, e->d_kmer, (uint64_t)n * sizeof(uint32_t),
                              hipMemcpyDeviceToDevice, s));
    HIP_TRY(e, launch_iota(e->d_kg_qs, n, s));
    {
        const uint64_t nh = 256ull * radix_blocks(n);
        DevBuf<uint32_t> hist, incl;
        if ((rc = dalloc(e, hist.p, nh)) || (rc = dalloc(e, incl.p, nh))) return rc;
        uint32_t *ka = e->d_kg_qk, *va = e->d_kg_qs, *kb2 = kb.p, *vb2 = vb.p;
        for (int shift = 0; shift < 2 * e->weight; shift += 8) {
            HIP_TRY(e, launch_radix_hist(ka, n, shift, hist.p, s));
            if ((rc = device_scan(e, hist.p, nh, incl.p, s))) return rc;
            HIP_TRY(e, launch_radix_scatter(ka, va, n, shift, incl.p, hist.p, kb2, vb2, s));
            std::swap(ka, kb2);
            std::swap(va, vb2);
        }
        if (ka != e->d_kg_qk) {  // an odd number of passes: the result is in kb / vb
            HIP_TRY(e, hipMemcpyAsync(e->d_kg_qk, ka, (uint64_t)n * sizeof(uint32_t),
                                      hipMemcpyDeviceToDevice, s));
            HIP_TRY(e, hipMemcpyAsync(e->d_kg_qs, va, (uint64_t)n * sizeof(uint32_t),
                                      hipMemcpyDeviceToDevice, s));
        }
    }
    if ((rc = dalloc(e, e->d_kg_qe, n))) return rc;
    HIP_TRY(e, launch_kg_gather(e->d_kg_qs, n, e->d_qend, e->d_kg_qe, s));
    {
        DevBuf<uint8_t> flag;
        if ((rc = dalloc(e, flag.p, n)) || (rc = dalloc(e, e->d_kg_runs, n)) ||
            (rc = ensure_compact(e, n)))
            return rc;
        HIP_TRY(e, launch_kg_run_flags(e->d_kg_qk, n, flag.p, s));
        HIP_TRY(e, launch_compact(flag.p, n, e->d_cblk, e->d_ctotal, e->d_kg_runs, nullptr,
                                  nullptr, n, s));
        HIP_TRY(e, hipMemcpyAsync(e->h_pinned, e->d_ctotal, sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, s));
        HIP_TRY(e, hipStreamSynchronize(s));
    }
    e->kg_n_runs = e->h_pinned[0];
    if ((rc = dalloc(e, e->d_kg_run_span, e->kg_n_runs))) return rc;
    HIP_TRY(e, launch_kg_run_span(e->d_kg_qs, n, e->d_kg_runs, e->kg_n_runs, e->d_kg_run_span,
                                  s));
    e->kg_built = true;
    return kg_run_info(e, s);
}

// Per-chunk scratch of the key-grouped stage for the current runs and n_waves waves.
int ensure_kg(Engine *e, uint64_t n_waves) {
    int rc;
    const uint64_t nr = std::max<uint64_t>(e->kg_n_runs, 1);
    if (nr > e->cap_kg || !e->d_kg_G) {
        const uint64_t nblk = (nr + kScanBlock - 1) / kScanBlock;
        if ((rc = dalloc(e, e->d_kg_G, nr)) ||
            (rc = dalloc(e, e->d_kg_a, nr)) || (rc = dalloc(e, e->d_kg_m, nr)) ||
            (rc = dalloc(e, e->d_kg_blksum, nblk)) || (rc = dalloc(e, e->d_kg_blkoff, nblk)) ||
            (rc = dalloc(e, e->d_kg_info, 1))) {
            e->cap_kg = 0;
            return rc;
        }
        e->cap_kg = nr;
    }
    if (n_waves > e->cap_kg_dir || !e->d_kg_dir) {
        const uint64_t want = std::max<uint64_t>({n_waves, 1024, e->cap_kg_dir + e->cap_kg_dir / 4});
        if ((rc = dalloc(e, e->d_kg_dir, want))) {
            e->cap_kg_dir = 0;
            return rc;
        }
        e->cap_kg_dir = want;
    }
    return HSPZ_OK;
}

}  // namespace

Engine::~Engine() {
    (void)hipSetDevice(device);
    dfree(d_end);
    dfree(d_ctab);
    dfree(d_cnib);
    for (uint32_t **q : {&d_kg_qk, &d_kg_qs, &d_kg_qe, &d_kg_runs, &d_kg_run_c, &d_kg_run_first,
                         &d_kg_G, &d_kg_a, &d_kg_m, &d_kg_dir, &d_kg_blkoff})
        dfree(*q);
    dfree(d_kg_blksum);
    dfree(d_kg_info);
    dfree(d_kg_run_span);
    dfree(d_pos);
    dfree(d_ref);
    dfree(d_qry);
    dfree(d_ref4);
    dfree(d_qry4);
    dfree(d_defer);
    dfree(d_defer_a);
    dfree(bb_flags);
    dfree(bb_anchors);
    dfree(bb_ids);
    dfree(d_defer_cnt);
    dfree(d_kmer);
    dfree(d_qend);
    dfree(d_count);
    dfree(d_first);
    dfree(d_prefix);
    dfree(d_blksum);
    dfree(d_blkoff);
    dfree(d_cblk);
    dfree(d_ctotal);
    if (mat) {
        dfree(mat->ka);
        dfree(mat->va);
        dfree(mat->kb);
        dfree(mat->vb);
        dfree(mat->hist);
        dfree(mat->incl);
        dfree(mat->side);
        dfree(mat->sum);
        dfree(mat->off);
        dfree(mat->info);
        dfree(mat->list);
        dfree(mat->lcnt);
        dfree(mat->sa);
        dfree(mat->sblk);
        delete mat;
    }
    dfree(d_bsa);
    dfree(d_bsi);
    dfree(d_bhist);
    dfree(d_bincl);
    dfree(d_bsum);
    dfree(d_boff);
    dfree(d_binfo);
    dfree(d_plan);
    dfree(d_dir);
    for (int b = 0; b < 2; b++) {
        dfree(rb_anchors[b]);
        dfree(rb_flags[b]);
        dfree(rb_ids[b]);
    }
    if (copy_s) (void)hipStreamSynchronize(copy_s);
    dfree(rb_hsp);
    dfree(rb_out[0]);
    dfree(rb_out[1]);
    dfree(rb_status);
    for (hipEvent_t ev : gate_ev)
        if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : count_ev)
        if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : copied_ev)
        if (ev) (void)hipEventDestroy(ev);
    if (plan_ev) (void)hipEventDestroy(plan_ev);
    if (copy_s) (void)hipStreamDestroy(copy_s);
    if (h_pinned) (void)hipHostFree(h_pinned);
    if (h_plan) (void)hipHostFree(h_plan);
    if (h_rec) (void)hipHostFree(h_rec);
}

void Engine::free_plan() {
    has_plan = false;
    plan_expandable = false;
    plan_aux = false;
    chunks.clear();
    total = 0;
}

}  // namespace hspz

using namespace hspz;

// Scratch of hspz_score_gate_noalloc, which allocates nothing: the two deferred-anchor
// lists of the window gate (each able to hold every anchor of a call) and its two
// counters, in one statically sized array that every GPU the library runs on holds until
// the process ends.  Layout in u32 words: [0, 16) counters, then list 1, then list 2.
constexpr uint64_t kNoAllocMaxAnchors = 1ull << 23;
constexpr uint64_t kNoAllocWords = 16 + 2 * kNoAllocMaxAnchors;  // 64 MiB + 64 B
static __device__ __align__(256) uint32_t scratch[kNoAllocWords];

// scratch's device address on each device, resolved once per device with that device
// current (the host-side name of the array is not a device address).
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint32_t *g_scratch_ptr[kMaxDevices] = {};

static int resolve_scratch(Engine *e) {
    if (e->device >= kMaxDevices)
        return fail(e, HSPZ_E_INVALID, "device %d beyond the scratch table", e->device);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[e->device]) return HSPZ_OK;
    void *ptr = nullptr;
    HIP_TRY(e, hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(e, HSPZ_E_HIP, "hipGetSymbolAddress returned NULL for scratch");
    g_scratch_ptr[e->device] = static_cast<uint32_t *>(ptr);
    return HSPZ_OK;
}

static int impl_hspz_engine_create(const hspz_params *p, hspz_engine **out) {
    if (!out) return fail(nullptr, HSPZ_E_INVALID, "out is NULL");
    *out = nullptr;
    if (!p || !p->seed_pattern) return fail(nullptr, HSPZ_E_INVALID, "params or pattern NULL");
    const size_t L = strlen(p->seed_pattern);
    std::vector<int32_t> care;
    for (size_t i = 0; i < L; i++) {
        if (p->seed_pattern[i] == '1') care.push_back((int32_t)i);
        else if (p->seed_pattern[i] != '0')
            return fail(nullptr, HSPZ_E_INVALID, "seed pattern may hold only '0' and '1'");
    }
    if (L == 0 || L > 64 || care.empty() || care.size() > 14 || p->seed_pattern[0] != '1' ||
        p->seed_pattern[L - 1] != '1')
        return fail(nullptr, HSPZ_E_INVALID,
                    "seed pattern must start and end with '1', weight 1..14, span <= 64");
    for (int i = 0; i < 16; i++)
        if (p->sub[i] > 10000 || p->sub[i] < -10000)
            return fail(nullptr, HSPZ_E_INVALID, "|sub| must be <= 10000");
    if (p->n_score > 10000 || p->n_score < -10000)
        return fail(nullptr, HSPZ_E_INVALID, "|n_score| must be <= 10000");
    if (p->xdrop < 0 || p->xdrop > 1000000)
        return fail(nullptr, HSPZ_E_INVALID, "xdrop must be in 0..1000000");
    // the device sums scores in 32 bits: a threshold up to 2^30 keeps R* + L* below 2^31
    // while the gate still needs both (each walk stops once the flag is known)
    if (p->hsp_threshold < 1 || p->hsp_threshold > (1 << 30))
        return fail(nullptr, HSPZ_E_INVALID, "hsp_threshold must be in 1..2^30");
    if (p->expand_mode < 0 || p->expand_mode > 2)
        return fail(nullptr, HSPZ_E_INVALID, "expand_mode must be 0, 1 or 2");
    if (p->chunk_walk < 0 || p->chunk_walk > 1)
        return fail(nullptr, HSPZ_E_INVALID, "chunk_walk must be 0 or 1");
    if (p->entropy_mode < 0 || p->entropy_mode > 1)
        return fail(nullptr, HSPZ_E_INVALID, "entropy_mode must be 0 or 1");
    if (p->ref_buckets < 0 || p->ref_buckets > 256)
        return fail(nullptr, HSPZ_E_INVALID, "ref_buckets must be in 0..256");
    if (p->materialize_mode < 0 || p->materialize_mode > 2)
        return fail(nullptr, HSPZ_E_INVALID, "materialize_mode must be 0, 1 or 2");
    if (p->gate_mode < 0 || p->gate_mode > 5)
        return fail(nullptr, HSPZ_E_INVALID, "gate_mode must be 0, 1, 2, 3, 4 or 5");

    Engine *e = new (std::nothrow) Engine();
    if (!e) return fail(nullptr, HSPZ_E_NOMEM, "engine allocation failed");
    e->params = *p;
    e->pattern = p->seed_pattern;
    e->params.seed_pattern = e->pattern.c_str();
    e->care = care;
    e->span = (int)L;
    e->weight = (int)care.size();
    e->device = p->device;
    e->T = keep_threshold(p->hsp_threshold);

    // Score table indexed by ref*8 + query (codes 0..3, N = 4, edge = 5).
    int32_t smax = std::max<int32_t>(p->n_score, 0);
    for (int r = 0; r < 8; r++) {
        for (int q = 0; q < 8; q++) {
            int32_t v;
            if (r == kCodeEdge || q == kCodeEdge || r > kCodeEdge || q > kCodeEdge)
                v = -(p->xdrop + 1);
            else if (r == kCodeN || q == kCodeN) v = p->n_score;
            else v = p->sub[r * 4 + q];
            e->sp.tab[(r << kRefShift) | q] = v;
        }
    }
    for (int i = 0; i < 16; i++) smax = std::max(smax, p->sub[i]);
    // Largest block B with (B - 1) * max score <= xdrop (see the gate kernel).
    e->block_bases = 1;
    for (int b : {8, 4, 2}) {
        if ((int64_t)(b - 1) * smax <= p->xdrop) {
            e->block_bases = b;
            break;
        }
    }
    e->sp.xdrop = p->xdrop;
    e->sp.T = e->T;
    e->sp.K = p->hsp_threshold;
    e->sp.entropy_mode = p->entropy_mode;
    // Windowed gate: exact when eight-base blocks are (B = 8 above) and every pair score,
    // the edge score included, fits 16 bits.
    e->window_ok = e->block_bases == 8 && p->xdrop + 1 <= 32767;
    for (int r = 0; r < 6; r++) {
        for (int q = 0; q < 16; q++) {
            const int32_t v = q < 6 ? e->sp.tab[(r << kRefShift) | q] : -(p->xdrop + 1);
            if (v < -32768 || v > 32767) e->window_ok = false;
            e->wp.tab[r * 16 + q] = (int16_t)v;
        }
    }
    e->wp.xdrop = p->xdrop;
    e->wp.T = e->T;
    if (p->gate_mode >= 2 && !e->window_ok) {
        delete e;
        return fail(nullptr, HSPZ_E_INVALID,
                    "gate_modes 2 to 5 need 7 * max score <= xdrop and 16-bit pair scores");
    }
    // the device last, so that every parameter error is reported as such on any machine
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || p->device < 0 || p->device >= ndev) {
        delete e;
        return fail(nullptr, HSPZ_E_INVALID, "device %d not available (%d devices)", p->device,
                    ndev);
    }
    int rc = set_device(e);
    if (rc) {
        g_create_error = e->err;
        delete e;
        return rc;
    }
    if (hipHostMalloc(reinterpret_cast<void **>(&e->h_pinned), 64 * sizeof(uint32_t)) !=
            hipSuccess ||
        hipHostMalloc(reinterpret_cast<void **>(&e->h_plan), sizeof(PlanBuf)) != hipSuccess ||
        dalloc(e, e->d_ctotal, 16) != HSPZ_OK || dalloc(e, e->d_defer_cnt, 16) != HSPZ_OK ||
        dalloc(e, e->d_plan, 1) != HSPZ_OK) {
        g_create_error = "pinned/device staging allocation failed";
        delete e;
        return HSPZ_E_NOMEM;
    }
    if ((rc = resolve_scratch(e))) {
        g_create_error = e->err;
        delete e;
        return rc;
    }
    *out = reinterpret_cast<hspz_engine *>(e);
    return HSPZ_OK;
}

HSPZ_API int hspz_engine_destroy(hspz_engine *engine) {
    delete reinterpret_cast<Engine *>(engine);
    return HSPZ_OK;
}

HSPZ_API int32_t hspz_keep_threshold(const hspz_engine *engine) {
    return engine ? reinterpret_cast<const Engine *>(engine)->T : 0;
}

HSPZ_API const char *hspz_last_error(const hspz_engine *engine) {
    if (!engine) return g_create_error.c_str();
    return reinterpret_cast<const Engine *>(engine)->err.c_str();
}

static int impl_hspz_upload_reference(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                                      void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!h_ascii && len) return fail(e, HSPZ_E_INVALID, "reference pointer is NULL");
    if (len >= 0xFFFFFFFFull - kPad) return fail(e, HSPZ_E_INVALID, "reference too long");
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    e->free_plan();
    e->has_ref = false;

    // Device indexer ("C. Hit discovery", C.1 index table): the valid windows' keys and
    // reference ends in position order; bucket sizes by an atomic histogram, cumulative
    // ends by a scan (leading 0), and the ends grouped by key with a stable radix sort, so
    // they ascend within each bucket.
    DevBuf<uint32_t> key, pos;
    uint32_t nwin = 0;
    if ((rc = seed_windows(e, h_ascii, len, 0, kRefShift, e->d_ref, e->d_ref4, &e->wp.ref4_alt,
                           key, pos, &nwin, s)))
        return rc;
    const uint64_t nb = 1ull << (2 * e->weight);
    DevBuf<uint32_t> ka, va, kb, vb, cnt;
    if ((rc = dalloc(e, ka.p, nwin)) || (rc = dalloc(e, va.p, nwin)) ||
        (rc = dalloc(e, kb.p, nwin)) || (rc = dalloc(e, vb.p, nwin)) ||
        (rc = dalloc(e, cnt.p, nb)) || (rc = dalloc(e, e->d_end, nb + 1)))
        return rc;
    HIP_TRY(e, launch_gather_pairs(pos.p, nwin, key.p, (uint32_t)e->span, ka.p, va.p, s));
    HIP_TRY(e, hipMemsetAsync(cnt.p, 0, nb * sizeof(uint32_t), s));
    HIP_TRY(e, launch_key_hist(ka.p, nwin, cnt.p, s));
    {
        // the scan's vector stores want a 16-byte aligned output, so scan into a
        // temporary and copy it behind the leading 0
        DevBuf<uint32_t> ends;
        if ((rc = dalloc(e, ends.p, nb))) return rc;
        if ((rc = device_scan(e, cnt.p, nb, ends.p, s))) return rc;
        HIP_TRY(e, launch_set_u32(e->d_end, 0u, s));
        HIP_TRY(e, hipMemcpyAsync(e->d_end + 1, ends.p, nb * sizeof(uint32_t),
                                  hipMemcpyDeviceToDevice, s));
        // the packed form the plan's lookups read (two uint4 per record)
        if ((rc = dalloc(e, e->d_ctab, 2ull * count_table_records(nb)))) return rc;
        HIP_TRY(e, launch_count_table(e->d_end, nb, e->d_ctab, s));
        // and the 4-bit counts the plan reads
        if ((rc = dalloc(e, e->d_cnib, count_nibble_words(nb)))) return rc;
        HIP_TRY(e, launch_count_nibbles(e->d_end, nb, e->d_cnib, s));
        HIP_TRY(e, hipStreamSynchronize(s));
    }
    const uint32_t nblk = radix_blocks(nwin);
    const uint64_t nh = 256ull * nblk;
    DevBuf<uint32_t> hist, incl;
    if ((rc = dalloc(e, hist.p, nh)) || (rc = dalloc(e, incl.p, nh))) return rc;
    for (int shift = 0; shift < 2 * e->weight; shift += 8) {
        HIP_TRY(e, launch_radix_hist(ka.p, nwin, shift, hist.p, s));
        if ((rc = device_scan(e, hist.p, nh, incl.p, s))) return rc;
        HIP_TRY(e, launch_radix_scatter(ka.p, va.p, nwin, shift, incl.p, hist.p, kb.p, vb.p, s));
        std::swap(ka.p, kb.p);
        std::swap(va.p, vb.p);
    }
    HIP_TRY(e, hipStreamSynchronize(s));
    dfree(e->d_pos);
    e->d_pos = va.release();
    if (!e->d_pos && (rc = dalloc(e, e->d_pos, 1))) return rc;
    e->n_index = nwin;
    e->n_ref = len;
    // bucketed gate: automatic slices of 2^22 bases (2 MiB of 4-bit codes, half of one
    // XCD's 4 MB L2), wider for references that would need more than 256 of them; or the
    // narrowest power-of-two width giving at most ref_buckets slices
    const uint64_t most = e->params.ref_buckets ? (uint64_t)e->params.ref_buckets : 256;
    e->slice_shift = e->params.ref_buckets ? 0 : 22;
    while ((len >> e->slice_shift) + 1 > most) e->slice_shift++;
    e->n_slices = (uint32_t)(len >> e->slice_shift) + 1;
    e->sp.n_ref = (uint32_t)len;
    e->wp.n_ref = (uint32_t)len;
    e->has_ref = true;
    return kg_run_info(e, s);  // the grouped seeds' buckets come from this reference
}

static int impl_hspz_upload_query(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                                  int32_t strand, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!h_ascii && len) return fail(e, HSPZ_E_INVALID, "query pointer is NULL");
    if (strand != 0 && strand != 1) return fail(e, HSPZ_E_INVALID, "strand must be 0 or 1");
    if (len >= 0xFFFFFFFFull - kPad) return fail(e, HSPZ_E_INVALID, "query too long");
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    e->free_plan();
    e->has_qry = false;

    // Device seeder: every valid window of the strand, in ascending position, with its
    // packed k-mer and query end.
    DevBuf<uint32_t> key, pos;
    uint32_t ns = 0;
    if ((rc = seed_windows(e, h_ascii, len, strand, 0, e->d_qry, e->d_qry4, &e->wp.qry4_alt, key,
                           pos, &ns, s)))
        return rc;
    if ((rc = dalloc(e, e->d_kmer, ns)) || (rc = dalloc(e, e->d_qend, ns))) return rc;
    HIP_TRY(e, launch_gather_pairs(pos.p, ns, key.p, (uint32_t)e->span, e->d_kmer, e->d_qend, s));
    e->h_seed_start.resize(ns);
    if (ns)
        HIP_TRY(e, hipMemcpyAsync(e->h_seed_start.data(), pos.p, (uint64_t)ns * sizeof(uint32_t),
                                  hipMemcpyDeviceToHost, s));
    HIP_TRY(e, hipStreamSynchronize(s));
    e->n_qry = len;
    e->sp.n_qry = (uint32_t)len;
    e->wp.n_qry = (uint32_t)len;
    e->n_seeds = ns;
    e->strand = strand;
    e->has_qry = true;
    return kg_build(e, s);
}

// Caller seeds in place of the device seeder's, for the current query strand.
static int impl_hspz_upload_seeds(hspz_engine *engine, const uint32_t *h_kmer,
                                  const uint32_t *h_q_end, uint64_t n, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_qry)
        return fail(e, HSPZ_E_STATE, "upload the query strand first: the walks read it");
    if (n && (!h_kmer || !h_q_end)) return fail(e, HSPZ_E_INVALID, "seed arrays are NULL");
    if (n >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "at most 2^32 - 2 seeds");
    const uint64_t nkeys = 1ull << (2 * e->weight);
    const uint64_t span = (uint64_t)e->span;
    for (uint64_t i = 0; i < n; i++) {
        if (h_kmer[i] >= nkeys)
            return fail(e, HSPZ_E_INVALID, "seed %llu: k-mer %u is not below 4^%d",
                        (unsigned long long)i, h_kmer[i], e->weight);
        if (h_q_end[i] < span || h_q_end[i] > e->n_qry)
            return fail(e, HSPZ_E_INVALID, "seed %llu: query end %u is outside [%llu, %llu]",
                        (unsigned long long)i, h_q_end[i], (unsigned long long)span,
                        (unsigned long long)e->n_qry);
        if (i && h_q_end[i] < h_q_end[i - 1])
            return fail(e, HSPZ_E_INVALID, "seed %llu: query ends must not decrease",
                        (unsigned long long)i);
    }
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    e->free_plan();
    std::vector<uint32_t> start(n);  // window starts, for hspz_seed_range
    for (uint64_t i = 0; i < n; i++) start[i] = h_q_end[i] - (uint32_t)span;
    e->n_seeds = 0;  // no seeds until the new ones have landed
    e->h_seed_start.clear();
    if ((rc = dalloc(e, e->d_kmer, n)) || (rc = dalloc(e, e->d_qend, n))) return rc;
    if (n) {
        HIP_TRY(e, hipMemcpyAsync(e->d_kmer, h_kmer, n * sizeof(uint32_t),
                                  hipMemcpyHostToDevice, s));
        HIP_TRY(e, hipMemcpyAsync(e->d_qend, h_q_end, n * sizeof(uint32_t),
                                  hipMemcpyHostToDevice, s));
    }
    HIP_TRY(e, hipStreamSynchronize(s));
    e->h_seed_start.swap(start);
    e->n_seeds = n;
    return kg_build(e, s);
}

HSPZ_API uint64_t hspz_num_seeds(const hspz_engine *engine) {
    const Engine *e = reinterpret_cast<const Engine *>(engine);
    return (e && e->has_qry) ? e->n_seeds : 0;
}

static int impl_hspz_seed_range(const hspz_engine *engine, uint64_t pos_lo, uint64_t pos_hi,
                                uint64_t *seed_lo, uint64_t *seed_hi) {
    const Engine *ce = reinterpret_cast<const Engine *>(engine);
    Engine *e = const_cast<Engine *>(ce);
    if (!e) return HSPZ_E_INVALID;
    if (!seed_lo || !seed_hi) return fail(e, HSPZ_E_INVALID, "NULL output");
    if (!e->has_qry) return fail(e, HSPZ_E_STATE, "no query uploaded");
    const auto &v = e->h_seed_start;
    auto lb = [&](uint64_t x) {
        if (x > 0xFFFFFFFFull) return (uint64_t)v.size();
        return (uint64_t)(std::lower_bound(v.begin(), v.end(), (uint32_t)x) - v.begin());
    };
    *seed_lo = lb(pos_lo);
    *seed_hi = std::max(*seed_lo, lb(pos_hi));
    return HSPZ_OK;
}

// hspz_plan, with finish_plan's queued hook (hspz_run_batch queues work there).
// The per-seed counts and bucket starts of the planned batch ("C. Hit discovery", C.1),
// which the plan leaves out: the same lookups again, writing those two arrays and no
// prefix.  Queued on s once per plan, by the first caller that reads them (the raw-order
// expansion and fused gate stage, hspz_get_plan_arrays).
static int ensure_plan_aux(Engine *e, hipStream_t s) {
    if (e->plan_aux) return HSPZ_OK;
    if (e->batch_n)
        HIP_TRY(e, launch_count_scan(e->d_kmer + e->batch_lo, nullptr, e->batch_n, e->d_end,
                                     e->d_ctab, e->d_count, e->d_first, nullptr, nullptr, s));
    e->plan_aux = true;
    return HSPZ_OK;
}

static int plan_batch(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi, void *stream,
                      uint64_t *total_hits, uint32_t *n_chunks,
                      const std::function<int()> &queued) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!total_hits || !n_chunks) return fail(e, HSPZ_E_INVALID, "NULL output");
    *total_hits = 0;
    *n_chunks = 0;
    if (!e->has_ref || !e->has_qry)
        return fail(e, HSPZ_E_STATE, "plan needs an uploaded reference and query");
    if (seed_lo > seed_hi || seed_hi > e->n_seeds)
        return fail(e, HSPZ_E_INVALID, "seed range [%llu, %llu) outside 0..%llu",
                    (unsigned long long)seed_lo, (unsigned long long)seed_hi,
                    (unsigned long long)e->n_seeds);
    int rc = set_device(e);
    if (rc) return rc;
    e->free_plan();
    hipStream_t s = as_stream(stream);
    const uint64_t n = seed_hi - seed_lo;
    if ((rc = ensure_batch(e, n))) return rc;
    e->batch_lo = seed_lo;
    e->batch_n = n;
    // the prefix alone: the per-seed counts and bucket starts only where a caller needs
    // them (ensure_plan_aux)
    HIP_TRY(e, launch_count_prefix(e->d_kmer + seed_lo, n, e->d_end, e->d_cnib, e->d_prefix,
                                   e->d_blksum, s));
    rc = finish_plan(e, n, s, total_hits, n_chunks, queued);
    if (rc) {
        *total_hits = 0;
        *n_chunks = 0;
        return rc;
    }
    e->plan_expandable = true;
    return HSPZ_OK;
}

static int impl_hspz_plan(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi, void *stream,
                          uint64_t *total_hits, uint32_t *n_chunks) {
    return plan_batch(engine, seed_lo, seed_hi, stream, total_hits, n_chunks, nullptr);
}

static int impl_hspz_debug_plan_counts(hspz_engine *engine, const uint32_t *h_counts, uint64_t n,
                                       void *stream, uint64_t *total_hits, uint32_t *n_chunks) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!total_hits || !n_chunks || (!h_counts && n))
        return fail(e, HSPZ_E_INVALID, "NULL argument");
    *total_hits = 0;
    *n_chunks = 0;
    int rc = set_device(e);
    if (rc) return rc;
    e->free_plan();
    hipStream_t s = as_stream(stream);
    if ((rc = ensure_batch(e, n))) return rc;
    e->batch_lo = 0;
    e->batch_n = n;
    if (n) {
        // counts are staged through the prefix buffer, then scanned into place
        HIP_TRY(e, hipMemcpyAsync(e->d_count, h_counts, n * sizeof(uint32_t),
                                  hipMemcpyHostToDevice, s));
        HIP_TRY(e, launch_count_scan(nullptr, e->d_count, n, nullptr, nullptr, e->d_count,
                                     nullptr, e->d_prefix, e->d_blksum, s));
    }
    rc = finish_plan(e, n, s, total_hits, n_chunks, nullptr);
    e->plan_aux = rc == HSPZ_OK;  // the counts are in place (this plan has no bucket starts)
    if (rc) {
        *total_hits = 0;
        *n_chunks = 0;
    }
    return rc;
}

static int impl_hspz_get_chunk(const hspz_engine *engine, uint32_t i, hspz_chunk *out) {
    Engine *e = const_cast<Engine *>(reinterpret_cast<const Engine *>(engine));
    if (!e) return HSPZ_E_INVALID;
    if (!out) return fail(e, HSPZ_E_INVALID, "NULL output");
    if (!e->has_plan) return fail(e, HSPZ_E_STATE, "no plan");
    if (i >= e->chunks.size()) return fail(e, HSPZ_E_INVALID, "chunk %u out of range", i);
    *out = e->chunks[i];
    return HSPZ_OK;
}

static int impl_hspz_get_plan_arrays(const hspz_engine *engine, uint32_t *h_counts,
                                     uint32_t *h_prefix) {
    Engine *e = const_cast<Engine *>(reinterpret_cast<const Engine *>(engine));
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_plan) return fail(e, HSPZ_E_STATE, "no plan");
    int rc = set_device(e);
    if (rc) return rc;
    if (e->batch_n) {
        if (h_counts) {
            // the counts' pass reads only the uploaded k-mers and table; the copy on the
            // same (null) stream waits for it
            if ((rc = ensure_plan_aux(e, nullptr))) return rc;
            HIP_TRY(e, hipMemcpy(h_counts, e->d_count, e->batch_n * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
        }
        if (h_prefix) {
            // the device keeps block-local prefixes and the blocks' offsets
            const uint64_t nblk = (e->batch_n + kScanBlock - 1) / kScanBlock;
            std::vector<uint32_t> off(nblk);
            HIP_TRY(e, hipMemcpy(h_prefix, e->d_prefix, e->batch_n * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
            HIP_TRY(e, hipMemcpy(off.data(), e->d_blkoff, nblk * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
            for (uint64_t i = 0; i < e->batch_n; i++) h_prefix[i] += off[i / kScanBlock];
        }
    }
    return HSPZ_OK;
}

static int impl_hspz_get_seeds(const hspz_engine *engine, uint64_t lo, uint64_t hi,
                               uint32_t *h_kmer, uint32_t *h_q_end) {
    Engine *e = const_cast<Engine *>(reinterpret_cast<const Engine *>(engine));
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_qry) return fail(e, HSPZ_E_STATE, "no query uploaded");
    if (lo > hi || hi > e->n_seeds) return fail(e, HSPZ_E_INVALID, "seed range out of bounds");
    int rc = set_device(e);
    if (rc) return rc;
    if (hi > lo) {
        if (h_kmer)
            HIP_TRY(e, hipMemcpy(h_kmer, e->d_kmer + lo, (hi - lo) * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
        if (h_q_end)
            HIP_TRY(e, hipMemcpy(h_q_end, e->d_qend + lo, (hi - lo) * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost));
    }
    return HSPZ_OK;
}

static int impl_hspz_get_index(const hspz_engine *engine, uint32_t *h_end, uint32_t *h_pos,
                               uint64_t *n_buckets, uint64_t *n_pos) {
    Engine *e = const_cast<Engine *>(reinterpret_cast<const Engine *>(engine));
    if (!e) return HSPZ_E_INVALID;
    if (!n_buckets || !n_pos) return fail(e, HSPZ_E_INVALID, "NULL size output");
    if (!e->has_ref) return fail(e, HSPZ_E_STATE, "no reference uploaded");
    const uint64_t nb = 1ull << (2 * e->weight);
    *n_buckets = nb;
    *n_pos = e->n_index;
    int rc = set_device(e);
    if (rc) return rc;
    if (h_end)
        HIP_TRY(e, hipMemcpy(h_end, e->d_end, (nb + 1) * sizeof(uint32_t), hipMemcpyDeviceToHost));
    if (h_pos && e->n_index)
        HIP_TRY(e, hipMemcpy(h_pos, e->d_pos, e->n_index * sizeof(uint32_t),
                             hipMemcpyDeviceToHost));
    return HSPZ_OK;
}

static int impl_hspz_find_hits(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors,
                               uint64_t cap, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_plan || !e->plan_expandable)
        return fail(e, HSPZ_E_STATE, "find_hits needs a plan from hspz_plan");
    if (chunk >= e->chunks.size()) return fail(e, HSPZ_E_INVALID, "chunk %u out of range", chunk);
    const hspz_chunk &c = e->chunks[chunk];
    if (cap < c.n_hits)
        return fail(e, HSPZ_E_CAPACITY, "anchor buffer holds %llu, chunk needs %llu",
                    (unsigned long long)cap, (unsigned long long)c.n_hits);
    if (!d_anchors && c.n_hits) return fail(e, HSPZ_E_INVALID, "anchor buffer is NULL");
    int rc = set_device(e);
    if (rc) return rc;
    const uint64_t ns = c.seed_hi - c.seed_lo + 1;
    bool dense;
    if (e->params.expand_mode == 1) dense = false;
    else if (e->params.expand_mode == 2) dense = true;
    else dense = c.n_hits >= 16 * ns;  // "C. Hit discovery", C.4 density rule
    const uint64_t local = c.seed_lo - e->batch_lo;
    if ((rc = ensure_plan_aux(e, as_stream(stream)))) return rc;
    HIP_TRY(e, launch_expand(dense, e->d_count + local, e->d_first + local,
                             e->d_qend + c.seed_lo,
                             PrefixView{e->d_prefix + local, e->d_blkoff, (uint32_t)local}, ns,
                             e->d_pos, (uint32_t)c.hit_lo, d_anchors, as_stream(stream)));
    return HSPZ_OK;
}

// The window gate's deferred lists (two of them) can each hold every anchor of a call.
static int ensure_defer(Engine *e, uint64_t n) {
    if (n <= e->cap_defer && e->d_defer) return HSPZ_OK;
    const uint64_t cap = std::max<uint64_t>(n + n / 4, 1u << 16);
    int rc = dalloc(e, e->d_defer, 2 * cap);
    if (rc) {
        e->cap_defer = 0;
        return rc;
    }
    e->cap_defer = cap;
    return HSPZ_OK;
}

// Bucketed gate scratch for n anchors.
static int ensure_bucket(Engine *e, uint64_t n) {
    if (!e->d_binfo) {
        int rc = dalloc(e, e->d_binfo, 1);
        if (rc) return rc;
    }
    if (n <= e->cap_bucket && e->d_bsa) return HSPZ_OK;
    const uint64_t cap = std::max<uint64_t>({n, 4096, e->cap_bucket + e->cap_bucket / 4});
    const uint64_t nh = 256ull * bucket_blocks((uint32_t)std::min<uint64_t>(cap, 0xFFFFFFFFull));
    const uint64_t ns = (nh + kScanBlock - 1) / kScanBlock;
    int rc;
    if ((rc = dalloc(e, e->d_bsa, cap)) || (rc = dalloc(e, e->d_bsi, cap)) ||
        (rc = dalloc(e, e->d_bhist, nh)) || (rc = dalloc(e, e->d_bincl, nh)) ||
        (rc = dalloc(e, e->d_bsum, ns)) || (rc = dalloc(e, e->d_boff, ns))) {
        e->cap_bucket = 0;
        return rc;
    }
    e->cap_bucket = cap;
    return HSPZ_OK;
}

// The fused first stage's per-wave owner directory for a chunk of n anchors.
static int ensure_dir(Engine *e, uint64_t n) {
    const uint64_t n_waves = gate_window_waves(n);
    if (n_waves <= e->cap_dir && e->d_dir) return HSPZ_OK;
    const uint64_t want = std::max<uint64_t>({n_waves, 1024, e->cap_dir + e->cap_dir / 4});
    int rc = dalloc(e, e->d_dir, want);
    if (rc) {
        e->cap_dir = 0;
        return rc;
    }
    e->cap_dir = want;
    return HSPZ_OK;
}

static int impl_hspz_score_gate(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                                uint8_t *d_flags, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_ref || !e->has_qry)
        return fail(e, HSPZ_E_STATE, "score_gate needs an uploaded reference and query");
    if (n >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "n must be < 2^32");
    if (n && (!d_anchors || !d_flags)) return fail(e, HSPZ_E_INVALID, "NULL buffer");
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    e->gate_deferred_valid = false;
    const bool window = e->window_ok && e->params.gate_mode != 1;
    if (!window) {
        HIP_TRY(e, launch_gate(e->block_bases, d_anchors, (uint32_t)n, d_flags, e->d_ref + kPad,
                               e->d_qry + kPad, e->sp, s));
        return HSPZ_OK;
    }
    if ((rc = ensure_defer(e, n))) return rc;
    uint32_t *list1 = e->d_defer, *list2 = e->d_defer + e->cap_defer;
    if (e->params.gate_mode == 4) {
        // stable sort by reference slice: slice-major histogram, its scan, the scatter
        if ((rc = ensure_bucket(e, n))) return rc;
        const uint32_t n32 = (uint32_t)n, nb = e->n_slices;
        const uint64_t nh = (uint64_t)nb * bucket_blocks(n32);
        HIP_TRY(e, launch_bucket_hist(d_anchors, n32, e->slice_shift, nb, e->d_bhist, s));
        if (nh) {
            HIP_TRY(e, launch_count_scan(nullptr, e->d_bhist, nh, nullptr, nullptr, e->d_bhist,
                                         nullptr, e->d_bincl, e->d_bsum, s));
            HIP_TRY(e, launch_scan_blocks(e->d_bsum, (nh + kScanBlock - 1) / kScanBlock,
                                          e->d_boff, e->d_binfo, s));
            HIP_TRY(e, launch_add_offsets(e->d_bincl, nh, e->d_boff, s));
        }
        HIP_TRY(e, launch_bucket_scatter(d_anchors, n32, e->slice_shift, nb, e->d_bincl,
                                         e->d_bhist, e->d_bsa, e->d_bsi, s));
        HIP_TRY(e, launch_gate_window_bucketed(d_anchors, n32, e->d_bsa, e->d_bsi, d_flags,
                                               e->d_ref4, e->d_qry4, e->wp, list1, list2,
                                               e->d_defer_cnt, s));
    } else {
        HIP_TRY(e, launch_gate_window(e->params.gate_mode == 3, d_anchors, (uint32_t)n, d_flags,
                                      e->d_ref4, e->d_qry4, e->wp, list1, list2, e->d_defer_cnt,
                                      s));
    }
    HIP_TRY(e, launch_gate_list_wave(d_anchors, list2, e->d_defer_cnt + 1, (uint32_t)n, d_flags,
                                     e->d_ref + kPad, e->d_qry + kPad, e->sp, s));
    e->gate_deferred_valid = true;
    return HSPZ_OK;
}

// hspz_score_gate with the deferred lists and counters in the static scratch array: no
// allocation of any kind.  The bucketed gate needs scratch proportional to n and is
// refused.
static int impl_hspz_score_gate_noalloc(hspz_engine *engine, const uint64_t *d_anchors,
                                        uint64_t n, uint8_t *d_flags, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_ref || !e->has_qry)
        return fail(e, HSPZ_E_STATE, "score_gate_noalloc needs an uploaded reference and query");
    if (n > kNoAllocMaxAnchors)
        return fail(e, HSPZ_E_CAPACITY, "score_gate_noalloc takes at most %llu anchors, got %llu",
                    (unsigned long long)kNoAllocMaxAnchors, (unsigned long long)n);
    if (n && (!d_anchors || !d_flags)) return fail(e, HSPZ_E_INVALID, "NULL buffer");
    if (e->params.gate_mode == 4)
        return fail(e, HSPZ_E_INVALID, "the bucketed gate (gate_mode 4) allocates; use "
                                       "hspz_score_gate");
    int rc = set_device(e);
    if (rc) return rc;
    uint32_t *ptr = e->device < kMaxDevices ? g_scratch_ptr[e->device] : nullptr;
    if (!ptr) return fail(e, HSPZ_E_STATE, "scratch not resolved on device %d", e->device);
    hipStream_t s = as_stream(stream);
    e->gate_deferred_valid = false;
    if (!(e->window_ok && e->params.gate_mode != 1)) {
        HIP_TRY(e, launch_gate(e->block_bases, d_anchors, (uint32_t)n, d_flags, e->d_ref + kPad,
                               e->d_qry + kPad, e->sp, s));
        return HSPZ_OK;
    }
    uint32_t *cnt = ptr, *list1 = ptr + 16, *list2 = ptr + 16 + kNoAllocMaxAnchors;
    HIP_TRY(e, launch_gate_window(e->params.gate_mode == 3, d_anchors, (uint32_t)n, d_flags,
                                  e->d_ref4, e->d_qry4, e->wp, list1, list2, cnt, s));
    HIP_TRY(e, launch_gate_list_wave(d_anchors, list2, cnt + 1, (uint32_t)n, d_flags,
                                     e->d_ref + kPad, e->d_qry + kPad, e->sp, s));
    return HSPZ_OK;
}

// The deferred-anchor list beside the first stage's list of deferred slots (both first
// stages of hspz_find_hits_gate pass their deferred anchors to the second stage in it).
static int ensure_defer_anchors(Engine *e) {
    if (e->cap_defer_a >= e->cap_defer && e->d_defer_a) return HSPZ_OK;
    int rc = dalloc(e, e->d_defer_a, e->cap_defer);
    if (rc) {
        e->cap_defer_a = 0;
        return rc;
    }
    e->cap_defer_a = e->cap_defer;
    return HSPZ_OK;
}

// Whether the key-grouped first stage serves a range of n_seeds seeds of the batch: it
// pays a pass over every k-mer run of the strand, so gate_mode 0 takes it when the range
// holds at least half as many seeds as there are runs, i.e. when same-k-mer seeds of the
// range share bucket windows; gate_mode 5 always (with the window gate's preconditions).
static bool key_grouped_suits(const Engine *e, uint64_t n_seeds) {
    return e->kg_ready && (e->params.gate_mode == 5 || 2 * n_seeds >= e->kg_n_runs);
}

// The window gate over seeds seed_lo .. seed_hi of the planned batch, whose n anchors are
// the batch's slots hit_lo .. hit_lo + n - 1, with the key-grouped first stage: flags
// receives their n flags, anchors (indexed from hit_lo) the anchor of every slot whose
// flag is 1.  A chunk of the plan, or the whole batch (hspz_run_batch).
static KeyGroups key_groups(const Engine *e) {
    return KeyGroups{e->d_kg_qs,        e->d_kg_qe,       e->d_kg_run_c,
                     e->d_kg_run_first, e->d_kg_run_span, e->kg_n_runs};
}

static KgScratch kg_scratch(const Engine *e) {
    return KgScratch{e->d_kg_G,      e->d_kg_a,      e->d_kg_m,   e->d_kg_dir,
                     e->d_kg_blksum, e->d_kg_blkoff, e->d_kg_info};
}

// groups_ready: the grouping pass for this seed range is already queued (hspz_run_batch
// queues it while the host waits for the plan).  bits: d_flags holds a bit per anchor
// (bit i % 32 of 32-bit word i / 32), for hspz_run_batch's own compaction.
static int gate_key_grouped(Engine *e, uint64_t seed_lo, uint64_t seed_hi, uint64_t hit_lo,
                            uint64_t n, uint64_t *d_anchors, uint8_t *d_flags, hipStream_t s,
                            bool groups_ready = false, bool bits = false) {
    int rc;
    if ((rc = ensure_defer(e, n)) || (rc = ensure_defer_anchors(e)) ||
        (rc = ensure_kg(e, gate_window_waves(n))))
        return rc;
    uint32_t *list1 = e->d_defer, *list2 = e->d_defer + e->cap_defer;
    const KeyGroups g = key_groups(e);
    const KgScratch ks = kg_scratch(e);
    HIP_TRY(e, launch_gate_window_kg(g, ks, PrefixView{e->d_prefix, e->d_blkoff, 0},
                                     (uint32_t)e->batch_lo,
                                     (uint32_t)seed_lo, (uint32_t)seed_hi, (uint32_t)hit_lo,
                                     (uint32_t)n, e->d_pos, d_anchors, d_flags, e->d_ref4,
                                     e->d_qry4, e->wp, list1, e->d_defer_a, list2,
                                     e->d_defer_cnt, e->sp, e->d_ref + kPad, e->d_qry + kPad,
                                     groups_ready, bits, s));
    HIP_TRY(e, launch_gate_list_wave(d_anchors, list2, e->d_defer_cnt + 1, (uint32_t)n, d_flags,
                                     e->d_ref + kPad, e->d_qry + kPad, e->sp, s, bits));
    e->gate_deferred_valid = true;
    return HSPZ_OK;
}

static int impl_hspz_find_hits_gate(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors,
                                    uint64_t cap, uint8_t *d_flags, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!e->has_plan || !e->plan_expandable)
        return fail(e, HSPZ_E_STATE, "find_hits_gate needs a plan from hspz_plan");
    if (chunk >= e->chunks.size()) return fail(e, HSPZ_E_INVALID, "chunk %u out of range", chunk);
    const hspz_chunk c = e->chunks[chunk];
    if (cap < c.n_hits)
        return fail(e, HSPZ_E_CAPACITY, "anchor buffer holds %llu, chunk needs %llu",
                    (unsigned long long)cap, (unsigned long long)c.n_hits);
    if (c.n_hits && (!d_anchors || !d_flags)) return fail(e, HSPZ_E_INVALID, "NULL buffer");
    // the exact gate and the bucketed gate read every anchor from memory
    if (!(e->window_ok && e->params.gate_mode != 1 && e->params.gate_mode != 4)) {
        int rc = hspz_find_hits(engine, chunk, d_anchors, cap, stream);
        return rc ? rc : hspz_score_gate(engine, d_anchors, c.n_hits, d_flags, stream);
    }
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    e->gate_deferred_valid = false;
    const uint64_t n = c.n_hits;
    if (n > 0 && key_grouped_suits(e, c.seed_hi - c.seed_lo + 1))
        return gate_key_grouped(e, c.seed_lo, c.seed_hi, c.hit_lo, n, d_anchors, d_flags, s);
    if ((rc = ensure_defer(e, n)) || (rc = ensure_defer_anchors(e))) return rc;
    uint32_t *list1 = e->d_defer, *list2 = e->d_defer + e->cap_defer;
    if ((rc = ensure_dir(e, n)) || (rc = ensure_plan_aux(e, s))) return rc;
    const uint64_t local = c.seed_lo - e->batch_lo;
    ChunkSeeds cs;
    cs.prefix = PrefixView{e->d_prefix + local, e->d_blkoff, (uint32_t)local};
    cs.first = e->d_first + local;
    cs.q_end = e->d_qend + c.seed_lo;
    cs.pos = e->d_pos;
    cs.dir = e->d_dir;
    cs.n_seeds = (uint32_t)(c.seed_hi - c.seed_lo + 1);
    cs.hit_lo = (uint32_t)c.hit_lo;
    HIP_TRY(e, launch_gate_window_fused(e->params.gate_mode == 3, cs, (uint32_t)n, d_anchors,
                                        d_flags, e->d_ref4, e->d_qry4, e->wp, list1,
                                        e->d_defer_a, list2, e->d_defer_cnt, s));
    HIP_TRY(e, launch_gate_list_wave(d_anchors, list2, e->d_defer_cnt + 1, (uint32_t)n, d_flags,
                                     e->d_ref + kPad, e->d_qry + kPad, e->sp, s));
    e->gate_deferred_valid = true;
    return HSPZ_OK;
}

static int compact_common(Engine *e, const uint8_t *d_flags, uint64_t n, uint32_t *ids,
                          const hspz_segment_pair *rin, hspz_segment_pair *rout, uint64_t cap,
                          uint64_t *n_out, hipStream_t s) {
    if (n >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "n must be < 2^32");
    if (n && !d_flags) return fail(e, HSPZ_E_INVALID, "NULL flags");
    int rc = set_device(e);
    if (rc) return rc;
    if ((rc = ensure_compact(e, n))) return rc;
    const uint32_t c32 = (uint32_t)std::min<uint64_t>(cap, 0xFFFFFFFFull);
    HIP_TRY(e, launch_compact(d_flags, (uint32_t)n, e->d_cblk, e->d_ctotal, ids, rin, rout, c32,
                              s));
    HIP_TRY(e, hipMemcpyAsync(e->h_pinned, e->d_ctotal, sizeof(uint32_t), hipMemcpyDeviceToHost,
                              s));
    HIP_TRY(e, hipStreamSynchronize(s));
    const uint64_t total = e->h_pinned[0];
    if (total > cap)
        return fail(e, HSPZ_E_CAPACITY, "%llu selected, capacity %llu",
                    (unsigned long long)total, (unsigned long long)cap);
    *n_out = total;
    return HSPZ_OK;
}

static int impl_hspz_compact(hspz_engine *engine, const uint8_t *d_flags, uint64_t n,
                             uint32_t *d_ids, uint64_t cap, uint64_t *n_out, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!n_out) return fail(e, HSPZ_E_INVALID, "NULL n_out");
    *n_out = 0;
    if (!d_ids && cap) return fail(e, HSPZ_E_INVALID, "NULL ids with nonzero capacity");
    int rc = compact_common(e, d_flags, n, d_ids, nullptr, nullptr, d_ids ? cap : 0, n_out,
                            as_stream(stream));
    if (rc) *n_out = 0;
    return rc;
}

// Diagonal-shared materialization: calls of at least this many survivors take it in
// materialize_mode 0.  Below it the sort's and scans' fixed launches (about 0.3 ms in
// all) cost more than the walks save: 66,579 survivors of the 50 Mb workload take
// 0.11 ms walked one by one.
constexpr uint64_t kMatSharedMin = 131072;

// Scratch of the diagonal-shared materialization for n survivors.  The per-side arrays
// (best, ext, term, ds, cnt, sum, pos: seven u32 each) are carved out
// of one allocation, each at a 16-byte aligned offset.
static uint64_t mat_stride(uint64_t cap) { return (cap + 3) / 4 * 4; }  // u32 words per array
static uint64_t mat_side_words(uint64_t cap) {
    return 7 * mat_stride(cap);  // a multiple of 4 words: 16-byte aligned sides
}

static int ensure_mat(Engine *e, uint64_t n) {
    if (!e->mat) {
        e->mat = new (std::nothrow) MatScratch();
        if (!e->mat) return fail(e, HSPZ_E_NOMEM, "out of host memory");
    }
    MatScratch &m = *e->mat;
    if (n <= m.cap && m.ka) return HSPZ_OK;
    const uint64_t cap = std::max<uint64_t>({n, 4096, m.cap + m.cap / 4});
    const uint64_t nh = 256ull * radix_blocks((uint32_t)std::min<uint64_t>(cap, 0xFFFFFFFFull));
    const uint64_t ns = (std::max(nh, cap) + kScanBlock - 1) / kScanBlock;
    int rc;
    if ((rc = dalloc(e, m.ka, cap)) || (rc = dalloc(e, m.va, cap)) ||
        (rc = dalloc(e, m.kb, cap)) || (rc = dalloc(e, m.vb, cap)) ||
        (rc = dalloc(e, m.hist, nh)) || (rc = dalloc(e, m.incl, nh)) ||
        (rc = dalloc(e, m.side, 2 * mat_side_words(cap))) ||
        (rc = dalloc(e, m.sum, ns)) || (rc = dalloc(e, m.off, ns)) ||
        (rc = dalloc(e, m.list, 2 * cap)) || (rc = dalloc(e, m.sa, cap)) ||
        (rc = dalloc(e, m.sblk,
                     4ull * mm_scan_blocks((uint32_t)std::min<uint64_t>(cap, 0xFFFFFFFFull)))) ||
        (!m.info && (rc = dalloc(e, m.info, 1))) ||
        (!m.lcnt && (rc = dalloc(e, m.lcnt, 2)))) {
        m.cap = 0;
        return rc;
    }
    m.cap = cap;
    return HSPZ_OK;
}

static MatSide mat_side(Engine *e, int side) {
    const uint64_t stride = mat_stride(e->mat->cap);
    uint32_t *b = e->mat->side + (uint64_t)side * mat_side_words(e->mat->cap);
    MatSide m;
    m.best = reinterpret_cast<int32_t *>(b);
    m.ext = b + stride;
    m.term = b + 2 * stride;
    m.ds = reinterpret_cast<int32_t *>(b + 3 * stride);
    m.cnt = b + 4 * stride;
    m.sum = b + 5 * stride;
    m.pos = b + 6 * stride;
    return m;
}

// Inclusive prefix sum (modulo 2^32) of n u32 values into out (16-byte aligned), on the
// materialization scratch.  in is written back unchanged.
static int mat_scan(Engine *e, uint32_t *in, uint64_t n, uint32_t *out, hipStream_t s) {
    if (n == 0) return HSPZ_OK;
    MatScratch &m = *e->mat;
    HIP_TRY(e, launch_count_scan(nullptr, in, n, nullptr, nullptr, in, nullptr, out, m.sum, s));
    HIP_TRY(e, launch_scan_blocks(m.sum, (n + kScanBlock - 1) / kScanBlock, m.off, m.info, s));
    HIP_TRY(e, launch_add_offsets(out, n, m.off, s));
    return HSPZ_OK;
}

static int bits_of(uint64_t v) {
    int b = 1;
    while (b < 64 && (v >> b)) b++;
    return b;
}

// Stable LSD radix sort of (ka, va) by the low `bits` bits of ka; the result ends in
// (ka, va) (the buffers are swapped as the passes go).
static int mat_radix(Engine *e, uint32_t *&ka, uint32_t *&va, uint32_t *&kb, uint32_t *&vb,
                     uint32_t n, int bits, hipStream_t s) {
    const uint64_t nh = 256ull * radix_blocks(n);
    int rc;
    for (int shift = 0; shift < bits; shift += 8) {
        HIP_TRY(e, launch_radix_hist(ka, n, shift, e->mat->hist, s));
        if ((rc = mat_scan(e, e->mat->hist, nh, e->mat->incl, s))) return rc;
        HIP_TRY(e, launch_radix_scatter(ka, va, n, shift, e->mat->incl, e->mat->hist, kb, vb, s));
        std::swap(ka, kb);
        std::swap(va, vb);
    }
    return HSPZ_OK;
}

// q_ordered: the survivors' query ends never decrease in id order (the pass's own
// survivors: anchors lie in slot order, seeds in query order), so on each diagonal the
// reference ends already ascend and the stable sort by diagonal alone keeps them so.
static int materialize_shared(Engine *e, const uint64_t *d_anchors, const uint32_t *d_ids,
                              uint32_t n, hspz_segment_pair *d_hsp, uint8_t *d_status,
                              bool q_ordered, hipStream_t s) {
    int rc;
    if ((rc = ensure_mat(e, n))) return rc;
    const uint32_t n_ref = (uint32_t)e->n_ref, n_qry = (uint32_t)e->n_qry;
    uint32_t *ka = e->mat->ka, *va = e->mat->va, *kb = e->mat->kb, *vb = e->mat->vb;
    HIP_TRY(e, launch_mm_keys(d_anchors, d_ids, n, n_ref, n_qry, ka, va, e->mat->lcnt, s));
    if (!q_ordered && (rc = mat_radix(e, ka, va, kb, vb, n, bits_of(n_ref), s))) return rc;
    HIP_TRY(e, launch_mm_diag(d_anchors, d_ids, va, n, n_ref, n_qry, ka, s));
    if ((rc = mat_radix(e, ka, va, kb, vb, n, bits_of((uint64_t)n_ref + n_qry + 1), s)))
        return rc;
    const MatSide right = mat_side(e, 0), left = mat_side(e, 1);
    uint64_t *sa = e->mat->sa;
    HIP_TRY(e, launch_mm_gather(d_anchors, d_ids, va, n, sa, s));
    // the lane stage needs exact eight-base blocks, as the windowed gate does
    HIP_TRY(e, launch_mm_walk(sa, ka, n, e->d_ref + kPad, e->d_qry + kPad,
                              e->d_ref4, e->d_qry4, e->sp, right, left, e->block_bases == 8,
                              e->mat->list, e->mat->lcnt, s));
    HIP_TRY(e, launch_mm_scan(right, left, n, e->mat->sblk, s));
    HIP_TRY(e, launch_mm_finish(sa, va, n, right, left, d_hsp, d_status,
                                e->d_ref + kPad, e->sp, s));
    return HSPZ_OK;
}

static int materialize(Engine *e, const uint64_t *d_anchors, const uint32_t *d_ids,
                       uint64_t n_surv, hspz_segment_pair *d_hsp, uint8_t *d_status,
                       bool q_ordered, void *stream) {
    if (!e->has_ref || !e->has_qry)
        return fail(e, HSPZ_E_STATE, "materialize needs an uploaded reference and query");
    if (n_surv >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "n_surv must be < 2^32");
    if (n_surv && (!d_anchors || !d_ids || !d_hsp || !d_status))
        return fail(e, HSPZ_E_INVALID, "NULL buffer");
    int rc = set_device(e);
    if (rc) return rc;
    // the diagonal keys r - q + n_qry must fit 32 bits for the shared walks
    const bool fits = (uint64_t)e->n_ref + e->n_qry + 2 < 0xFFFFFFFFull;
    const int mode = e->params.materialize_mode;
    if (fits && n_surv && (mode == 2 || (mode == 0 && n_surv >= kMatSharedMin)))
        return materialize_shared(e, d_anchors, d_ids, (uint32_t)n_surv, d_hsp, d_status,
                                  q_ordered, as_stream(stream));
    HIP_TRY(e, launch_materialize(d_anchors, d_ids, (uint32_t)n_surv, d_hsp, d_status,
                                  e->d_ref + kPad, e->d_ref4, e->d_qry4, e->sp,
                                  as_stream(stream)));
    return HSPZ_OK;
}

static int impl_hspz_materialize(hspz_engine *engine, const uint64_t *d_anchors,
                                 const uint32_t *d_ids, uint64_t n_surv, hspz_segment_pair *d_hsp,
                                 uint8_t *d_status, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    return materialize(e, d_anchors, d_ids, n_surv, d_hsp, d_status, false, stream);
}

static int impl_hspz_compact_hsps(hspz_engine *engine, const hspz_segment_pair *d_hsp,
                                  const uint8_t *d_status, uint64_t n, hspz_segment_pair *d_out,
                                  uint64_t cap, uint64_t *n_out, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!n_out) return fail(e, HSPZ_E_INVALID, "NULL n_out");
    *n_out = 0;
    if (n && !d_hsp) return fail(e, HSPZ_E_INVALID, "NULL records");
    if (!d_out && cap) return fail(e, HSPZ_E_INVALID, "NULL output with nonzero capacity");
    int rc = compact_common(e, d_status, n, nullptr, d_hsp, d_out, d_out ? cap : 0, n_out,
                            as_stream(stream));
    if (rc) *n_out = 0;
    return rc;
}

// Grow both sets of whole-batch chunk buffers to n anchors, and the survivor buffers to s
// survivors (a quarter of headroom).
static int ensure_run_buffers(Engine *e, uint64_t n, uint64_t ns) {
    int rc;
    if (n > e->rb_cap_a || !e->rb_anchors[0]) {
        const uint64_t cap = std::max<uint64_t>({n, 1024, e->rb_cap_a + e->rb_cap_a / 4});
        for (int b = 0; b < 2; b++)
            if ((rc = dalloc(e, e->rb_anchors[b], cap)) ||
                (rc = dalloc(e, e->rb_flags[b], cap + 16)) || (rc = dalloc(e, e->rb_ids[b], cap))) {
                e->rb_cap_a = 0;
                return rc;
            }
        e->rb_cap_a = cap;
    }
    if (ns > e->rb_cap_s || !e->rb_hsp) {
        const uint64_t cap = std::max<uint64_t>({ns, 1024, e->rb_cap_s + e->rb_cap_s / 4});
        if ((rc = dalloc(e, e->rb_hsp, cap)) || (rc = dalloc(e, e->rb_out[0], cap)) ||
            (rc = dalloc(e, e->rb_out[1], cap)) || (rc = dalloc(e, e->rb_status, cap + 16))) {
            e->rb_cap_s = 0;
            return rc;
        }
        e->rb_cap_s = cap;
    }
    return HSPZ_OK;
}

// The whole-batch gate's buffers for n anchors.
static int ensure_batch_buffers(Engine *e, uint64_t n) {
    if (n <= e->bb_cap && e->bb_flags) return HSPZ_OK;
    int rc;
    // flags one bit per anchor (32-bit words)
    if ((rc = dalloc(e, e->bb_flags, (n + 31) / 32 * 4 + 16)) || (rc = dalloc(e, e->bb_anchors, n)) ||
        (rc = dalloc(e, e->bb_ids, n))) {
        e->bb_cap = 0;
        return rc;
    }
    e->bb_cap = n;
    return HSPZ_OK;
}

// Room for n records in the pinned staging; the first keep records are carried over.
static int ensure_record_staging(Engine *e, uint64_t n, uint64_t keep, hipStream_t s) {
    if (n <= e->h_rec_cap && e->h_rec) return HSPZ_OK;
    const uint64_t cap = std::max<uint64_t>({n, 4096, e->h_rec_cap + e->h_rec_cap / 2});
    hspz_segment_pair *p = nullptr;
    if (hipHostMalloc(reinterpret_cast<void **>(&p), cap * sizeof(hspz_segment_pair)) !=
        hipSuccess)
        return fail(e, HSPZ_E_NOMEM, "pinned record staging of %llu records failed",
                    (unsigned long long)cap);
    if (e->h_rec) {
        HIP_TRY(e, hipStreamSynchronize(s));  // copies into the old staging have landed
        if (e->copy_s) HIP_TRY(e, hipStreamSynchronize(e->copy_s));
        if (keep) memcpy(p, e->h_rec, keep * sizeof(hspz_segment_pair));
        (void)hipHostFree(e->h_rec);
    }
    e->h_rec = p;
    e->h_rec_cap = cap;
    return HSPZ_OK;
}

// Queue a compaction whose count lands in pinned slot `slot` (0: survivors, 1: records),
// with count_ev[slot] recorded behind the copy; count_wait() reads it back.
static int count_queue(Engine *e, const uint8_t *flags, uint64_t n, uint32_t *ids,
                       const hspz_segment_pair *rin, hspz_segment_pair *rout, uint64_t cap,
                       int slot, hipStream_t s, bool bits = false) {
    if (n >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "n must be < 2^32");
    if ((n + kCompactBlock - 1) / kCompactBlock + 1 > e->cap_cblk)
        return fail(e, HSPZ_E_INVALID, "compaction scratch not sized for %llu",
                    (unsigned long long)n);
    uint32_t *d_total = e->d_ctotal + 4 * (slot + 1);
    uint32_t *h_total = e->h_pinned + 16 + 4 * slot;
    const uint32_t c32 = (uint32_t)std::min<uint64_t>(cap, 0xFFFFFFFFull);
    if (bits)  // ids of the set bits (flags as 32-bit words)
        HIP_TRY(e, launch_compact_bits(reinterpret_cast<const uint32_t *>(flags), (uint32_t)n,
                                       e->d_cblk, d_total, ids, c32, s));
    else
        HIP_TRY(e, launch_compact(flags, (uint32_t)n, e->d_cblk, d_total, ids, rin, rout, c32,
                                  s));
    HIP_TRY(e, hipMemcpyAsync(h_total, d_total, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
    HIP_TRY(e, hipEventRecord(e->count_ev[slot], s));
    return HSPZ_OK;
}

static int count_wait(Engine *e, int slot, uint64_t cap, uint64_t *n_out) {
    HIP_TRY(e, hipEventSynchronize(e->count_ev[slot]));
    const uint64_t total = e->h_pinned[16 + 4 * slot];
    if (total > cap)
        return fail(e, HSPZ_E_CAPACITY, "%llu selected, capacity %llu", (unsigned long long)total,
                    (unsigned long long)cap);
    *n_out = total;
    return HSPZ_OK;
}

constexpr uint64_t kWholeBatchMax = 1ull << 30;  // anchors of a whole-batch gate call
constexpr uint64_t kWholeChunkMin = 1ull << 22;  // and the least anchors per chunk

static int impl_hspz_run_batch(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi,
                               int32_t time_gate, hspz_batch_stats *stats, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!stats) return fail(e, HSPZ_E_INVALID, "NULL stats");
    *stats = hspz_batch_stats{};
    e->h_rec_n = 0;
    hipStream_t s = as_stream(stream);
    uint64_t total = 0;
    uint32_t nch = 0;
    if (time_gate)
        for (hipEvent_t &ev : e->gate_ev)
            if (!ev) HIP_TRY(e, hipEventCreate(&ev));
    // A batch of large MAX_HITS chunks (below) is gated at once with the key-grouped
    // stage, whose first pass depends on the seed range alone: it is queued behind the
    // plan's copy to the host, so that it runs while the host waits for the plan.
    bool spec = false;
    auto queued = [&]() -> int {
        if (!(key_grouped_suits(e, seed_hi - seed_lo) && seed_hi > seed_lo &&
              (e->params.max_hits == 0 || e->params.max_hits >= kWholeChunkMin)))
            return HSPZ_OK;
        if (ensure_kg(e, 0) != HSPZ_OK) {  // not enough memory now: no head start
            (void)hipGetLastError();
            e->err.clear();
            return HSPZ_OK;
        }
        if (time_gate) HIP_TRY(e, hipEventRecord(e->gate_ev[0], s));
        HIP_TRY(e, launch_kg_groups(key_groups(e), kg_scratch(e), (uint32_t)seed_lo,
                                    (uint32_t)(seed_hi - 1), s));
        spec = true;
        return HSPZ_OK;
    };
    int rc = plan_batch(engine, seed_lo, seed_hi, stream, &total, &nch, queued);
    if (rc) return rc;
    stats->n_anchors = total;
    stats->n_chunks = nch;
    uint64_t maxn = 0;
    for (const hspz_chunk &c : e->chunks) maxn = std::max<uint64_t>(maxn, c.n_hits);
    // The whole batch at once: where the key-grouped stage serves the batch, one gate call
    // covers the slots of every chunk (the batch's flags, kept anchors and survivor ids in
    // one buffer each; the chunk cut bounds memory on small GPUs, and up to 2^30 anchors
    // fit here), so a k-mer's seeds in every chunk share their reference windows and the
    // stage runs once; the survivors are then compacted and materialized in one call
    // each (below).  Batches of small chunks (under 2^22 anchors on average) go chunk by
    // chunk: there each chunk's gate, queued ahead, covers the host's wait for the
    // previous chunk's counts.
    bool whole = nch > 1 && total <= kWholeBatchMax && total / nch >= kWholeChunkMin &&
                 key_grouped_suits(e, e->batch_n);
    if (whole) {
        // its buffers (flags, kept anchors, survivor ids, both deferred lists, compaction
        // blocks) are sized for the batch; where the device cannot hold them the batch
        // goes chunk by chunk after all
        if ((rc = ensure_batch_buffers(e, total)) || (rc = ensure_defer(e, total)) ||
            (rc = ensure_defer_anchors(e)) || (rc = ensure_kg(e, gate_window_waves(total))) ||
            (rc = ensure_compact(e, total))) {
            if (rc != HSPZ_E_NOMEM) return rc;
            (void)hipGetLastError();  // the failed allocation's error is not the next call's
            e->err.clear();
            dfree(e->bb_flags);
            dfree(e->bb_anchors);
            dfree(e->bb_ids);
            dfree(e->d_defer);
            dfree(e->d_defer_a);
            e->bb_cap = e->cap_defer = e->cap_defer_a = 0;
            whole = false;
        }
    }
    // Scratch that queued work may still be using is never regrown inside the loop: size
    // the gate's lists and directory and the compaction blocks for the largest chunk now.
    if (!whole && ((rc = ensure_run_buffers(e, maxn, 0)) || (rc = ensure_defer(e, maxn)) ||
                   (rc = ensure_defer_anchors(e)) || (rc = ensure_dir(e, maxn)) ||
                   (rc = ensure_compact(e, maxn))))
        return rc;
    for (hipEvent_t &ev : e->count_ev)
        if (!ev) HIP_TRY(e, hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    for (hipEvent_t &ev : e->copied_ev)
        if (!ev) HIP_TRY(e, hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    if (!e->copy_s) HIP_TRY(e, hipStreamCreateWithFlags(&e->copy_s, hipStreamNonBlocking));
    // every return below, error or not, first lets the record copies land
    struct CopyDrain {
        Engine *e;
        ~CopyDrain() {
            (void)hipStreamSynchronize(e->copy_s);
            e->copy_pending[0] = e->copy_pending[1] = false;
        }
    } drain{e};

    stats->whole_batch_gate = whole ? 1 : 0;
    if (whole) {
        if (time_gate && !spec) HIP_TRY(e, hipEventRecord(e->gate_ev[0], s));
        if ((rc = set_device(e)) ||
            (rc = gate_key_grouped(e, e->batch_lo, e->batch_lo + e->batch_n - 1, 0, total,
                                   e->bb_anchors, e->bb_flags, s, spec, true)))
            return rc;
        if (time_gate) HIP_TRY(e, hipEventRecord(e->gate_ev[1], s));
        // The survivors of every chunk at once: their ids are batch slots, ascending, so
        // chunk by chunk in chunk order and within a chunk in slot order; their anchors
        // are in query order, so they are materialized in one call and the accepted
        // records leave in one copy -- the records of the chunks one after another.
        uint64_t ns = 0, na = 0;
        if ((rc = count_queue(e, e->bb_flags, total, e->bb_ids, nullptr, nullptr, e->bb_cap, 0,
                              s, true)) ||
            (rc = count_wait(e, 0, e->bb_cap, &ns)))
            return rc;
        if (time_gate) {
            float ms = 0.f;
            HIP_TRY(e, hipEventElapsedTime(&ms, e->gate_ev[0], e->gate_ev[1]));
            stats->gate_ms = ms;
            stats->gate_calls = 1;
        }
        // the accepted records are compacted straight into the pinned host staging (sized
        // for every survivor), so the host's one wait, for their count, ends the batch
        if ((rc = ensure_run_buffers(e, 0, ns)) || (rc = ensure_record_staging(e, ns, 0, s)))
            return rc;
        hspz_segment_pair *d_rec = nullptr;
        HIP_TRY(e, hipHostGetDevicePointer(reinterpret_cast<void **>(&d_rec), e->h_rec, 0));
        if ((rc = materialize(e, e->bb_anchors, e->bb_ids, ns, e->rb_hsp, e->rb_status, true,
                              stream)) ||
            (rc = count_queue(e, e->rb_status, ns, nullptr, e->rb_hsp, d_rec, e->h_rec_cap, 1,
                              s)) ||
            (rc = count_wait(e, 1, e->h_rec_cap, &na)))
            return rc;
        stats->n_survivors = ns;
        stats->n_accepted = na;
        e->h_rec_n = na;
        return HSPZ_OK;
    }

    // One stream, queued one chunk ahead: chunk c + 1's expansion+gate and survivor
    // compaction are queued before the host waits on chunk c's counts, so the GPU has work
    // while the host reads them.  Chunk c uses buffer set c & 1; stream order keeps every
    // read of a set ahead of the next write to it.  Chunk c's accepted records go to the
    // host on copy_s, behind its record count, while the next chunks run; the compaction
    // of chunk c + 2 into the same record buffer waits for that copy.
    auto gate = [&](uint32_t c) -> int {
        const int b = c & 1;
        if (time_gate) HIP_TRY(e, hipEventRecord(e->gate_ev[2 * b], s));
        int r = hspz_find_hits_gate(engine, c, e->rb_anchors[b], e->rb_cap_a, e->rb_flags[b],
                                    stream);
        if (r) return r;
        if (time_gate) HIP_TRY(e, hipEventRecord(e->gate_ev[2 * b + 1], s));
        return HSPZ_OK;
    };
    auto survivors = [&](uint32_t c) -> int {
        const int b = c & 1;
        return count_queue(e, e->rb_flags[b], e->chunks[c].n_hits, e->rb_ids[b], nullptr,
                           nullptr, e->rb_cap_a, 0, s);
    };
    if (nch && ((rc = gate(0)) || (rc = survivors(0)))) return rc;
    uint64_t acc = 0;
    for (uint32_t c = 0; c < nch; c++) {
        const int b = c & 1;
        if (c + 1 < nch && (rc = gate(c + 1))) return rc;
        uint64_t ns = 0, na = 0;
        if ((rc = count_wait(e, 0, e->rb_cap_a, &ns))) return rc;
        if (time_gate) {  // the survivor count lands after the chunk's gate events
            float ms = 0.f;
            HIP_TRY(e, hipEventElapsedTime(&ms, e->gate_ev[2 * b], e->gate_ev[2 * b + 1]));
            stats->gate_ms += ms;
            stats->gate_calls++;
        }
        if (ns > e->rb_cap_s) {  // the survivor buffers grow only once both streams are idle
            HIP_TRY(e, hipStreamSynchronize(s));
            HIP_TRY(e, hipStreamSynchronize(e->copy_s));
            e->copy_pending[0] = e->copy_pending[1] = false;
            if ((rc = ensure_run_buffers(e, maxn, ns))) return rc;
        }
        // the chunk's own survivors, in slot order: query ends never decrease
        if ((rc = materialize(e, e->rb_anchors[b], e->rb_ids[b], ns, e->rb_hsp, e->rb_status,
                              true, stream)))
            return rc;
        if (e->copy_pending[b]) {  // chunk c - 2's records are still being read out of it
            HIP_TRY(e, hipStreamWaitEvent(s, e->copied_ev[b], 0));
            e->copy_pending[b] = false;
        }
        if ((rc = count_queue(e, e->rb_status, ns, nullptr, e->rb_hsp, e->rb_out[b],
                              e->rb_cap_s, 1, s)))
            return rc;
        if (c + 1 < nch && (rc = survivors(c + 1))) return rc;
        if ((rc = count_wait(e, 1, e->rb_cap_s, &na))) return rc;
        if (na) {
            if ((rc = ensure_record_staging(e, acc + na, acc, s))) return rc;
            // count_ev[1] stands behind this chunk's record compaction
            HIP_TRY(e, hipStreamWaitEvent(e->copy_s, e->count_ev[1], 0));
            HIP_TRY(e, hipMemcpyAsync(e->h_rec + acc, e->rb_out[b],
                                      na * sizeof(hspz_segment_pair), hipMemcpyDeviceToHost,
                                      e->copy_s));
            HIP_TRY(e, hipEventRecord(e->copied_ev[b], e->copy_s));
            e->copy_pending[b] = true;
        }
        stats->n_survivors += ns;
        acc += na;
    }
    HIP_TRY(e, hipStreamSynchronize(s));
    HIP_TRY(e, hipStreamSynchronize(e->copy_s));
    stats->n_accepted = acc;
    e->h_rec_n = acc;
    return HSPZ_OK;
}

static int impl_hspz_get_batch_records(const hspz_engine *engine, hspz_segment_pair *h_out,
                                       uint64_t cap, uint64_t *n) {
    Engine *e = const_cast<Engine *>(reinterpret_cast<const Engine *>(engine));
    if (!e) return HSPZ_E_INVALID;
    if (!n || (!h_out && cap)) return fail(e, HSPZ_E_INVALID, "NULL argument");
    *n = e->h_rec_n;
    if (!h_out) return HSPZ_OK;  // size query
    const uint64_t k = std::min<uint64_t>(cap, e->h_rec_n);
    if (k) memcpy(h_out, e->h_rec, k * sizeof(hspz_segment_pair));
    if (cap < e->h_rec_n)
        return fail(e, HSPZ_E_CAPACITY, "%llu records, room for %llu",
                    (unsigned long long)e->h_rec_n, (unsigned long long)cap);
    return HSPZ_OK;
}

namespace {

struct RecordHash {
    size_t operator()(const hspz_segment_pair &r) const {
        uint64_t a = ((uint64_t)r.ref_start << 32) | r.query_start;
        uint64_t b = ((uint64_t)r.len << 32) | (uint32_t)r.score;
        uint64_t x = a ^ (b * 0x9E3779B97F4A7C15ull);  // splitmix64 finaliser of the mix
        x ^= x >> 30;
        x *= 0xBF58476D1CE4E5B9ull;
        x ^= x >> 27;
        x *= 0x94D049BB133111EBull;
        return (size_t)(x ^ (x >> 31));
    }
};
struct RecordEq {
    bool operator()(const hspz_segment_pair &x, const hspz_segment_pair &y) const {
        return x.ref_start == y.ref_start && x.query_start == y.query_start && x.len == y.len &&
               x.score == y.score;
    }
};

int no_engine_fail(int code, const char *msg) {
    g_create_error = msg;
    return code;
}

}  // namespace

static int impl_hspz_dedup_records(const hspz_segment_pair *h_in, uint64_t n,
                                   hspz_segment_pair *h_out, uint64_t cap, uint64_t *n_out) {
    if (!n_out) return no_engine_fail(HSPZ_E_INVALID, "NULL n_out");
    *n_out = 0;
    if (n && (!h_in || !h_out)) return no_engine_fail(HSPZ_E_INVALID, "NULL records");
    std::vector<uint8_t> first;
    uint64_t kept = 0;
    try {
        first.assign(n, 0);
        std::unordered_set<hspz_segment_pair, RecordHash, RecordEq> seen;
        seen.reserve((size_t)n);
        for (uint64_t i = 0; i < n; i++)
            if (seen.insert(h_in[i]).second) {
                first[i] = 1;
                kept++;
            }
    } catch (const std::bad_alloc &) {
        return no_engine_fail(HSPZ_E_NOMEM, "dedup: host allocation failed");
    }
    *n_out = kept;
    if (kept > cap) return no_engine_fail(HSPZ_E_CAPACITY, "dedup: output capacity too small");
    uint64_t k = 0;  // k <= i throughout, so h_out == h_in is safe
    for (uint64_t i = 0; i < n; i++)
        if (first[i]) h_out[k++] = h_in[i];
    return HSPZ_OK;
}

static int impl_hspz_debug_walk_steps(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                                      uint64_t *total_steps, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!total_steps) return fail(e, HSPZ_E_INVALID, "NULL output");
    *total_steps = 0;
    if (!e->has_ref || !e->has_qry)
        return fail(e, HSPZ_E_STATE, "walk statistics need an uploaded reference and query");
    if (n >= 0xFFFFFFFFull) return fail(e, HSPZ_E_INVALID, "n must be < 2^32");
    if (n && !d_anchors) return fail(e, HSPZ_E_INVALID, "NULL anchors");
    if (n == 0) return HSPZ_OK;
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    const uint32_t nb = walk_steps_blocks((uint32_t)n);
    uint64_t *d_part = nullptr;
    if ((rc = dalloc(e, d_part, nb))) return rc;
    std::vector<uint64_t> part(nb);
    hipError_t st = launch_walk_steps(d_anchors, (uint32_t)n, e->d_ref + kPad, e->d_qry + kPad,
                                      e->sp, d_part, s);
    if (st == hipSuccess)
        st = hipMemcpyAsync(part.data(), d_part, nb * sizeof(uint64_t), hipMemcpyDeviceToHost, s);
    if (st == hipSuccess) st = hipStreamSynchronize(s);
    dfree(d_part);
    if (st != hipSuccess)
        return fail(e, HSPZ_E_HIP, "walk statistics failed: %s", hipGetErrorString(st));
    uint64_t t = 0;
    for (uint64_t v : part) t += v;
    *total_steps = t;
    return HSPZ_OK;
}

static int impl_hspz_debug_gate_deferred(hspz_engine *engine, uint64_t *n_stage2,
                                         uint64_t *n_exact, void *stream) {
    Engine *e = reinterpret_cast<Engine *>(engine);
    if (!e) return HSPZ_E_INVALID;
    if (!n_stage2 || !n_exact) return fail(e, HSPZ_E_INVALID, "NULL output");
    *n_stage2 = 0;
    *n_exact = 0;
    if (!e->gate_deferred_valid)
        return fail(e, HSPZ_E_STATE, "the last score_gate call did not take the window path");
    int rc = set_device(e);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    HIP_TRY(e, hipMemcpyAsync(e->h_pinned, e->d_defer_cnt, 4 * sizeof(uint32_t),
                              hipMemcpyDeviceToHost, s));
    HIP_TRY(e, hipStreamSynchronize(s));
    // the listed stages plus the ones the first stage's workgroups ran themselves
    *n_stage2 = (uint64_t)e->h_pinned[0] + e->h_pinned[2];
    *n_exact = (uint64_t)e->h_pinned[1] + e->h_pinned[3];
    return HSPZ_OK;
}

// ---- exception barrier ----------------------------------------------------------------
// Every int-returning entry point runs its implementation inside a handler, so that no
// C++ exception (an allocation failure in a host-side vector or string) crosses the C ABI:
// it becomes HSPZ_E_NOMEM with a fixed message.
static int api_exception(Engine *e) noexcept {
    try {
        fail(e, HSPZ_E_NOMEM, "host allocation failed");
    } catch (...) {
    }
    return HSPZ_E_NOMEM;
}

HSPZ_API int hspz_engine_create(const hspz_params *p, hspz_engine **out) {
    try {
        return impl_hspz_engine_create(p, out);
    } catch (...) {
        return api_exception(nullptr);
    }
}

HSPZ_API int hspz_upload_reference(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                                   void *stream) {
    try {
        return impl_hspz_upload_reference(engine, h_ascii, len, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_upload_query(hspz_engine *engine, const uint8_t *h_ascii, uint64_t len,
                               int32_t strand, void *stream) {
    try {
        return impl_hspz_upload_query(engine, h_ascii, len, strand, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_seed_range(const hspz_engine *engine, uint64_t pos_lo, uint64_t pos_hi,
                             uint64_t *seed_lo, uint64_t *seed_hi) {
    try {
        return impl_hspz_seed_range(engine, pos_lo, pos_hi, seed_lo, seed_hi);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_plan(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi, void *stream,
                       uint64_t *total_hits, uint32_t *n_chunks) {
    try {
        return impl_hspz_plan(engine, seed_lo, seed_hi, stream, total_hits, n_chunks);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_debug_plan_counts(hspz_engine *engine, const uint32_t *h_counts, uint64_t n,
                                    void *stream, uint64_t *total_hits, uint32_t *n_chunks) {
    try {
        return impl_hspz_debug_plan_counts(engine, h_counts, n, stream, total_hits, n_chunks);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_get_chunk(const hspz_engine *engine, uint32_t i, hspz_chunk *out) {
    try {
        return impl_hspz_get_chunk(engine, i, out);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_get_plan_arrays(const hspz_engine *engine, uint32_t *h_counts,
                                  uint32_t *h_prefix) {
    try {
        return impl_hspz_get_plan_arrays(engine, h_counts, h_prefix);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_get_seeds(const hspz_engine *engine, uint64_t lo, uint64_t hi,
                            uint32_t *h_kmer, uint32_t *h_q_end) {
    try {
        return impl_hspz_get_seeds(engine, lo, hi, h_kmer, h_q_end);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_get_index(const hspz_engine *engine, uint32_t *h_end, uint32_t *h_pos,
                            uint64_t *n_buckets, uint64_t *n_pos) {
    try {
        return impl_hspz_get_index(engine, h_end, h_pos, n_buckets, n_pos);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_find_hits(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors,
                            uint64_t cap, void *stream) {
    try {
        return impl_hspz_find_hits(engine, chunk, d_anchors, cap, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_score_gate(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                             uint8_t *d_flags, void *stream) {
    try {
        return impl_hspz_score_gate(engine, d_anchors, n, d_flags, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_score_gate_noalloc(hspz_engine *engine, const uint64_t *d_anchors,
                                     uint64_t n, uint8_t *d_flags, void *stream) {
    try {
        return impl_hspz_score_gate_noalloc(engine, d_anchors, n, d_flags, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_find_hits_gate(hspz_engine *engine, uint32_t chunk, uint64_t *d_anchors,
                                 uint64_t cap, uint8_t *d_flags, void *stream) {
    try {
        return impl_hspz_find_hits_gate(engine, chunk, d_anchors, cap, d_flags, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_compact(hspz_engine *engine, const uint8_t *d_flags, uint64_t n,
                          uint32_t *d_ids, uint64_t cap, uint64_t *n_out, void *stream) {
    try {
        return impl_hspz_compact(engine, d_flags, n, d_ids, cap, n_out, stream);
    } catch (...) {
        if (n_out) *n_out = 0;
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_materialize(hspz_engine *engine, const uint64_t *d_anchors,
                              const uint32_t *d_ids, uint64_t n_surv, hspz_segment_pair *d_hsp,
                              uint8_t *d_status, void *stream) {
    try {
        return impl_hspz_materialize(engine, d_anchors, d_ids, n_surv, d_hsp, d_status, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_compact_hsps(hspz_engine *engine, const hspz_segment_pair *d_hsp,
                               const uint8_t *d_status, uint64_t n, hspz_segment_pair *d_out,
                               uint64_t cap, uint64_t *n_out, void *stream) {
    try {
        return impl_hspz_compact_hsps(engine, d_hsp, d_status, n, d_out, cap, n_out, stream);
    } catch (...) {
        if (n_out) *n_out = 0;
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_run_batch(hspz_engine *engine, uint64_t seed_lo, uint64_t seed_hi,
                            int32_t time_gate, hspz_batch_stats *stats, void *stream) {
    try {
        return impl_hspz_run_batch(engine, seed_lo, seed_hi, time_gate, stats, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_get_batch_records(const hspz_engine *engine, hspz_segment_pair *h_out,
                                    uint64_t cap, uint64_t *n) {
    try {
        return impl_hspz_get_batch_records(engine, h_out, cap, n);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_dedup_records(const hspz_segment_pair *h_in, uint64_t n,
                                hspz_segment_pair *h_out, uint64_t cap, uint64_t *n_out) {
    try {
        return impl_hspz_dedup_records(h_in, n, h_out, cap, n_out);
    } catch (...) {
        if (n_out) *n_out = 0;
        return api_exception(nullptr);
    }
}

HSPZ_API int hspz_debug_walk_steps(hspz_engine *engine, const uint64_t *d_anchors, uint64_t n,
                                   uint64_t *total_steps, void *stream) {
    try {
        return impl_hspz_debug_walk_steps(engine, d_anchors, n, total_steps, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_debug_gate_deferred(hspz_engine *engine, uint64_t *n_stage2,
                                      uint64_t *n_exact, void *stream) {
    try {
        return impl_hspz_debug_gate_deferred(engine, n_stage2, n_exact, stream);
    } catch (...) {
        return api_exception(const_cast<Engine *>(reinterpret_cast<const Engine *>(engine)));
    }
}

HSPZ_API int hspz_upload_seeds(hspz_engine *engine, const uint32_t *h_kmer,
                               const uint32_t *h_q_end, uint64_t n, void *stream) {
    try {
        return impl_hspz_upload_seeds(engine, h_kmer, h_q_end, n, stream);
    } catch (...) {
        return api_exception(reinterpret_cast<Engine *>(engine));
    }
}
