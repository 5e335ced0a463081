// Hit counting and the device half of the global prefix ("C. Hit discovery", C.1-C.2).
//
// k_count_scan: one workgroup per kScanBlock (1024) seeds.  Each seed's count is the
// difference of adjacent cumulative bucket ends.  The block scans its counts locally
// (64-bit partial sums, so a block total can never wrap) and publishes its block sum.
// The plan writes only that prefix: the per-seed counts and bucket starts (the lower
// ends, which the raw-order expansion reads in seed order instead of gathering them from
// the 4^w-entry table again) are written by a second pass of the same kernel, with no
// prefix, only when a caller needs them; the key-grouped gate reads neither, and on the
// 50 Mb workload leaving out those 8 bytes per seed took 0.12 ms off a 4.4 ms pass.
// k_scan_blocks scans the block sums in 64 bits in one workgroup (the host refuses a
// batch whose total is over 2^32 - 1) and k_add_offsets adds each block's exclusive
// offset back, giving the inclusive prefix.
//
// The per-seed lookup reads a packed form of the cumulative bucket ends (k_count_table):
// one 32-byte record per 28 consecutive keys, holding the bucket start of the first key
// and the count of each key in a byte, eight times smaller than the 4^w-entry table.
// Every lookup is one random line either way; random lines come faster from a smaller
// region (an XCD's 4 MB L2 holds a larger share of it, and address translation reaches
// it with fewer entries).  A record in which some key has 255 or more hits is marked,
// and its keys are looked up in the full table.
//
// The plan itself needs counts only, so it reads a smaller table still (k_count_nibbles):
// each key's count in four bits, eight keys to a dword, 15 meaning "15 or more: look it
// up in the full table".  For 12-mers that is 8.4 MB against the records' 19 MB, and an
// XCD's 4 MB L2 holds about half of it instead of a fifth.
//
// k_chunk_walk: the MAX_HITS cut ("C. Hit discovery", C.3) on the device, by one wave.
// Each boundary is the first seed whose prefix reaches H + MAX_HITS, found by a 64-way
// search: every round the lanes read the last prefix of 64 equal segments of the range
// and a ballot picks the first segment that reaches the target, so a boundary costs
// about log64(n) dependent reads.
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kScanBlock / kThreads;  // 4
static_assert(kPerThread == 4, "uint4 stores assume four seeds per thread");

constexpr uint32_t kCtMarked = 0xFFFFFFFFu;  // record with a count over 254

// Record g of the packed count table from the cumulative ends end_tbl[0 .. nb].
__global__ __launch_bounds__(kThreads) void k_count_table(const uint32_t *__restrict__ end_tbl,
                                                          uint64_t nb, uint32_t n_rec,
                                                          uint4 *__restrict__ ctab) {
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= n_rec) return;
    const uint64_t k0 = (uint64_t)g * kCountTableKeys;
    uint32_t w[8] = {end_tbl[min<uint64_t>(k0, nb)], 0, 0, 0, 0, 0, 0, 0};
    bool marked = false;
    for (uint32_t j = 0; j < kCountTableKeys; j++) {
        const uint64_t k = k0 + j;
        const uint32_t c = k < nb ? end_tbl[k + 1] - end_tbl[k] : 0u;
        marked |= c > 254u;
        w[1 + j / 4] |= min(c, 255u) << (8 * (j % 4));
    }
    if (marked) w[0] = kCtMarked;
    ctab[2 * (uint64_t)g] = make_uint4(w[0], w[1], w[2], w[3]);
    ctab[2 * (uint64_t)g + 1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Dword g of the 4-bit count table: key 8g + j's count, capped at 15, in bits 4j .. 4j+3.
__global__ __launch_bounds__(kThreads) void k_count_nibbles(const uint32_t *__restrict__ end_tbl,
                                                            uint64_t nb, uint32_t n_words,
                                                            uint32_t *__restrict__ cnib) {
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= n_words) return;
    uint32_t w = 0;
    for (uint32_t j = 0; j < 8; j++) {
        const uint64_t k = (uint64_t)g * 8 + j;
        const uint32_t c = k < nb ? end_tbl[k + 1] - end_tbl[k] : 0u;
        w |= min(c, 15u) << (4 * j);
    }
    cnib[g] = w;
}

// Bucket start and hit count of the key at offset i (0 .. 27) of an unmarked record
// (dwords a.x .. b.w): the record's start plus the counts of the keys before it.
__device__ __forceinline__ void count_record(const uint4 a, const uint4 b, uint32_t i,
                                             uint32_t &start, uint32_t &cnt) {
    const uint32_t w[7] = {a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t sum = 0, mine = 0;
#pragma unroll
    for (int d = 0; d < 7; d++) {
        // bytes of word d that belong to keys before i
        const int below = min(max((int)i - 4 * d, 0), 4);
        const uint32_t mask = below == 4 ? 0xFFFFFFFFu : (1u << (8 * below)) - 1u;
        sum = __builtin_amdgcn_sad_u8(w[d] & mask, 0u, sum);
        mine = (int)(i >> 2) == d ? w[d] : mine;
    }
    start = a.x + sum;
    cnt = (mine >> (8 * (i & 3u))) & 0xFFu;
}

// Mode: 0 = injected counts (counts_in), 1 = k-mers looked up in end_tbl, 2 = k-mers
// looked up in the packed table, 3 = counts alone from the 4-bit table (cnib; no bucket
// starts).  The four seeds' loads are issued together, with no branch between them, so
// that a thread keeps four lookups in flight.
template <int Mode>
__global__ __launch_bounds__(kThreads) void k_count_scan(
    const uint32_t *__restrict__ kmer, const uint32_t *counts_in, uint64_t n,
    const uint32_t *__restrict__ end_tbl, const uint4 *__restrict__ ctab,
    const uint32_t *__restrict__ cnib, uint32_t *count, uint32_t *__restrict__ first_out,
    uint32_t *__restrict__ prefix, uint64_t *__restrict__ blksum) {
    // counts_in may alias count (injected counts are scanned in place): each thread
    // reads its own four entries before writing them.
    __shared__ uint64_t wave_tot[kThreads / 64];
    const int t = threadIdx.x;
    const uint64_t first = (uint64_t)blockIdx.x * kScanBlock + (uint64_t)t * kPerThread;

    uint32_t c[kPerThread], b[kPerThread];
    bool in[kPerThread];
    uint64_t sc[kPerThread];  // the seed, clamped into range (n > 0)
#pragma unroll
    for (int i = 0; i < kPerThread; i++) {
        in[i] = first + i < n;
        sc[i] = in[i] ? first + i : n - 1;
    }
    if (Mode == 0) {
#pragma unroll
        for (int i = 0; i < kPerThread; i++) {
            const uint32_t v = counts_in[sc[i]];
            c[i] = in[i] ? v : 0u;
            b[i] = 0;
        }
    } else {
        uint32_t k[kPerThread];
#pragma unroll
        for (int i = 0; i < kPerThread; i++) k[i] = kmer[sc[i]];
        if (Mode == 3) {
            uint32_t wv[kPerThread];
#pragma unroll
            for (int i = 0; i < kPerThread; i++) wv[i] = cnib[k[i] >> 3];
#pragma unroll
            for (int i = 0; i < kPerThread; i++) {
                c[i] = (wv[i] >> (4 * (k[i] & 7u))) & 15u;
                if (c[i] == 15u) c[i] = end_tbl[k[i] + 1] - end_tbl[k[i]];  // 15 or more
                if (!in[i]) c[i] = 0;
                b[i] = 0;
            }
        } else if (Mode == 1) {
            uint32_t lo[kPerThread], hi[kPerThread];
#pragma unroll
            for (int i = 0; i < kPerThread; i++) {
                lo[i] = end_tbl[k[i]];
                hi[i] = end_tbl[k[i] + 1];
            }
#pragma unroll
            for (int i = 0; i < kPerThread; i++) {
                b[i] = in[i] ? lo[i] : 0u;
                c[i] = in[i] ? hi[i] - lo[i] : 0u;
            }
        } else {
            uint4 ra[kPerThread], rb[kPerThread];
            uint32_t g[kPerThread];
#pragma unroll
            for (int i = 0; i < kPerThread; i++) {
                g[i] = (uint32_t)(((uint64_t)(k[i] >> 2) * 613566757ull) >> 32);  // k / 28
                ra[i] = ctab[2 * (uint64_t)g[i]];
                rb[i] = ctab[2 * (uint64_t)g[i] + 1];
            }
#pragma unroll
            for (int i = 0; i < kPerThread; i++) {
                count_record(ra[i], rb[i], k[i] - g[i] * kCountTableKeys, b[i], c[i]);
                if (ra[i].x == kCtMarked) {  // a key of this record has over 254 hits
                    b[i] = end_tbl[k[i]];
                    c[i] = end_tbl[k[i] + 1] - b[i];
                }
                if (!in[i]) b[i] = c[i] = 0;
            }
        }
    }
    uint64_t run[kPerThread];
    uint64_t acc = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; i++) {
        acc += c[i];
        run[i] = acc;
    }
    const uint64_t incl = wave_incl_sum_u64(acc);
    if (lane_id() == 63) wave_tot[t >> 6] = incl;
    __syncthreads();
    uint64_t base = incl - acc;
    for (int w = 0; w < (t >> 6); w++) base += wave_tot[w];

    if (first + kPerThread <= n) {
        if (count) *reinterpret_cast<uint4 *>(count + first) = make_uint4(c[0], c[1], c[2], c[3]);
        if (first_out)
            *reinterpret_cast<uint4 *>(first_out + first) = make_uint4(b[0], b[1], b[2], b[3]);
        if (prefix)
            *reinterpret_cast<uint4 *>(prefix + first) =
                make_uint4((uint32_t)(base + run[0]), (uint32_t)(base + run[1]),
                           (uint32_t)(base + run[2]), (uint32_t)(base + run[3]));
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; i++) {
            if (first + i < n) {
                if (count) count[first + i] = c[i];
                if (first_out) first_out[first + i] = b[i];
                if (prefix) prefix[first + i] = (uint32_t)(base + run[i]);
            }
        }
    }
    if (blksum && t == kThreads - 1) {
        uint64_t tot = 0;
        for (int w = 0; w < kThreads / 64; w++) tot += wave_tot[w];
        blksum[blockIdx.x] = tot;
    }
}

__global__ __launch_bounds__(kThreads) void k_add_offsets(uint32_t *__restrict__ prefix,
                                                          uint64_t n,
                                                          const uint32_t *__restrict__ blkoff) {
    const uint64_t first = (uint64_t)blockIdx.x * kScanBlock + (uint64_t)threadIdx.x * kPerThread;
    const uint32_t off = blkoff[blockIdx.x];
    if (off == 0) return;
    if (first + kPerThread <= n) {
        uint4 v = *reinterpret_cast<uint4 *>(prefix + first);
        v.x += off;
        v.y += off;
        v.z += off;
        v.w += off;
        *reinterpret_cast<uint4 *>(prefix + first) = v;
    } else {
        for (int i = 0; i < kPerThread; i++)
            if (first + i < n) prefix[first + i] += off;
    }
}

constexpr int kScanThreads = 1024;

// One workgroup: tiles of kScanThreads * kScanTile block sums are read coalesced (all of
// a thread's reads in flight together) into LDS, where each thread scans kScanTile
// consecutive sums, and the offsets go back out coalesced; the tile totals carry on.
constexpr int kScanTile = 8;
__global__ __launch_bounds__(kScanThreads) void k_scan_blocks(const uint64_t *__restrict__ blksum,
                                                             uint64_t nblk,
                                                             uint32_t *__restrict__ blkoff,
                                                             PlanInfo *__restrict__ info) {
    __shared__ uint64_t tile[kScanThreads * kScanTile];
    __shared__ uint64_t wave_tot[kScanThreads / 64];
    const int t = threadIdx.x;
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nblk; base += kScanThreads * kScanTile) {
        uint64_t v[kScanTile];
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            const uint64_t i = base + (uint64_t)k * kScanThreads + t;
            v[k] = i < nblk ? blksum[i] : 0;
        }
#pragma unroll
        for (int k = 0; k < kScanTile; k++) tile[k * kScanThreads + t] = v[k];
        __syncthreads();
        uint64_t loc[kScanTile], sum = 0;
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            loc[k] = tile[t * kScanTile + k];
            sum += loc[k];
        }
        const uint64_t incl = wave_incl_sum_u64(sum);
        if (lane_id() == 63) wave_tot[t >> 6] = incl;
        __syncthreads();
        uint64_t acc = carry + incl - sum, tile_total = 0;
        for (int w = 0; w < kScanThreads / 64; w++) {
            if (w < (t >> 6)) acc += wave_tot[w];
            tile_total += wave_tot[w];
        }
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            tile[t * kScanTile + k] = acc;
            acc += loc[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            const uint64_t i = base + (uint64_t)k * kScanThreads + t;
            if (i < nblk) blkoff[i] = (uint32_t)tile[k * kScanThreads + t];
        }
        carry += tile_total;
        __syncthreads();  // the next tile reuses tile and wave_tot
    }
    if (t == 0) info->total = carry;
}

__global__ __launch_bounds__(64) void k_chunk_walk(PrefixView P, uint64_t n,
                                                   uint64_t max_hits, uint64_t batch_lo,
                                                   PlanBuf *__restrict__ buf) {
    const int lane = lane_id();
    const uint64_t total = buf->info.total;
    uint32_t c = 0;
    if (total > 0 && total <= 0xFFFFFFFFull) {
        uint64_t s0 = 0, H = 0;
        while (s0 < n && c <= kChunkCap) {
            uint64_t e;
            if (max_hits == 0 || total - H <= max_hits) {
                e = n - 1;
            } else {
                // first e >= s0 with P[e] >= target; P[n - 1] = total > target
                const uint32_t target = (uint32_t)(H + max_hits);
                uint64_t lo = s0, hi = n - 1;
                while (hi - lo >= 64) {
                    const uint64_t step = (hi - lo + 64) / 64;  // ceil(span / 64)
                    const uint64_t idx = min(lo + (uint64_t)(lane + 1) * step - 1, hi);
                    // lane 63 reads P[hi] >= target, so the mask is never empty
                    const uint64_t m = __ballot(P.at(idx) >= target);
                    const uint64_t f = (uint64_t)__builtin_ctzll(m);
                    hi = min(lo + (f + 1) * step - 1, hi);
                    lo = lo + f * step;
                }
                const uint64_t idx = lo + (uint64_t)lane;
                const uint64_t m = __ballot(idx <= hi && P.at(min(idx, hi)) >= target);
                e = lo + (uint64_t)__builtin_ctzll(m);
            }
            const uint32_t Pe = P.at(e);
            if (lane == 0 && c < kChunkCap) {
                hspz_chunk ch;
                ch.seed_lo = batch_lo + s0;
                ch.seed_hi = batch_lo + e;
                ch.hit_lo = H;
                ch.n_hits = (uint64_t)Pe - H;
                buf->chunks[c] = ch;
            }
            c++;
            H = Pe;
            s0 = e + 1;
        }
    }
    if (lane == 0) buf->info.n_chunks = c;
}

}  // namespace

hipError_t launch_scan_blocks(const uint64_t *blksum, uint64_t nblk, uint32_t *blkoff,
                              PlanInfo *info, hipStream_t s) {
    hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(kScanThreads), 0, s, blksum, nblk, blkoff,
                       info);
    return hipGetLastError();
}

hipError_t launch_chunk_walk(PrefixView P, uint64_t n, uint64_t max_hits, uint64_t batch_lo,
                             PlanBuf *buf, hipStream_t s) {
    hipLaunchKernelGGL(k_chunk_walk, dim3(1), dim3(64), 0, s, P, n, max_hits, batch_lo, buf);
    return hipGetLastError();
}

hipError_t launch_count_scan(const uint32_t *kmer, const uint32_t *counts_in, uint64_t n,
                             const uint32_t *end_tbl, const uint4 *ctab, uint32_t *count,
                             uint32_t *first, uint32_t *prefix, uint64_t *blksum,
                             hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + kScanBlock - 1) / kScanBlock;
    if (!kmer)
        hipLaunchKernelGGL(k_count_scan<0>, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                           counts_in, n, end_tbl, ctab, nullptr, count, first, prefix, blksum);
    else if (!ctab)
        hipLaunchKernelGGL(k_count_scan<1>, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                           counts_in, n, end_tbl, ctab, nullptr, count, first, prefix, blksum);
    else
        hipLaunchKernelGGL(k_count_scan<2>, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                           counts_in, n, end_tbl, ctab, nullptr, count, first, prefix, blksum);
    return hipGetLastError();
}

hipError_t launch_count_prefix(const uint32_t *kmer, uint64_t n, const uint32_t *end_tbl,
                               const uint32_t *cnib, uint32_t *prefix, uint64_t *blksum,
                               hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(k_count_scan<3>, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                       nullptr, n, end_tbl, nullptr, cnib, nullptr, nullptr, prefix, blksum);
    return hipGetLastError();
}

uint32_t count_table_records(uint64_t nb) {
    return (uint32_t)((nb + kCountTableKeys - 1) / kCountTableKeys);
}

hipError_t launch_count_table(const uint32_t *end_tbl, uint64_t nb, uint4 *ctab,
                              hipStream_t s) {
    const uint32_t n_rec = count_table_records(nb);
    hipLaunchKernelGGL(k_count_table, dim3((n_rec + kThreads - 1) / kThreads), dim3(kThreads),
                       0, s, end_tbl, nb, n_rec, ctab);
    return hipGetLastError();
}

uint64_t count_nibble_words(uint64_t nb) { return (nb + 7) / 8; }

hipError_t launch_count_nibbles(const uint32_t *end_tbl, uint64_t nb, uint32_t *cnib,
                                hipStream_t s) {
    const uint64_t nw = count_nibble_words(nb);
    hipLaunchKernelGGL(k_count_nibbles, dim3((uint32_t)((nw + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, end_tbl, nb, (uint32_t)nw, cnib);
    return hipGetLastError();
}

hipError_t launch_add_offsets(uint32_t *prefix, uint64_t n, const uint32_t *blkoff,
                              hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(k_add_offsets, dim3((uint32_t)blocks), dim3(kThreads), 0, s, prefix,
                       n, blkoff);
    return hipGetLastError();
}

}  // namespace hspz
