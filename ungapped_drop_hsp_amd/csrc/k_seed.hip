// Device seeder and reference indexer: the inputs of "C. Hit discovery", C.1 (the packed
// k-mer of every query seed, and the reference index table: cumulative bucket ends plus
// the concatenated buckets of reference end coordinates, ascending within a bucket).
//
//   k_encode_bytes / k_encode_nibbles  ASCII -> padded byte and 4-bit code arrays, either
//                                      strand (the reverse strand is the reverse
//                                      complement in its own coordinates)
//   k_window_keys                      valid flag and packed key of every window
//   k_gather_pairs                     (key, window end) of the valid windows, listed in
//                                      ascending position by the stable compaction
//   k_key_hist                         bucket sizes (atomic histogram over the keys)
//   k_rs_hist / k_rs_scatter           stable LSD radix sort of (key, end) pairs by key,
//                                      8 bits per pass, so ends stay ascending per bucket
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
// Pairs per thread per radix pass.  Sorting 1.04 M survivors by diagonal, 16 (one
// workgroup per CU) left the scatter waiting on memory; 8 and 4 measured 2% faster per
// step on tandem-rich input, 2 no faster.
constexpr int kRsItems = 8;
constexpr int kRsBlock = kThreads * kRsItems;     // 2048 pairs per workgroup

__device__ __forceinline__ uint32_t ascii_code(uint8_t c) {
    switch (c) {
    case 'A': case 'a': return 0;
    case 'C': case 'c': return 1;
    case 'G': case 'g': return 2;
    case 'T': case 't': return 3;
    default: return kCodeN;
    }
}

// Code of base b (0 <= b < n) of the strand.
__device__ __forceinline__ uint32_t strand_code(const uint8_t *__restrict__ ascii, uint64_t n,
                                                int strand, uint64_t b) {
    if (strand == 0) return ascii_code(ascii[b]);
    const uint32_t c = ascii_code(ascii[n - 1 - b]);
    return c < 4 ? 3u - c : kCodeN;
}

__global__ __launch_bounds__(kThreads) void k_encode_bytes(const uint8_t *__restrict__ ascii,
                                                           uint64_t n, int strand, int shift,
                                                           uint8_t *__restrict__ out) {
    const uint64_t j = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= n + 2 * (uint64_t)kPad) return;
    const int64_t b = (int64_t)j - kPad;
    const uint32_t c = (b >= 0 && (uint64_t)b < n) ? strand_code(ascii, n, strand, (uint64_t)b)
                                                   : (uint32_t)kCodeEdge;
    out[j] = (uint8_t)(c << shift);
}

__global__ __launch_bounds__(kThreads) void k_encode_nibbles(const uint8_t *__restrict__ ascii,
                                                             uint64_t n, int strand,
                                                             uint64_t words,
                                                             uint32_t *__restrict__ out) {
    const uint64_t w = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (w >= words) return;
    uint32_t v = 0;
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const int64_t b = (int64_t)(8 * w + m) - kPad4;
        const uint32_t c = (b >= 0 && (uint64_t)b < n)
                               ? strand_code(ascii, n, strand, (uint64_t)b)
                               : (uint32_t)kCodeEdge;
        v |= c << (4 * m);
    }
    out[w] = v;
}

// Window p is valid when every care position holds A/C/G/T; its key packs the care
// codes two bits each, the first care position most significant.
__global__ __launch_bounds__(kThreads) void k_window_keys(const uint8_t *__restrict__ codes,
                                                          int shift, uint64_t nw, SeedShape sh,
                                                          uint8_t *__restrict__ valid,
                                                          uint32_t *__restrict__ key) {
    const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= nw) return;
    uint32_t k = 0;
    bool ok = true;
    for (int i = 0; i < sh.weight; i++) {
        const uint32_t c = (uint32_t)codes[p + sh.care[i]] >> shift;
        ok = ok && c < 4;
        k = (k << 2) | (c & 3u);
    }
    valid[p] = ok ? 1 : 0;
    key[p] = k;
}

__global__ __launch_bounds__(kThreads) void k_gather_pairs(const uint32_t *__restrict__ pos,
                                                           uint32_t count,
                                                           const uint32_t *__restrict__ key,
                                                           uint32_t span,
                                                           uint32_t *__restrict__ key_out,
                                                           uint32_t *__restrict__ end_out) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= count) return;
    const uint32_t p = pos[i];
    key_out[i] = key[p];
    end_out[i] = p + span;
}

__global__ __launch_bounds__(kThreads) void k_key_hist(const uint32_t *__restrict__ key,
                                                       uint32_t n, uint32_t *__restrict__ cnt) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) atomicAdd(&cnt[key[i]], 1u);
}

__global__ void k_set_u32(uint32_t *p, uint32_t v) { *p = v; }

// Grouping the query's seeds by k-mer (the key-grouped first gate stage): v[i] = i, the
// seed indices that the stable sort by k-mer reorders.
__global__ __launch_bounds__(kThreads) void k_iota(uint32_t *__restrict__ v, uint32_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) v[i] = (uint32_t)i;
}

// 1 where a run of equal keys starts in the sorted key list.
__global__ __launch_bounds__(kThreads) void k_kg_run_flags(const uint32_t *__restrict__ qk,
                                                           uint32_t n,
                                                           uint8_t *__restrict__ flag) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) flag[i] = (i == 0 || qk[i] != qk[i - 1]) ? 1 : 0;
}

// The query end of each seed in grouped order.
__global__ __launch_bounds__(kThreads) void k_kg_gather(const uint32_t *__restrict__ qs,
                                                        uint32_t n,
                                                        const uint32_t *__restrict__ q_end,
                                                        uint32_t *__restrict__ qe) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) qe[i] = q_end[qs[i]];
}

// Each run's range in the grouped order and its first and last seed, in one record.
__global__ __launch_bounds__(kThreads) void k_kg_run_span(const uint32_t *__restrict__ qs,
                                                          uint32_t n,
                                                          const uint32_t *__restrict__ runs,
                                                          uint32_t n_runs,
                                                          uint4 *__restrict__ run_span) {
    const uint64_t r = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (r >= n_runs) return;
    const uint32_t a = runs[r];
    const uint32_t b = r + 1 < n_runs ? runs[r + 1] : n;
    run_span[r] = make_uint4(a, b, qs[a], qs[b - 1]);
}

// Each run's k-mer bucket: its size and start in the reference index.
__global__ __launch_bounds__(kThreads) void k_kg_run_info(const uint32_t *__restrict__ qk,
                                                          const uint32_t *__restrict__ runs,
                                                          uint32_t n_runs,
                                                          const uint32_t *__restrict__ end_tbl,
                                                          uint32_t *__restrict__ run_c,
                                                          uint32_t *__restrict__ run_first) {
    const uint64_t r = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (r >= n_runs) return;
    const uint32_t k = qk[runs[r]];
    const uint32_t b = end_tbl[k];
    run_first[r] = b;
    run_c[r] = end_tbl[k + 1] - b;
}

// Digit histogram of each 2,048-pair block, stored digit-major: hist[d * nblk + block].
__global__ __launch_bounds__(kThreads) void k_rs_hist(const uint32_t *__restrict__ key,
                                                      uint32_t n, int shift, uint32_t nblk,
                                                      uint32_t *__restrict__ hist) {
    __shared__ uint32_t h[256];
    const int t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kRsBlock;
#pragma unroll
    for (int r = 0; r < kRsItems; r++) {
        const uint64_t i = base + (uint64_t)r * kThreads + t;
        if (i < n) atomicAdd(&h[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    hist[(uint64_t)t * nblk + blockIdx.x] = h[t];
}

// Stable scatter: pairs keep their order among equal digits.  The block's first pair of
// digit d goes to incl[d * nblk + block] - hist[d * nblk + block] (the inclusive scan of
// the digit-major histogram, minus the entry itself).  A block takes its pairs in rounds of
// 256 in index order; inside a round each wave ranks its lanes per digit with eight
// ballots, waves are ranked in order through LDS counts, and a running count per digit
// carries over to the next round.
__global__ __launch_bounds__(kThreads) void k_rs_scatter(
    const uint32_t *__restrict__ key_in, const uint32_t *__restrict__ val_in, uint32_t n,
    int shift, uint32_t nblk, const uint32_t *__restrict__ incl,
    const uint32_t *__restrict__ hist, uint32_t *__restrict__ key_out,
    uint32_t *__restrict__ val_out) {
    __shared__ uint32_t running[256];
    __shared__ uint32_t wcnt[kThreads / 64][256];
    const int t = threadIdx.x;
    const int w = t >> 6;
    const int lane = lane_id();
    const uint64_t hi = (uint64_t)t * nblk + blockIdx.x;
    running[t] = incl[hi] - hist[hi];
#pragma unroll
    for (int v = 0; v < kThreads / 64; v++) wcnt[v][t] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * kRsBlock;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r = 0; r < kRsItems; r++) {
        const uint64_t i = base + (uint64_t)r * kThreads + t;
        const bool ok = i < n;
        const uint32_t k = ok ? key_in[i] : 0u;
        const uint32_t v = ok ? val_in[i] : 0u;
        const uint32_t d = (k >> shift) & 255u;
        uint64_t m = __ballot(ok);
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const bool bit = (d >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const uint32_t rank = (uint32_t)__popcll(m & below);
        if (ok && rank == 0) wcnt[w][d] = (uint32_t)__popcll(m);
        __syncthreads();
        if (ok) {
            uint32_t dst = running[d] + rank;
            for (int v2 = 0; v2 < w; v2++) dst += wcnt[v2][d];
            key_out[dst] = k;
            val_out[dst] = v;
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int v2 = 0; v2 < kThreads / 64; v2++) {
            add += wcnt[v2][t];
            wcnt[v2][t] = 0;
        }
        running[t] += add;
        __syncthreads();
    }
}

inline uint32_t grid_of(uint64_t n) { return (uint32_t)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_encode(const uint8_t *ascii, uint64_t n, int strand, uint8_t *bytes, int shift,
                         uint32_t *nibbles, uint64_t nibble_words, hipStream_t s) {
    hipLaunchKernelGGL(k_encode_bytes, dim3(grid_of(n + 2 * (uint64_t)kPad)), dim3(kThreads), 0,
                       s, ascii, n, strand, shift, bytes);
    hipLaunchKernelGGL(k_encode_nibbles, dim3(grid_of(nibble_words)), dim3(kThreads), 0, s,
                       ascii, n, strand, nibble_words, nibbles);
    return hipGetLastError();
}

hipError_t launch_window_keys(const uint8_t *codes, int shift, uint64_t nw, const SeedShape &sh,
                              uint8_t *valid, uint32_t *key, hipStream_t s) {
    if (nw == 0) return hipSuccess;
    hipLaunchKernelGGL(k_window_keys, dim3(grid_of(nw)), dim3(kThreads), 0, s, codes, shift, nw,
                       sh, valid, key);
    return hipGetLastError();
}

hipError_t launch_gather_pairs(const uint32_t *pos, uint32_t count, const uint32_t *key,
                               uint32_t span, uint32_t *key_out, uint32_t *end_out,
                               hipStream_t s) {
    if (count == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_pairs, dim3(grid_of(count)), dim3(kThreads), 0, s, pos, count,
                       key, span, key_out, end_out);
    return hipGetLastError();
}

hipError_t launch_key_hist(const uint32_t *key, uint32_t n, uint32_t *cnt, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_key_hist, dim3(grid_of(n)), dim3(kThreads), 0, s, key, n, cnt);
    return hipGetLastError();
}

hipError_t launch_set_u32(uint32_t *p, uint32_t v, hipStream_t s) {
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, s, p, v);
    return hipGetLastError();
}

uint32_t radix_blocks(uint32_t n) { return (uint32_t)(((uint64_t)n + kRsBlock - 1) / kRsBlock); }

hipError_t launch_iota(uint32_t *v, uint32_t n, hipStream_t s) {
    if (n) hipLaunchKernelGGL(k_iota, dim3(grid_of(n)), dim3(kThreads), 0, s, v, n);
    return hipGetLastError();
}

hipError_t launch_kg_run_flags(const uint32_t *qk, uint32_t n, uint8_t *flag, hipStream_t s) {
    if (n) hipLaunchKernelGGL(k_kg_run_flags, dim3(grid_of(n)), dim3(kThreads), 0, s, qk, n, flag);
    return hipGetLastError();
}

hipError_t launch_kg_gather(const uint32_t *qs, uint32_t n, const uint32_t *q_end, uint32_t *qe,
                            hipStream_t s) {
    if (n)
        hipLaunchKernelGGL(k_kg_gather, dim3(grid_of(n)), dim3(kThreads), 0, s, qs, n, q_end, qe);
    return hipGetLastError();
}

hipError_t launch_kg_run_span(const uint32_t *qs, uint32_t n, const uint32_t *runs,
                              uint32_t n_runs, uint4 *run_span, hipStream_t s) {
    if (n_runs)
        hipLaunchKernelGGL(k_kg_run_span, dim3(grid_of(n_runs)), dim3(kThreads), 0, s, qs, n,
                           runs, n_runs, run_span);
    return hipGetLastError();
}

hipError_t launch_kg_run_info(const uint32_t *qk, const uint32_t *runs, uint32_t n_runs,
                              const uint32_t *end_tbl, uint32_t *run_c, uint32_t *run_first,
                              hipStream_t s) {
    if (n_runs)
        hipLaunchKernelGGL(k_kg_run_info, dim3(grid_of(n_runs)), dim3(kThreads), 0, s, qk, runs,
                           n_runs, end_tbl, run_c, run_first);
    return hipGetLastError();
}

hipError_t launch_radix_hist(const uint32_t *key, uint32_t n, int shift, uint32_t *hist,
                             hipStream_t s) {
    const uint32_t nblk = radix_blocks(n);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rs_hist, dim3(nblk), dim3(kThreads), 0, s, key, n, shift, nblk, hist);
    return hipGetLastError();
}

hipError_t launch_radix_scatter(const uint32_t *key_in, const uint32_t *val_in, uint32_t n,
                                int shift, const uint32_t *incl, const uint32_t *hist,
                                uint32_t *key_out, uint32_t *val_out, hipStream_t s) {
    const uint32_t nblk = radix_blocks(n);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_rs_scatter, dim3(nblk), dim3(kThreads), 0, s, key_in, val_in, n, shift,
                       nblk, incl, hist, key_out, val_out);
    return hipGetLastError();
}

}  // namespace hspz
