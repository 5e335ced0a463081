// Stable compaction ("D. Score gate", D.4; reused for the accepted records of
// "E. X-drop materialization", E.5).
//
// k_count: each workgroup counts the non-zero bytes of its kCompactBlock (8192) flags.
// k_scan:  one workgroup turns the block counts into exclusive offsets plus the total.
//          (The pages move the block counts to the host for this scan; on one MI355X a
//          single device workgroup does it without a round trip.)
// k_emit:  each workgroup re-reads its flags, ranks the non-zero bytes in index order
//          (per-thread counts, then a block scan) and writes their indices, or copies
//          the selected 16-byte records.  Blocks without survivors return at once.
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kBytes = kCompactBlock / kThreads;  // 32 flag bytes per thread
constexpr int kScanThreads = 1024;

__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    return (uint32_t)__popc((((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u);
}

// The 32 flag bytes of one thread as 8 dwords (bytes past n read as 0).
__device__ __forceinline__ void load_flags(const uint8_t *__restrict__ f, uint64_t start,
                                           uint32_t n, bool aligned, uint32_t (&w)[8]) {
    if (aligned && start + kBytes <= n) {
        const uint4 *p = reinterpret_cast<const uint4 *>(f + start);
        const uint4 a = p[0], b = p[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) {
            uint32_t v = 0;
            for (int j = 0; j < 4; j++) {
                const uint64_t i = start + 4 * k + j;
                const uint32_t byte = i < n ? f[i] : 0u;
                v |= byte << (8 * j);
            }
            w[k] = v;
        }
    }
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t &total) {
    const int t = threadIdx.x;
    const uint32_t incl = wave_incl_sum_u32(v);
    if (lane_id() == 63) sh[t >> 6] = incl;
    __syncthreads();
    uint32_t base = 0;
    total = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) {
        if (w < (t >> 6)) base += sh[w];
        total += sh[w];
    }
    return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void k_count(const uint8_t *__restrict__ f, uint32_t n,
                                                    int aligned, uint32_t *__restrict__ blk) {
    __shared__ uint32_t sh[kThreads / 64];
    const uint64_t start = (uint64_t)blockIdx.x * kCompactBlock + (uint64_t)threadIdx.x * kBytes;
    uint32_t w[8];
    load_flags(f, start, n, aligned != 0, w);
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) c += nonzero_bytes(w[k]);
    uint32_t total;
    block_excl_scan(c, sh, total);
    if (threadIdx.x == 0) blk[blockIdx.x] = total;
}

// In place: blk[0..nblk) counts -> exclusive offsets, blk[nblk] = *total = sum.  Tiles of
// kScanThreads * kScanTile counts are read coalesced into LDS (a thread's reads in flight
// together), scanned there kScanTile consecutive counts per thread, and written back.
constexpr int kScanTile = 8;
__global__ __launch_bounds__(kScanThreads) void k_scan(uint32_t *__restrict__ blk, uint32_t nblk,
                                                       uint32_t *__restrict__ total_out) {
    __shared__ uint32_t tile[kScanThreads * kScanTile];
    __shared__ uint32_t sh[kScanThreads / 64];
    const int t = threadIdx.x;
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nblk; base += kScanThreads * kScanTile) {
        uint32_t v[kScanTile];
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            const uint32_t i = base + k * kScanThreads + t;
            v[k] = i < nblk ? blk[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kScanTile; k++) tile[k * kScanThreads + t] = v[k];
        __syncthreads();
        uint32_t loc[kScanTile], sum = 0;
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            loc[k] = tile[t * kScanTile + k];
            sum += loc[k];
        }
        uint32_t tile_total;
        uint32_t acc = carry + block_excl_scan(sum, sh, tile_total);
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            tile[t * kScanTile + k] = acc;
            acc += loc[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScanTile; k++) {
            const uint32_t i = base + k * kScanThreads + t;
            if (i < nblk) blk[i] = tile[k * kScanThreads + t];
        }
        carry += tile_total;
        __syncthreads();  // the next tile reuses tile and sh
    }
    if (t == 0) {
        blk[nblk] = carry;
        *total_out = carry;
    }
}

__global__ __launch_bounds__(kThreads) void k_emit(const uint8_t *__restrict__ f, uint32_t n,
                                                   int aligned, const uint32_t *__restrict__ off,
                                                   uint32_t *__restrict__ ids,
                                                   const hspz_segment_pair *__restrict__ rin,
                                                   hspz_segment_pair *__restrict__ rout,
                                                   uint32_t cap) {
    __shared__ uint32_t sh[kThreads / 64];
    const uint32_t b0 = off[blockIdx.x];
    if (off[blockIdx.x + 1] == b0) return;  // no survivor in this block (uniform)
    const uint64_t start = (uint64_t)blockIdx.x * kCompactBlock + (uint64_t)threadIdx.x * kBytes;
    uint32_t w[8];
    load_flags(f, start, n, aligned != 0, w);
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) c += nonzero_bytes(w[k]);
    uint32_t total;
    uint32_t o = b0 + block_excl_scan(c, sh, total);
    if (c == 0) return;
    for (int k = 0; k < 8; k++) {
        for (int j = 0; j < 4; j++) {
            if ((w[k] >> (8 * j)) & 0xFFu) {
                const uint32_t i = (uint32_t)(start + 4 * k + j);
                if (o < cap) {
                    if (rout) rout[o] = rin[i];
                    else ids[o] = i;
                }
                o++;
            }
        }
    }
}

// The same for flags held one bit per element: a workgroup's kCompactBlock flags are its
// threads' 32-bit words, one each.
__global__ __launch_bounds__(kThreads) void k_count_bits(const uint32_t *__restrict__ bits,
                                                         uint32_t words,
                                                         uint32_t *__restrict__ blk) {
    __shared__ uint32_t sh[kThreads / 64];
    const uint64_t w = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint32_t c = w < words ? (uint32_t)__popc(bits[w]) : 0u;
    uint32_t total;
    block_excl_scan(c, sh, total);
    if (threadIdx.x == 0) blk[blockIdx.x] = total;
}

__global__ __launch_bounds__(kThreads) void k_emit_bits(const uint32_t *__restrict__ bits,
                                                        uint32_t words,
                                                        const uint32_t *__restrict__ off,
                                                        uint32_t *__restrict__ ids,
                                                        uint32_t cap) {
    __shared__ uint32_t sh[kThreads / 64];
    const uint32_t b0 = off[blockIdx.x];
    if (off[blockIdx.x + 1] == b0) return;  // no set flag in this block (uniform)
    const uint64_t w = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t v = w < words ? bits[w] : 0u;
    uint32_t total;
    uint32_t o = b0 + block_excl_scan((uint32_t)__popc(v), sh, total);
    while (v) {
        const uint32_t j = (uint32_t)__builtin_ctz(v);
        if (o < cap) ids[o] = (uint32_t)(w * 32u + j);
        o++;
        v &= v - 1u;
    }
}

}  // namespace

hipError_t launch_compact_bits(const uint32_t *bits, uint32_t n, uint32_t *blk,
                               uint32_t *d_total, uint32_t *ids, uint32_t cap, hipStream_t s) {
    const uint32_t nblk = (uint32_t)(((uint64_t)n + kCompactBlock - 1) / kCompactBlock);
    const uint32_t words = (uint32_t)(((uint64_t)n + 31) / 32);
    static_assert(kCompactBlock == 32 * kThreads, "one flag word per thread");
    if (nblk > 0)
        hipLaunchKernelGGL(k_count_bits, dim3(nblk), dim3(kThreads), 0, s, bits, words, blk);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, blk, nblk, d_total);
    if (nblk > 0)
        hipLaunchKernelGGL(k_emit_bits, dim3(nblk), dim3(kThreads), 0, s, bits, words, blk, ids,
                           cap);
    return hipGetLastError();
}

hipError_t launch_compact(const uint8_t *flags, uint32_t n, uint32_t *blk, uint32_t *d_total,
                          uint32_t *ids, const hspz_segment_pair *rec_in,
                          hspz_segment_pair *rec_out, uint32_t cap, hipStream_t s) {
    const uint32_t nblk = (uint32_t)(((uint64_t)n + kCompactBlock - 1) / kCompactBlock);
    const int aligned = ((reinterpret_cast<uintptr_t>(flags) & 15) == 0) ? 1 : 0;
    if (nblk > 0)
        hipLaunchKernelGGL(k_count, dim3(nblk), dim3(kThreads), 0, s, flags, n, aligned, blk);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, blk, nblk, d_total);
    if (nblk > 0)
        hipLaunchKernelGGL(k_emit, dim3(nblk), dim3(kThreads), 0, s, flags, n, aligned, blk, ids,
                           rec_in, rec_out, cap);
    return hipGetLastError();
}

}  // namespace hspz
