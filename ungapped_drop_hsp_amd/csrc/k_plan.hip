// Hit counting and the device half of the global prefix ("C. Hit discovery", C.1-C.2).
//
// k_count_scan: one workgroup per kScanBlock (1024) seeds.  Each seed's count is the
// difference of adjacent cumulative bucket ends; the bucket start (the lower end) is
// kept per seed so that the expansion reads it in seed order instead of gathering it
// from the 4^w-entry table again.  The block scans its counts locally
// (64-bit partial sums, so a block total can never wrap) and publishes its block sum.
// The host scans the block sums in 64 bits (refusing a batch over 2^32 - 1) and
// k_add_offsets adds each block's exclusive offset back, giving the inclusive prefix.
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kScanBlock / kThreads;  // 4
static_assert(kPerThread == 4, "uint4 stores assume four seeds per thread");

__global__ __launch_bounds__(kThreads) void k_count_scan(
    const uint32_t *__restrict__ kmer, const uint32_t *counts_in, uint64_t n,
    const uint32_t *__restrict__ end_tbl, uint32_t *count, uint32_t *__restrict__ first_out,
    uint32_t *__restrict__ prefix, uint64_t *__restrict__ blksum) {
    // counts_in may alias count (injected counts are scanned in place): each thread
    // reads its own four entries before writing them.
    __shared__ uint64_t wave_tot[kThreads / 64];
    const int t = threadIdx.x;
    const uint64_t first = (uint64_t)blockIdx.x * kScanBlock + (uint64_t)t * kPerThread;

    uint32_t c[kPerThread], b[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; i++) {
        const uint64_t s = first + i;
        c[i] = 0;
        b[i] = 0;
        if (s < n) {
            if (kmer) {
                const uint32_t k = kmer[s];
                b[i] = end_tbl[k];
                c[i] = end_tbl[k + 1] - b[i];
            } else {
                c[i] = counts_in[s];
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
        *reinterpret_cast<uint4 *>(count + first) = make_uint4(c[0], c[1], c[2], c[3]);
        if (first_out)
            *reinterpret_cast<uint4 *>(first_out + first) = make_uint4(b[0], b[1], b[2], b[3]);
        *reinterpret_cast<uint4 *>(prefix + first) =
            make_uint4((uint32_t)(base + run[0]), (uint32_t)(base + run[1]),
                       (uint32_t)(base + run[2]), (uint32_t)(base + run[3]));
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; i++) {
            if (first + i < n) {
                count[first + i] = c[i];
                if (first_out) first_out[first + i] = b[i];
                prefix[first + i] = (uint32_t)(base + run[i]);
            }
        }
    }
    if (t == kThreads - 1) {
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

}  // namespace

hipError_t launch_count_scan(const uint32_t *kmer, const uint32_t *counts_in, uint64_t n,
                             const uint32_t *end_tbl, uint32_t *count, uint32_t *first,
                             uint32_t *prefix, uint64_t *blksum, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint64_t blocks = (n + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(k_count_scan, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                       counts_in, n, end_tbl, count, first, prefix, blksum);
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
