// Backward bucket expansion ("C. Hit discovery", C.4-C.5).
//
// Occurrence j of seed s (bucket start b, inclusive prefix P[s]) becomes the packed
// anchor  pos[b + j] | (q_end[s] << 32)  at chunk-local slot  P[s] - 1 - hit_lo - j.
// Two mappings write identical bytes:
//   sparse: one thread per seed walks its bucket;
//   dense:  a 16-lane group per seed strides its bucket, so a wave reads four buckets
//           with unit-stride lanes (the page's warp-per-seed path; a quarter wave keeps
//           lanes busy at the ~16-40 hits per seed where the density rule switches).
#include "hspz_internal.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 16;

__global__ __launch_bounds__(kThreads) void k_expand_sparse(
    const uint32_t *__restrict__ kmer, const uint32_t *__restrict__ q_end,
    const uint32_t *__restrict__ prefix, uint64_t n_seeds,
    const uint32_t *__restrict__ end_tbl, const uint32_t *__restrict__ pos, uint32_t hit_lo,
    uint64_t *__restrict__ anchors) {
    const uint64_t s = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (s >= n_seeds) return;
    const uint32_t k = kmer[s];
    const uint32_t b = end_tbl[k];
    const uint32_t cnt = end_tbl[k + 1] - b;
    if (cnt == 0) return;
    const uint32_t slot0 = prefix[s] - 1u - hit_lo;
    const uint64_t hi = (uint64_t)q_end[s] << 32;
    for (uint32_t j = 0; j < cnt; j++) anchors[slot0 - j] = (uint64_t)pos[b + j] | hi;
}

__global__ __launch_bounds__(kThreads) void k_expand_dense(
    const uint32_t *__restrict__ kmer, const uint32_t *__restrict__ q_end,
    const uint32_t *__restrict__ prefix, uint64_t n_seeds,
    const uint32_t *__restrict__ end_tbl, const uint32_t *__restrict__ pos, uint32_t hit_lo,
    uint64_t *__restrict__ anchors) {
    const uint64_t s = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) / kGroup;
    const uint32_t g = threadIdx.x % kGroup;
    if (s >= n_seeds) return;
    const uint32_t k = kmer[s];
    const uint32_t b = end_tbl[k];
    const uint32_t cnt = end_tbl[k + 1] - b;
    const uint32_t slot0 = prefix[s] - 1u - hit_lo;
    const uint64_t hi = (uint64_t)q_end[s] << 32;
    for (uint32_t j = g; j < cnt; j += kGroup) anchors[slot0 - j] = (uint64_t)pos[b + j] | hi;
}

}  // namespace

hipError_t launch_expand(bool dense, const uint32_t *kmer, const uint32_t *q_end,
                         const uint32_t *prefix, uint64_t n_seeds, const uint32_t *end_tbl,
                         const uint32_t *pos, uint32_t hit_lo, uint64_t *anchors,
                         hipStream_t s) {
    if (n_seeds == 0) return hipSuccess;
    if (dense) {
        const uint64_t blocks = (n_seeds * kGroup + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(k_expand_dense, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                           q_end, prefix, n_seeds, end_tbl, pos, hit_lo, anchors);
    } else {
        const uint64_t blocks = (n_seeds + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(k_expand_sparse, dim3((uint32_t)blocks), dim3(kThreads), 0, s, kmer,
                           q_end, prefix, n_seeds, end_tbl, pos, hit_lo, anchors);
    }
    return hipGetLastError();
}

}  // namespace hspz
