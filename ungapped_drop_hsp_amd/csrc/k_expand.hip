// Backward bucket expansion ("C. Hit discovery", C.4-C.5).
//
// Occurrence j of seed s (bucket start b, inclusive prefix P[s]) becomes the packed
// anchor  pos[b + j] | (q_end[s] << 32)  at chunk-local slot  P[s] - 1 - hit_lo - j.
// The count kernel already stored each seed's count and bucket start, so both mappings
// read per-seed data in seed order.  They write identical bytes:
//   sparse: one lane per seed.  The lanes of a wave own 64 consecutive seeds, whose
//           anchors fill one contiguous slot range; the wave writes that range
//           cooperatively, 64 consecutive slots per round, each lane finding the seed
//           that owns its slot by a binary search over the wave's inclusive hit counts
//           in LDS.  Stores and bucket reads are unit-stride, however the hits are spread
//           over the seeds.
//   dense:  a 16-lane group per seed strides its bucket, so a wave covers four buckets
//           with unit-stride lanes (the page's warp-per-seed path; a quarter wave keeps
//           lanes busy at the ~16-40 hits per seed where the density rule switches).
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroup = 16;

__global__ __launch_bounds__(kThreads) void k_expand_sparse(
    const uint32_t *__restrict__ count, const uint32_t *__restrict__ first,
    const uint32_t *__restrict__ q_end, PrefixView prefix, uint64_t n_seeds,
    const uint32_t *__restrict__ pos, uint32_t hit_lo, uint64_t *__restrict__ anchors) {
    __shared__ uint32_t s_incl[kWaves][64];  // inclusive hit count over the wave's seeds
    __shared__ uint32_t s_b[kWaves][64];     // bucket start
    __shared__ uint32_t s_top[kWaves][64];   // slot of occurrence 0: P[s] - 1 - hit_lo
    __shared__ uint32_t s_qe[kWaves][64];    // query end
    const int w = threadIdx.x >> 6;
    const int lane = lane_id();
    const uint64_t s = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t cnt = 0, b = 0, top = 0, qe = 0;
    if (s < n_seeds) {
        cnt = count[s];
        b = first[s];
        top = prefix.at(s) - 1u - hit_lo;
        qe = q_end[s];
    }
    const uint32_t incl = wave_incl_sum_u32(cnt);
    const uint32_t total = __shfl(incl, 63, 64);
    if (total == 0) return;  // wave-uniform; no block barrier follows
    s_incl[w][lane] = incl;
    s_b[w][lane] = b;
    s_top[w][lane] = top;
    s_qe[w][lane] = qe;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // first slot of the wave: P[s0] - hit_lo - count[s0] (lane 0 always holds a seed here)
    const uint32_t start = __shfl(top + 1u - incl, 0, 64);
    const uint32_t *incl_w = s_incl[w];
    for (uint32_t u = lane; u < total; u += 64) {
        // owner = number of the wave's seeds whose inclusive count is <= u
        int L = 0;
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1)
            if (incl_w[L + step - 1] <= u) L += step;
        const uint32_t t = start + u;
        const uint32_t j = s_top[w][L] - t;
        anchors[t] = (uint64_t)pos[s_b[w][L] + j] | ((uint64_t)s_qe[w][L] << 32);
    }
}

__global__ __launch_bounds__(kThreads) void k_expand_dense(
    const uint32_t *__restrict__ count, const uint32_t *__restrict__ first,
    const uint32_t *__restrict__ q_end, PrefixView prefix, uint64_t n_seeds,
    const uint32_t *__restrict__ pos, uint32_t hit_lo, uint64_t *__restrict__ anchors) {
    const uint64_t s = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) / kGroup;
    const uint32_t g = threadIdx.x % kGroup;
    if (s >= n_seeds) return;
    const uint32_t cnt = count[s];
    const uint32_t b = first[s];
    const uint32_t slot0 = prefix.at(s) - 1u - hit_lo;
    const uint64_t hi = (uint64_t)q_end[s] << 32;
    for (uint32_t j = g; j < cnt; j += kGroup) anchors[slot0 - j] = (uint64_t)pos[b + j] | hi;
}

}  // namespace

hipError_t launch_expand(bool dense, const uint32_t *count, const uint32_t *first,
                         const uint32_t *q_end, PrefixView prefix, uint64_t n_seeds,
                         const uint32_t *pos, uint32_t hit_lo, uint64_t *anchors,
                         hipStream_t s) {
    if (n_seeds == 0) return hipSuccess;
    if (dense) {
        const uint64_t blocks = (n_seeds * kGroup + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(k_expand_dense, dim3((uint32_t)blocks), dim3(kThreads), 0, s, count,
                           first, q_end, prefix, n_seeds, pos, hit_lo, anchors);
    } else {
        const uint64_t blocks = (n_seeds + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(k_expand_sparse, dim3((uint32_t)blocks), dim3(kThreads), 0, s, count,
                           first, q_end, prefix, n_seeds, pos, hit_lo, anchors);
    }
    return hipGetLastError();
}

}  // namespace hspz
