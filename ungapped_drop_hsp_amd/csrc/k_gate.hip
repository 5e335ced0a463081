// Score-only X-drop gate ("D. Score gate", D.1-D.3).
//
// Mapping (designed for wave64, not the pages' warp-per-anchor tiles): every lane walks
// one anchor at a time, base by base, and a wave refills finished lanes from its own
// tile of kTile consecutive anchors (ranks from a ballot).  A random anchor scores only
// ~60 bases in total, so spreading one anchor over a whole wave would idle most lanes;
// one anchor per lane keeps every lane on useful bases.
//
// Per lane and per block of B bases the walk keeps, for the running score s and best
// score b, only the drawdown d = b - s (d' = max(d - sigma, 0)), its block maximum and
// s.  A drop inside the block shows as max(d) > xdrop at the block end.  B is chosen by
// the host so that (B - 1) * max(sigma) <= xdrop: after a drop the score cannot climb
// back above the best inside the same block, so b = s + d at the block end is exactly
// the maximum before the first drop, with no per-base branch.  Walks past a sequence
// end read edge bytes whose score -(xdrop + 1) forces that drop.
//
// Phase 1 walks every anchor of the tile to the right and parks R* in LDS; phase 2
// walks left and decides the flag, stopping early once R* + (best so far) reaches T
// (the flag cannot change after that).  Flags are staged in LDS and written per tile.
#include "hspz_internal.h"
#include "wave.h"

namespace hspz {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPerLane = 8;
constexpr int kTile = 64 * kPerLane;  // anchors per wave

// Eight consecutive bytes starting at p, any alignment: three aligned dwords and two
// byte funnels.  Reads [p - 3, p + 12).
__device__ __forceinline__ void load8(const uint8_t *p, uint32_t &lo, uint32_t &hi) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t *w = reinterpret_cast<const uint32_t *>(a & ~uintptr_t(3));
    const uint32_t sh = (uint32_t)(a & 3);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    lo = __builtin_amdgcn_alignbyte(w1, w0, sh);
    hi = __builtin_amdgcn_alignbyte(w2, w1, sh);
}

// Score B bases in walk direction D starting at (rp, qp) (right: rp[0..B), left:
// rp[-1] down to rp[-B]).
template <int D, int B>
__device__ __forceinline__ void block_step(const int32_t *tab, const uint8_t *rp,
                                           const uint8_t *qp, int32_t &d, int32_t &dmax,
                                           int32_t &s) {
    uint32_t rl, rh, ql, qh;
    load8(D > 0 ? rp : rp - B, rl, rh);
    load8(D > 0 ? qp : qp - B, ql, qh);
    const uint32_t pl = rl | ql, ph = rh | qh;
#pragma unroll
    for (int i = 0; i < B; i++) {
        const int bi = D > 0 ? i : B - 1 - i;
        const uint32_t idx = (bi < 4 ? (pl >> (8 * bi)) : (ph >> (8 * (bi - 4)))) & 0xFFu;
        const int32_t sg = tab[idx];
        const int32_t t = d - sg;
        dmax = max(dmax, t);
        d = max(t, 0);
        s += sg;
    }
}

template <int D, int B>
__device__ __forceinline__ void walk_phase(const uint64_t *__restrict__ an, int cnt,
                                           const int32_t *tab, const uint8_t *ref,
                                           const uint8_t *qry, const ScoreParams &sp,
                                           int32_t *rstar, uint8_t *fl8) {
    const int lane = lane_id();
    int next = 64;
    int cur = lane < cnt ? lane : -1;
    const uint8_t *rp = ref, *qp = qry;
    int32_t d = 0, dmax = 0, s = 0, other = 0;

    auto start = [&](int i) {
        const uint64_t a = an[i];
        uint32_t r = (uint32_t)a, q = (uint32_t)(a >> 32);
        if (r > sp.n_ref || q > sp.n_qry) {  // outside the sequences: both sides score 0
            r = D > 0 ? sp.n_ref : 0;
            q = D > 0 ? sp.n_qry : 0;
        }
        rp = ref + r;
        qp = qry + q;
        d = 0;
        dmax = 0;
        s = 0;
        other = D > 0 ? 0 : rstar[i];
    };
    if (cur >= 0) start(cur);

    for (;;) {
        if (__ballot(cur >= 0) == 0) break;
        bool done = false;
        if (cur >= 0) {
            block_step<D, B>(tab, rp, qp, d, dmax, s);
            rp += D * B;
            qp += D * B;
            const int32_t best = s + d;
            const bool keep = (int64_t)other + best >= (int64_t)sp.T;
            done = dmax > sp.xdrop || (D < 0 && keep);
            if (done) {
                if (D > 0) rstar[cur] = best;
                else fl8[cur] = keep ? 1 : 0;
            }
        }
        const uint64_t dm = __ballot(done);
        if (dm) {
            if (done) {
                cur = next + lane_rank(dm);
                if (cur < cnt) start(cur);
                else cur = -1;
            }
            next += __popcll(dm);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <int B>
__global__ __launch_bounds__(kThreads) void k_gate(const uint64_t *__restrict__ anchors,
                                                   uint32_t n, uint8_t *__restrict__ flags,
                                                   const uint8_t *__restrict__ ref,
                                                   const uint8_t *__restrict__ qry,
                                                   ScoreParams sp, int aligned8) {
    __shared__ int32_t tab[kTabSize];
    __shared__ int32_t rstar[kWaves][kTile];
    __shared__ uint32_t flg[kWaves][kTile / 4];
    if (threadIdx.x < kTabSize) tab[threadIdx.x] = sp.tab[threadIdx.x];
    __syncthreads();

    const int w = threadIdx.x >> 6;
    const int lane = lane_id();
    const uint64_t tile0 = ((uint64_t)blockIdx.x * kWaves + w) * kTile;
    if (tile0 >= n) return;
    const int cnt = (int)min<uint64_t>((uint64_t)kTile, (uint64_t)n - tile0);
    const uint64_t *an = anchors + tile0;
    uint8_t *fl8 = reinterpret_cast<uint8_t *>(flg[w]);

    walk_phase<+1, B>(an, cnt, tab, ref, qry, sp, rstar[w], fl8);
    walk_phase<-1, B>(an, cnt, tab, ref, qry, sp, rstar[w], fl8);

    if (cnt == kTile && aligned8) {
        const uint2 v = reinterpret_cast<const uint2 *>(flg[w])[lane];
        reinterpret_cast<uint2 *>(flags + tile0)[lane] = v;
    } else {
        for (int i = lane; i < cnt; i += 64) flags[tile0 + i] = fl8[i];
    }
}

}  // namespace

hipError_t launch_gate(int block_bases, const uint64_t *anchors, uint32_t n, uint8_t *flags,
                       const uint8_t *ref, const uint8_t *qry, const ScoreParams &sp,
                       hipStream_t s) {
    if (n == 0) return hipSuccess;
    const uint32_t per_block = kWaves * kTile;
    const uint32_t blocks = (uint32_t)(((uint64_t)n + per_block - 1) / per_block);
    const int aligned8 = ((reinterpret_cast<uintptr_t>(flags) & 7) == 0) ? 1 : 0;
    switch (block_bases) {
    case 8:
        hipLaunchKernelGGL(k_gate<8>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    case 4:
        hipLaunchKernelGGL(k_gate<4>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    case 2:
        hipLaunchKernelGGL(k_gate<2>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    default:
        hipLaunchKernelGGL(k_gate<1>, dim3(blocks), dim3(kThreads), 0, s, anchors, n, flags,
                           ref, qry, sp, aligned8);
        break;
    }
    return hipGetLastError();
}

}  // namespace hspz
