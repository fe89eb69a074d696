// team_sample.hip -- draft tokens and their confidences.
//
// The shared verification pool ranks prefixes by what the drafter's output distribution
// says of them (AngelSpec tutorial page, section "Runtime adaptation: verification as a
// shared pool", the D-cut paragraph); these kernels produce what it ranks.  For drafter row
// (r, k): x ~ q = softmax(z / T) by inverse CDF at u = U(Philox(seed; r, k, DRAFT, step)) and
// conf = q(x).  At T = 0 the token is the first argmax and the confidence is the drafter's
// probability of it at T = 1.
//
// sample_stream_kernel  rows x S members.  Member j streams its 16384-logit chunk of the row
//                       once into registers and publishes, without waiting: stochastic, the
//                       mass of each 4096-logit wave range against the member's reference
//                       (its largest wave maximum) and that reference; greedy, the chunk's
//                       maximum and its first index, and the chunk's (M, s) at T = 1.
// sample_finalize_kernel one wave per row: merges the published words in member order, picks
//                       the range holding u R and re-reads it, 64 consecutive logits per lane
//                       (the inverse-CDF draw of the verification's bonus token, laid out for
//                       one wave); the confidence is the drawn token's weight.  The last row
//                       advances the call epoch.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "team.hpp"
#include "team_device.hpp"
#include "team_sample.hpp"

namespace sv {
namespace {

constexpr float kLog2eF = 1.44269504088896341f;   // c at T = 1

template <int DT, bool GREEDY, bool FULL>
__device__ __forceinline__ void sample_member(const TeamArgs &a, int j, int64_t row, TeamRed &red) {
    const int S = a.S;
    const int V = a.V;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *drow = row_ptr<DT>(a.draft, row, a.ld_d);
    const uint32_t epoch = load_uniform(a.epoch);
    LaneRow<DT> dr;
    dr.template load<FULL>(drow, base, V);
    sched_fence();
    const uint32_t tag = epoch + 1;
    if constexpr (GREEDY) {
        const float m = dr.max();
        float wm = m, wz = neg_inf();
        int i0 = 0, i1 = 0;
        block_amax2(wm, i0, wz, i1, red);   // chunk maximum
        int im = (m == wm && m != neg_inf()) ? dr.first_index(m, base) : 0x7fffffff;
        float fm = wm, fz = neg_inf();
        int iz = 0x7fffffff;
        block_amax2(fm, im, fz, iz, red);   // its lowest index
        // (M, s) at T = 1 against the wave maximum, for the confidence
        const float mw = wave_max(m);
        float M = (mw == neg_inf()) ? neg_inf() : mw * kLog2eF;
        float s = (mw == neg_inf()) ? 0.f : dr.exp_sum(kLog2eF, M);
        float Mz = neg_inf(), sz = 0.f;
        block_ms2(M, s, Mz, sz, red);
        if (threadIdx.x == 0) {
            putf(part + 4 * S + j, wm, tag);
            put(part + 5 * S + j, (uint32_t)im, tag);
            putf(part + j, M, tag);
            putf(part + S + j, s, tag);
        }
    } else {
        float M, sm;
        dr.lane_ms(a.c, M, sm);
        sm = wave_sum(sm);   // M is the wave's
        if (lane_id() == 0) red.f[0][w] = M;
        __syncthreads();
        float Mj = red.f[0][0];
        for (int q = 1; q < kTeamWaves; ++q) Mj = fmaxf(Mj, red.f[0][q]);
        if (lane_id() == 0) {
            putf(a.dir + row * a.nseg + j * kTeamWaves + w, (M == neg_inf()) ? 0.f : sm * exp2_fast(M - Mj), tag);
            if (w == 0) putf(part + j, Mj, tag);
        }
    }
}

}  // namespace

template <int DT, bool GREEDY>
__global__ __launch_bounds__(kTeamThreads) void sample_stream_kernel(TeamArgs a) {
    __shared__ TeamRed red;
    const int S = a.S;
    const int j = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)S));
    const int64_t row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)S));
    if ((j + 1) * kTeamChunk <= a.V) sample_member<DT, GREEDY, true>(a, j, row, red);
    else sample_member<DT, GREEDY, false>(a, j, row, red);
}

namespace {

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kRowsPerFinalize = kTeamThreads / kWave;   // one wave per row
constexpr int kGatherMax = 5;                             // words per lane: S + nseg <= 5 * 64

// Words p0[0..n0) then p1[0..n1) (n0 + n1 <= kGatherMax * 64), written by an earlier kernel on
// the stream, to dst[0..n0 + n1) in one pass whose loads all issue before any returns.
// Returns false (every lane) when any of them lacks the tag.
__device__ bool wave_gather(const uint64_t *p0, int n0, const uint64_t *p1, int n1, uint32_t tag, uint32_t *dst) {
    const int lane = lane_id();
    const int n = n0 + n1;
    uint64_t w[kGatherMax];
#pragma unroll
    for (int b = 0; b < kGatherMax; ++b) {
        const int i = lane + b * kWave;
        w[b] = i < n0 ? p0[i] : (i < n ? p1[i - n0] : 0);
    }
    bool ok = true;
#pragma unroll
    for (int b = 0; b < kGatherMax; ++b) {
        const int i = lane + b * kWave;
        if (i < n) {
            dst[i] = (uint32_t)w[b];
            ok = ok && (uint32_t)(w[b] >> 32) == tag;
        }
    }
    return __all(ok);
}
constexpr int kFinLane = kTeamSeg / kWave;              // logits of a range per lane (64)

// Token of the range sidx of a row at target rem inside the range, by one wave: lane l holds
// kFinLane consecutive logits; their weights sum in order, the lane sums scan in lane order,
// and the lane holding the crossing scans its weights.  If rounding runs past the range, the
// last logit with positive weight.  Returns the token (every lane); *w: its weight.
template <int DT>
__device__ int wave_draw_range(const void *row, int V, float c, Norm2 nb, int sidx, double rem, float *w) {
    const int lane = lane_id();
    const int e0 = sidx * kTeamSeg + lane * kFinLane;
    const int vend = min(V, (sidx + 1) * kTeamSeg);
    float wt[kFinLane];
    double my = 0.0;
#pragma unroll
    for (int e8 = 0; e8 < kFinLane; e8 += 8) {
        float z[8];
        load8<DT>(row, e0 + e8, vend, z);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wt[e8 + e] = exp2_fast(log2prob(z[e], c, nb));
            my += (double)wt[e8 + e];
        }
    }
    const double incl = wave_incl_scan(my);
    const uint64_t hit = __ballot(incl > rem && my > 0.0);
    int tok = -1;
    float wsel = 0.f;
    if (hit) {
        const int l = __builtin_ctzll(hit);
        if (lane == l) {
            double run = incl - my;
            int k = kFinLane - 1;
            for (int e = 0; e < kFinLane; ++e) {
                run += (double)wt[e];
                if (run > rem) { k = e; break; }
            }
            tok = e0 + k;
#pragma unroll
            for (int e = 0; e < kFinLane; ++e)
                if (e == k) wsel = wt[e];
        }
        tok = __shfl(tok, l, kWave);
        wsel = __shfl(wsel, l, kWave);
    } else {
        // the last logit of the range with positive weight
        int last = -1;
        for (int e = kFinLane - 1; e >= 0; --e)
            if (wt[e] > 0.f) { last = e; break; }
        const uint64_t pos = __ballot(last >= 0);
        if (pos) {
            const int l = 63 - __builtin_clzll(pos);
            if (lane == l) {
                tok = e0 + last;
#pragma unroll
                for (int e = 0; e < kFinLane; ++e)
                    if (e == last) wsel = wt[e];
            }
            tok = __shfl(tok, l, kWave);
            wsel = __shfl(wsel, l, kWave);
        } else {
            tok = min(sidx * kTeamSeg, V - 1);
        }
    }
    *w = wsel;
    return tok;
}

}  // namespace

// One wave per row (kRowsPerFinalize rows per workgroup, no workgroup barrier): merges the
// row's published words in member order, picks the range holding u R, and re-reads it.
template <int DT, bool GREEDY>
__global__ __launch_bounds__(kTeamThreads) void sample_finalize_kernel(TeamArgs a, int32_t *tokens, float *conf) {
    __shared__ uint32_t pay_all[kRowsPerFinalize][5 * 64 + 8];   // S + nseg <= 320 words, or 4S <= 256
    __shared__ float mass_all[kRowsPerFinalize][4 * 64 + 8];
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * kRowsPerFinalize + w;
    if (row >= a.rows) return;
    uint32_t *pay = pay_all[w];
    float *mass = mass_all[w];
    const int S = a.S;
    const int nseg = a.nseg;
    const int r = (int)(row / a.K), k = (int)(row % a.K);
    const uint32_t tag = read_epoch(a.epoch) + 1;
    const uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *drow = row_ptr<DT>(a.draft, row, a.ld_d);
    // the stream kernel has completed: every word is there, so one pass reads them
    bool got;
    if constexpr (GREEDY) got = wave_gather(part, 2 * S, part + 4 * S, 2 * S, tag, pay);
    else got = wave_gather(part, S, a.dir + row * nseg, nseg, tag, pay);
    if (!got && lane == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
    wave_sync();
    int tok = 0;
    float cf = 0.f;
    if constexpr (GREEDY) {
        float bv = neg_inf(), M = neg_inf(), s = 0.f;
        int bi = 0x7fffffff;
        for (int m = 0; m < S; ++m) {   // every lane, the same order
            amax_merge(bv, bi, __uint_as_float(pay[2 * S + m]), (int)pay[3 * S + m]);
            ms_merge(M, s, __uint_as_float(pay[m]), __uint_as_float(pay[S + m]));
        }
        tok = bi == 0x7fffffff ? 0 : bi;
        cf = exp2_fast(log2prob(load1<DT>(drow, tok), kLog2eF, norm2(M, log2f(s))));
    } else {
        // pay[0..S): member references Mj; pay[S + j * W + w]: range masses against Mj
        float M = neg_inf(), sm = 0.f;
        for (int m = lane; m < S; m += kWave) {
            float sj = 0.f;
            for (int q = 0; q < kTeamWaves; ++q) sj += __uint_as_float(pay[S + m * kTeamWaves + q]);
            ms_merge(M, sm, __uint_as_float(pay[m]), sj);
        }
        wave_ms(M, sm);
        const Norm2 nb = norm2(M, log2f(sm));
        double part_sum = 0.0;
        for (int q = lane; q < nseg; q += kWave) {
            const float Mq = __uint_as_float(pay[q / kTeamWaves]);
            mass[q] = (Mq == neg_inf()) ? 0.f : __uint_as_float(pay[S + q]) * exp2_fast((Mq - nb.hi) - nb.lo);
            part_sum += (double)mass[q];
        }
        wave_sync();
        // R: lane partials summed in lane order; the range by inverse CDF in range order
        const double R = __shfl(wave_incl_scan(part_sum), kWave - 1, kWave);
        const float u = uniform24(a.seed, (uint64_t)r, (uint64_t)k, kPurposeDraft, a.step);
        const double t = (double)u * R;
        double ex = 0.0;
        const int sidx = wave_find([&](int q) { return mass[q]; }, nseg, t, &ex);
        if (sidx >= 0) tok = wave_draw_range<DT>(drow, a.V, a.c, nb, sidx, t - ex, &cf);
    }
    if (lane == 0) {
        tokens[row] = tok;
        conf[row] = cf;
        // the last row of the call advances the epoch for the next call
        if (last_arrival(a, row, a.rows)) __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int DT>
static hipError_t launch_sample_t(const TeamArgs &a, int32_t *tokens, float *conf, hipStream_t s) {
    const unsigned grid = (unsigned)((uint64_t)a.rows * (uint64_t)a.S);
    const unsigned fblocks = (unsigned)((a.rows + kRowsPerFinalize - 1) / kRowsPerFinalize);
    if (a.c == 0.f) {
        hipLaunchKernelGGL((sample_stream_kernel<DT, true>), dim3(grid), dim3(kTeamThreads), 0, s, a);
        hipLaunchKernelGGL((sample_finalize_kernel<DT, true>), dim3(fblocks), dim3(kTeamThreads), 0, s, a, tokens,
                           conf);
    } else {
        hipLaunchKernelGGL((sample_stream_kernel<DT, false>), dim3(grid), dim3(kTeamThreads), 0, s, a);
        hipLaunchKernelGGL((sample_finalize_kernel<DT, false>), dim3(fblocks), dim3(kTeamThreads), 0, s, a, tokens,
                           conf);
    }
    return hipGetLastError();
}

hipError_t team_launch_sample(const TeamArgs &a, int dtype_d, int32_t *tokens, float *conf, hipStream_t s) {
    if (dtype_d == SV_BF16) return launch_sample_t<kDtBF16>(a, tokens, conf, s);
    return launch_sample_t<kDtF32>(a, tokens, conf, s);
}

}  // namespace sv
