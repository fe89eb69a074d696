// team_sample.hip -- draft tokens and their confidences.
//
// The shared verification pool ranks prefixes by what the drafter's output distribution
// says of them (AngelSpec tutorial page, section "Runtime adaptation: verification as a
// shared pool", the D-cut paragraph); these kernels produce what it ranks.  For drafter row
// (r, k): x ~ q = softmax(z / T) by inverse CDF at u = U(Philox(seed; r, k, DRAFT, step)) and
// conf = q(x).  At T = 0 the token is the first argmax and the confidence is the drafter's
// probability of it at T = 1.
//
// sample_kernel, one launch per call:
//   rows x S members.  Member j streams its 16384-logit chunk of the row once into registers
//   and publishes, without waiting: stochastic, the mass of each 4096-logit wave range
//   against the member's reference (its largest wave maximum) and that reference; greedy, the
//   chunk's maximum and its first index, and the chunk's (M, s) at T = 1.
//   then ceil(rows / 4) finalize workgroups, one wave per row, dispatched after every member:
//   the wave gathers the row's published words as they arrive (bounded wait), merges them in
//   member order, picks the range holding u R and re-reads it, 64 consecutive logits per lane
//   (the inverse-CDF draw of the verification's bonus token, laid out for one wave); the
//   confidence is the drawn token's weight.  Once a row's words are all in, no workgroup
//   that writes them still has to read the call epoch: the row arrives, and the last
//   arrival advances the epoch.
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
    if (epoch_poisoned(epoch)) return;   // the workspace samples nothing
    const uint32_t tag = epoch_tag(epoch);
    if constexpr (GREEDY) {
        float m;
        int im;
        dr.max_first(base, m, im);
        float wm = m, wz = neg_inf();
        int iz = 0x7fffffff;
        block_amax2(wm, im, wz, iz, red);   // chunk maximum; equal values: lowest index
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

namespace {

constexpr int kRowsPerFinalize = kTeamThreads / kWave;   // one wave per row
constexpr int kGatherMax = 5;                             // words per lane: S + nseg <= 5 * 64

// Words p0[0..n0) then p1[0..n1) (n0 + n1 <= kGatherMax * 64) to dst[0..n0 + n1), by one wave,
// as they are published: each sweep re-reads the words still without the tag, all its loads
// issued before any returns.  Bounded by `limit` 10-ns ticks; false (every lane) on timeout.
__device__ bool wave_gather(const uint64_t *p0, int n0, const uint64_t *p1, int n1, uint32_t tag, uint32_t *dst,
                            int64_t limit) {
    const int lane = lane_id();
    const int n = n0 + n1;
    uint32_t pend = 0;
#pragma unroll
    for (int b = 0; b < kGatherMax; ++b)
        if (lane + b * kWave < n) pend |= 1u << b;
    const uint64_t t0 = wall_clock64();
    while (true) {
        uint64_t w[kGatherMax];
#pragma unroll
        for (int b = 0; b < kGatherMax; ++b) {
            const int i = lane + b * kWave;
            w[b] = ((pend >> b) & 1u) ? peek(i < n0 ? p0 + i : p1 + (i - n0)) : 0;
        }
#pragma unroll
        for (int b = 0; b < kGatherMax; ++b) {
            if (((pend >> b) & 1u) && (uint32_t)(w[b] >> 32) == tag) {
                dst[lane + b * kWave] = (uint32_t)w[b];
                pend &= ~(1u << b);
            }
        }
        if (__all(pend == 0)) return true;
        if ((int64_t)(wall_clock64() - t0) > limit) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}
constexpr int kFinLane = kTeamSeg / kWave;              // logits of a range per lane (64)

// Weight of one logit of the range: both passes of the draw below compute it with this one
// function, so they see the same binary32 values.
__device__ __forceinline__ float range_weight(float z, float c, Norm2 nb) { return exp2_fast(log2prob(z, c, nb)); }

// Token of the range sidx of a row at target rem inside the range, by one wave: lane l sums
// the weights of its kFinLane consecutive logits in order and the lane sums scan in lane
// order; then the wave reads the logits of the lane holding the crossing again (from cache),
// one per lane, and scans their weights in binary64.  If rounding runs past the range, the
// last logit with positive weight.  Returns the token (every lane); *w: its weight.  No
// lane keeps its weights between the passes, so the draw fits the member workgroups'
// register budget of the kernel it runs in.
template <int DT>
__device__ int wave_draw_range(const void *row, int V, float c, Norm2 nb, int sidx, double rem, float *w) {
    const int lane = lane_id();
    const int vend = min(V, (sidx + 1) * kTeamSeg);
    double my = 0.0;
    const int e0 = sidx * kTeamSeg + lane * kFinLane;
    if (DT == kDtBF16 && e0 + kFinLane <= vend) {
        // all 8 loads in flight at once, kept packed (bfloat16 pairs, element 2i low)
        u32x4 q[kFinLane / 8];
        const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(row) + e0);
#pragma unroll
        for (int g = 0; g < kFinLane / 8; ++g) q[g] = p[g];
#pragma unroll
        for (int g = 0; g < kFinLane / 8; ++g) {
            const uint32_t ws[4] = {q[g].x, q[g].y, q[g].z, q[g].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                my += (double)range_weight(bf16_lo(ws[h]), c, nb);
                my += (double)range_weight(bf16_hi(ws[h]), c, nb);
            }
        }
    } else {
#pragma unroll 2
        for (int e8 = 0; e8 < kFinLane; e8 += 8) {
            float z[8];
            load8<DT>(row, e0 + e8, vend, z);
#pragma unroll
            for (int e = 0; e < 8; ++e) my += (double)range_weight(z[e], c, nb);
        }
    }
    const double incl = wave_incl_scan(my);
    const uint64_t hit = __ballot(incl > rem && my > 0.0);
    const uint64_t pos = __ballot(my > 0.0);
    if (!pos) {
        *w = 0.f;
        return min(sidx * kTeamSeg, V - 1);
    }
    // the lane whose logits hold the token: the crossing, else the last with positive weight
    const int l = hit ? __builtin_ctzll(hit) : 63 - __builtin_clzll(pos);
    const int base = sidx * kTeamSeg + l * kFinLane;
    const int v = base + lane;
    const float x = range_weight(v < vend ? load1<DT>(row, v) : neg_inf(), c, nb);
    int k;
    if (hit) {
        const double before = readlane_d(incl - my, l);
        const uint64_t h = __ballot(before + wave_incl_scan((double)x) > rem);
        k = h ? __builtin_ctzll(h) : kFinLane - 1;   // rounding ran past the lane's logits: its last
    } else {
        k = 63 - __builtin_clzll(__ballot(x > 0.f) | 1ull);
    }
    *w = readlane_f(x, k);
    return base + k;
}

// LDS of a finalize workgroup: one slice per wave (row)
struct SampleFinShared {
    uint32_t pay[kRowsPerFinalize][5 * 64 + 8];   // S + nseg <= 320 words, or 4S <= 256
    float mass[kRowsPerFinalize][4 * 64 + 8];
};
union SampleShared {
    TeamRed red;
    SampleFinShared f;
};


// One wave per row (kRowsPerFinalize rows per workgroup, no workgroup barrier): gathers the
// row's published words, merges them in member order, picks the range holding u R, and
// re-reads it.
template <int DT, bool GREEDY>
__device__ __forceinline__ void sample_finalize(const TeamArgs &a, int fb, SampleFinShared &sh, int32_t *tokens,
                                                float *conf) {
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t row = (int64_t)fb * kRowsPerFinalize + w;
    if (row >= a.rows) return;
    uint32_t *pay = sh.pay[w];
    float *mass = sh.mass[w];
    const int S = a.S;
    const int nseg = a.nseg;
    const int r = (int)(row / a.K), k = (int)(row % a.K);
    const uint32_t epoch = read_epoch(a.epoch);
    if (epoch_poisoned(epoch)) {   // nothing sampled: token -1, confidence 0, flag raised
        if (lane == 0) {
            tokens[row] = -1;
            conf[row] = 0.f;
            atomicOr(a.err, SV_DEVERR_POISONED);
        }
        return;
    }
    const uint32_t tag = epoch_tag(epoch);
    const uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *drow = row_ptr<DT>(a.draft, row, a.ld_d);
    // the draw's uniform depends on the row alone: drawn before the wait for the members
    const float u = GREEDY ? 0.f : uniform24(a.seed, (uint64_t)r, (uint64_t)k, kPurposeDraft, a.step);
    bool got;
    if constexpr (GREEDY) got = wave_gather(part, 2 * S, part + 4 * S, 2 * S, tag, pay, a.fin_ticks);
    else got = wave_gather(part, S, a.dir + row * nseg, nseg, tag, pay, a.fin_ticks);
    if (lane == 0) {
        if (!got) atomicOr(a.err, SV_DEVERR_TIMEOUT);
        // every member of the row has published (unless the wait gave up: then the call ends
        // with the epoch poisoned): the row arrives, the last one advancing the epoch while
        // the draws still run
        const Arrival ar = last_arrival(a, row, a.rows, !got);
        if (ar.last) __hip_atomic_store(a.epoch, epoch_after(tag, ar.gave_up), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wave_lds_sync();
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
        wave_lds_sync();
        // R: lane partials summed in lane order; the range by inverse CDF in range order
        const double R = readlane_d(wave_incl_scan(part_sum), kWave - 1);
        const double t = (double)u * R;
        double ex = 0.0;
        const int sidx = wave_find([&](int q) { return mass[q]; }, nseg, t, &ex);
        if (sidx >= 0) tok = wave_draw_range<DT>(drow, a.V, a.c, nb, sidx, t - ex, &cf);
    }
    if (lane == 0) {
        tokens[row] = tok;
        conf[row] = cf;
    }
}

}  // namespace

// Members (rows x S workgroups), then the finalize workgroups.  bfloat16: at most 64
// registers per lane, so eight waves share each SIMD (binary32 chunks take 64 on their own).
template <int DT, bool GREEDY>
__global__ __launch_bounds__(kTeamThreads) __attribute__((amdgpu_waves_per_eu(DT == kDtBF16 ? 8 : 5))) void sample_kernel(
    TeamArgs a, int32_t *tokens, float *conf) {
    __shared__ SampleShared sh;
    const int S = a.S;
    const unsigned members = (unsigned)a.rows * (unsigned)S;
    if (blockIdx.x >= members) {
        sample_finalize<DT, GREEDY>(opaque_args(), (int)(blockIdx.x - members), sh.f, tokens, conf);
        return;
    }
    const int j = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)S));
    const int64_t row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)S));
    if ((j + 1) * kTeamChunk <= a.V) sample_member<DT, GREEDY, true>(a, j, row, sh.red);
    else sample_member<DT, GREEDY, false>(a, j, row, sh.red);
}

template <int DT>
static hipError_t launch_sample_t(const TeamArgs &a, int32_t *tokens, float *conf, hipStream_t s) {
    const unsigned fblocks = (unsigned)((a.rows + kRowsPerFinalize - 1) / kRowsPerFinalize);
    const unsigned grid = (unsigned)((uint64_t)a.rows * (uint64_t)a.S + fblocks);
    if (a.c == 0.f)
        hipLaunchKernelGGL((sample_kernel<DT, true>), dim3(grid), dim3(kTeamThreads), 0, s, a, tokens, conf);
    else
        hipLaunchKernelGGL((sample_kernel<DT, false>), dim3(grid), dim3(kTeamThreads), 0, s, a, tokens, conf);
    return hipGetLastError();
}

hipError_t team_launch_sample(const TeamArgs &a, int dtype_d, int32_t *tokens, float *conf, hipStream_t s) {
    if (dtype_d == SV_BF16) return launch_sample_t<kDtBF16>(a, tokens, conf, s);
    return launch_sample_t<kDtF32>(a, tokens, conf, s);
}

}  // namespace sv
