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
// sample_finalize_kernel one workgroup per row: merges the published words in member order,
//                       picks the range holding u R and re-reads it (the same inverse-CDF
//                       draw as the bonus token of verification); the confidence is the drawn
//                       token's weight.  The last workgroup advances the call epoch.
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

template <int DT, bool GREEDY>
__global__ __launch_bounds__(kTeamThreads) void sample_finalize_kernel(TeamArgs a, int32_t *tokens, float *conf) {
    __shared__ TeamRed red;
    __shared__ uint32_t pay[8 * 64 + 8];        // 4S <= 256 published words, then nseg <= 256
    __shared__ float s_mass[4 * 64 + 8];
    __shared__ Norm2 s_n;
    __shared__ float s_conf;
    const int S = a.S;
    const int nseg = a.nseg;
    const int64_t row = blockIdx.x;
    const int r = (int)(row / a.K), k = (int)(row % a.K);
    const uint32_t tag = read_epoch(a.epoch) + 1;
    const uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *drow = row_ptr<DT>(a.draft, row, a.ld_d);
    // the stream kernel has completed: every word is there, so one pass reads them
    if (threadIdx.x < kWave) {
        bool got;
        if constexpr (GREEDY) got = wave_poll(part, 2 * S, tag, pay, 0) && wave_poll(part + 4 * S, 2 * S, tag, pay + 2 * S, 0);
        else got = wave_poll(part, S, tag, pay, 0) && wave_poll(a.dir + row * nseg, nseg, tag, pay + S, 0);
        if (!got && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
    }
    if (threadIdx.x == 0) s_conf = 0.f;
    __syncthreads();
    float cf = 0.f;
    int tok = 0;
    if constexpr (GREEDY) {
        if (threadIdx.x == 0) {
            float bv = neg_inf(), M = neg_inf(), s = 0.f;
            int bi = 0x7fffffff;
            for (int m = 0; m < S; ++m) {
                amax_merge(bv, bi, __uint_as_float(pay[2 * S + m]), (int)pay[3 * S + m]);
                ms_merge(M, s, __uint_as_float(pay[m]), __uint_as_float(pay[S + m]));
            }
            tok = bi == 0x7fffffff ? 0 : bi;
            cf = exp2_fast(log2prob(load1<DT>(drow, tok), kLog2eF, norm2(M, log2f(s))));
        }
    } else {
        // pay[0..S): member references Mj; pay[S + j * W + w]: range masses against Mj
        if (threadIdx.x < kWave) {
            float M = neg_inf(), sm = 0.f;
            for (int m = threadIdx.x; m < S; m += kWave) {
                float sj = 0.f;
                for (int w = 0; w < kTeamWaves; ++w) sj += __uint_as_float(pay[S + m * kTeamWaves + w]);
                ms_merge(M, sm, __uint_as_float(pay[m]), sj);
            }
            wave_ms(M, sm);
            if (threadIdx.x == 0) s_n = norm2(M, log2f(sm));
        }
        __syncthreads();
        const Norm2 nb = s_n;
        for (int q = threadIdx.x; q < nseg; q += kTeamThreads) {
            const float Mq = __uint_as_float(pay[q / kTeamWaves]);
            s_mass[q] = (Mq == neg_inf()) ? 0.f : __uint_as_float(pay[S + q]) * exp2_fast((Mq - nb.hi) - nb.lo);
        }
        __syncthreads();
        const float u = uniform24(a.seed, (uint64_t)r, (uint64_t)k, kPurposeDraft, a.step);
        // the confidence is the weight of the token drawn, from the thread that holds it
        tok = draw_ranges<DT, DT, false>(drow, nullptr, a.V, a.c, nb, Norm2{0.f, 0.f}, s_mass, nseg, u, red, &s_conf);
        if (tok < 0) tok = 0;
        cf = s_conf;
    }
    if (threadIdx.x == 0) {
        tokens[row] = tok;
        conf[row] = cf;
        // the last workgroup of the call advances the epoch for the next call
        if (atomicAdd(a.gdone, 1) == (int)gridDim.x - 1) {
            __hip_atomic_store(a.gdone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT>
static hipError_t launch_sample_t(const TeamArgs &a, int32_t *tokens, float *conf, hipStream_t s) {
    const unsigned grid = (unsigned)((uint64_t)a.rows * (uint64_t)a.S);
    if (a.c == 0.f) {
        hipLaunchKernelGGL((sample_stream_kernel<DT, true>), dim3(grid), dim3(kTeamThreads), 0, s, a);
        hipLaunchKernelGGL((sample_finalize_kernel<DT, true>), dim3((unsigned)a.rows), dim3(kTeamThreads), 0, s, a,
                           tokens, conf);
    } else {
        hipLaunchKernelGGL((sample_stream_kernel<DT, false>), dim3(grid), dim3(kTeamThreads), 0, s, a);
        hipLaunchKernelGGL((sample_finalize_kernel<DT, false>), dim3((unsigned)a.rows), dim3(kTeamThreads), 0, s, a,
                           tokens, conf);
    }
    return hipGetLastError();
}

hipError_t team_launch_sample(const TeamArgs &a, int dtype_d, int32_t *tokens, float *conf, hipStream_t s) {
    if (dtype_d == SV_BF16) return launch_sample_t<kDtBF16>(a, tokens, conf, s);
    return launch_sample_t<kDtF32>(a, tokens, conf, s);
}

}  // namespace sv
