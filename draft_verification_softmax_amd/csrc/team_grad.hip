// team_grad.hip -- gradient of the end-to-end TV objective in the drafter logits.
//
// The loss is L_e2e = 1 - (1/(|I| D)) sum_i sum_{m<D} prod_{k<=m} alpha_{i,k} (AngelSpec
// tutorial page, section "From KL to an end-to-end TV loss", the L_e2e equation); the second
// training stage fine-tunes the drafter on it (same section, the paragraph after the
// equation).  By the chain rule, for row (i, k) and token v:
//   dL/dz^d_v = s_{i,k} q_v ([q_v < p_v] - beta_{i,k}),   beta_{i,k} = sum_{w: q_w < p_w} q_w,
//   s_{i,k} = -w_{i,k} / (|I| D T),   w_{i,k} = sum_{m>=k} prod_{j<=m, j!=k} alpha_{i,j},
// the slope of min(p, q) in q being read as [q < p] (0 at a tie).
//
// Kernels, in stream order:
//   weights_kernel  one thread per sequence: w_{i,k} = A_k R_k with the prefix product
//                   A_k = prod_{j<k} alpha_{i,j} and R_k = 1 + alpha_{i,k+1} R_{k+1}
//                   (R_{D-1} = 1), so O(D) per sequence and no division by alpha_{i,k}.
//   grad_kernel     rows x S members.  Member j holds its chunk of the target and drafter
//                   rows in registers (as the verification stream kernel does) and exchanges
//                   two rounds of tagged partials with its team: (M, s) of both rows, then
//                   its share of beta.  It then writes its chunk of the gradient with
//                   16-byte non-temporal stores.  HBM traffic: one read of each logit row,
//                   one write of the gradient row.
//   fixup_kernel    one thread per row checks that every member marked itself done; the
//                   workgroup recomputes any row that has a member which gave up a bounded
//                   wait (it then wrote nothing), streaming the row from HBM.  The last
//                   workgroup advances the call epoch.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "team.hpp"
#include "team_device.hpp"
#include "team_grad.hpp"

namespace sv {
namespace {

constexpr uint32_t kDone = 1u;   // payload of a member's done word (part word 4S + j)

// float -> bfloat16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const __bf16 h = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// beta share of a lane: sum of q over its slots where q < p (compared in log2 domain)
template <int DTT, int DTD>
__device__ __forceinline__ float beta_sum(LaneRow<DTT> &t, LaneRow<DTD> &d, float c, Norm2 nt, Norm2 nd) {
    float b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int g = 0; g < kTeamE; g += 8) {
        t.refresh8(g);
        d.refresh8(g);
#pragma unroll
        for (int i = g; i < g + 8; i += 2) {
            const float xt0 = log2prob(t.get(i), c, nt), xd0 = log2prob(d.get(i), c, nd);
            const float xt1 = log2prob(t.get(i + 1), c, nt), xd1 = log2prob(d.get(i + 1), c, nd);
            b0 += (xd0 < xt0) ? exp2_fast(xd0) : 0.f;
            b1 += (xd1 < xt1) ? exp2_fast(xd1) : 0.f;
        }
        sched_fence();
    }
    return b0 + b1;
}

// The dot2 form of the two gradient passes over bfloat16 rows (as in the overlap pass of the
// verification): v_dot2_f32_bf16 with beta = bf16(c) in one half of its second operand widens
// one logit and applies the scale and the normaliser in one instruction, y = z beta - N.hi /
// gamma, so x = z c - N.hi is y gamma, and q < p is yd < yt (gamma > 0).  The low parts of the
// normalisers are left out (the caller takes this form only when both are below 2^-20).  A
// masked (-inf) logit in the other half of a packed word makes y NaN: a NaN-propagating running
// maximum of every y tells the caller to take the FMA form for the wave instead.
// Eight products of two packed words of each row: yt[e], yd[e] for slots 2q + e (words q, q+1
// of the lane; e = 0, 1 from word q, e = 2, 3 from word q + 1).  A DOT result read by another
// VALU instruction needs three wait states, which the closing s_nop gives the last ones.
__device__ __forceinline__ void dot2_y8(uint32_t t0, uint32_t t1, uint32_t d0, uint32_t d1, uint32_t blo,
                                        uint32_t bhi, float ct, float cd, float (&yt)[4], float (&yd)[4]) {
    asm("v_dot2_f32_bf16 %0, %8, %12, %14\n\t"
        "v_dot2_f32_bf16 %1, %8, %13, %14\n\t"
        "v_dot2_f32_bf16 %2, %9, %12, %14\n\t"
        "v_dot2_f32_bf16 %3, %9, %13, %14\n\t"
        "v_dot2_f32_bf16 %4, %10, %12, %15\n\t"
        "v_dot2_f32_bf16 %5, %10, %13, %15\n\t"
        "v_dot2_f32_bf16 %6, %11, %12, %15\n\t"
        "v_dot2_f32_bf16 %7, %11, %13, %15\n\t"
        "s_nop 2"
        : "=&v"(yt[0]), "=&v"(yt[1]), "=&v"(yt[2]), "=&v"(yt[3]), "=&v"(yd[0]), "=&v"(yd[1]), "=&v"(yd[2]),
          "=&v"(yd[3])
        : "v"(t0), "v"(t1), "v"(d0), "v"(d1), "s"(blo), "s"(bhi), "v"(ct), "v"(cd));
}

// beta_sum in the dot2 form; chk: the running NaN-propagating maximum of every y.
__device__ __forceinline__ float beta_sum_dot2(LaneRow<kDtBF16> &t, LaneRow<kDtBF16> &d, Norm2 nt, Norm2 nd,
                                               const Dot2Scale &ds, float &chk) {
    float ct = neg_over_gamma(nt.hi, ds), cd = neg_over_gamma(nd.hi, ds);
    // wait states between the VALU writes of ct, cd and the first DOT that reads them
    asm volatile("s_nop 4" : "+v"(ct), "+v"(cd));
    float b0 = 0.f, b1 = 0.f;
    chk = neg_inf();
#pragma unroll
    for (int q = 0; q < LaneRow<kDtBF16>::kWords; q += 2) {
        float yt[4], yd[4];
        dot2_y8(t.w[q], t.w[q + 1], d.w[q], d.w[q + 1], ds.blo, ds.bhi, ct, cd, yt, yd);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            b0 += (yd[e] < yt[e]) ? exp2_fast(yd[e] * ds.gamma) : 0.f;
            b1 += (yd[e + 1] < yt[e + 1]) ? exp2_fast(yd[e + 1] * ds.gamma) : 0.f;
            chk = __builtin_elementwise_maximum(chk, __builtin_elementwise_maximum(yt[e], yd[e]));
            chk = __builtin_elementwise_maximum(chk, __builtin_elementwise_maximum(yt[e + 1], yd[e + 1]));
        }
    }
    return b0 + b1;
}

// Gradient of a member's chunk: slot i of lane l in wave w is token
// base + (i / 8) * 512 + l * 8 + i % 8 (base = chunk start + w * kTeamSeg).
// D2: the dot2 form (bfloat16 rows, low parts below 2^-20, no NaN in the wave's y).
template <int DTT, int DTD, int DTG, bool FULL, bool D2>
__device__ __forceinline__ void write_chunk(LaneRow<DTT> &t, LaneRow<DTD> &d, float c, Norm2 nt, Norm2 nd,
                                            float beta, float scale, void *grow, int base, int V,
                                            const Dot2Scale &ds) {
    float ct = 0.f, cd = 0.f;
    // the lane index through an opaque copy: the store addresses are formed here, so the
    // compiler does not keep the row loads' per-lane addresses live through the passes
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    if constexpr (D2) {
        ct = neg_over_gamma(nt.hi, ds);
        cd = neg_over_gamma(nd.hi, ds);
        asm volatile("s_nop 4" : "+v"(ct), "+v"(cd));
    }
#pragma unroll
    for (int g = 0; g < kTeamE; g += 8) {
        float gv[8];
        if constexpr (D2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = g / 2 + 2 * h;   // words q, q + 1: slots g + 4 h .. g + 4 h + 3
                float yt[4], yd[4];
                dot2_y8(t.w[q], t.w[q + 1], d.w[q], d.w[q + 1], ds.blo, ds.bhi, ct, cd, yt, yd);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gv[4 * h + e] = scale * exp2_fast(yd[e] * ds.gamma) * ((yd[e] < yt[e] ? 1.f : 0.f) - beta);
            }
        } else {
            t.refresh8(g);
            d.refresh8(g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xt = log2prob(t.get(g + e), c, nt), xd = log2prob(d.get(g + e), c, nd);
                gv[e] = scale * exp2_fast(xd) * ((xd < xt ? 1.f : 0.f) - beta);
            }
        }
        const int v0 = base + g * 64 + lane * 8;
        if (FULL || v0 + 8 <= V) {
            if constexpr (DTG == kDtBF16) {
                u32x4 q;
                q.x = bf16_bits(gv[0]) | bf16_bits(gv[1]) << 16;
                q.y = bf16_bits(gv[2]) | bf16_bits(gv[3]) << 16;
                q.z = bf16_bits(gv[4]) | bf16_bits(gv[5]) << 16;
                q.w = bf16_bits(gv[6]) | bf16_bits(gv[7]) << 16;
                __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(grow) + (v0 >> 3));
            } else {
                u32x4 q0, q1;
                q0.x = __float_as_uint(gv[0]); q0.y = __float_as_uint(gv[1]);
                q0.z = __float_as_uint(gv[2]); q0.w = __float_as_uint(gv[3]);
                q1.x = __float_as_uint(gv[4]); q1.y = __float_as_uint(gv[5]);
                q1.z = __float_as_uint(gv[6]); q1.w = __float_as_uint(gv[7]);
                u32x4 *p = reinterpret_cast<u32x4 *>(grow) + (v0 >> 2);
                __builtin_nontemporal_store(q0, p);
                __builtin_nontemporal_store(q1, p + 1);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (v0 + e < V) {
                    if constexpr (DTG == kDtBF16) static_cast<uint16_t *>(grow)[v0 + e] = (uint16_t)bf16_bits(gv[e]);
                    else static_cast<float *>(grow)[v0 + e] = gv[e];
                }
            }
        }
        sched_fence();
    }
}

template <int DTG>
__device__ __forceinline__ void *grad_row(const GradArgs &g, int64_t row) {
    return static_cast<char *>(g.grad) + (size_t)(row * g.ld_g) * (DTG == kDtBF16 ? 2 : 4);
}

// One member's work on row `row` (= i * D + k).  FULL: its chunk lies inside the row.
template <int DTT, int DTD, int DTG, bool FULL>
__device__ __forceinline__ void grad_member(const TeamArgs &a, const GradArgs &g, int j, int64_t row, TeamRed &red,
                                            uint32_t *pay, Norm2 *s_tot, int *s_ok, float *s_bs) {
    const int S = a.S;
    const int V = a.V;
    const float c = a.c;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *trow = row_ptr<DTT>(a.target, row, a.ld_t);
    const void *drow = row_ptr<DTD>(a.draft, row, a.ld_d);
    const uint32_t epoch = load_uniform(a.epoch);

    LaneRow<DTT> tr;
    LaneRow<DTD> dr;
    tr.template load<FULL>(trow, base, V);
    dr.template load<FULL>(drow, base, V);
    sched_fence();
    const uint32_t tag = epoch_tag(epoch);

    // ---- first exchange: the row normalisers ----
    ThreadStats ts;
    tr.lane_ms(c, ts.Mt, ts.st);
    dr.lane_ms(c, ts.Md, ts.sd);
    publish_partials(part, S, j, ts, tag, red);
    if (threadIdx.x < kWave) {
        const bool got = wave_poll(part, 4 * S, tag, pay, a.spin_ticks);   // wave-uniform
        if (got) {
            Norm2 nt, nd;
            team_totals(pay, S, nt, nd);
            if (threadIdx.x == 0) { s_tot[0] = nt; s_tot[1] = nd; }
        }
        if (threadIdx.x == 0) *s_ok = got ? 1 : 0;
    }
    __syncthreads();
    if (!*s_ok) {   // no share from this member: its teammates write nothing either
        if (threadIdx.x == 0) put(a.apart + row * S + j, kGaveUp, tag);
        return;
    }
    const Norm2 nt = s_tot[0], nd = s_tot[1];

    // ---- second exchange: beta ----
    // the dot2 form for bfloat16 rows when both low parts are negligible and no y of the
    // wave is NaN (no masked logit next to another in a packed word); else the FMA form
    bool d2 = false;
    float bl;
    if constexpr (DTT == kDtBF16 && DTD == kDtBF16) {
        const Dot2Scale ds = dot2_scale(opaque_args());
        const bool small_lo = __builtin_fabsf(nt.lo) <= kLoNegligible && __builtin_fabsf(nd.lo) <= kLoNegligible;
        if (ds.ok && small_lo) {
            float chk;
            bl = beta_sum_dot2(tr, dr, nt, nd, ds, chk);
            d2 = !__ballot(__builtin_isnan(chk));   // wave-uniform
        }
    }
    if (!d2) bl = beta_sum(tr, dr, c, nt, nd);
    const float b = block_sumf(bl, red);
    if (threadIdx.x == 0) putf(a.apart + row * S + j, b, tag);
    if (threadIdx.x < kWave) {
        const bool got = wave_poll(a.apart + row * S, S, tag, pay, a.spin_ticks);
        if (threadIdx.x == 0) {
            bool ok = got;
            double beta = 0.0;   // member order, so every member gets the same value
            for (int m = 0; m < S && ok; ++m) {
                ok = pay[m] != kGaveUp;
                beta += (double)__uint_as_float(pay[m]);
            }
            *s_ok = ok ? 1 : 0;
            s_bs[0] = (float)beta;
            s_bs[1] = load_uniform(g.scale + row);
            if (ok) put(part + 4 * S + j, kDone, tag);
        }
    }
    __syncthreads();
    if (!*s_ok) return;
    if constexpr (DTT == kDtBF16 && DTD == kDtBF16) {
        if (d2) {
            write_chunk<DTT, DTD, DTG, FULL, true>(tr, dr, c, nt, nd, s_bs[0], s_bs[1], grad_row<DTG>(g, row), base, V,
                                                   dot2_scale(opaque_args()));
            return;
        }
    }
    write_chunk<DTT, DTD, DTG, FULL, false>(tr, dr, c, nt, nd, s_bs[0], s_bs[1], grad_row<DTG>(g, row), base, V,
                                            Dot2Scale{});
}

}  // namespace

// One thread per sequence: s_{i,k} = -grad_loss * w_{i,k} / (|I| D T).
__global__ __launch_bounds__(kTeamThreads) void weights_kernel(const float *alpha, const float *grad_loss, int I,
                                                               int D, double inv_idt, float *scale) {
    const int i = blockIdx.x * kTeamThreads + threadIdx.x;
    if (i >= I) return;
    const float *al = alpha + (size_t)i * D;
    float *sc = scale + (size_t)i * D;
    const double gl = grad_loss ? (double)*grad_loss : 1.0;
    double R = 1.0;   // R_k = sum_{m>=k} prod_{k<j<=m} alpha_j, from the end
    for (int k = D - 1; k >= 0; --k) {
        sc[k] = (float)R;
        R = 1.0 + (double)al[k] * R;
    }
    double A = 1.0;   // A_k = prod_{j<k} alpha_j
    for (int k = 0; k < D; ++k) {
        sc[k] = (float)(-gl * inv_idt * A * (double)sc[k]);
        A *= (double)al[k];
    }
}

template <int DTT, int DTD, int DTG>
__global__ __launch_bounds__(kTeamThreads) void grad_kernel(TeamArgs a, GradArgs g) {
    __shared__ TeamRed red;
    __shared__ uint32_t pay[4 * 128];
    __shared__ Norm2 s_tot[2];
    __shared__ int s_ok;
    __shared__ float s_bs[2];
    const int S = a.S;
    const int j = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)S));
    const int64_t row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)S));
    if ((j + 1) * kTeamChunk <= a.V) grad_member<DTT, DTD, DTG, true>(a, g, j, row, red, pay, s_tot, &s_ok, s_bs);
    else grad_member<DTT, DTD, DTG, false>(a, g, j, row, red, pay, s_tot, &s_ok, s_bs);
}

// Rows with a member that did not write: recomputed whole by the workgroup, chunk by chunk
// (normalisers, then beta, then the gradient), each pass re-reading the row.
template <int DTT, int DTD, int DTG>
__global__ __launch_bounds__(kTeamThreads) void fixup_kernel(TeamArgs a, GradArgs g) {
    __shared__ TeamRed red;
    __shared__ int s_list[kTeamThreads], s_n;
    const int64_t rows = a.rows;
    const int64_t row = (int64_t)blockIdx.x * kTeamThreads + threadIdx.x;
    const uint32_t tag = epoch_tag(read_epoch(a.epoch));
    const int S = a.S;
    const float c = a.c;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    if (row < rows) {
        bool done = true;
        for (int m = 0; m < S && done; ++m) {
            const uint64_t w = peek(a.part + row * 8 * S + 4 * S + m);
            done = (uint32_t)(w >> 32) == tag && (uint32_t)w == kDone;
        }
        if (!done) s_list[atomicAdd(&s_n, 1)] = threadIdx.x;
    }
    __syncthreads();
    const int w = threadIdx.x / kWave;
    for (int q = 0; q < s_n; ++q) {
        const int64_t rr = (int64_t)blockIdx.x * kTeamThreads + s_list[q];
        const void *trow = row_ptr<DTT>(a.target, rr, a.ld_t);
        const void *drow = row_ptr<DTD>(a.draft, rr, a.ld_d);
        // normalisers: chunk partials merged in chunk order, as the team reduction does
        float Tt = neg_inf(), Ts = 0.f, Dt = neg_inf(), Ds = 0.f;
        for (int m = 0; m < S; ++m) {
            LaneRow<DTT> tr;
            LaneRow<DTD> dr;
            tr.template load<false>(trow, m * kTeamChunk + w * kTeamSeg, a.V);
            dr.template load<false>(drow, m * kTeamChunk + w * kTeamSeg, a.V);
            ThreadStats ts;
            tr.lane_ms(c, ts.Mt, ts.st);
            dr.lane_ms(c, ts.Md, ts.sd);
            block_ms2(ts.Mt, ts.st, ts.Md, ts.sd, red);
            ms_merge(Tt, Ts, ts.Mt, ts.st);
            ms_merge(Dt, Ds, ts.Md, ts.sd);
        }
        const Norm2 nt = norm2(Tt, log2f(Ts)), nd = norm2(Dt, log2f(Ds));
        double beta = 0.0;
        for (int m = 0; m < S; ++m) {
            LaneRow<DTT> tr;
            LaneRow<DTD> dr;
            tr.template load<false>(trow, m * kTeamChunk + w * kTeamSeg, a.V);
            dr.template load<false>(drow, m * kTeamChunk + w * kTeamSeg, a.V);
            beta += (double)block_sumf(beta_sum(tr, dr, c, nt, nd), red);
        }
        const float scale = g.scale[rr];
        for (int m = 0; m < S; ++m) {
            LaneRow<DTT> tr;
            LaneRow<DTD> dr;
            const int base = m * kTeamChunk + w * kTeamSeg;
            tr.template load<false>(trow, base, a.V);
            dr.template load<false>(drow, base, a.V);
            write_chunk<DTT, DTD, DTG, false, false>(tr, dr, c, nt, nd, (float)beta, scale, grad_row<DTG>(g, rr), base,
                                                     a.V, Dot2Scale{});
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        // the last workgroup of the call advances the epoch for the next call (every
        // workgroup that reads the epoch has arrived by then: the member grid is complete)
        if (last_arrival(a, blockIdx.x, gridDim.x, false).last)
            __hip_atomic_store(a.epoch, epoch_after(tag, false), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int DTT, int DTD, int DTG>
static hipError_t launch_grad_t(const TeamArgs &a, const GradArgs &g, hipStream_t s) {
    const unsigned wblocks = (unsigned)((a.B + kTeamThreads - 1) / kTeamThreads);
    hipLaunchKernelGGL(weights_kernel, dim3(wblocks), dim3(kTeamThreads), 0, s, g.alpha, g.grad_loss, a.B, a.K,
                       g.inv_idt, g.scale);
    const unsigned grid = (unsigned)((uint64_t)a.rows * (uint64_t)a.S);
    hipLaunchKernelGGL((grad_kernel<DTT, DTD, DTG>), dim3(grid), dim3(kTeamThreads), 0, s, a, g);
    const unsigned fblocks = (unsigned)((a.rows + kTeamThreads - 1) / kTeamThreads);
    hipLaunchKernelGGL((fixup_kernel<DTT, DTD, DTG>), dim3(fblocks), dim3(kTeamThreads), 0, s, a, g);
    return hipGetLastError();
}

template <int DTT, int DTD>
static hipError_t launch_grad_dg(const TeamArgs &a, const GradArgs &g, int dg, hipStream_t s) {
    if (dg == SV_BF16) return launch_grad_t<DTT, DTD, kDtBF16>(a, g, s);
    return launch_grad_t<DTT, DTD, kDtF32>(a, g, s);
}

hipError_t team_launch_grad(const TeamArgs &a, const GradArgs &g, int dt, int dd, int dg, hipStream_t s) {
    if (dt == SV_BF16 && dd == SV_BF16) return launch_grad_dg<kDtBF16, kDtBF16>(a, g, dg, s);
    if (dt == SV_F32 && dd == SV_F32) return launch_grad_dg<kDtF32, kDtF32>(a, g, dg, s);
    if (dt == SV_BF16 && dd == SV_F32) return launch_grad_dg<kDtBF16, kDtF32>(a, g, dg, s);
    return launch_grad_dg<kDtF32, kDtBF16>(a, g, dg, s);
}

}  // namespace sv
