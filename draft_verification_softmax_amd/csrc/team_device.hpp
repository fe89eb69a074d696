// team_device.hpp -- device helpers shared by the kernels in which a team of workgroups
// shares one row pair (verification, L_e2e and its gradient): tagged-word exchange, fixed-
// order workgroup reductions, a member's register-resident chunk of a row pair and its
// passes, and the row normalisers reduced from the members' partials.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "sv_device.hpp"
#include "team.hpp"

namespace sv {
namespace {

constexpr uint32_t kGaveUp = 0xffffffffu;  // share payload of a member that did not finish

// ---- tagged words --------------------------------------------------------------------
__device__ __forceinline__ void put(uint64_t *p, uint32_t payload, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void putf(uint64_t *p, float v, uint32_t tag) { put(p, __float_as_uint(v), tag); }
__device__ __forceinline__ uint64_t peek(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave waits until words p[0..n) carry `tag` (n <= 2048), copying their payloads to
// dst[0..n).  Bounded by `limit` 10-ns ticks; returns false on timeout.  Every lane of the
// wave must call it.
__device__ inline bool wave_poll(const uint64_t *p, int n, uint32_t tag, uint32_t *dst, int64_t limit) {
    const int l = lane_id();
    uint32_t missing = 0;
    for (int i = l, b = 0; i < n; i += kWave, ++b) missing |= 1u << b;
    const uint64_t t0 = wall_clock64();
    while (true) {
        for (int i = l, b = 0; i < n; i += kWave, ++b) {
            if ((missing >> b) & 1u) {
                const uint64_t w = peek(p + i);
                if ((uint32_t)(w >> 32) == tag) {
                    dst[i] = (uint32_t)w;
                    missing &= ~(1u << b);
                }
            }
        }
        if (__all(missing == 0)) return true;
        if ((int64_t)(wall_clock64() - t0) > limit) return false;
        __builtin_amdgcn_s_sleep(4);   // ~256 cycles between sweeps
    }
}

__device__ __forceinline__ uint32_t read_epoch(const uint32_t *e) {
    return __hip_atomic_load(const_cast<uint32_t *>(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival of unit i of n (one thread per unit) at the end of a call, on the workspace's
// counters: Arrival::last for exactly one unit, whose arrival completes the call, with
// Arrival::gave_up when a unit of the call gave up a wait.  Up to kArriveSingle units share
// the second-level counter directly (one returning atomic on the last unit's path); more land
// on kArriveSlots first-level counters, so at most about n / kArriveSlots + kArriveSlots
// returning atomics queue on one address.
__device__ inline Arrival last_arrival(const TeamArgs &a, int64_t i, int64_t n, bool gave_up) {
    return arrive(
        i, n, gave_up, a.gdone, [&](int s) { return a.arrive + s * kArriveStride; }, kArriveSingle, kArriveSlots,
        [](uint32_t *p, uint32_t v) { return atomicAdd(p, v); }, [](uint32_t *p, uint32_t v) { return atomicOr(p, v); },
        [](uint32_t *p) { __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); });
}

// The kernel's argument block (a TeamArgs, the kernel's first parameter, at the start of the
// kernarg segment) through a pointer the compiler cannot see through: reads through it are
// scalar loads of their own (the pointer still carries the constant address space the loads
// need).  A kernel whose workgroups take one of two paths gives one path this view, so the
// compiler does not merge the two paths' argument loads and hoist them above the branch,
// where they would stay live, and spill, through the other path.
__device__ __forceinline__ const TeamArgs &opaque_args() {
    auto kp = (const __attribute__((address_space(4))) TeamArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    return *(const TeamArgs *)kp;
}

// Scalar load of a value that stays constant while the kernel runs (written, if at all, by
// an earlier kernel on the stream), at a workgroup-uniform address.  It uses the scalar
// counter, so waiting for it never waits for the vector loads of the chunk.
template <class T>
__device__ __forceinline__ T load_uniform(const T *p) {
    return *(const __attribute__((address_space(4))) T *)(uintptr_t)p;
}

// One logit at a workgroup-uniform index i of a row by a scalar load of the 4-byte word that
// holds it (rows are 16-byte aligned with a pitch of a multiple of 16 bytes, so that word
// lies inside the row): the value lands in a scalar register, so no vector register holds
// it while the passes run.
template <int DT>
__device__ __forceinline__ float load1_uniform(const void *row, int i) {
    if constexpr (DT == kDtBF16) {
        const uint32_t w = load_uniform(static_cast<const uint32_t *>(row) + (i >> 1));
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __uint_as_float(load_uniform(static_cast<const uint32_t *>(row) + i));
    }
}

// ---- row chunk loads -----------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- workgroup reductions (fixed order) ------------------------------------------------
struct TeamRed {
    float f[8][kTeamWaves];
    int i[4][kTeamWaves];
    double d[kTeamWaves];
};

// (M, s) pairs in base 2: s = sum 2^{x - M}
__device__ __forceinline__ void ms_merge(float &M, float &s, float M2, float s2) { lse_merge(M, s, M2, s2, 1.0f); }

// (M, s) pairs whose references differ from lane to lane
__device__ __forceinline__ void wave_ms(float &M, float &s) { wave_lse(M, s, 1.0f); }

// The four waves' (M, s) of both rows merged in wave order, into every thread.
__device__ inline void block_merge2(float &Mt, float &st, float &Md, float &sd, TeamRed &red) {
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) { red.f[0][w] = Mt; red.f[1][w] = st; red.f[2][w] = Md; red.f[3][w] = sd; }
    __syncthreads();
    Mt = red.f[0][0]; st = red.f[1][0]; Md = red.f[2][0]; sd = red.f[3][0];
    for (int q = 1; q < kTeamWaves; ++q) { ms_merge(Mt, st, red.f[0][q], red.f[1][q]); ms_merge(Md, sd, red.f[2][q], red.f[3][q]); }
    __syncthreads();
}

// Workgroup (M, s) of both rows from lane states whose reference M is uniform across each
// wave: the lane sums add up without rescaling.
__device__ inline void block_ms2(float &Mt, float &st, float &Md, float &sd, TeamRed &red) {
    st = wave_sum(st);
    sd = wave_sum(sd);
    block_merge2(Mt, st, Md, sd, red);
}

// The same from lane states with a reference per lane.
__device__ inline void block_ms2_lanes(float &Mt, float &st, float &Md, float &sd, TeamRed &red) {
    wave_ms(Mt, st);
    wave_ms(Md, sd);
    block_merge2(Mt, st, Md, sd, red);
}

__device__ inline void block_amax2(float &vt, int &it, float &vd, int &id, TeamRed &red) {
    wave_amax(vt, it);
    wave_amax(vd, id);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) { red.f[4][w] = vt; red.i[0][w] = it; red.f[5][w] = vd; red.i[1][w] = id; }
    __syncthreads();
    vt = red.f[4][0]; it = red.i[0][0]; vd = red.f[5][0]; id = red.i[1][0];
    for (int q = 1; q < kTeamWaves; ++q) { amax_merge(vt, it, red.f[4][q], red.i[0][q]); amax_merge(vd, id, red.f[5][q], red.i[1][q]); }
    __syncthreads();
}

__device__ inline float block_sumf(float x, TeamRed &red) {
    x = wave_sum(x);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) red.f[6][w] = x;
    __syncthreads();
    float t = red.f[6][0];
    for (int q = 1; q < kTeamWaves; ++q) t += red.f[6][q];
    __syncthreads();
    return t;
}

// A wave's pass-1 lane sums against its provisional reference stay below this, else the wave
// takes its exact maximum.
constexpr float kRefSumMax = 0x1p64f;

// ---- one member's chunk, kept as loaded ----------------------------------------------
// Lane l of wave w of member j holds logits base + g * 512 + l * 8 + (0..7), g < kTeamE / 8,
// base = j * kTeamChunk + w * kTeamSeg: bfloat16 as packed pairs, binary32 as is.
template <int DT>
struct LaneRow {
    static constexpr int kWords = DT == kDtBF16 ? kTeamE / 2 : kTeamE;
    uint32_t w[kWords];

    // Widen slot i (bfloat16: a shift or a mask of its packed word).
    __device__ __forceinline__ float get(int i) const {
        if constexpr (DT == kDtBF16) {
            return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
        } else {
            return __uint_as_float(w[i]);
        }
    }

    // Called at the start of every pass over each group of slots: the packed words become
    // opaque to the compiler, so each pass widens them afresh instead of the compiler keeping the
    // widened values of an earlier pass live (which would double the registers the chunk
    // occupies).  Emits no instruction.
    // Per group of 8 slots (one 16-byte load of bfloat16), so that a pass can start on the
    // first groups while later loads are still in flight.
    __device__ __forceinline__ void refresh8(int i) {
        constexpr int kPer8 = DT == kDtBF16 ? 4 : 8;
#pragma unroll
        for (int q = 0; q < kPer8; ++q) asm volatile("" : "+v"(w[(i / 8) * kPer8 + q]));
    }

    // FULL: the range lies inside the row.  Then no load sits under a condition, so the
    // compiler can wait for each one on its own as the passes consume them.
    template <bool FULL>
    __device__ __forceinline__ void load(const void *row, int base, int V) {
#pragma unroll
        for (int g = 0; g < kTeamE / 8; ++g) {
            const int v0 = base + g * 512 + lane_id() * 8;
            if (FULL || v0 + 8 <= V) {
                if constexpr (DT == kDtBF16) {
                    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + (v0 >> 3));
                    w[g * 4 + 0] = q.x; w[g * 4 + 1] = q.y; w[g * 4 + 2] = q.z; w[g * 4 + 3] = q.w;
                } else {
                    const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + (v0 >> 2);
                    const u32x4 q0 = __builtin_nontemporal_load(p), q1 = __builtin_nontemporal_load(p + 1);
                    w[g * 8 + 0] = q0.x; w[g * 8 + 1] = q0.y; w[g * 8 + 2] = q0.z; w[g * 8 + 3] = q0.w;
                    w[g * 8 + 4] = q1.x; w[g * 8 + 5] = q1.y; w[g * 8 + 6] = q1.z; w[g * 8 + 7] = q1.w;
                }
            } else {
                // ragged end of the row: -inf past V
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = v0 + e;
                    if constexpr (DT == kDtBF16) {
                        const uint32_t h = v < V ? (uint32_t) static_cast<const uint16_t *>(row)[v] : 0xff80u;
                        if (e & 1) w[g * 4 + (e >> 1)] |= h << 16;
                        else w[g * 4 + (e >> 1)] = h;
                    } else {
                        w[g * 8 + e] = v < V ? static_cast<const uint32_t *>(row)[v] : 0xff800000u;
                    }
                }
            }
        }
    }

    __device__ __forceinline__ float max() {
        float m0 = neg_inf(), m1 = neg_inf();
#pragma unroll
        for (int g = 0; g < kTeamE; g += 8) {
            refresh8(g);
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                m0 = fmaxf(m0, get(i));
                m1 = fmaxf(m1, get(i + 1));
            }
            sched_fence();
        }
        return fmaxf(m0, m1);
    }

    // The lane's maximum and the vocabulary index of its first occurrence (0x7fffffff when
    // every logit is -inf), in one pass.  Two running maxima over the even and the odd slots
    // keep the dependency chains short; each keeps the first slot of its maximum (slots are
    // visited in vocabulary order), and equal maxima resolve to the lower slot.
    __device__ __forceinline__ void max_first(int base, float &m, int &idx) {
        float m0 = neg_inf(), m1 = neg_inf();
        int s0 = -1, s1 = -1;
#pragma unroll
        for (int g = 0; g < kTeamE; g += 8) {
            refresh8(g);
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                const float z0 = get(i), z1 = get(i + 1);
                if (z0 > m0) { m0 = z0; s0 = i; }
                if (z1 > m1) { m1 = z1; s1 = i + 1; }
            }
            sched_fence();
        }
        const bool take1 = m1 > m0 || (m1 == m0 && s1 >= 0 && s1 < s0);
        m = take1 ? m1 : m0;
        const int sl = take1 ? s1 : s0;
        idx = sl < 0 ? 0x7fffffff : base + (sl >> 3) * 512 + lane_id() * 8 + (sl & 7);
    }

    // The wave's first logit (lane 0, slot 0), the same value in every lane: the packed word
    // is read into a scalar register and widened there.
    __device__ __forceinline__ float wave_first() const {
        const uint32_t u = __builtin_amdgcn_readfirstlane(w[0]);
        if constexpr (DT == kDtBF16) {
            return __uint_as_float(u << 16);
        } else {
            return __uint_as_float(u);
        }
    }

    // (M, s) of this lane's logits in base 2 (s = sum_i 2^{x_i c - M}) without a pass for
    // the maximum.  The reference M is the same for the whole wave, c times the wave's first
    // logit, so the wave's sums add up without rescaling; as that logit is one of the wave's,
    // the wave's largest term is at least 1 and none that matters underflows.  Should some
    // lane's sum reach 2^64 (or the first logit be -inf or NaN), the wave takes its exact
    // maximum instead.  The bound also keeps the exponent x c - M of every term that counts
    // below 64, where the fma's rounding moves a term by at most 2^-19 ln 2 relative.  Every
    // lane of the wave must call it.
    __device__ __forceinline__ void lane_ms(float c, float &M, float &s) {
        refresh8(0);
        const float mw = wave_first();
        M = (mw == neg_inf()) ? neg_inf() : mw * c;
        s = (mw == neg_inf()) ? 0.f : exp_sum(c, M);
        if (__ballot(mw == neg_inf() || !(s < kRefSumMax))) {   // wave-uniform
            const float m = wave_max(max());
            M = (m == neg_inf()) ? neg_inf() : m * c;
            s = (m == neg_inf()) ? 0.f : exp_sum(c, M);
        }
    }

    // sum_i 2^{x_i c - M}, each term kept in e[i] (M = -inf: every logit is -inf, every term 0).
    __device__ __forceinline__ float exp_keep(float c, float M, float (&e)[kTeamE]) {
        const float Mf = M == neg_inf() ? 0.f : M;
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int g = 0; g < kTeamE; g += 8) {
            refresh8(g);
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                e[i] = exp2_fast(__builtin_fmaf(get(i), c, -Mf));
                e[i + 1] = exp2_fast(__builtin_fmaf(get(i + 1), c, -Mf));
                a0 += e[i];
                a1 += e[i + 1];
            }
            sched_fence();
        }
        return a0 + a1;
    }

    // lane_ms with the terms kept in e.  The packed words are dead once e holds the terms:
    // should the first-logit reference fail, the chunk is read again from the row.
    template <bool FULL>
    __device__ __forceinline__ void lane_ms_keep(float c, float &M, float &s, float (&e)[kTeamE], const void *row,
                                                 int base, int V) {
        refresh8(0);
        const float mw = wave_first();
        M = (mw == neg_inf()) ? neg_inf() : mw * c;
        s = exp_keep(c, M, e);
        if (__ballot(mw == neg_inf() || !(s < kRefSumMax))) {   // wave-uniform
            load<FULL>(row, base, V);
            const float m = wave_max(max());
            M = (m == neg_inf()) ? neg_inf() : m * c;
            s = exp_keep(c, M, e);
        }
    }

    // sum_i 2^{x_i c - M}
    __device__ __forceinline__ float exp_sum(float c, float M) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int g = 0; g < kTeamE; g += 8) {
            refresh8(g);
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                a0 += exp2_fast(__builtin_fmaf(get(i), c, -M));
                a1 += exp2_fast(__builtin_fmaf(get(i + 1), c, -M));
            }
            sched_fence();
        }
        return a0 + a1;
    }
};

// A row normaliser in base 2, log2 sum_v 2^{z_v c}, kept as an unevaluated sum hi + lo.
// At low temperature it reaches several hundred, where one binary32 value would be off by
// up to 2^-15 and so every probability by ~2e-5 relative; in two parts a probability is
// 2^{fma(z, c, -hi) - lo}: the fma leaves a small argument, and lo (|lo| <= half an ulp
// of hi) is applied after it.
struct Norm2 {
    float hi, lo;
};

// hi + lo = M + l exactly (Knuth's two-sum); lo = 0 when the sum is not finite.
__device__ __forceinline__ Norm2 norm2(float M, float l) {
    Norm2 n;
    n.hi = M + l;
    const float bv = n.hi - M;
    const float e = (M - (n.hi - bv)) + (l - bv);
    n.lo = __builtin_isfinite(n.hi) ? e : 0.f;
    return n;
}

// log2 of the probability of logit z under the row normaliser n
__device__ __forceinline__ float log2prob(float z, float c, Norm2 n) { return __builtin_fmaf(z, c, -n.hi) - n.lo; }

// A low part this small moves a probability by at most 2^-20 ln 2 < 6.6e-7 relative; it is
// always so when |hi| < 32 (half an ulp of hi).
constexpr float kLoNegligible = 0x1p-20f;

// sum_i min(p_i, q_i) with p = 2^{t c - Nt}, q = 2^{d c - Nd}, as
// 2^{-Nt.lo} sum_i 2^{min(fma(t, c, -Nt.hi), fma(d, c, -Nd.hi) + Nt.lo - Nd.lo)} when `split`
// (uniform), else with both low parts left out (each at most kLoNegligible).  The choice is
// made per group of slots, after the group's words are refreshed, so both arms read the
// same registers.
template <int DTT, int DTD>
__device__ __forceinline__ float min_sum(LaneRow<DTT> &t, LaneRow<DTD> &d, float c, Norm2 nt, Norm2 nd, int split) {
    const float dl = nt.lo - nd.lo;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int g = 0; g < kTeamE; g += 8) {
        t.refresh8(g);
        d.refresh8(g);
        if (split) {
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                a0 += exp2_fast(fminf(__builtin_fmaf(t.get(i), c, -nt.hi), __builtin_fmaf(d.get(i), c, -nd.hi) + dl));
                a1 += exp2_fast(fminf(__builtin_fmaf(t.get(i + 1), c, -nt.hi), __builtin_fmaf(d.get(i + 1), c, -nd.hi) + dl));
            }
        } else {
#pragma unroll
            for (int i = g; i < g + 8; i += 2) {
                a0 += exp2_fast(fminf(__builtin_fmaf(t.get(i), c, -nt.hi), __builtin_fmaf(d.get(i), c, -nd.hi)));
                a1 += exp2_fast(fminf(__builtin_fmaf(t.get(i + 1), c, -nt.hi), __builtin_fmaf(d.get(i + 1), c, -nd.hi)));
            }
        }
        sched_fence();
    }
    return split ? (a0 + a1) * exp2_fast(-nt.lo) : a0 + a1;
}

// Four logit pairs (two packed words of each row) of the dot2 form of the overlap pass: per
// pair, the NaN-propagating minimum of dot2(t, beta, ct) and dot2(d, beta, cd), where
// v_dot2_f32_bf16 in its three-operand form gives a.lo * b.lo + a.hi * b.hi + c with exact
// products and one rounding (beta sits in one half of blo / bhi, 0 in the other).  Inline
// assembly keeps the compiler from choosing the two-operand accumulating form, which needs a
// copy of c into the destination before each use.  A DOT result read by another VALU
// instruction needs three wait states, which the compiler does not know to leave after
// assembly it cannot see into: so the eight products come first and each minimum reads them
// at least three instructions later.  m[0..3]: words (t0, d0) low, high halves, then
// (t1, d1) low, high.
__device__ __forceinline__ void dot2_min4(uint32_t t0, uint32_t t1, uint32_t d0, uint32_t d1, uint32_t blo,
                                          uint32_t bhi, float ct, float cd, float (&m)[4]) {
    float y0, y1, y2, y3, y4, y5, y6, y7;
    asm("v_dot2_f32_bf16 %4, %12, %16, %18\n\t"
        "v_dot2_f32_bf16 %5, %14, %16, %19\n\t"
        "v_dot2_f32_bf16 %6, %12, %17, %18\n\t"
        "v_dot2_f32_bf16 %7, %14, %17, %19\n\t"
        "v_dot2_f32_bf16 %8, %13, %16, %18\n\t"
        "v_dot2_f32_bf16 %9, %15, %16, %19\n\t"
        "v_dot2_f32_bf16 %10, %13, %17, %18\n\t"
        "v_dot2_f32_bf16 %11, %15, %17, %19\n\t"
        "v_minimum3_f32 %0, %4, %5, %5\n\t"
        "v_minimum3_f32 %1, %6, %7, %7\n\t"
        "v_minimum3_f32 %2, %8, %9, %9\n\t"
        "v_minimum3_f32 %3, %10, %11, %11"
        : "=v"(m[0]), "=v"(m[1]), "=v"(m[2]), "=v"(m[3]), "=&v"(y0), "=&v"(y1), "=&v"(y2), "=&v"(y3),
          "=&v"(y4), "=&v"(y5), "=&v"(y6), "=&v"(y7)
        : "v"(t0), "v"(t1), "v"(d0), "v"(d1), "s"(blo), "s"(bhi), "v"(ct), "v"(cd));
}

// The scale c = log2(e) / T as beta * gamma for the dot2 form of the overlap pass (beta a
// bfloat16, gamma = c / beta), from the kernel arguments.
struct Dot2Scale {
    uint32_t blo, bhi;   // beta in the low / high half of a bfloat16 pair, 0 in the other
    float gamma, rgamma;
    bool ok;
};
__device__ __forceinline__ Dot2Scale dot2_scale(const TeamArgs &a) {
    return Dot2Scale{a.d2_blo, a.d2_blo << 16, a.d2_gamma, a.d2_rgamma, a.d2_ok != 0};
}

// -n / gamma with about half an ulp of error: the product with 1 / gamma, then one correction
// step from its residual (so that gamma times the result gives -n back to within an ulp).
__device__ __forceinline__ float neg_over_gamma(float n, const Dot2Scale &ds) {
    const float q = -n * ds.rgamma;
    const float r = __builtin_fmaf(q, ds.gamma, n);   // gamma q + n, the error of q times gamma
    return __builtin_fmaf(-r, ds.rgamma, q);
}

// sum_i min(p_i, q_i) of bfloat16 rows with both low parts left out (as in min_sum's unsplit
// form), in the dot2 form: per logit pair, the minimum of dot2(t, beta, -Nt/gamma) and
// dot2(d, beta, -Nd/gamma) (each the logit times beta less the row's normaliser over gamma,
// one rounding, centred near 0 for the terms that matter), times gamma, into 2^x: six
// instructions per pair instead of seven.  A logit pair whose other half is infinite (a masked
// logit) gives a NaN there, which the NaN-propagating minimum carries into the sum: the caller
// then takes the fma form for the wave.
__device__ __forceinline__ float min_sum_dot2(LaneRow<kDtBF16> &t, LaneRow<kDtBF16> &d, Norm2 nt, Norm2 nd,
                                             const Dot2Scale &ds) {
    float ct = neg_over_gamma(nt.hi, ds), cd = neg_over_gamma(nd.hi, ds);
    // wait states between the VALU writes of ct, cd and the first DOT that reads them
    asm volatile("s_nop 4" : "+v"(ct), "+v"(cd));
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int q = 0; q < LaneRow<kDtBF16>::kWords; q += 2) {
        // no refresh: the packed words are consumed as they are, nothing widened is kept
        float m[4];
        dot2_min4(t.w[q], t.w[q + 1], d.w[q], d.w[q + 1], ds.blo, ds.bhi, ct, cd, m);
        a0 += exp2_fast(m[0] * ds.gamma);
        a1 += exp2_fast(m[1] * ds.gamma);
        a0 += exp2_fast(m[2] * ds.gamma);
        a1 += exp2_fast(m[3] * ds.gamma);
    }
    return a0 + a1;
}

// Pass 1 of a lane: base-2 log-sum-exp state (M, s = sum 2^{x c - M}) per row, M uniform
// across the wave.
struct ThreadStats {
    float Mt, st, Md, sd;
};

// From the lane maxima mt, md: the wave's maxima are the references.
template <int DTT, int DTD>
__device__ __forceinline__ ThreadStats pass1(LaneRow<DTT> &t, LaneRow<DTD> &d, float mt, float md, float c) {
    mt = wave_max(mt);
    md = wave_max(md);
    ThreadStats s;
    s.Mt = (mt == neg_inf()) ? neg_inf() : mt * c;
    s.Md = (md == neg_inf()) ? neg_inf() : md * c;
    s.st = (mt == neg_inf()) ? 0.f : t.exp_sum(c, s.Mt);
    s.sd = (md == neg_inf()) ? 0.f : d.exp_sum(c, s.Md);
    return s;
}

// Pass 2 of a lane: its share of alpha and of the residual mass sum max(p - q, 0).
template <int DTT, int DTD>
__device__ __forceinline__ void pass2(LaneRow<DTT> &t, LaneRow<DTD> &d, const ThreadStats &s, float c,
                                      Norm2 nt, Norm2 nd, float &alpha, float &resid, const Dot2Scale &ds) {
    // the low parts matter only at large |hi| (low temperatures); the test is uniform
    const int split = __builtin_amdgcn_readfirstlane(
        (__builtin_fabsf(nt.lo) > kLoNegligible || __builtin_fabsf(nd.lo) > kLoNegligible) ? 1 : 0);
    if constexpr (DTT == kDtBF16 && DTD == kDtBF16) {
        if (!split && ds.ok) {
            alpha = min_sum_dot2(t, d, nt, nd, ds);
            if (!__ballot(__builtin_isnan(alpha))) {   // wave-uniform: no infinite logit in the wave's range
                const float P = (s.Mt == neg_inf()) ? 0.f : s.st * exp2_fast((s.Mt - nt.hi) - nt.lo);
                resid = P - alpha;
                return;
            }
        }
    }
    alpha = min_sum(t, d, c, nt, nd, split);
    const float P = (s.Mt == neg_inf()) ? 0.f : s.st * exp2_fast((s.Mt - nt.hi) - nt.lo);   // this lane's target mass
    resid = P - alpha;
}

// Pass 1 from the lane maxima, the terms kept in et, ed.
template <int DTT, int DTD>
__device__ __forceinline__ ThreadStats pass1_keep(LaneRow<DTT> &t, LaneRow<DTD> &d, float mt, float md, float c,
                                                  float (&et)[kTeamE], float (&ed)[kTeamE]) {
    mt = wave_max(mt);
    md = wave_max(md);
    ThreadStats s;
    s.Mt = (mt == neg_inf()) ? neg_inf() : mt * c;
    s.Md = (md == neg_inf()) ? neg_inf() : md * c;
    s.st = t.exp_keep(c, s.Mt, et);
    s.sd = d.exp_keep(c, s.Md, ed);
    return s;
}

// Pass 2 over the kept terms.  With p_i = et_i A and q_i = ed_i B (A = 2^{Mt - Nt},
// B = 2^{Md - Nd}, both uniform over the wave), sum min(p_i, q_i) is taken as
// A sum min(et_i, ed_i B/A) when A >= B, else B sum min(et_i A/B, ed_i): one multiply, a
// min and an add per pair, and the ratio is at most 1, so no product overflows.
__device__ __forceinline__ void pass2_keep(const float (&et)[kTeamE], const float (&ed)[kTeamE], const ThreadStats &s,
                                           Norm2 nt, Norm2 nd, float &alpha, float &resid) {
    const float lA = __uint_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_uint(s.Mt == neg_inf() ? neg_inf() : (s.Mt - nt.hi) - nt.lo)));
    const float lB = __uint_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_uint(s.Md == neg_inf() ? neg_inf() : (s.Md - nd.hi) - nd.lo)));
    float a0 = 0.f, a1 = 0.f;
    alpha = 0.f;
    if (lA == neg_inf() || lB == neg_inf()) {
        // one of the rows has no mass in this wave's range: no overlap
    } else if (lA >= lB) {
        const float R = exp2_fast(lB - lA);
#pragma unroll
        for (int i = 0; i < kTeamE; i += 2) {
            a0 += fminf(et[i], ed[i] * R);
            a1 += fminf(et[i + 1], ed[i + 1] * R);
        }
        alpha = (a0 + a1) * exp2_fast(lA);
    } else {
        const float R = exp2_fast(lA - lB);
#pragma unroll
        for (int i = 0; i < kTeamE; i += 2) {
            a0 += fminf(et[i] * R, ed[i]);
            a1 += fminf(et[i + 1] * R, ed[i + 1]);
        }
        alpha = (a0 + a1) * exp2_fast(lB);
    }
    const float P = (s.Mt == neg_inf()) ? 0.f : s.st * exp2_fast(lA);   // this lane's target mass
    resid = P - alpha;
}

// A wave-uniform pair held in scalar registers.
__device__ __forceinline__ Norm2 uniform_norm(Norm2 n) {
    return Norm2{__uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(n.hi))),
                 __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(n.lo)))};
}

// Orders this wave's LDS writes before its lanes' later LDS reads of each other's words.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Row normalisers (base 2) from the S member partials (S <= 64) in pay, by one whole wave:
// lane q takes member q; the maxima and then the rescaled sums reduce in a fixed tree order.
// The members and the finalize (which recomputes them when a member handed over) both call
// this on the same payloads, so they agree bit for bit.  Every lane of the wave must call it;
// every lane gets the result.
__device__ __forceinline__ void team_totals(const uint32_t *pay, int S, Norm2 &nt, Norm2 &nd) {
    wave_lds_sync();
    const int q = lane_id();
    const float mt = q < S ? __uint_as_float(pay[q]) : neg_inf();
    const float st = q < S ? __uint_as_float(pay[S + q]) : 0.f;
    const float md = q < S ? __uint_as_float(pay[2 * S + q]) : neg_inf();
    const float sd = q < S ? __uint_as_float(pay[3 * S + q]) : 0.f;
    const float Mt = wave_max(mt), Md = wave_max(md);
    const float Ts = wave_sum(mt == neg_inf() ? 0.f : st * exp2_fast(mt - Mt));
    const float Ds = wave_sum(md == neg_inf() ? 0.f : sd * exp2_fast(md - Md));
    nt = norm2(Mt, log2f(Ts));
    nd = norm2(Md, log2f(Ds));
}

template <int DT>
__device__ __forceinline__ const void *row_ptr(const void *base, int64_t row, int64_t ld) {
    return static_cast<const char *>(base) + (size_t)(row * ld) * (DT == kDtBF16 ? 2 : 4);
}

// Workgroup-cooperative load of n tagged words into dst (payloads); returns the number of
// words whose tag is not `tag` (their payload is replaced by `missing`).
__device__ inline int load_tagged(const uint64_t *p, int n, uint32_t tag, uint32_t *dst, uint32_t missing) {
    constexpr int U = 8;
    int bad = 0;
    for (int i0 = 0; i0 < n; i0 += U * kTeamThreads) {
        uint64_t w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kTeamThreads + threadIdx.x;
            w[u] = i < n ? peek(p + i) : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kTeamThreads + threadIdx.x;
            if (i < n) {
                const bool ok = (uint32_t)(w[u] >> 32) == tag;
                dst[i] = ok ? (uint32_t)w[u] : missing;
                bad += ok ? 0 : 1;
            }
        }
    }
    return bad;
}

// LDS scratch of draw_ranges (part of the caller's shared block, so that kernels which
// run other work in other workgroups can overlay it).
struct DrawShared {
    double scan[kTeamThreads];
    double ex;
    int seg, tok;
};

// Token drawn by inverse CDF at target t over weights w: the residual max(p - q, 0) after
// a rejection (RESID), else p (the bonus token).  The per-range masses (one per
// kTeamSeg-logit wave range) pick the range; the workgroup re-reads that range and scans
// it in binary64.
// The total R of the range masses is summed in binary64 in range order and the target is
// u * R; -1 when every mass is zero.  w_sel (LDS, optional, set beforehand by the caller):
// receives the weight of the token drawn.
template <int DTT, int DTD, bool RESID>
__device__ int draw_ranges(const void *trow, const void *drow, int V, float c, Norm2 nt, Norm2 nd,
                           const float *dirv, int nseg, float u, DrawShared &ds, float *w_sel = nullptr) {
    int &s_seg = ds.seg;
    double &s_ex = ds.ex;
    double *s_scan = ds.scan;
    int &s_tok = ds.tok;
    const int w = threadIdx.x / kWave;
    if (w == 0) {
        const int lane = lane_id();
        double ex = 0.0;
        int sidx = -1;
        if (nseg <= kWave) {
            // one pass: the inclusive scan gives R at its last lane and the crossing at once
            const double x = lane < nseg ? (double)dirv[lane] : 0.0;
            const double incl = wave_incl_scan(x);
            const double t = (double)u * readlane_d(incl, kWave - 1);
            const uint64_t hit = __ballot(incl > t);
            const uint64_t pos = __ballot(x > 0.0);
            const int l = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
            ex = readlane_d(incl - x, l);
            sidx = (hit || pos) ? l : -1;
            if (lane == 0) s_ex = t - ex;
        } else {
            double part = 0.0;
            for (int q = lane; q < nseg; q += kWave) part += (double)dirv[q];
            // fixed order: lane partials summed in lane order
            const double R = readlane_d(wave_incl_scan(part), kWave - 1);
            const double t = (double)u * R;
            sidx = wave_find([&](int q) { return dirv[q]; }, nseg, t, &ex);
            if (lane == 0) s_ex = t - ex;
        }
        if (lane == 0) s_seg = sidx;
    }
    __syncthreads();
    const int sidx = s_seg;
    if (sidx < 0) return -1;
    const double rem = s_ex;
    // the range's kTeamSeg logits, kPer consecutive ones per thread
    constexpr int kPer = kTeamSeg / kTeamThreads;
    const int e0 = sidx * kTeamSeg + threadIdx.x * kPer;
    const int vend = min(V, (sidx + 1) * kTeamSeg);
    float wt[kPer];
    double my = 0.0;
#pragma unroll
    for (int e8 = 0; e8 < kPer; e8 += 8) {
        float zt[8], zd[8];
        load8<DTT>(trow, e0 + e8, vend, zt);
        if constexpr (RESID) load8<DTD>(drow, e0 + e8, vend, zd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = exp2_fast(log2prob(zt[e], c, nt));
            if constexpr (RESID) {
                const float q = exp2_fast(log2prob(zd[e], c, nd));
                wt[e8 + e] = p - fminf(p, q);
            } else {
                wt[e8 + e] = p;
            }
            my += (double)wt[e8 + e];
        }
    }
    // inclusive scan of per-thread sums in thread order
    double incl = wave_incl_scan(my);
    if (lane_id() == kWave - 1) s_scan[w] = incl;
    __syncthreads();
    double off = 0.0;
    for (int q = 0; q < w; ++q) off += s_scan[q];
    incl += off;
    __syncthreads();
    if (threadIdx.x == 0) s_tok = 0x7fffffff;
    __syncthreads();
    if (incl > rem && incl - my <= rem) {
        // this thread's 8 logits hold the crossing
        double run = incl - my;
        int k = kPer - 1;
        for (int e = 0; e < kPer; ++e) {
            run += (double)wt[e];
            if (run > rem) { k = e; break; }
        }
        atomicMin(&s_tok, e0 + k);
    }
    __syncthreads();
    int tok = s_tok;
    if (tok == 0x7fffffff) {
        // rounding ran past the range: the last logit of the range with positive weight
        int last = -1;
        for (int e = kPer - 1; e >= 0; --e)
            if (wt[e] > 0.f) { last = e0 + e; break; }
        s_scan[threadIdx.x] = (double)last;
        __syncthreads();
        if (threadIdx.x == 0) {
            int best = min(sidx * kTeamSeg, V - 1);
            for (int q = kTeamThreads - 1; q >= 0; --q)
                if (s_scan[q] >= 0.0) { best = (int)s_scan[q]; break; }
            s_tok = best;
        }
        __syncthreads();
        tok = s_tok;
    }
    if (w_sel) {   // the weight of the token drawn, from the thread that holds it (w_sel: LDS)
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (e0 + e == tok) *w_sel = wt[e];
    }
    __syncthreads();
    return tok;
}

// Token of one row drawn from p = softmax(row / T) at target u * R by inverse CDF (the
// single-row draw of the finalize's empty-residual case and of the stand-alone sampler):
// one sweep keeps (max, sum) of every kBonusSeg-logit segment in `seg` (2 nseg floats of
// workspace or LDS, this workgroup only), then a wave finds the segment and re-reads it.
template <int DT>
__device__ __forceinline__ int draw_from_row(const void *row, int V, float c, float u, float *seg, int nseg, TeamRed &red, int &s_tok) {
    const int w = threadIdx.x / kWave;
    float M = neg_inf(), s = 0.f;
    int it = 0;
    for (int base = 0; base < V; base += kTeamThreads * 8, ++it) {
        float z[8];
        load8<DT>(row, base + threadIdx.x * 8, V, z);
        float cm = neg_inf();
#pragma unroll
        for (int e = 0; e < 8; ++e) cm = fmaxf(cm, z[e]);
        const float cM = (cm == neg_inf()) ? neg_inf() : cm * c;   // base-2 reference
        float cs = 0.f;
        if (cm != neg_inf()) {
#pragma unroll
            for (int e = 0; e < 8; ++e) cs += exp2_fast(__builtin_fmaf(z[e], c, -cM));
        }
        ms_merge(M, s, cM, cs);
        float wM = cM, ws = cs;
        wave_ms(wM, ws);
        if (lane_id() == 0) {
            const int sidx = it * kTeamWaves + w;
            if (sidx < nseg) { seg[sidx] = wM; seg[nseg + sidx] = ws; }
        }
    }
    float Md = neg_inf(), sd = 0.f;
    block_ms2_lanes(M, s, Md, sd, red);
    const Norm2 nb = norm2(M, log2f(s));
    __threadfence_block();
    __syncthreads();
    for (int q = threadIdx.x; q < nseg; q += kTeamThreads) {
        const float sM = seg[q], ss = seg[nseg + q];
        seg[q] = (sM == neg_inf()) ? 0.f : ss * exp2_fast((sM - nb.hi) - nb.lo);
    }
    __threadfence_block();
    __syncthreads();
    if (w == 0) {
        double part = 0.0;
        for (int q = lane_id(); q < nseg; q += kWave) part += (double)seg[q];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) part += __shfl_xor(part, d, kWave);
        const double R = part;
        const double t = (double)u * R;
        double ex;
        const int sidx = wave_find([&](int q) { return seg[q]; }, nseg, t, &ex);
        int tok = 0;
        if (sidx >= 0) {
            const int e0 = sidx * kBonusSeg;
            const int n = min(kBonusSeg, V - e0);
            double ex2;
            const int k = wave_find([&](int q) { return exp2_fast(log2prob(load1<DT>(row, e0 + q), c, nb)); }, n,
                                    t - ex, &ex2);
            tok = k < 0 ? e0 : e0 + k;
        }
        if (lane_id() == 0) s_tok = tok;
    }
    __syncthreads();
    return s_tok;
}

}  // namespace

// Phase 1 of a row: the workgroup merges its lanes' (M, s) states of both rows (references
// uniform across each wave) and thread 0 publishes the member's partials.
__device__ __forceinline__ void publish_partials(uint64_t *part, int S, int j, const ThreadStats &ts, uint32_t tag,
                                                 TeamRed &red) {
    const float st = wave_sum(ts.st), sd = wave_sum(ts.sd);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) { red.f[0][w] = ts.Mt; red.f[1][w] = st; red.f[2][w] = ts.Md; red.f[3][w] = sd; }
    __syncthreads();
    if (threadIdx.x < kWave) {   // only the publisher needs the merged values
        // lane q < 4 takes wave q: the maxima, then the rescaled sums, over the quad
        const int q = lane_id();
        const float mt = q < kTeamWaves ? red.f[0][q] : neg_inf(), tt = q < kTeamWaves ? red.f[1][q] : 0.f;
        const float md = q < kTeamWaves ? red.f[2][q] : neg_inf(), dd = q < kTeamWaves ? red.f[3][q] : 0.f;
        float Mt = fmaxf(mt, dpp_f<0xB1>(mt)), Md = fmaxf(md, dpp_f<0xB1>(md));
        Mt = fmaxf(Mt, dpp_f<0x4E>(Mt));
        Md = fmaxf(Md, dpp_f<0x4E>(Md));
        float Tt = (mt == neg_inf()) ? 0.f : tt * exp2_fast(mt - Mt);
        float Dd = (md == neg_inf()) ? 0.f : dd * exp2_fast(md - Md);
        Tt += dpp_f<0xB1>(Tt);
        Dd += dpp_f<0xB1>(Dd);
        Tt += dpp_f<0x4E>(Tt);
        Dd += dpp_f<0x4E>(Dd);
        if (q == 0) {
            putf(part + 0 * S + j, Mt, tag);
            putf(part + 1 * S + j, Tt, tag);
            putf(part + 2 * S + j, Md, tag);
            putf(part + 3 * S + j, Dd, tag);
        }
    }
}

}  // namespace sv
