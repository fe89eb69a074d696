// sv_device.hpp -- device building blocks for gfx950 (CDNA4, wave64).
//
// Logit loads (binary32 / bfloat16), the Philox4x64-10 counter-based generator, the
// log-sum-exp merge, wave64 reductions and scans, and the wave-level inverse-CDF search.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kDtF32 = 0;
constexpr int kDtBF16 = 1;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// bfloat16 is the upper half of a binary32: widening is exact.  Element 2i of a bf16 row
// sits in the low half of 32-bit word i (little endian).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v_exp_f32: 2^x, about 1 ulp; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT>
__device__ __forceinline__ float load1(const void *row, int64_t i) {
    if constexpr (DT == kDtBF16) {
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(row)[i] << 16);
    } else {
        return static_cast<const float *>(row)[i];
    }
}

// Eight consecutive logits starting at element e (e a multiple of 8, row 16-byte aligned);
// elements at or past V read as -inf.
template <int DT>
__device__ __forceinline__ void load8(const void *row, int e, int V, float (&z)[8]) {
    if (e + 8 <= V) {
        if constexpr (DT == kDtBF16) {
            const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(row) + e);
            z[0] = bf16_lo(w.x); z[1] = bf16_hi(w.x);
            z[2] = bf16_lo(w.y); z[3] = bf16_hi(w.y);
            z[4] = bf16_lo(w.z); z[5] = bf16_hi(w.z);
            z[6] = bf16_lo(w.w); z[7] = bf16_hi(w.w);
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(row) + e);
            const float4 a = p[0], b = p[1];
            z[0] = a.x; z[1] = a.y; z[2] = a.z; z[3] = a.w;
            z[4] = b.x; z[5] = b.y; z[6] = b.z; z[7] = b.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[j] = (e + j < V) ? load1<DT>(row, e + j) : neg_inf();
    }
}

// ---------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 64x64->128-bit
// products of counter words 0 and 2 by the published multipliers, a word permutation
// xored with the key, and a Weyl-sequence key schedule between rounds.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t philox_word0(uint64_t seed, uint64_t c0, uint64_t c1,
                                                 uint64_t c2, uint64_t c3) {
    const uint64_t MA = 0xD2E7470EE14C6C93ull, MB = 0xCA5A826395121157ull;
    const uint64_t WA = 0x9E3779B97F4A7C15ull, WB = 0xBB67AE8584CAA73Bull;
    uint64_t k0 = seed, k1 = 0;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) { k0 += WA; k1 += WB; }
        const uint64_t ha = __umul64hi(MA, c0), la = MA * c0;
        const uint64_t hb = __umul64hi(MB, c2), lb = MB * c2;
        const uint64_t n0 = hb ^ c1 ^ k0, n2 = ha ^ c3 ^ k1;
        c0 = n0; c1 = lb; c2 = n2; c3 = la;
    }
    return c0;
}

// Uniform in [0,1) from the top 24 bits of word 0: exactly representable in binary32.
__device__ __forceinline__ float uniform24(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2,
                                           uint64_t c3) {
    return (float)(philox_word0(seed, c0, c1, c2, c3) >> 40) * 0x1p-24f;
}

constexpr uint64_t kPurposeAccept = 0;
constexpr uint64_t kPurposeCorrection = 1;
constexpr uint64_t kPurposeDraft = 2;

// ---------------------------------------------------------------------------------------
// Log-sum-exp state in base 2: (m, s) stands for sum_v 2^{(z_v - m) c}; c = log2(e) / T.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2, float c) {
    const float mn = fmaxf(m, m2);
    if (mn == neg_inf()) { m = mn; s = 0.f; return; }
    s = s * exp2_fast((m - mn) * c) + s2 * exp2_fast((m2 - mn) * c);
    m = mn;
}

// Argmax state: larger value wins, equal values -> lower index.
__device__ __forceinline__ void amax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void amax_update8(float &v, int &i, const float (&z)[8], int e) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (z[j] > v) { v = z[j]; i = e + j; }
}

// ---------------------------------------------------------------------------------------
// wave64 collectives
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Lane exchange inside rows of 16 lanes (DPP): CTRL 0xB1 / 0x4E swap lanes xor 1 / xor 2
// (quad permutations), 0x141 mirrors each half-row, 0x140 each row.  Every source lane
// is valid for these patterns.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) { return __int_as_float(dpp_i<CTRL>(__float_as_int(x))); }
__device__ __forceinline__ float readlane_f(float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); }

// Wave reductions: a butterfly inside each row of 16 lanes (every lane of a row ends with
// the row's value), then the four row values, read from lanes 0, 16, 32 and 48, are merged
// in row order.  The result is wave-uniform.  Scheduling fences keep the compiler from
// filling the exchange latency with independent work hoisted from later code, which
// would keep that work's values live (and raise the register count) across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ float wave_sum(float x) {
    sched_fence();
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    x = (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
    sched_fence();
    return x;
}

// Order-preserving map of binary32 bit patterns (no NaN) to unsigned integers: positive
// values get the top bit set, negative ones are complemented.  The unsigned maximum of keys
// is the key of the floating maximum, and an integer maximum needs no NaN quieting of its
// operands, so each exchange step is one DPP-fused instruction.
__device__ __forceinline__ uint32_t fkey(float x) {
    const uint32_t b = __float_as_uint(x);
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) { return __uint_as_float(k ^ ((k >> 31) ? 0x80000000u : 0xffffffffu)); }

template <int CTRL>
__device__ __forceinline__ uint32_t kmax_step(uint32_t k) {
    const uint32_t o = (uint32_t)dpp_i<CTRL>((int)k);
    return k > o ? k : o;
}

__device__ __forceinline__ float wave_max(float x) {
    sched_fence();
    uint32_t k = fkey(x);
    k = kmax_step<0xB1>(k);
    k = kmax_step<0x4E>(k);
    k = kmax_step<0x141>(k);
    k = kmax_step<0x140>(k);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)k, 48);
    const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
    x = fkey_inv(a > b ? a : b);
    sched_fence();
    return x;
}

template <int CTRL>
__device__ __forceinline__ void lse_step(float &m, float &s, float c) {
    const float m2 = dpp_f<CTRL>(m), s2 = dpp_f<CTRL>(s);
    lse_merge(m, s, m2, s2, c);
}

__device__ __forceinline__ void wave_lse(float &m, float &s, float c) {
    sched_fence();
    lse_step<0xB1>(m, s, c);
    lse_step<0x4E>(m, s, c);
    lse_step<0x141>(m, s, c);
    lse_step<0x140>(m, s, c);
    float M = readlane_f(m, 0), S = readlane_f(s, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) lse_merge(M, S, readlane_f(m, 16 * r), readlane_f(s, 16 * r), c);
    m = M;
    s = S;
    sched_fence();
}

template <int CTRL>
__device__ __forceinline__ void amax_step(float &v, int &i) {
    const float v2 = dpp_f<CTRL>(v);
    const int i2 = dpp_i<CTRL>(i);
    amax_merge(v, i, v2, i2);
}

__device__ __forceinline__ void wave_amax(float &v, int &i) {
    sched_fence();
    amax_step<0xB1>(v, i);
    amax_step<0x4E>(v, i);
    amax_step<0x141>(v, i);
    amax_step<0x140>(v, i);
    float V = readlane_f(v, 0);
    int I = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) amax_merge(V, I, readlane_f(v, 16 * r), __builtin_amdgcn_readlane(i, 16 * r));
    v = V;
    i = I;
    sched_fence();
}

// A double from the lane DPP control CTRL selects, 0 where there is none (rows outside
// ROW_MASK also read 0).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_d(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// A double from lane l, l the same in every lane of the wave (two scalar reads).
__device__ __forceinline__ double readlane_d(double x, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive scan over the wave in lane order, in registers: shifts by 1, 2, 4 and 8 inside
// each row of 16 lanes, then the last lane of row 0 (2) is added to row 1 (3), and the last
// lane of row 1 to rows 2 and 3.  Every lane of the wave must call it.
__device__ __forceinline__ double wave_incl_scan(double x) {
    x += dpp_d<0x111>(x);        // row_shr:1
    x += dpp_d<0x112>(x);        // row_shr:2
    x += dpp_d<0x114>(x);        // row_shr:4
    x += dpp_d<0x118>(x);        // row_shr:8
    x += dpp_d<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_d<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Inverse-CDF search by one full wave: the smallest index i in [0, n) whose inclusive
// prefix of the non-negative weights weight(i) exceeds t.  Prefix sums run in binary64 in
// index order (64 per round).  If none exceeds t (rounding at the very end), the last
// index with a positive weight is taken; -1 if every weight is zero.  *excl receives the
// prefix before the returned index.  Every lane of the wave must call it.
template <class F>
__device__ int wave_find(F weight, int n, double t, double *excl) {
    const int lane = lane_id();
    double base = 0.0;
    int last_pos = -1;
    double last_pos_excl = 0.0;
    for (int b = 0; b < n; b += kWave) {
        const int i = b + lane;
        const double x = (i < n) ? (double)weight(i) : 0.0;
        const double incl = base + wave_incl_scan(x);
        const uint64_t hit = __ballot(incl > t);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            const double e = readlane_d(incl - x, l);
            *excl = e;
            return b + l;
        }
        const uint64_t pos = __ballot(x > 0.0);
        if (pos) {
            const int l = 63 - __builtin_clzll(pos);
            last_pos = b + l;
            last_pos_excl = readlane_d(incl - x, l);
        }
        base = readlane_d(incl, kWave - 1);
    }
    *excl = last_pos_excl;
    return last_pos;
}

}  // namespace sv
