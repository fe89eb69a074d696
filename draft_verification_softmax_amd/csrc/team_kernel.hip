// team_kernel.hip -- fused batched verification, one team of workgroups per row pair.
//
// Grid: (row slots) x S members; member j of row (r, k) owns logits
// [j * 8192, (j + 1) * 8192) of target row (r, k) and drafter row (r, k).  Wave w of a member
// owns the contiguous range [j * 8192 + w * 2048, +2048); lane l of that wave holds
// logits base + g * 512 + l * 8 + (0..7), g = 0..3, in registers (16-byte non-temporal loads).
//
// Definitions (AngelSpec tutorial page, section "From KL to an end-to-end TV loss"): the
// overlap alpha = sum_v min(p_v, q_v); a rejected draft voids the later ones; the L_e2e
// equation.  Rejection sampling itself and the residual/bonus draw follow the standard
// speculative-sampling rule, the one that keeps the target distribution (abstract).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"
#include "team.hpp"

namespace sv {

TeamLayout team_layout(int B, int K, int V, size_t ws_bytes) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    TeamLayout L;
    L.S = (V + kTeamChunk - 1) / kTeamChunk;
    L.nseg = L.S * kTeamWaves;
    L.nseg_b = (V + kBonusSeg - 1) / kBonusSeg;
    L.rows = (int64_t)(B > 0 ? B : 1) * (K > 0 ? K : 1);
    L.n_grp = (int)((L.rows + 255) / 256);
    const size_t nB = (size_t)(B > 0 ? B : 1);
    // counters, from the start
    L.off_err = 0;
    L.off_epoch = 64;
    L.off_gdone = 128;
    L.off_grp = 256;
    L.off_rowcnt = al(L.off_grp + sizeof(int32_t) * (size_t)L.n_grp);
    L.off_reqcnt = al(L.off_rowcnt + sizeof(int32_t) * (size_t)L.rows);
    const size_t counters = al(L.off_reqcnt + sizeof(int32_t) * nB);
    // tagged words and scratch, relative to their own base
    size_t o = 0;
    L.off_part = o;  o = al(o + sizeof(uint64_t) * 8 * (size_t)L.S * (size_t)L.rows);
    L.off_apart = o; o = al(o + sizeof(uint64_t) * (size_t)L.S * (size_t)L.rows);
    L.off_dir = o;   o = al(o + sizeof(uint64_t) * (size_t)L.nseg * (size_t)L.rows);
    L.off_rec = o;   o = al(o + sizeof(uint64_t) * 4 * (size_t)L.rows);
    L.off_bonus = o; o = al(o + sizeof(float) * 2 * (size_t)L.nseg_b * nB);
    L.off_alpha = o; o = al(o + sizeof(float) * (size_t)L.rows);
    const size_t tagged = o;
    L.total = counters + tagged;
    const size_t size = ws_bytes >= L.total ? ws_bytes : L.total;
    const size_t base = (size - tagged) & ~(size_t)255;   // >= counters since size >= total
    L.off_part += base; L.off_apart += base; L.off_dir += base;
    L.off_rec += base; L.off_bonus += base; L.off_alpha += base;
    return L;
}

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
__device__ bool wave_poll(const uint64_t *p, int n, uint32_t tag, uint32_t *dst, int64_t limit) {
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
        __builtin_amdgcn_s_sleep(1);
    }
}

__device__ __forceinline__ uint32_t read_epoch(const uint32_t *e) {
    return __hip_atomic_load(const_cast<uint32_t *>(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- row chunk loads -----------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight logits at v0 (multiple of 8) of a 16-byte-aligned row, -inf past V.
template <int DT>
__device__ __forceinline__ void load8nt(const void *row, int v0, int V, float *z) {
    if (v0 + 8 <= V) {
        if constexpr (DT == kDtBF16) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + (v0 >> 3));
            z[0] = bf16_lo(w.x); z[1] = bf16_hi(w.x); z[2] = bf16_lo(w.y); z[3] = bf16_hi(w.y);
            z[4] = bf16_lo(w.z); z[5] = bf16_hi(w.z); z[6] = bf16_lo(w.w); z[7] = bf16_hi(w.w);
        } else {
            const u32x4 *q = reinterpret_cast<const u32x4 *>(row) + (v0 >> 2);
            const u32x4 w0 = __builtin_nontemporal_load(q), w1 = __builtin_nontemporal_load(q + 1);
            z[0] = __uint_as_float(w0.x); z[1] = __uint_as_float(w0.y); z[2] = __uint_as_float(w0.z); z[3] = __uint_as_float(w0.w);
            z[4] = __uint_as_float(w1.x); z[5] = __uint_as_float(w1.y); z[6] = __uint_as_float(w1.z); z[7] = __uint_as_float(w1.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (v0 + e < V) ? load1<DT>(row, v0 + e) : neg_inf();
    }
}

// Vocabulary index of register slot i (group i / 8, element i % 8) of this lane.
__device__ __forceinline__ int slot_index(int base, int i) { return base + (i >> 3) * 512 + lane_id() * 8 + (i & 7); }

// ---- workgroup reductions (fixed order) ------------------------------------------------
struct TeamRed {
    float f[8][kTeamWaves];
    int i[4][kTeamWaves];
    double d[kTeamWaves];
};

// (M, s) pairs in base 2: s = sum 2^{x - M}
__device__ __forceinline__ void ms_merge(float &M, float &s, float M2, float s2) { lse_merge(M, s, M2, s2, 1.0f); }

__device__ __forceinline__ void wave_ms(float &M, float &s) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float M2 = __shfl_xor(M, d, kWave), s2 = __shfl_xor(s, d, kWave);
        ms_merge(M, s, M2, s2);
    }
}

__device__ void block_ms2(float &Mt, float &st, float &Md, float &sd, TeamRed &red) {
    wave_ms(Mt, st);
    wave_ms(Md, sd);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) { red.f[0][w] = Mt; red.f[1][w] = st; red.f[2][w] = Md; red.f[3][w] = sd; }
    __syncthreads();
    Mt = red.f[0][0]; st = red.f[1][0]; Md = red.f[2][0]; sd = red.f[3][0];
    for (int q = 1; q < kTeamWaves; ++q) { ms_merge(Mt, st, red.f[0][q], red.f[1][q]); ms_merge(Md, sd, red.f[2][q], red.f[3][q]); }
    __syncthreads();
}

__device__ void block_amax2(float &vt, int &it, float &vd, int &id, TeamRed &red) {
    wave_amax(vt, it);
    wave_amax(vd, id);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) { red.f[4][w] = vt; red.i[0][w] = it; red.f[5][w] = vd; red.i[1][w] = id; }
    __syncthreads();
    vt = red.f[4][0]; it = red.i[0][0]; vd = red.f[5][0]; id = red.i[1][0];
    for (int q = 1; q < kTeamWaves; ++q) { amax_merge(vt, it, red.f[4][q], red.i[0][q]); amax_merge(vd, id, red.f[5][q], red.i[1][q]); }
    __syncthreads();
}

__device__ float block_sumf(float x, TeamRed &red) {
    x = wave_sum(x);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) red.f[6][w] = x;
    __syncthreads();
    float t = red.f[6][0];
    for (int q = 1; q < kTeamWaves; ++q) t += red.f[6][q];
    __syncthreads();
    return t;
}

// ---- one member's chunk ----------------------------------------------------------------
struct Chunk {
    float xt[kTeamE], xd[kTeamE];
};

template <int DTT, int DTD>
__device__ __forceinline__ void load_chunk(Chunk &ch, const void *trow, const void *drow, int base, int V) {
#pragma unroll
    for (int g = 0; g < kTeamE / 8; ++g) {
        const int v0 = base + g * 512 + lane_id() * 8;
        load8nt<DTT>(trow, v0, V, ch.xt + g * 8);
        load8nt<DTD>(drow, v0, V, ch.xd + g * 8);
    }
}

__device__ __forceinline__ float max_of(const float *x) {
    float m0 = neg_inf(), m1 = neg_inf(), m2 = neg_inf(), m3 = neg_inf();
#pragma unroll
    for (int i = 0; i < kTeamE; i += 4) { m0 = fmaxf(m0, x[i]); m1 = fmaxf(m1, x[i + 1]); m2 = fmaxf(m2, x[i + 2]); m3 = fmaxf(m3, x[i + 3]); }
    return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}

// First register slot holding value m (slots are in increasing vocabulary order).
__device__ __forceinline__ int first_index_of(const float *x, float m, int base) {
    int idx = 0x7fffffff;
#pragma unroll
    for (int i = kTeamE - 1; i >= 0; --i)
        if (x[i] == m) idx = slot_index(base, i);
    return idx;
}

// In place: x_i <- 2^{x_i c - M}; returns the sum in a fixed association order.
__device__ __forceinline__ float exp_sum(float *x, float c, float M) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < kTeamE; i += 4) {
        x[i] = exp2_fast(__builtin_fmaf(x[i], c, -M));
        x[i + 1] = exp2_fast(__builtin_fmaf(x[i + 1], c, -M));
        x[i + 2] = exp2_fast(__builtin_fmaf(x[i + 2], c, -M));
        x[i + 3] = exp2_fast(__builtin_fmaf(x[i + 3], c, -M));
        a0 += x[i]; a1 += x[i + 1]; a2 += x[i + 2]; a3 += x[i + 3];
    }
    return (a0 + a1) + (a2 + a3);
}

// sum_i min(et_i, ed_i * rho), same association as exp_sum (so it never exceeds it).
__device__ __forceinline__ float min_sum(const float *et, const float *ed, float rho) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int i = 0; i < kTeamE; i += 4) {
        a0 += fminf(et[i], ed[i] * rho);
        a1 += fminf(et[i + 1], ed[i + 1] * rho);
        a2 += fminf(et[i + 2], ed[i + 2] * rho);
        a3 += fminf(et[i + 3], ed[i + 3] * rho);
    }
    return (a0 + a1) + (a2 + a3);
}

// Pass 1 on a loaded chunk: thread reference M = max * c (-inf if empty), exps in place.
struct ThreadStats {
    float Mt, st, Md, sd;   // base-2 log-sum-exp states of this lane's slice
};

__device__ __forceinline__ ThreadStats pass1(Chunk &ch, float c) {
    ThreadStats s;
    const float mt = max_of(ch.xt), md = max_of(ch.xd);
    s.Mt = (mt == neg_inf()) ? neg_inf() : mt * c;
    s.Md = (md == neg_inf()) ? neg_inf() : md * c;
    s.st = exp_sum(ch.xt, c, s.Mt == neg_inf() ? 0.f : s.Mt);
    s.sd = exp_sum(ch.xd, c, s.Md == neg_inf() ? 0.f : s.Md);
    return s;
}

// Pass 2: this lane's share of sum_v min(p_v, q_v) and of the residual mass
// sum_v max(p_v - q_v, 0), given the row normalisers L2t, L2d (base 2).
__device__ __forceinline__ void pass2(const Chunk &ch, const ThreadStats &s, float L2t, float L2d, float &alpha,
                                      float &resid) {
    alpha = 0.f;
    resid = 0.f;
    if (s.Mt == neg_inf()) return;             // no target mass in this slice
    const float lrt = s.Mt - L2t;              // log2 of the factor turning x_t into p
    const float lrd = (s.Md == neg_inf()) ? neg_inf() : s.Md - L2d;
    const float rho = exp2_fast(fminf(lrd - lrt, 126.f));
    const float sm = min_sum(ch.xt, ch.xd, rho);
    const float rt = exp2_fast(lrt);
    alpha = rt * sm;
    resid = rt * (s.st - sm);
}

// ---- request-level helpers --------------------------------------------------------------

// Token of one row drawn from p = softmax(row / T) at target u * R by inverse CDF: one sweep
// keeps (max, sum) of every 512-logit segment in `seg` (workspace, this workgroup only),
// then a wave finds the segment and re-reads it.
template <int DT>
__device__ int draw_from_row(const void *row, int V, float c, float u, float *seg, int nseg, TeamRed &red) {
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
    block_ms2(M, s, Md, sd, red);
    const float L2 = M + log2f(s);
    __threadfence_block();
    __syncthreads();
    for (int q = threadIdx.x; q < nseg; q += kTeamThreads) {
        const float sM = seg[q], ss = seg[nseg + q];
        seg[q] = (sM == neg_inf()) ? 0.f : ss * exp2_fast(sM - L2);
    }
    __threadfence_block();
    __syncthreads();
    __shared__ int s_tok;
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
            const int k = wave_find([&](int q) { return exp2_fast(__builtin_fmaf(load1<DT>(row, e0 + q), c, -L2)); }, n,
                                    t - ex, &ex2);
            tok = k < 0 ? e0 : e0 + k;
        }
        if (lane_id() == 0) s_tok = tok;
    }
    __syncthreads();
    return s_tok;
}

template <int DT>
__device__ int row_argmax(const void *row, int V, TeamRed &red) {
    float v = neg_inf(), vd = neg_inf();
    int i = 0x7fffffff, id = 0x7fffffff;
    for (int base = 0; base < V; base += kTeamThreads * 8) {
        const int e = base + threadIdx.x * 8;
        float z[8];
        load8<DT>(row, e, V, z);
        amax_update8(v, i, z, e);
    }
    block_amax2(v, i, vd, id, red);
    return i == 0x7fffffff ? 0 : i;
}

// Correction token after a rejection at row tau: inverse CDF of w = max(p - q, 0) at
// u * R.  The directory (residual mass of each 2048-logit wave range) picks the range; the
// workgroup re-reads it (8 logits per thread) and scans it in binary64.
template <int DTT, int DTD>
__device__ int draw_residual(const void *trow, const void *drow, int V, float c, float L2t, float L2d,
                             const float *dirv, int nseg, double t, TeamRed &red) {
    __shared__ int s_seg;
    __shared__ double s_ex;
    __shared__ double s_scan[kTeamThreads];
    __shared__ int s_tok;
    const int w = threadIdx.x / kWave;
    if (w == 0) {
        double ex;
        const int sidx = wave_find([&](int q) { return dirv[q]; }, nseg, t, &ex);
        if (lane_id() == 0) { s_seg = sidx; s_ex = ex; }
    }
    __syncthreads();
    const int sidx = s_seg;
    if (sidx < 0) return -1;
    const double rem = t - s_ex;
    const int e0 = sidx * kTeamSeg + threadIdx.x * 8;
    float wt[8];
    double my = 0.0;
    {
        float zt[8], zd[8];
        load8<DTT>(trow, e0, V, zt);
        load8<DTD>(drow, e0, V, zd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = exp2_fast(__builtin_fmaf(zt[e], c, -L2t));
            const float q = exp2_fast(__builtin_fmaf(zd[e], c, -L2d));
            wt[e] = p - fminf(p, q);
            my += (double)wt[e];
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
        int k = 7;
        for (int e = 0; e < 8; ++e) {
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
        for (int e = 7; e >= 0; --e)
            if (wt[e] > 0.f) { last = e0 + e; break; }
        s_scan[threadIdx.x] = (double)last;
        __syncthreads();
        if (threadIdx.x == 0) {
            int best = sidx * kTeamSeg;
            for (int q = kTeamThreads - 1; q >= 0; --q)
                if (s_scan[q] >= 0.0) { best = (int)s_scan[q]; break; }
            s_tok = best;
        }
        __syncthreads();
        tok = s_tok;
    }
    __syncthreads();
    return tok;
}

template <int DTT, int DTD, int MODE>
__device__ void request_finalize(const TeamArgs &a, int r, int L, uint32_t tag, TeamRed &red, uint32_t *pay) {
    __shared__ int s_tau, s_tok;
    const int K = a.K;
    const int slots = K > 0 ? K : 1;
    const int64_t row0 = (int64_t)r * slots;
    const int64_t rows = (int64_t)a.B * slots;
    bool ok = true;
    // first-reject scan over the accept words of rows 0..L-1
    if (threadIdx.x == 0) s_tau = L;
    __syncthreads();
    for (int k0 = 0; k0 < L; k0 += 2048) {
        const int n = min(2048, L - k0);
        if (threadIdx.x < kWave) {
            const bool got = wave_poll(a.rec + row0 + k0, n, tag, pay, a.spin_ticks_max);
            if (!got && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
        }
        __syncthreads();
        for (int q = threadIdx.x; q < n; q += kTeamThreads)
            if (pay[q] == 0) atomicMin(&s_tau, k0 + q);
        __syncthreads();
    }
    const int tau = s_tau;
    (void)ok;

    int tok = 0;
    const void *trow = static_cast<const char *>(a.target) +
                       (size_t)((r * (int64_t)a.trows + tau) * a.ld_t) * (DTT == kDtBF16 ? 2 : 4);
    if constexpr (MODE == kTeamGreedy) {
        if (tau < L) {
            if (threadIdx.x < kWave) wave_poll(a.rec + rows + row0 + tau, 1, tag, pay, a.spin_ticks_max);
            __syncthreads();
            tok = (int)pay[0];
            __syncthreads();
        } else {
            tok = row_argmax<DTT>(trow, a.V, red);
        }
    } else {
        const float u = uniform24(a.seed, (uint64_t)r, (uint64_t)tau, kPurposeCorrection, a.step);
        bool done = false;
        if (tau < L) {
            const int64_t row = row0 + tau;
            const int nseg = a.nseg;
            // payloads: [0, nseg) directory, nseg: L2t, nseg + 1: L2d
            if (threadIdx.x < kWave) {
                bool g1 = wave_poll(a.dir + row * nseg, nseg, tag, pay, a.spin_ticks_max);
                bool g2 = wave_poll(a.rec + 2 * rows + row, 1, tag, pay + nseg, a.spin_ticks_max);
                bool g3 = wave_poll(a.rec + 3 * rows + row, 1, tag, pay + nseg + 1, a.spin_ticks_max);
                if (!(g1 && g2 && g3) && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
            }
            __syncthreads();
            float *dirv = reinterpret_cast<float *>(pay);
            const float L2t = dirv[nseg], L2d = dirv[nseg + 1];
            double R = 0.0;
            for (int q = 0; q < nseg; ++q) R += (double)dirv[q];
            if (R > 0.0) {
                const void *drow = static_cast<const char *>(a.draft) +
                                   (size_t)((row0 + tau) * a.ld_d) * (DTD == kDtBF16 ? 2 : 4);
                const int t = draw_residual<DTT, DTD>(trow, drow, a.V, a.c, L2t, L2d, dirv, nseg, (double)u * R, red);
                if (t >= 0) { tok = t; done = true; }
            }
            __syncthreads();
        }
        if (!done) tok = draw_from_row<DTT>(trow, a.V, a.c, u, a.bonus + (size_t)r * 2 * a.nseg_b, a.nseg_b, red);
    }
    if (threadIdx.x == 0) s_tok = tok;
    __syncthreads();
    tok = s_tok;

    int32_t *o = a.out_tokens + (size_t)r * (K + 1);
    for (int q = threadIdx.x; q <= K; q += kTeamThreads)
        o[q] = q < tau ? a.tokens[(size_t)r * K + q] : (q == tau ? tok : -1);
    for (int k = L + threadIdx.x; k < K; k += kTeamThreads) {
        const size_t i = (size_t)r * K + k;
        a.alpha[i] = 0.f;
        a.accept[i] = 0;
        if (a.lse_t) a.lse_t[i] = 0.f;
        if (a.lse_d) a.lse_d[i] = 0.f;
        if (a.amax_t) a.amax_t[i] = -1;
        if (a.amax_d) a.amax_d[i] = -1;
    }
    if (threadIdx.x == 0) {
        a.accept_len[r] = tau;
        a.n_out[r] = tau + 1;
        // the last request of the call advances the epoch for the next call
        const int old = atomicAdd(a.gdone, 1);
        if (old == a.B - 1) {
            __hip_atomic_store(a.gdone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Recompute member j's share of a row from HBM (used only when that member gave up).
template <int DTT, int DTD>
__device__ float recompute_share(const TeamArgs &a, const void *trow, const void *drow, int j, float L2t, float L2d,
                                 int64_t row, uint32_t tag, TeamRed &red, bool publish_dir) {
    Chunk ch;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    load_chunk<DTT, DTD>(ch, trow, drow, base, a.V);
    const ThreadStats s = pass1(ch, a.c);
    float al, rs;
    pass2(ch, s, L2t, L2d, al, rs);
    rs = wave_sum(rs);
    if (publish_dir && lane_id() == 0) putf(a.dir + row * a.nseg + j * kTeamWaves + w, rs, tag);
    return block_sumf(al, red);
}

}  // namespace

template <int DTT, int DTD, int MODE>
__global__ __launch_bounds__(kTeamThreads) void team_kernel(TeamArgs a) {
    __shared__ TeamRed red;
    __shared__ uint32_t pay[2048 + 8];
    __shared__ int s_flag, s_rank;
    __shared__ float s_tot[8];

    const int S = a.S;
    const int j = blockIdx.x % S;
    const int64_t row = blockIdx.x / S;
    const int K = a.K;
    const int slots = K > 0 ? K : 1;
    const int r = (int)(row / slots);
    const int k = (int)(row % slots);
    int L = K;
    if (MODE != kTeamAlpha && a.draft_len) {
        L = a.draft_len[r];
        if (L < 0 || L > K) {
            if (threadIdx.x == 0 && k == 0 && j == 0) atomicOr(a.err, SV_DEVERR_DRAFT_LEN);
            L = L < 0 ? 0 : K;
        }
    }
    if (k >= L) {
        if (MODE != kTeamAlpha && L == 0 && k == 0 && j == 0) {
            const uint32_t tag = read_epoch(a.epoch) + 1;
            request_finalize<DTT, DTD, MODE>(a, r, 0, tag, red, pay);
        }
        return;
    }
    const uint32_t tag = read_epoch(a.epoch) + 1;
    const int64_t rows = (int64_t)a.B * slots;
    const size_t et = DTT == kDtBF16 ? 2 : 4, ed = DTD == kDtBF16 ? 2 : 4;
    const void *trow = static_cast<const char *>(a.target) + (size_t)(((int64_t)r * a.trows + k) * a.ld_t) * et;
    const void *drow = static_cast<const char *>(a.draft) + (size_t)(row * a.ld_d) * ed;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    const float c = a.c;

    Chunk ch;
    load_chunk<DTT, DTD>(ch, trow, drow, base, a.V);

    // ---------------- phase 1: per-member partials ----------------
    uint64_t *part = a.part + row * (int64_t)(8 * S);
    const bool want_amax = (MODE == kTeamGreedy) || a.want_amax;
    float vt = neg_inf(), vd = neg_inf();
    int it = 0x7fffffff, id = 0x7fffffff;
    if (want_amax) {
        vt = max_of(ch.xt);
        vd = max_of(ch.xd);
        it = vt == neg_inf() ? 0x7fffffff : first_index_of(ch.xt, vt, base);
        id = vd == neg_inf() ? 0x7fffffff : first_index_of(ch.xd, vd, base);
        block_amax2(vt, it, vd, id, red);
    }
    ThreadStats ts{};
    float Mt = neg_inf(), st = 0.f, Md = neg_inf(), sd = 0.f;
    if constexpr (MODE != kTeamGreedy) {
        ts = pass1(ch, c);
        Mt = ts.Mt; st = ts.st; Md = ts.Md; sd = ts.sd;
        block_ms2(Mt, st, Md, sd, red);
    }
    int my_rank = -1;
    if (threadIdx.x == 0) {
        if constexpr (MODE != kTeamGreedy) {
            putf(part + 0 * S + j, Mt, tag);
            putf(part + 1 * S + j, st, tag);
            putf(part + 2 * S + j, Md, tag);
            putf(part + 3 * S + j, sd, tag);
        }
        if (want_amax) {
            putf(part + 4 * S + j, vt, tag);
            put(part + 5 * S + j, (uint32_t)it, tag);
            putf(part + 6 * S + j, vd, tag);
            put(part + 7 * S + j, (uint32_t)id, tag);
        }
        my_rank = atomicAdd(a.row_cnt + row, 1);
    }

    if constexpr (MODE == kTeamGreedy) {
        if (threadIdx.x == 0) s_rank = my_rank;
        __syncthreads();
        if (s_rank != S - 1) return;
    }

    // ---------------- row normalisers: every member reduces all partials ----------------
    float L2t = 0.f, L2d = 0.f;
    if constexpr (MODE != kTeamGreedy) {
        if (threadIdx.x < kWave) {
            bool got = wave_poll(part, 4 * S, tag, pay, a.spin_ticks);
            int flag = got ? 1 : 0;
            if (!got) {
                // only the last arriver is sure that every partial has been written
                const int rank = __shfl(my_rank, 0, kWave);
                if (rank == S - 1) {
                    got = wave_poll(part, 4 * S, tag, pay, a.spin_ticks_max);
                    if (!got && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
                    flag = 1;
                }
            }
            if (threadIdx.x == 0) {
                float Tt = neg_inf(), Ts = 0.f, Dt = neg_inf(), Ds = 0.f;
                for (int q = 0; q < S; ++q) {
                    ms_merge(Tt, Ts, __uint_as_float(pay[q]), __uint_as_float(pay[S + q]));
                    ms_merge(Dt, Ds, __uint_as_float(pay[2 * S + q]), __uint_as_float(pay[3 * S + q]));
                }
                s_tot[0] = Tt + log2f(Ts);
                s_tot[1] = Dt + log2f(Ds);
                s_flag = flag;
                s_rank = my_rank;
            }
        }
        __syncthreads();
        if (!s_flag) {
            // gave up waiting: hand this member's share to the last arriver
            if (threadIdx.x == 0) put(a.apart + row * S + j, kGaveUp, tag);
            return;
        }
        L2t = s_tot[0];
        L2d = s_tot[1];

        // ---------------- phase 2: this member's share of alpha and residual mass -------------
        float al, rs;
        pass2(ch, ts, L2t, L2d, al, rs);
        if constexpr (MODE == kTeamStoch) {
            rs = wave_sum(rs);
            if (lane_id() == 0) putf(a.dir + row * a.nseg + j * kTeamWaves + w, rs, tag);
        }
        al = block_sumf(al, red);
        if (threadIdx.x == 0) putf(a.apart + row * S + j, al, tag);
        if (s_rank != S - 1) return;
    }

    // ---------------- the last arriver completes the row ----------------
    float alpha = 0.f;
    int at = 0, ad = 0;
    if (want_amax) {
        if (threadIdx.x < kWave) {
            const bool got = wave_poll(part + 4 * S, 4 * S, tag, pay, a.spin_ticks_max);
            if (!got && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
            if (threadIdx.x == 0) {
                float bv = neg_inf(), bd = neg_inf();
                int bi = 0x7fffffff, bj = 0x7fffffff;
                for (int q = 0; q < S; ++q) {
                    amax_merge(bv, bi, __uint_as_float(pay[q]), (int)pay[S + q]);
                    amax_merge(bd, bj, __uint_as_float(pay[2 * S + q]), (int)pay[3 * S + q]);
                }
                red.i[2][0] = bi == 0x7fffffff ? 0 : bi;
                red.i[3][0] = bj == 0x7fffffff ? 0 : bj;
            }
        }
        __syncthreads();
        at = red.i[2][0];
        ad = red.i[3][0];
        __syncthreads();
    }
    if constexpr (MODE != kTeamGreedy) {
        if (threadIdx.x < kWave) {
            const bool got = wave_poll(a.apart + row * S, S, tag, pay, a.spin_ticks_max);
            if (!got && threadIdx.x == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
        }
        __syncthreads();
        // members that gave up: recompute their shares (and directory entries) from HBM
        for (int q = 0; q < S; ++q) {
            if (pay[q] == kGaveUp) {
                const float sh = recompute_share<DTT, DTD>(a, trow, drow, q, L2t, L2d, row, tag, red, MODE == kTeamStoch);
                __syncthreads();
                if (threadIdx.x == 0) pay[q] = __float_as_uint(sh);
                __syncthreads();
            }
        }
        if (threadIdx.x == 0) {
            double s = 0.0;
            for (int q = 0; q < S; ++q) s += (double)__uint_as_float(pay[q]);
            s_tot[2] = (float)s;
        }
        __syncthreads();
        alpha = s_tot[2];
    }

    if constexpr (MODE == kTeamAlpha) {
        if (threadIdx.x == 0) {
            a.alpha[row] = alpha;
            __hip_atomic_store(a.row_cnt + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // epoch advance once every row of the call is complete (grouped counters)
            const int g = (int)(row / 256);
            const int gsize = (int)min((int64_t)256, rows - (int64_t)g * 256);
            if (atomicAdd(a.grp_cnt + g, 1) == gsize - 1) {
                __hip_atomic_store(a.grp_cnt + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (atomicAdd(a.gdone, 1) == a.n_grp - 1) {
                    __hip_atomic_store(a.gdone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(a.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        return;
    } else {
        if (threadIdx.x == 0) {
            const size_t i = (size_t)r * K + k;
            const int x = a.tokens[i];
            const bool okx = (x >= 0 && x < a.V);
            if (!okx) atomicOr(a.err, SV_DEVERR_TOKEN);
            int acc = 0;
            if constexpr (MODE == kTeamGreedy) {
                acc = okx && x == at;
                alpha = (at == ad) ? 1.f : 0.f;
            } else if (okx) {
                // accept iff u * q(x) < p(x)
                const float lpt = __builtin_fmaf(load1<DTT>(trow, x), c, -L2t);
                const float lpd = __builtin_fmaf(load1<DTD>(drow, x), c, -L2d);
                const float u = uniform24(a.seed, (uint64_t)r, (uint64_t)k, kPurposeAccept, a.step);
                acc = u < exp2f(lpt - lpd);
            }
            a.alpha[i] = alpha;
            a.accept[i] = (uint8_t)acc;
            if (a.lse_t) a.lse_t[i] = (MODE == kTeamStoch) ? L2t * 0.69314718055994531f : 0.f;
            if (a.lse_d) a.lse_d[i] = (MODE == kTeamStoch) ? L2d * 0.69314718055994531f : 0.f;
            if (a.amax_t) a.amax_t[i] = want_amax ? at : -1;
            if (a.amax_d) a.amax_d[i] = want_amax ? ad : -1;
            put(a.rec + 0 * rows + row, (uint32_t)acc, tag);
            put(a.rec + 1 * rows + row, (uint32_t)at, tag);
            putf(a.rec + 2 * rows + row, L2t, tag);
            putf(a.rec + 3 * rows + row, L2d, tag);
            __hip_atomic_store(a.row_cnt + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int old = atomicAdd(a.req_cnt + r, 1);
            s_flag = (old == L - 1);
            if (s_flag) __hip_atomic_store(a.req_cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_flag) request_finalize<DTT, DTD, MODE>(a, r, L, tag, red, pay);
    }
}

template <int DTT, int DTD>
static hipError_t launch_mode(const TeamArgs &a, int mode, unsigned grid, hipStream_t s) {
    if (mode == kTeamStoch) hipLaunchKernelGGL((team_kernel<DTT, DTD, kTeamStoch>), dim3(grid), dim3(kTeamThreads), 0, s, a);
    else if (mode == kTeamGreedy) hipLaunchKernelGGL((team_kernel<DTT, DTD, kTeamGreedy>), dim3(grid), dim3(kTeamThreads), 0, s, a);
    else hipLaunchKernelGGL((team_kernel<DTT, DTD, kTeamAlpha>), dim3(grid), dim3(kTeamThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t team_launch(const TeamArgs &a, int dt, int dd, int mode, unsigned grid, hipStream_t s) {
    if (dt == SV_BF16 && dd == SV_BF16) return launch_mode<kDtBF16, kDtBF16>(a, mode, grid, s);
    if (dt == SV_F32 && dd == SV_F32) return launch_mode<kDtF32, kDtF32>(a, mode, grid, s);
    if (dt == SV_BF16 && dd == SV_F32) return launch_mode<kDtBF16, kDtF32>(a, mode, grid, s);
    return launch_mode<kDtF32, kDtBF16>(a, mode, grid, s);
}

}  // namespace sv
