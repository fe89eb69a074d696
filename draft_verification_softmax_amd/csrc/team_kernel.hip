// team_kernel.hip -- fused batched verification, one team of workgroups per row pair.
//
// Grid: (row slots) x S members, then (verification) one finalize workgroup per request.
// A grid that fits on the device at once runs a variant whose lanes keep pass 1's terms in
// binary32 for pass 2 (fewer instructions, fewer waves per SIMD).
// Member j of row (r, k) owns logits [j * 16384, (j + 1) * 16384) of target row (r, k) and
// drafter row (r, k).  Wave w of a member owns the contiguous range [j * 16384 + w * 4096,
// +4096); lane l of that wave holds logits base + g * 512 + l * 8 + (0..7), g = 0..7, in
// registers (16-byte non-temporal loads).
//
// Definitions (AngelSpec tutorial page, section "From KL to an end-to-end TV loss"): the
// overlap alpha = sum_v min(p_v, q_v); a rejected draft voids the later ones; the L_e2e
// equation.  Rejection sampling itself and the residual/bonus draw follow the standard
// speculative-sampling rule, the one that keeps the target distribution (abstract).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "specverify.h"
#include "sv_device.hpp"
#include "team.hpp"
#include "team_device.hpp"

namespace sv {

TeamLayout team_layout(int B, int slots, int V, size_t ws_bytes) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    TeamLayout L;
    L.S = (V + kTeamChunk - 1) / kTeamChunk;
    L.nseg = L.S * kTeamWaves;
    L.nseg_b = (V + kBonusSeg - 1) / kBonusSeg;
    L.rows = (int64_t)(B > 0 ? B : 1) * (slots > 0 ? slots : 1);
    const size_t nB = (size_t)(B > 0 ? B : 1);
    // counters, from the start
    L.off_err = kOffErr;
    L.off_epoch = kOffEpoch;
    L.off_gdone = kOffGdone;
    L.off_arrive = kOffArrive;
    const size_t counters = kOffArrive + sizeof(int32_t) * kArriveSlots * kArriveStride;
    // tagged words and scratch, relative to their own base
    size_t o = 0;
    L.off_part = o;  o = al(o + sizeof(uint64_t) * 8 * (size_t)L.S * (size_t)L.rows);
    L.off_apart = o; o = al(o + sizeof(uint64_t) * (size_t)L.S * (size_t)L.rows);
    L.off_dir = o;   o = al(o + sizeof(uint64_t) * (size_t)L.nseg * (size_t)L.rows);
    L.off_acc = o;   o = al(o + sizeof(uint64_t) * kAccWords * (size_t)L.rows);
    L.off_bonus = o; o = al(o + sizeof(float) * 2 * (size_t)L.nseg_b * nB);
    L.off_alpha = o; o = al(o + sizeof(float) * (size_t)L.rows);
    const size_t tagged = o;
    L.total = counters + tagged;
    const size_t size = ws_bytes >= L.total ? ws_bytes : L.total;
    const size_t base = (size - tagged) & ~(size_t)255;   // >= counters since size >= total
    L.off_part += base; L.off_apart += base; L.off_dir += base;
    L.off_acc += base; L.off_bonus += base; L.off_alpha += base;
    return L;
}

namespace {

// A grid of at most this many workgroups per compute unit runs with the kept terms (three
// waves per SIMD, one wave of each workgroup on each SIMD).
constexpr int kKeepWgPerCu = 3;
constexpr int kMaxDevices = 64;

// ---- request-level helpers --------------------------------------------------------------

// Row normalisers in LDS words 1..4 of a row's accept record (the layout the stream
// kernel publishes: flag, t.hi, d.hi, t.lo, d.lo).
__device__ __forceinline__ void put_norms(uint32_t *w, Norm2 nt, Norm2 nd) {
    w[1] = __float_as_uint(nt.hi); w[2] = __float_as_uint(nd.hi);
    w[3] = __float_as_uint(nt.lo); w[4] = __float_as_uint(nd.lo);
}
__device__ __forceinline__ void get_norms(const uint32_t *w, Norm2 &nt, Norm2 &nd) {
    nt = Norm2{__uint_as_float(w[1]), __uint_as_float(w[3])};
    nd = Norm2{__uint_as_float(w[2]), __uint_as_float(w[4])};
}
// natural log-sum-exp of z / T from the base-2 normaliser
__device__ __forceinline__ float ln_of(Norm2 n) {
    constexpr float kLn2 = 0.69314718055994531f;
    return __builtin_fmaf(n.hi, kLn2, n.lo * kLn2);
}

__device__ __forceinline__ int row_limit(const TeamArgs &a, int r) {
    int L = a.draft_len ? a.draft_len[r] : a.K;
    return L < 0 ? 0 : (L > a.K ? a.K : L);
}

// Accept iff u * q(x) < p(x), i.e. u < 2^{log2 p(x) - log2 q(x)}.
// u: the accept uniform of the row, accept_uniform(seed, r, k, step).
__device__ __forceinline__ int accept_test(float zt, float zd, float c, Norm2 nt, Norm2 nd, float u) {
    const float lpt = log2prob(zt, c, nt);
    const float lpd = log2prob(zd, c, nd);
    return u < exp2f(lpt - lpd) ? 1 : 0;
}
__device__ __forceinline__ float accept_uniform(uint64_t seed, int r, int k, uint64_t step) {
    return uniform24(seed, (uint64_t)r, (uint64_t)k, kPurposeAccept, step);
}

}  // namespace

// =======================================================================================
// Stream kernel: one member workgroup per (row pair, vocabulary chunk)
// =======================================================================================
// Phase 2 of a row: wait (bounded) for the team's partials, reduce them in member order to
// the row normalisers, then publish this member's share of alpha, its residual-mass
// directory entries and (member holding the drafted token) the accept flag.  s_tot[2] and
// s_ok are this row's own LDS slots.  KEEP: pass 2 runs over the terms pass 1 kept in et, ed
// instead of the packed words.
template <int DTT, int DTD, int MODE, bool KEEP>
__device__ __forceinline__ void finish_row(const TeamArgs &a, int64_t row, int j, LaneRow<DTT> &tr,
                                           LaneRow<DTD> &dr, const float (&et)[kTeamE],
                                           const float (&ed)[kTeamE], const ThreadStats &ts, bool owner, float zx_t,
                                           float zx_d, float ua, uint32_t tag, TeamRed &red, uint32_t *pay,
                                           Norm2 *s_tot, int *s_ok) {
    const int S = a.S;
    const float c = a.c;
    const int w = threadIdx.x / kWave;
    const uint64_t *part = a.part + row * (int64_t)(8 * S);
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
    if (!*s_ok) {
        if (threadIdx.x == 0) put(a.apart + row * S + j, kGaveUp, tag);   // the finalize takes over
        return;
    }
    // the row normalisers are uniform: scalar registers, so no vector register holds them
    // through pass 2
    const Norm2 nt = uniform_norm(s_tot[0]), nd = uniform_norm(s_tot[1]);
    float al, rs;
    if constexpr (KEEP) pass2_keep(et, ed, ts, nt, nd, al, rs);
    else pass2(tr, dr, ts, c, nt, nd, al, rs, dot2_scale(opaque_args()));   // read here, not held from the start
    if constexpr (MODE == kTeamStoch) {
        rs = fmaxf(wave_sum(rs), 0.f);
        if (lane_id() == 0) putf(a.dir + row * a.nseg + j * kTeamWaves + w, rs, tag);
    }
    al = block_sumf(al, red);
    if (threadIdx.x == 0) {
        putf(a.apart + row * S + j, al, tag);
        if (MODE == kTeamStoch && owner) {   // accept test and the row normalisers of this row
            uint64_t *ac = a.acc + kAccWords * row;
            put(ac, (uint32_t)accept_test(zx_t, zx_d, c, nt, nd, ua), tag);
            putf(ac + 1, nt.hi, tag);
            putf(ac + 2, nd.hi, tag);
            putf(ac + 3, nt.lo, tag);
            putf(ac + 4, nd.lo, tag);
        }
    }
}

// The token's two logits, read by scalar loads at a clamped index (only the member whose
// chunk holds the token uses them; thread 0 of that member is the owner).
template <int DTT, int DTD>
__device__ __forceinline__ void token_logits(const void *trow, const void *drow, int x, int V, int j, float &zx_t,
                                             float &zx_d, bool &owner) {
    const int xs = x < 0 ? 0 : (x >= V ? V - 1 : x);
    zx_t = load1_uniform<DTT>(trow, xs);
    zx_d = load1_uniform<DTD>(drow, xs);
    owner = threadIdx.x == 0 && x >= 0 && x < V && x / kTeamChunk == j;
}

// One member's work on a verified row pair (not a bonus slot).  FULL: its chunk lies inside
// the row.  KEEP: pass 1 keeps its terms for pass 2 (more registers per lane, less issue).
template <int DTT, int DTD, int MODE, bool AMAX, bool FULL, bool KEEP>
__device__ __forceinline__ void row_member(const TeamArgs &a, int j, int64_t row, int r, int k, TeamRed &red,
                                           uint32_t *pay, Norm2 *s_tot, int *s_ok) {
    const int S = a.S;
    const int K = a.K;
    const int V = a.V;
    const float c = a.c;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *trow = row_ptr<DTT>(a.target, (int64_t)r * a.trows + k, a.ld_t);
    const void *drow = row_ptr<DTD>(a.draft, (int64_t)r * K + k, a.ld_d);

    // The drafted token and the call epoch come by scalar loads; the token's two logits are
    // fetched after the chunk, so no wait for them holds up the passes.
    int x = 0;
    if constexpr (MODE == kTeamStoch) x = load_uniform(a.tokens + (size_t)r * K + k);
    const uint32_t epoch = load_uniform(a.epoch);

    LaneRow<DTT> tr;
    LaneRow<DTD> dr;
    tr.template load<FULL>(trow, base, V);
    dr.template load<FULL>(drow, base, V);
    sched_fence();   // what uses the scalar loads goes after the chunk loads, not before
    const uint32_t tag = epoch_tag(epoch);

    float zx_t = 0.f, zx_d = 0.f;
    bool owner = false;
    // The accept uniform depends on the row alone: the member holding the token draws it now,
    // while its chunk loads are in flight, rather than after pass 2.
    float ua = 0.f;
    if constexpr (MODE == kTeamStoch) {
        token_logits<DTT, DTD>(trow, drow, x, V, j, zx_t, zx_d, owner);
        if (x >= 0 && x < V && x / kTeamChunk == j) ua = accept_uniform(a.seed, r, k, a.step);
    }

    // a poisoned workspace verifies nothing: the member publishes nothing
    if (MODE != kTeamAlpha && epoch_poisoned(epoch)) return;

    constexpr bool want_amax = MODE == kTeamGreedy || AMAX;
    float mt = 0.f, md = 0.f;
    // ---- argmax partials: chunk maximum and the first index holding it ----
    if constexpr (want_amax) {
        int it, id;
        tr.max_first(base, mt, it);
        dr.max_first(base, md, id);
        float wt = mt, wd = md;
        block_amax2(wt, it, wd, id, red);   // larger value; equal values: lowest index
        if (threadIdx.x == 0) {
            putf(part + 4 * S + j, wt, tag);
            put(part + 5 * S + j, (uint32_t)it, tag);
            putf(part + 6 * S + j, wd, tag);
            put(part + 7 * S + j, (uint32_t)id, tag);
        }
    }
    if constexpr (MODE == kTeamGreedy) return;

    // ---- phase 1 (the exact maxima serve as the references when they were needed anyway) ----
    ThreadStats ts;
    float et[kTeamE], ed[kTeamE];
    if constexpr (KEEP) {
        if constexpr (want_amax) {
            ts = pass1_keep(tr, dr, mt, md, c, et, ed);
        } else {
            tr.template lane_ms_keep<FULL>(c, ts.Mt, ts.st, et, trow, base, V);
            dr.template lane_ms_keep<FULL>(c, ts.Md, ts.sd, ed, drow, base, V);
        }
    } else if constexpr (want_amax) {
        ts = pass1(tr, dr, mt, md, c);
    } else {
        tr.lane_ms(c, ts.Mt, ts.st);
        dr.lane_ms(c, ts.Md, ts.sd);
    }
    publish_partials(part, S, j, ts, tag, red);
    // ---- phase 2 ----
    finish_row<DTT, DTD, MODE, KEEP>(a, row, j, tr, dr, et, ed, ts, owner, zx_t, zx_d, ua, tag, red, pay, s_tot,
                                     s_ok);
}

// Bonus slot of request r (target row L): per-wave-range masses against the member's
// reference (stochastic) or the argmax partials (greedy), published without waiting.
template <int DTT, int MODE>
__device__ __forceinline__ void bonus_member(const TeamArgs &a, int j, int64_t row, int r, int L, TeamRed &red) {
    const int S = a.S;
    const int V = a.V;
    const float c = a.c;
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg;
    uint64_t *part = a.part + row * (int64_t)(8 * S);
    const void *brow = row_ptr<DTT>(a.target, (int64_t)r * a.trows + L, a.ld_t);
    const uint32_t epoch = load_uniform(a.epoch);
    LaneRow<DTT> br;
    br.template load<false>(brow, base, V);
    sched_fence();
    if (epoch_poisoned(epoch)) return;
    const uint32_t tag = epoch_tag(epoch);
    if constexpr (MODE == kTeamGreedy) {
        float wb;
        int ib;
        br.max_first(base, wb, ib);
        float wz = neg_inf();
        int iz = 0x7fffffff;
        block_amax2(wb, ib, wz, iz, red);   // larger value; equal values: lowest index
        if (threadIdx.x == 0) {
            putf(part + 4 * S + j, wb, tag);
            put(part + 5 * S + j, (uint32_t)ib, tag);
        }
    } else {
        // per wave range: sum 2^{z c - Mj} against the member's reference Mj (the largest
        // wave maximum), so the finalize needs one directory word per range
        float M, sm;
        br.lane_ms(c, M, sm);
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

// Request r's draft length (r workgroup-uniform): a scalar load, so the member's chunk loads
// that follow do not wait behind it on the vector memory counter.
__device__ __forceinline__ int request_limit(const TeamArgs &a, int r, bool report) {
    int L = a.K;
    if (a.draft_len) {
        const int l0 = load_uniform(a.draft_len + r);
        if ((l0 < 0 || l0 > a.K) && report) atomicOr(a.err, SV_DEVERR_DRAFT_LEN);
        L = l0 < 0 ? 0 : (l0 > a.K ? a.K : l0);
    }
    return L;
}

namespace {

// Recompute member j's share of a row (alpha, and the residual directory entries of its
// wave ranges when dir_row is given) from HBM, once the row normalisers are known: one
// streaming pass over the member's chunk in the member layout, 8 logits of each row at a
// time.  Used only when that member handed its share over, so it keeps few registers live
// rather than the chunk (it runs inside the verification kernel, under its register bound).
template <int DTT, int DTD>
__device__ __forceinline__ float recompute_share(const void *trow, const void *drow, int V, float c, int j, Norm2 nt,
                                                 Norm2 nd, uint64_t *dir_row, uint32_t tag, TeamRed &red) {
    const int w = threadIdx.x / kWave;
    const int base = j * kTeamChunk + w * kTeamSeg + lane_id() * 8;
    float al = 0.f, rs = 0.f;
#pragma unroll 1
    for (int g = 0; g < kTeamE / 8; ++g) {
        float zt[8], zd[8];
        load8<DTT>(trow, base + g * 512, V, zt);
        load8<DTD>(drow, base + g * 512, V, zd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = exp2_fast(log2prob(zt[e], c, nt));
            const float m = fminf(p, exp2_fast(log2prob(zd[e], c, nd)));
            al += m;
            rs += p - m;
        }
    }
    rs = wave_sum(rs);
    if (dir_row && lane_id() == 0) putf(dir_row + j * kTeamWaves + w, rs, tag);
    return block_sumf(al, red);
}

constexpr int kMaxS = (SV_V_MAX + kTeamChunk - 1) / kTeamChunk;   // members per row at most
constexpr int kFinWords = 4096;     // LDS words staged per batch of rows
constexpr int kAccUsed = 5;         // words of an accept record: flag, t.hi, d.hi, t.lo, d.lo
constexpr uint32_t kAbsent = 0xfffffffeu;   // staged payload of a word not published (yet)

// LDS of a member workgroup (one row pair's chunk)
struct MemberShared {
    TeamRed red;
    uint32_t pay[4 * kMaxS];
    Norm2 tot[2];
    int ok;
};

// LDS of a request's finalize workgroup
struct FinShared {
    TeamRed red;
    DrawShared draw;
    uint32_t stage[kFinWords];
    uint32_t pay[6 * kMaxS + 8];
    float mass[4 * kMaxS + 8];
    float u[kTeamThreads];     // correction/bonus uniform for each candidate tau
    int x[kTeamThreads];       // drafted tokens of the rows of a batch
    Norm2 n[2];                // normalisers of the row the draw uses (target, drafter)
    int tau, tok, flags, at;
    int gave;                  // (thread 0) a wait before the arrival gave up
};

// Members and finalize workgroups run the same kernel: their LDS overlays.  The L_e2e grid
// has members only.
union TeamShared {
    MemberShared m;
    FinShared f;
};
template <int MODE>
struct KernelShared {
    using type = TeamShared;
};
template <>
struct KernelShared<kTeamAlpha> {
    using type = MemberShared;
};
__device__ __forceinline__ MemberShared &member_lds(TeamShared &u) { return u.m; }
__device__ __forceinline__ MemberShared &member_lds(MemberShared &m) { return m; }

// One wave (every lane) waits for words p[0..n) with the call's tag; on timeout it flags
// the call and returns false (wave-uniform).
__device__ __forceinline__ bool wave_wait(const TeamArgs &a, const uint64_t *p, int n, uint32_t tag, uint32_t *dst) {
    const bool got = wave_poll(p, n, tag, dst, a.fin_ticks);
    if (!got && lane_id() == 0) atomicOr(a.err, SV_DEVERR_TIMEOUT);
    return got;
}

}  // namespace

// The outputs of request r on a poisoned workspace: nothing verified (accept_len 0, no output
// token, alpha and accept 0, log-sum-exps 0, argmax -1), and the device error flag raised.
__device__ __forceinline__ void nothing_verified(const TeamArgs &a, int r) {
    const int K = a.K;
    for (int q = threadIdx.x; q <= K; q += kTeamThreads) a.out_tokens[(size_t)r * (K + 1) + q] = -1;
    for (int k = threadIdx.x; k < K; k += kTeamThreads) {
        const size_t i = (size_t)r * K + k;
        a.alpha[i] = 0.f;
        a.accept[i] = 0;
        if (a.lse_t) a.lse_t[i] = 0.f;
        if (a.lse_d) a.lse_d[i] = 0.f;
        if (a.amax_t) a.amax_t[i] = -1;
        if (a.amax_d) a.amax_d[i] = -1;
    }
    if (threadIdx.x == 0) {
        a.accept_len[r] = 0;
        a.n_out[r] = 0;
        atomicOr(a.err, SV_DEVERR_POISONED);
    }
}

// =======================================================================================
// Finalize: the last B workgroups of the verification grid, one per request
// =======================================================================================
// Request r's workgroup is dispatched after every member workgroup of the call.  It gathers
// its rows' tagged words as they are published (bounded wait), sums the shares in member
// order, recomputes handed-over shares from HBM, and runs the first-reject scan and the
// correction / bonus draw while the rest of the grid is still streaming.  Before it arrives
// at the call's end it has seen the final word of every workgroup of its request that read
// the call epoch (the shares of its rows, or their argmax words, and the bonus slot's
// references), so the epoch advances only once no workgroup of the call still has to read
// it.
template <int DTT, int DTD, int MODE>
__device__ __forceinline__ void finalize_request(const TeamArgs &a, int r, FinShared &sh) {
    TeamRed &red = sh.red;
    const int K = a.K;
    const int S = a.S;
    const int nseg = a.nseg;
    const int L = row_limit(a, r);
    const uint32_t epoch = read_epoch(a.epoch);
    if (epoch_poisoned(epoch)) {
        nothing_verified(a, r);
        return;
    }
    const uint32_t tag = epoch_tag(epoch);
    const int64_t row0 = (int64_t)r * a.slots;
    const int64_t brow = row0 + K;   // the bonus slot
    const float c = a.c;
    const bool want_amax = (MODE == kTeamGreedy) || a.want_amax;

    // The uniform of the draw after the scan, for every candidate tau <= K: computed up front
    // if K + 1 <= kTeamThreads (the request's rows are usually still streaming), else on
    // demand.
    const bool pre_u = MODE == kTeamStoch && K + 1 <= kTeamThreads;
    auto tau_u = [&](int t) {
        return pre_u ? sh.u[t] : uniform24(a.seed, (uint64_t)r, (uint64_t)t, kPurposeCorrection, a.step);
    };
    if (threadIdx.x == 0) { sh.tau = L; sh.at = 0; sh.gave = 0; sh.n[0] = sh.n[1] = Norm2{0.f, 0.f}; }
    if (pre_u && threadIdx.x <= K)
        sh.u[threadIdx.x] = uniform24(a.seed, (uint64_t)r, (uint64_t)threadIdx.x, kPurposeCorrection, a.step);
    __syncthreads();

    // Rows are staged in batches: acc [nb][kAccUsed] | shares [nb][S] | directory [nb][nseg] |
    // argmax words [nb][4S].
    const int nA = (MODE == kTeamStoch) ? kAccUsed : 0;
    const int nB = (MODE != kTeamGreedy) ? S : 0;
    const int nC = (MODE == kTeamStoch) ? nseg : 0;
    const int nD = want_amax ? 4 * S : 0;
    // The last batch also stages the bonus slot's final words (its members' references,
    // greedy: their argmax indices), which must be seen before the arrival below.
    const int per_row = nA + nB + nC + nD;
    const int batch = max(1, min(kTeamThreads, (kFinWords - S) / max(per_row, 1)));
    const uint64_t *bonus_final = a.part + brow * 8 * S + (MODE == kTeamGreedy ? 5 * S : 0);
    for (int k0 = 0; k0 < L; k0 += batch) {
        const int nb = min(batch, L - k0);
        uint32_t *sx = sh.stage;             // [nb][kAccUsed]
        uint32_t *sa = sx + nb * nA;         // [nb][S]
        uint32_t *sd = sa + nb * nB;         // [nb][nseg]
        uint32_t *sm = sd + nb * nC;         // [nb][4S]
        const int n = nb * per_row + (k0 + nb == L ? S : 0);   // + [S] bonus final words
        if (threadIdx.x < nb) sh.x[threadIdx.x] = a.tokens[(size_t)r * K + k0 + threadIdx.x];

        auto src = [&](int i) -> const uint64_t * {
            if (i < nb * nA) return a.acc + kAccWords * (row0 + k0 + i / kAccUsed) + i % kAccUsed;
            i -= nb * nA;
            if (i < nb * nB) return a.apart + (row0 + k0) * S + i;
            i -= nb * nB;
            if (i < nb * nC) return a.dir + (row0 + k0) * nseg + i;
            i -= nb * nC;
            if (i < nb * nD) return a.part + (row0 + k0 + i / (4 * S)) * 8 * S + 4 * S + i % (4 * S);
            return bonus_final + (i - nb * nD);
        };
        // A staged word is settled once published, or once it is known not to come: the
        // directory words of a member that handed its share over, and the accept record of a
        // row whose token is out of range or whose owner member handed over.
        auto settled = [&](int i) -> bool {
            if (sh.stage[i] != kAbsent) return true;
            if (i < nb * nA) {
                const int q = i / kAccUsed;
                const int x = sh.x[q];
                return x < 0 || x >= a.V || sa[q * S + x / kTeamChunk] == kGaveUp;
            }
            i -= nb * nA;
            if (i < nb * nB) return false;
            i -= nb * nB;
            if (i < nb * nC) return sa[(i / nseg) * S + (i % nseg) / kTeamWaves] == kGaveUp;
            return false;
        };

        // Sweeps until every word is settled: each thread owns words threadIdx.x + u * 256
        // (u < 16) and re-reads those still pending.
        uint32_t pend = 0;
        for (int u = 0; u * kTeamThreads + (int)threadIdx.x < n; ++u) pend |= 1u << u;
        const uint64_t t0 = wall_clock64();
        while (true) {
            for (int u0 = 0; u0 < kFinWords / kTeamThreads; u0 += 4) {
                if (!(pend >> u0)) break;
                uint64_t wv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    wv[u] = ((pend >> (u0 + u)) & 1u) ? peek(src((u0 + u) * kTeamThreads + threadIdx.x)) : 0;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if ((pend >> (u0 + u)) & 1u)
                        sh.stage[(u0 + u) * kTeamThreads + threadIdx.x] =
                            (uint32_t)(wv[u] >> 32) == tag ? (uint32_t)wv[u] : kAbsent;
            }
            __syncthreads();
            for (int u = 0; u < kFinWords / kTeamThreads; ++u)
                if (((pend >> u) & 1u) && settled(u * kTeamThreads + threadIdx.x)) pend &= ~(1u << u);
            if (!__syncthreads_or(pend != 0)) break;
            if ((int64_t)(wall_clock64() - t0) > a.fin_ticks) {
                // Not published within the bound: shares (and the shares of members whose
                // directory words are missing) are recomputed here; an incomplete accept
                // record sends the row to the partials below.
                if (threadIdx.x == 0) {
                    atomicOr(a.err, SV_DEVERR_TIMEOUT);
                    sh.gave = 1;
                }
                for (int u = 0; u < kFinWords / kTeamThreads; ++u) {
                    if (!((pend >> u) & 1u)) continue;
                    int i = u * kTeamThreads + (int)threadIdx.x - nb * nA;
                    if (i >= 0 && i < nb * nB) sa[i] = kGaveUp;
                    i -= nb * nB;
                    if (i >= 0 && i < nb * nC) sa[(i / nseg) * S + (i % nseg) / kTeamWaves] = kGaveUp;
                }
                __syncthreads();
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }

        // any row whose accept record is incomplete, or any handed-over share?
        if (threadIdx.x == 0) sh.flags = 0;
        __syncthreads();
        {
            int f = 0;
            if (MODE == kTeamStoch)
                for (int q = threadIdx.x; q < nb * kAccUsed; q += kTeamThreads) f |= (sx[q] == kAbsent) ? 1 : 0;
            if (MODE != kTeamGreedy)
                for (int q = threadIdx.x; q < nb * S; q += kTeamThreads) f |= (sa[q] == kGaveUp) ? 2 : 0;
            if (f) atomicOr(&sh.flags, f);
        }
        __syncthreads();
        const int flags = sh.flags;
        // rows whose accept record is incomplete (a member handed over, or the drafted token
        // is out of range): the normalisers from the partials, the accept test below
        if (MODE == kTeamStoch && (flags & 1)) {
            for (int q = 0; q < nb; ++q) {
                bool whole = true;
                for (int e = 0; e < kAccUsed; ++e) whole = whole && sx[q * kAccUsed + e] != kAbsent;
                if (whole) continue;
                if (threadIdx.x < kWave) {
                    const bool got = wave_poll(a.part + (row0 + k0 + q) * 8 * S, 4 * S, tag, sh.pay, a.fin_ticks);
                    if (!got && threadIdx.x == 0) {   // the row was never streamed
                        atomicOr(a.err, SV_DEVERR_DRAFT_LEN);
                        sh.gave = 1;
                    }
                }
                __syncthreads();
                if (threadIdx.x < kWave) {
                    Norm2 nt, nd;
                    team_totals(sh.pay, S, nt, nd);
                    if (threadIdx.x == 0) {
                        sx[q * kAccUsed] = kAbsent;   // the test runs here
                        put_norms(sx + q * kAccUsed, nt, nd);
                    }
                }
                __syncthreads();
            }
        }
        // handed-over shares: recompute them (and their directory entries) from HBM
        if (MODE != kTeamGreedy && (flags & 2)) {
            for (int q = 0; q < nb; ++q) {
                for (int m = 0; m < S; ++m) {
                    if (sa[q * S + m] != kGaveUp) continue;
                    Norm2 nt, nd;
                    if (MODE == kTeamStoch) {
                        get_norms(sx + q * kAccUsed, nt, nd);
                    } else {
                        if (threadIdx.x < kWave && !wave_wait(a, a.part + (row0 + k0 + q) * 8 * S, 4 * S, tag, sh.pay) &&
                            threadIdx.x == 0)
                            sh.gave = 1;
                        __syncthreads();
                        team_totals(sh.pay, S, nt, nd);
                    }
                    const int k = k0 + q;
                    const void *trow = row_ptr<DTT>(a.target, (int64_t)r * a.trows + k, a.ld_t);
                    const void *drow = row_ptr<DTD>(a.draft, (int64_t)r * K + k, a.ld_d);
                    const float share = recompute_share<DTT, DTD>(
                        trow, drow, a.V, c, m, nt, nd, MODE == kTeamStoch ? a.dir + (row0 + k) * nseg : nullptr, tag, red);
                    __syncthreads();
                    if (threadIdx.x == 0) sa[q * S + m] = __float_as_uint(share);
                    if (MODE == kTeamStoch) {   // the fresh directory entries of this member
                        load_tagged(a.dir + (row0 + k) * nseg + m * kTeamWaves, kTeamWaves, tag,
                                    sd + q * nseg + m * kTeamWaves, 0u);
                    }
                    __syncthreads();
                }
            }
        }

        // one thread per row of the batch
        Norm2 nt{0.f, 0.f}, nd{0.f, 0.f};
        int at = 0;
        if (threadIdx.x < nb) {
            const int q = threadIdx.x;
            const int k = k0 + q;
            const size_t i = (size_t)r * K + k;
            int ad = 0;
            if (want_amax) {
                const uint32_t *pp = sm + q * 4 * S;
                float bv = neg_inf(), bd = neg_inf();
                int bi = 0x7fffffff, bj = 0x7fffffff;
                for (int m = 0; m < S; ++m) {
                    amax_merge(bv, bi, __uint_as_float(pp[m]), (int)pp[S + m]);
                    amax_merge(bd, bj, __uint_as_float(pp[2 * S + m]), (int)pp[3 * S + m]);
                }
                at = bi == 0x7fffffff ? 0 : bi;
                ad = bj == 0x7fffffff ? 0 : bj;
            }
            const int x = sh.x[q];
            const bool okx = x >= 0 && x < a.V;
            if (!okx) atomicOr(a.err, SV_DEVERR_TOKEN);
            float alpha;
            int acc;
            if constexpr (MODE == kTeamGreedy) {
                alpha = (at == ad) ? 1.f : 0.f;
                acc = okx && x == at;
            } else {
                double sum = 0.0;
                for (int m = 0; m < S; ++m) sum += (double)__uint_as_float(sa[q * S + m]);
                alpha = (float)sum;
                get_norms(sx + q * kAccUsed, nt, nd);
                if (sx[q * kAccUsed] != kAbsent) {
                    acc = (int)sx[q * kAccUsed];
                } else if (okx) {   // the owner member handed over: run the test here
                    const float zt = load1<DTT>(row_ptr<DTT>(a.target, (int64_t)r * a.trows + k, a.ld_t), x);
                    const float zd = load1<DTD>(row_ptr<DTD>(a.draft, (int64_t)r * K + k, a.ld_d), x);
                    acc = accept_test(zt, zd, c, nt, nd, accept_uniform(a.seed, r, k, a.step));
                } else {
                    acc = 0;
                }
            }
            a.alpha[i] = alpha;
            a.accept[i] = (uint8_t)acc;
            if (a.lse_t) a.lse_t[i] = (MODE == kTeamStoch) ? ln_of(nt) : 0.f;
            if (a.lse_d) a.lse_d[i] = (MODE == kTeamStoch) ? ln_of(nd) : 0.f;
            if (a.amax_t) a.amax_t[i] = want_amax ? at : -1;
            if (a.amax_d) a.amax_d[i] = want_amax ? ad : -1;
            if (!acc) atomicMin(&sh.tau, k);
        }
        __syncthreads();
        const int tau = sh.tau;
        if (tau >= k0 && tau < k0 + nb) {
            // keep what the draw after the rejection at tau needs
            if (threadIdx.x == tau - k0) {
                sh.n[0] = nt;
                sh.n[1] = nd;
                sh.at = at;
            }
            if (MODE == kTeamStoch)
                for (int q = threadIdx.x; q < nseg; q += kTeamThreads) sh.mass[q] = __uint_as_float(sd[(tau - k0) * nseg + q]);
        }
        __syncthreads();
    }

    // The bonus slot's members read the epoch too: see their final words (staged with the
    // last batch of rows when there were rows).  After that no workgroup of the call still
    // reads the epoch, so the request arrives now, and the last arrival advances it while
    // the draws still run.
    // If a wait before the arrival gave up, a workgroup of the request may not have read the
    // epoch yet: the call then ends with the epoch poisoned.
    bool gave = false;
    if (L == 0 && threadIdx.x < kWave) gave = !wave_wait(a, bonus_final, S, tag, sh.pay);
    if (threadIdx.x == 0) {
        const Arrival ar = last_arrival(a, r, a.B, gave || sh.gave != 0);
        if (ar.last) __hip_atomic_store(a.epoch, epoch_after(tag, ar.gave_up), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const int tau = sh.tau;
    int tok = 0;
    const void *trow = row_ptr<DTT>(a.target, (int64_t)r * a.trows + tau, a.ld_t);
    if (tau == L) {
        // every draft accepted: the bonus token from the bonus slot's published states
        if (threadIdx.x < kWave) {
            // greedy: argmax words 4S..6S only
            if (MODE == kTeamGreedy) wave_wait(a, a.part + brow * 8 * S + 4 * S, 2 * S, tag, sh.pay + 4 * S);
            else wave_wait(a, a.part + brow * 8 * S, S, tag, sh.pay);
        }
        __syncthreads();
        if constexpr (MODE == kTeamGreedy) {
            if (threadIdx.x == 0) {
                float bv = neg_inf();
                int bi = 0x7fffffff;
                for (int m = 0; m < S; ++m) amax_merge(bv, bi, __uint_as_float(sh.pay[4 * S + m]), (int)sh.pay[5 * S + m]);
                sh.at = bi == 0x7fffffff ? 0 : bi;
            }
            __syncthreads();
            tok = sh.at;
        } else {
            if (threadIdx.x < kWave) wave_wait(a, a.dir + brow * nseg, nseg, tag, sh.pay + S);
            __syncthreads();
            // pay[0..S): member references Mj; pay[S + j * W + w]: range sums against Mj
            if (threadIdx.x < kWave) {
                float M = neg_inf(), sm = 0.f;
                for (int m = threadIdx.x; m < S; m += kWave) {
                    float sj = 0.f;
                    for (int w = 0; w < kTeamWaves; ++w) sj += __uint_as_float(sh.pay[S + m * kTeamWaves + w]);
                    ms_merge(M, sm, __uint_as_float(sh.pay[m]), sj);
                }
                wave_ms(M, sm);
                if (threadIdx.x == 0) sh.n[0] = norm2(M, log2f(sm));
            }
            __syncthreads();
            const Norm2 nb = sh.n[0];
            for (int q = threadIdx.x; q < nseg; q += kTeamThreads) {
                const float Mq = __uint_as_float(sh.pay[q / kTeamWaves]);
                sh.mass[q] = (Mq == neg_inf()) ? 0.f : __uint_as_float(sh.pay[S + q]) * exp2_fast((Mq - nb.hi) - nb.lo);
            }
            __syncthreads();
            tok = draw_ranges<DTT, DTD, false>(trow, nullptr, a.V, c, nb, Norm2{0.f, 0.f}, sh.mass, nseg, tau_u(tau),
                                               sh.draw);
            if (tok < 0) tok = 0;
        }
    } else if constexpr (MODE == kTeamGreedy) {
        tok = sh.at;
    } else {
        // rejection at tau: the residual max(p - q, 0) of row tau
        const float u = tau_u(tau);
        bool done = false;
        {
            const void *drow = row_ptr<DTD>(a.draft, (int64_t)r * K + tau, a.ld_d);
            const int t = draw_ranges<DTT, DTD, true>(trow, drow, a.V, c, sh.n[0], sh.n[1], sh.mass, nseg, u, sh.draw);
            if (t >= 0) { tok = t; done = true; }
        }
        __syncthreads();
        // an empty residual (p == q everywhere in binary32): draw from p_tau
        if (!done)
            tok = draw_from_row<DTT>(trow, a.V, c, u, a.bonus + (size_t)r * 2 * a.nseg_b, a.nseg_b, red, sh.tok);
    }
    if (threadIdx.x == 0) sh.tok = tok;
    __syncthreads();
    tok = sh.tok;

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
    }
}

// =======================================================================================
// Verification grid: one member workgroup per (row pair, vocabulary chunk), then the
// bonus slots, then one finalize workgroup per request
// =======================================================================================
// AMAX: also publish the argmax partials (always in greedy mode; on request otherwise).
// Bfloat16 rows: at most 96 registers per lane, so five waves share each SIMD.  A binary32
// row takes 64 registers of chunk instead of 32: four waves (128 registers) with one such row,
// three with two, so that the chunk stays in registers.  KEEP (not greedy): each lane
// keeps pass 1's terms in binary32 for pass 2, which then costs a multiply, a min and an add per
// logit pair instead of two widenings, two FMAs, a min, an exponential and an add; the terms
// take ~160 registers, so three waves share a SIMD.  The launch takes it only for a grid that
// fits on the device at once at that occupancy, where fewer waves per SIMD cost nothing.
template <int DTT, int DTD>
constexpr int kStreamWaves = 2 + (DTT == kDtBF16 ? 1 : 0) + (DTD == kDtBF16 ? 1 : 0) + (DTT == kDtBF16 && DTD == kDtBF16 ? 1 : 0);

template <int DTT, int DTD, int MODE, bool AMAX, bool KEEP>
__global__ __launch_bounds__(kTeamThreads) __attribute__((amdgpu_waves_per_eu(KEEP ? 3 : kStreamWaves<DTT, DTD>))) void stream_kernel(
    TeamArgs a) {
    __shared__ typename KernelShared<MODE>::type sh;

    // The S members of a team are consecutive workgroups: round-robin dispatch spreads them
    // over the XCDs, whose dispatchers start them at nearly the same time.
    // Work items in grid order: the verified rows (r, k < K) request by request, then every
    // request's bonus slot, so the short bonus workgroups are dispatched last and fill the
    // tail of the grid, then (verification) the finalize workgroups, which run their
    // requests' scans and draws beside the tail.  (Divisions by runtime values are done on
    // the vector unit: readfirstlane returns the uniform results to scalar registers.)
    const int S = a.S;
    const int K = a.K;
    const int slots = a.slots;
    // With a row list, the verified items are the listed rows only.
    const int nv = a.selected ? a.n_rows : a.B * K;
    if constexpr (MODE != kTeamAlpha) {
        const unsigned members = (unsigned)(nv + a.B) * (unsigned)S;
        if (blockIdx.x >= members) {
            // The finalize reads the arguments through an opaque pointer to the kernel's own
            // argument block (the one parameter sits at its start), so none of its scalar
            // loads is merged with the members' and hoisted above the branch, where they would
            // stay live, and spill, through the member path.
            const TeamArgs &fa = opaque_args();
            finalize_request<DTT, DTD, MODE>(fa, (int)(blockIdx.x - members), sh.f);
            return;
        }
    }
    MemberShared &ms = member_lds(sh);
    const int j = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)S));
    const int item = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (unsigned)S));
    int r = item - nv, k = K;
    if (item < nv) {
        const int f = a.selected ? load_uniform(a.row_list + item) : item;
        if (f < 0 || f >= a.B * K) {   // not a row of this batch: nothing to do
            if (threadIdx.x == 0 && j == 0) atomicOr(a.err, SV_DEVERR_DRAFT_LEN);
            return;
        }
        r = f / K;
        k = f - r * K;
    }
    r = __builtin_amdgcn_readfirstlane(r);
    k = __builtin_amdgcn_readfirstlane(k);
    const int64_t row = (int64_t)r * slots + k;
    const bool bonus = (MODE != kTeamAlpha) && k == K;
    const int L = (MODE != kTeamAlpha) ? request_limit(a, r, bonus && j == 0 && threadIdx.x == 0) : K;
    if (!bonus && k >= L) return;
    if (bonus) {
        bonus_member<DTT, MODE>(a, j, row, r, L, ms.red);
        return;
    }
    if ((j + 1) * kTeamChunk <= a.V)
        row_member<DTT, DTD, MODE, AMAX, true, KEEP>(a, j, row, r, k, ms.red, ms.pay, ms.tot, &ms.ok);
    else
        row_member<DTT, DTD, MODE, AMAX, false, KEEP>(a, j, row, r, k, ms.red, ms.pay, ms.tot, &ms.ok);
}

// =======================================================================================
// L_e2e: alpha of each row from the member shares (one thread per row)
// =======================================================================================
template <int DTT, int DTD>
__global__ __launch_bounds__(kTeamThreads) void e2e_alpha_kernel(TeamArgs a) {
    __shared__ TeamRed red;
    __shared__ int s_list[kTeamThreads], s_n;
    __shared__ uint32_t pay[4 * 128 + 8];
    const int64_t rows = (int64_t)a.B * a.K;
    const int64_t row = (int64_t)blockIdx.x * kTeamThreads + threadIdx.x;
    const uint32_t tag = read_epoch(a.epoch) + 1;
    const int S = a.S;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    double sum = 0.0;
    bool handed = false;
    if (row < rows) {
        for (int m = 0; m < S; ++m) {
            const uint64_t w = peek(a.apart + row * S + m);
            if ((uint32_t)(w >> 32) != tag || (uint32_t)w == kGaveUp) { handed = true; break; }
            sum += (double)__uint_as_float((uint32_t)w);
        }
        if (handed) s_list[atomicAdd(&s_n, 1)] = threadIdx.x;
        else a.alpha[row] = (float)sum;
    }
    __syncthreads();
    // rows with a handed-over share: recompute the whole row's alpha (rare)
    for (int q = 0; q < s_n; ++q) {
        const int64_t rr = (int64_t)blockIdx.x * kTeamThreads + s_list[q];
        load_tagged(a.part + rr * 8 * S, 4 * S, tag, pay, 0u);
        __syncthreads();
        Norm2 nt, nd;
        team_totals(pay, S, nt, nd);
        const int ri = (int)(rr / a.K), ki = (int)(rr % a.K);
        const void *trow = row_ptr<DTT>(a.target, (int64_t)ri * a.trows + ki, a.ld_t);
        const void *drow = row_ptr<DTD>(a.draft, rr, a.ld_d);
        double t = 0.0;
        for (int m = 0; m < S; ++m)
            t += (double)recompute_share<DTT, DTD>(trow, drow, a.V, a.c, m, nt, nd, nullptr, tag, red);
        if (threadIdx.x == 0) a.alpha[rr] = (float)t;
        __syncthreads();
    }
}

// Compute units of the current device, read once per device (0 when unknown).
static int device_cus() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cached[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}

template <int DTT, int DTD, bool KEEP>
static void launch_stream_k(const TeamArgs &a, int mode, unsigned grid, hipStream_t s) {
    if (mode == kTeamStoch && a.want_amax)
        hipLaunchKernelGGL((stream_kernel<DTT, DTD, kTeamStoch, true, KEEP>), dim3(grid), dim3(kTeamThreads), 0, s, a);
    else if (mode == kTeamStoch)
        hipLaunchKernelGGL((stream_kernel<DTT, DTD, kTeamStoch, false, KEEP>), dim3(grid), dim3(kTeamThreads), 0, s, a);
    else
        hipLaunchKernelGGL((stream_kernel<DTT, DTD, kTeamAlpha, false, KEEP>), dim3(grid), dim3(kTeamThreads), 0, s, a);
}

template <int DTT, int DTD>
static hipError_t launch_stream_t(const TeamArgs &a, int mode, hipStream_t s) {
    // verification: member workgroups of the verified rows and the bonus slots, then one
    // finalize workgroup per request; L_e2e: member workgroups only
    const uint64_t items = a.selected ? (uint64_t)a.n_rows + (uint64_t)a.B : (uint64_t)a.rows;
    const unsigned grid = (unsigned)(items * (uint64_t)a.S + (mode == kTeamAlpha ? 0u : (uint64_t)a.B));
    if (grid == 0) return hipSuccess;
    if (mode == kTeamGreedy) {
        hipLaunchKernelGGL((stream_kernel<DTT, DTD, kTeamGreedy, true, false>), dim3(grid), dim3(kTeamThreads), 0, s,
                           a);
    } else if ((uint64_t)grid <= (uint64_t)kKeepWgPerCu * (uint64_t)device_cus()) {
        launch_stream_k<DTT, DTD, true>(a, mode, grid, s);   // every workgroup resident at once
    } else {
        launch_stream_k<DTT, DTD, false>(a, mode, grid, s);
    }
    return hipGetLastError();
}

template <int DTT, int DTD>
static hipError_t launch_e2e_t(const TeamArgs &a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.K;
    hipLaunchKernelGGL((e2e_alpha_kernel<DTT, DTD>), dim3((unsigned)((rows + kTeamThreads - 1) / kTeamThreads)),
                       dim3(kTeamThreads), 0, s, a);
    return hipGetLastError();
}

#define SV_DISPATCH(F, ...)                                                        \
    if (dt == SV_BF16 && dd == SV_BF16) return F<kDtBF16, kDtBF16>(__VA_ARGS__);   \
    if (dt == SV_F32 && dd == SV_F32) return F<kDtF32, kDtF32>(__VA_ARGS__);       \
    if (dt == SV_BF16 && dd == SV_F32) return F<kDtBF16, kDtF32>(__VA_ARGS__);     \
    return F<kDtF32, kDtBF16>(__VA_ARGS__);

hipError_t team_launch_stream(const TeamArgs &a, int dt, int dd, int mode, hipStream_t s) {
    SV_DISPATCH(launch_stream_t, a, mode, s)
}
hipError_t team_launch_e2e_alpha(const TeamArgs &a, int dt, int dd, hipStream_t s) { SV_DISPATCH(launch_e2e_t, a, s) }

}  // namespace sv
