// specverify.hip -- batched speculative-decoding draft verification for MI355X (gfx950).
//
// Kernels (all wave64):
//   team_kernel          (team_kernel.hip) fused verification and L_e2e alpha: one team
//                        of workgroups per row pair, each row read from HBM once.
//   residual_kernel      stand-alone correction/bonus draw per request.
//   e2e_reduce_kernel    L_e2e from the alpha table, fixed summation order.
//   budget_kernel        cumulative confidences, sort, selected prefix lengths.
//   accept_len_kernel    first-reject prefix per request.
//
// The definitions come from the AngelSpec pages: the overlap equation and the serial
// acceptance argument and the L_e2e equation (tutorial page, section "From KL to an
// end-to-end TV loss"), the shared verification budget (same page, section "Runtime
// adaptation: verification as a shared pool"), target-distribution preservation (abstract).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sv_device.hpp"
#include "specverify.h"
#include "team.hpp"
#include "team_device.hpp"
#include "team_grad.hpp"
#include "team_sample.hpp"

namespace sv {

// ---------------------------------------------------------------------------------------
// Stand-alone correction / bonus draw (sv_residual_sample): one workgroup per request runs
// the finalize's draws on the row pair at its accepted length
// ---------------------------------------------------------------------------------------
struct ResidualArgs {
    const void *target, *draft;
    const int32_t *draft_len, *accept_len;
    int32_t *out_tokens;
    int64_t ld_t, ld_d;
    int32_t K, V;
    float c;   // log2(e) / T (0: greedy)
    uint64_t seed, step;
};

constexpr int kResidualSegMax = (SV_V_MAX + kBonusSeg - 1) / kBonusSeg;   // draw_from_row segments
constexpr int kRowStep = kTeamThreads * 8;                                 // logits per workgroup sweep step

template <int DTT, int DTD>
__global__ __launch_bounds__(kTeamThreads) void residual_kernel(ResidualArgs a) {
    __shared__ TeamRed red;
    __shared__ DrawShared draw;
    __shared__ float seg[2 * kResidualSegMax];   // range masses, then draw_from_row's segments
    __shared__ int s_tok;
    const int r = blockIdx.x;
    const int K = a.K, V = a.V;
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    int L = a.draft_len ? a.draft_len[r] : K;
    if (L < 0 || L > K) L = L < 0 ? 0 : K;
    int tau = a.accept_len[r];
    if (tau < 0 || tau > L) tau = tau < 0 ? 0 : L;
    const void *trow = row_ptr<DTT>(a.target, (int64_t)r * (K + 1) + tau, a.ld_t);
    int tok = -1;
    if (a.c == 0.f) {
        // greedy: the lowest index of the target row's maximum
        float v = neg_inf(), vd = neg_inf();
        int i = 0x7fffffff, id = 0x7fffffff;
        for (int base = 0; base < V; base += kRowStep) {
            float z[8];
            load8<DTT>(trow, base + threadIdx.x * 8, V, z);
            amax_update8(v, i, z, base + threadIdx.x * 8);
        }
        block_amax2(v, i, vd, id, red);
        tok = i == 0x7fffffff ? 0 : i;
    } else {
        const float c = a.c;
        const float u = uniform24(a.seed, (uint64_t)r, (uint64_t)tau, kPurposeCorrection, a.step);
        if (tau < L) {
            // rejection at tau: the residual max(p - q, 0) of the row pair.  Normalisers of
            // both rows in base 2, then the residual mass of each kTeamSeg-logit range (wave
            // w takes ranges w, w + 4, ...), then the finalize's range draw.
            const void *drow = row_ptr<DTD>(a.draft, (int64_t)r * K + tau, a.ld_d);
            float Mt = neg_inf(), st = 0.f, Md = neg_inf(), sd = 0.f;
            auto lane_ms8 = [&](const float (&z)[8], float &M, float &s) {
                float cm = neg_inf();
#pragma unroll
                for (int e = 0; e < 8; ++e) cm = fmaxf(cm, z[e]);
                if (cm == neg_inf()) return;
                const float cM = cm * c;
                float cs = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) cs += exp2_fast(__builtin_fmaf(z[e], c, -cM));
                ms_merge(M, s, cM, cs);
            };
            for (int base = 0; base < V; base += kRowStep) {
                float zt[8], zd[8];
                load8<DTT>(trow, base + threadIdx.x * 8, V, zt);
                load8<DTD>(drow, base + threadIdx.x * 8, V, zd);
                lane_ms8(zt, Mt, st);
                lane_ms8(zd, Md, sd);
            }
            block_ms2_lanes(Mt, st, Md, sd, red);
            const Norm2 nt = norm2(Mt, log2f(st)), nd = norm2(Md, log2f(sd));
            const int nr = (V + kTeamSeg - 1) / kTeamSeg;
            for (int q = w; q < nr; q += kTeamWaves) {
                float m = 0.f;
                for (int e8 = lane * 8; e8 < kTeamSeg; e8 += kWave * 8) {
                    const int e = q * kTeamSeg + e8;
                    float zt[8], zd[8];
                    load8<DTT>(trow, e, V, zt);
                    load8<DTD>(drow, e, V, zd);
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const float p = exp2_fast(log2prob(zt[k], c, nt));
                        m += p - fminf(p, exp2_fast(log2prob(zd[k], c, nd)));
                    }
                }
                m = wave_sum(m);
                if (lane == 0) seg[q] = m;
            }
            __syncthreads();
            tok = draw_ranges<DTT, DTD, true>(trow, drow, V, c, nt, nd, seg, nr, u, draw);
            __syncthreads();
        }
        // the bonus row (tau = L), or an empty residual (p == q in binary32): a draw from p_tau
        if (tok < 0) tok = draw_from_row<DTT>(trow, V, c, u, seg, (V + kBonusSeg - 1) / kBonusSeg, red, s_tok);
    }
    if (threadIdx.x == 0) a.out_tokens[r] = tok;
}

// ---------------------------------------------------------------------------------------
// L_e2e = 1 - (1/(|I| D)) sum_i sum_{m<D} prod_{k<=m} alpha_{i,k}, fixed summation order
// ---------------------------------------------------------------------------------------
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void e2e_reduce_kernel(const float *alpha, int I, int D, float *loss,
                                                                    uint32_t *epoch) {
    __shared__ double part[kReduceThreads];
    double acc = 0.0;
    for (int i = threadIdx.x; i < I; i += kReduceThreads) {
        double prod = 1.0, row = 0.0;
        for (int m = 0; m < D; ++m) {
            prod *= (double)alpha[(size_t)i * D + m];
            row += prod;
        }
        acc += row;
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kReduceThreads / 2; h > 0; h >>= 1) {
        if (threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *loss = (float)(1.0 - part[0] / ((double)I * (double)D));
        // the team kernels of this call are complete: advance the workspace epoch
        __hip_atomic_store(epoch, epoch_after(epoch_tag(*epoch), false), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------------------
// Batch verification budget
// ---------------------------------------------------------------------------------------
// D-cut choice of the budget (when cost != nullptr): among n = 0..min(n_cost - 1, total)
// with a finite positive cost[n], the n maximising E(n) / cost[n], E(n) = B + the sum of the
// first n candidates' C (binary64); the smallest n on ties, 0 if none qualifies.  The sum
// runs as a block scan: each thread adds a contiguous run of candidates, then the run
// totals are scanned.
__device__ int dcut_choose(const uint64_t *keys, int total, int B, const float *cost, int n_cost, double *dscan,
                           double *s_ratio, int *s_n, double *s_E, int32_t *n_chosen, double *utility) {
    const int nmax = min(n_cost - 1, total);
    const int count = nmax + 1;   // values of n
    const int per = (count + kReduceThreads - 1) / kReduceThreads;
    const int m0 = threadIdx.x * per, m1 = min(count, m0 + per);
    auto Cof = [&](int m) { return (double)__uint_as_float(~(uint32_t)(keys[m] >> 32)); };
    double run = 0.0;   // this thread's candidates m0..m1-1 that precede a later n
    for (int m = m0; m < m1 && m < nmax; ++m) run += Cof(m);
    // exclusive scan of the runs in thread order
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    double incl = run;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const double y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) dscan[wv] = incl;
    __syncthreads();
    double before = 0.0;
    for (int q = 0; q < wv; ++q) before += dscan[q];
    double P = before + incl - run;
    // this thread's best n
    double best_r = -1.0, best_E = (double)B;
    int best_n = 0x7fffffff;
    for (int m = m0; m < m1; ++m) {
        const double E = (double)B + P;
        const double cm = (double)cost[m];
        if (isfinite(cm) && cm > 0.0) {
            const double ratio = E / cm;
            if (ratio > best_r) { best_r = ratio; best_n = m; best_E = E; }
        }
        if (m < nmax) P += Cof(m);
    }
    // block argmax: larger ratio, then smaller n
    for (int d = 32; d >= 1; d >>= 1) {
        const double r2 = __shfl_xor(best_r, d, kWave);
        const int n2 = __shfl_xor(best_n, d, kWave);
        const double e2 = __shfl_xor(best_E, d, kWave);
        if (r2 > best_r || (r2 == best_r && n2 < best_n)) { best_r = r2; best_n = n2; best_E = e2; }
    }
    __syncthreads();
    if (lane == 0) { s_ratio[wv] = best_r; s_n[wv] = best_n; s_E[wv] = best_E; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double r = s_ratio[0], e = s_E[0];
        int n = s_n[0];
        for (int q = 1; q < kReduceThreads / kWave; ++q)
            if (s_ratio[q] > r || (s_ratio[q] == r && s_n[q] < n)) { r = s_ratio[q]; n = s_n[q]; e = s_E[q]; }
        if (n == 0x7fffffff) { n = 0; e = (double)B; }   // no usable cost entry
        s_n[0] = n;
        *n_chosen = n;
        *utility = e;
    }
    __syncthreads();
    return s_n[0];
}

// Bitonic sort of keys[0..np2), ascending (np2 a power of two); every thread of the block calls it.
__device__ void sort_keys(uint64_t *keys, int np2) {
    if (np2 <= kReduceThreads) {
        // one key per thread in registers: exchanges within a wave (partner distance < 64)
        // by lane shuffles, wider ones through LDS
        const int i = threadIdx.x;
        uint64_t key = i < np2 ? keys[i] : ~0ull;
        for (int size = 2; size <= np2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                uint64_t other;
                if (stride >= kWave) {
                    keys[i] = key;
                    __syncthreads();
                    other = keys[i ^ stride];
                    __syncthreads();
                } else {
                    other = __shfl_xor(key, stride, kWave);
                }
                // the lower index of a pair keeps the minimum in an ascending block
                const bool up = (i & size) == 0, lower = (i & stride) == 0;
                key = (lower == up) ? (key < other ? key : other) : (key < other ? other : key);
            }
        }
        keys[i] = key;
        __syncthreads();
    } else {
        for (int size = 2; size <= np2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = threadIdx.x; i < np2; i += kReduceThreads) {
                    const int j = i ^ stride;
                    if (j > i) {
                        const bool up = (i & size) == 0;
                        const uint64_t a = keys[i], b = keys[j];
                        if ((a > b) == up) { keys[i] = b; keys[j] = a; }
                    }
                }
                __syncthreads();
            }
        }
    }
}

// The kth smallest (0-based) of keys[0..n) (distinct keys) by radix selection, 8-bit digits
// from the top: per digit a histogram of the digit values of the keys that agree with the
// digits chosen so far (LDS atomic adds into 256 bins), then one wave scans it, four bins a
// lane, for the value whose running count passes the rank.  A digit value held by a single
// candidate ends the search: that key is the one.  Every thread of the block calls it, and
// every thread gets the result.
__device__ uint64_t select_kth(const uint64_t *keys, int n, int kth, int *hist, uint64_t *s_prefix, int *s_rank,
                               int *s_one) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    uint64_t prefix = 0;
    int rank = kth;
    for (int shift = 56; shift >= 0; shift -= 8) {
        const uint64_t known = shift == 56 ? 0ull : ~0ull << (shift + 8);   // digits chosen so far
        if (threadIdx.x < 256) hist[threadIdx.x] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kReduceThreads) {
            const uint64_t key = keys[i];
            if ((key & known) == prefix) atomicAdd(&hist[(int)((key >> shift) & 255u)], 1);
        }
        __syncthreads();
        if (wv == 0) {
            const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
            const int local = h0 + h1 + h2 + h3;
            int incl = local;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int y = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += y;
            }
            // the first lane whose running count passes rank, then the bin inside it
            const uint64_t hit = __ballot(incl > rank);
            const int l = hit ? __builtin_ctzll(hit) : kWave - 1;
            if (lane == l) {
                int before = incl - local, b = 3, hb = h3;
                if (before + h0 > rank) {
                    b = 0;
                    hb = h0;
                } else if (before + h0 + h1 > rank) {
                    b = 1;
                    hb = h1;
                    before += h0;
                } else if (before + h0 + h1 + h2 > rank) {
                    b = 2;
                    hb = h2;
                    before += h0 + h1;
                } else {
                    before += h0 + h1 + h2;
                }
                *s_prefix = prefix | ((uint64_t)(4 * l + b) << shift);
                *s_rank = rank - before;
                *s_one = hb == 1 ? 1 : 0;
            }
        }
        __syncthreads();
        prefix = *s_prefix;
        rank = *s_rank;
        if (*s_one != 0 && shift > 0) {   // the one key that agrees with the chosen digits
            const uint64_t mask = ~0ull << shift;
            __syncthreads();   // every thread has read s_prefix before it is overwritten
            for (int i = threadIdx.x; i < n; i += kReduceThreads)
                if ((keys[i] & mask) == prefix) *s_prefix = keys[i];
            __syncthreads();
            prefix = *s_prefix;
            break;
        }
    }
    __syncthreads();   // s_prefix and hist may be reused by the caller
    return prefix;
}

__global__ __launch_bounds__(kReduceThreads) void budget_kernel(const float *conf, const int32_t *draft_len,
                                                                int B, int K, int N, int32_t *lens,
                                                                int32_t *row_off, int32_t *row_list,
                                                                uint32_t *err, const float *cost, int n_cost,
                                                                int32_t *n_chosen, double *utility) {
    __shared__ uint64_t keys[SV_BUDGET_MAX];
    __shared__ int cnt[SV_BUDGET_MAX];
    __shared__ int scan[kReduceThreads];
    __shared__ int s_total;
    const int n = B * K;
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    if (threadIdx.x == 0) s_total = 0;
    for (int i = threadIdx.x; i < np2; i += kReduceThreads) keys[i] = ~0ull;
    for (int r = threadIdx.x; r < B; r += kReduceThreads) cnt[r] = 0;
    __syncthreads();
    // cumulative confidence per request: one thread per request, sequential binary32 products
    // (the confidences read from global memory 32 at a time, ahead of the products)
    int local_total = 0;
    for (int r = threadIdx.x; r < B; r += kReduceThreads) {
        int L = draft_len ? draft_len[r] : K;
        if (L < 0 || L > K) {
            if (err) atomicOr(err, SV_DEVERR_DRAFT_LEN);
            L = L < 0 ? 0 : K;
        }
        float C = 1.f;
        for (int k0 = 0; k0 < L; k0 += 32) {
            // every load of the batch issued before the products use them, at clamped (valid)
            // indices so that no load sits under a branch
            float ck[32];
            const int last = r * K + L - 1;
#pragma unroll
            for (int e = 0; e < 32; ++e) ck[e] = conf[min(r * K + k0 + e, last)];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const int k = k0 + e;
                if (k >= L) break;
                C = (k == 0) ? ck[e] : __fmul_rn(C, ck[e]);
                // ascending key = descending C (non-negative binary32 bits are monotone), then (r, k);
                // stored position-major (k * B + r: the requests' threads write consecutive words),
                // since nothing below depends on where a key sits
                keys[k * B + r] = ((uint64_t)(~__float_as_uint(C)) << 32) | (uint32_t)(r * K + k);
            }
        }
        local_total += L;
    }
    // one LDS atomic per wave that holds requests, not one per thread on the same word
    if (threadIdx.x < ((B + kWave - 1) / kWave) * kWave) {
        for (int d = kWave / 2; d >= 1; d >>= 1) local_total += __shfl_xor(local_total, d, kWave);
        if ((threadIdx.x & (kWave - 1)) == 0) atomicAdd(&s_total, local_total);
    }
    __syncthreads();
    __shared__ double dscan[kReduceThreads / kWave], s_ratio[kReduceThreads / kWave], s_E[kReduceThreads / kWave];
    __shared__ int s_n[kReduceThreads / kWave];
    __shared__ int hist[256], s_rank, s_one;
    __shared__ uint64_t s_prefix;
    int keep;
    uint64_t thr = 0;   // the keep-th smallest key: the selection is every key <= thr
    if (!cost) {
        keep = min(N, s_total);
        if (keep > 0) thr = select_kth(keys, n, keep - 1, hist, &s_prefix, &s_rank, &s_one);
    } else {
        sort_keys(keys, np2);   // the D-cut choice sums the candidates in order
        keep = dcut_choose(keys, s_total, B, cost, n_cost, dscan, s_ratio, s_n, s_E, n_chosen, utility);
        if (keep > 0) thr = keys[keep - 1];
    }
    // selected rows per request: the keys <= thr, wherever they sit in keys[]
    if (keep > 0) {
        for (int i = threadIdx.x; i < n; i += kReduceThreads) {
            const uint64_t key = keys[i];
            if (key <= thr) atomicAdd(&cnt[(int)(key & 0xffffffffu) / K], 1);
        }
    }
    __syncthreads();
    // exclusive scan of cnt over B: contiguous chunk per thread, then a scan of chunk sums
    const int per = (B + kReduceThreads - 1) / kReduceThreads;
    const int b0 = threadIdx.x * per, b1 = min(B, b0 + per);
    int sum = 0;
    for (int r = b0; r < b1; ++r) sum += cnt[r];
    // inclusive scan of the chunk sums in thread order: within each wave by shuffles, then
    // the wave totals
    int incl = sum;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
    }
    if (lane == kWave - 1) scan[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int q = 0; q < wv; ++q) before += scan[q];
    incl += before;
    __syncthreads();
    scan[threadIdx.x] = incl;
    __syncthreads();
    int off = incl - sum;
    for (int r = b0; r < b1; ++r) {
        lens[r] = cnt[r];
        row_off[r] = off;
        if (row_list)
            for (int k = 0; k < cnt[r]; ++k) row_list[off + k] = r * K + k;
        off += cnt[r];
    }
    if (threadIdx.x == kReduceThreads - 1) row_off[B] = scan[kReduceThreads - 1];
}

// ---------------------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------------------
__global__ void accept_len_kernel(const uint8_t *accept, const int32_t *draft_len, int B, int K,
                                  int32_t *accept_len, uint32_t *err) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= B) return;
    int L = draft_len ? draft_len[r] : K;
    if (L < 0 || L > K) L = L < 0 ? 0 : K;
    int tau = L;
    for (int k = 0; k < L; ++k)
        if (!accept[(size_t)r * K + k]) { tau = k; break; }
    accept_len[r] = tau;
}

__global__ void uniforms_kernel(uint64_t seed, const uint64_t *ctr, int n, float *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = uniform24(seed, ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
}

// Read-only streaming reference: workgroup b reads 16-byte words [b * 2048, (b + 1) * 2048)
// once (eight non-temporal loads in flight per lane) and exits, the access pattern of the
// verification members without their arithmetic.  The loads feed an xor that reaches memory
// only when it equals an arbitrary constant, so the compiler cannot drop them.
constexpr int kStreamLoads = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *p, size_t n16, uint32_t *sink) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const size_t base = (size_t)blockIdx.x * (256 * kStreamLoads) + threadIdx.x;
    u32x4 v[kStreamLoads];
#pragma unroll
    for (int u = 0; u < kStreamLoads; ++u) {
        const size_t i = base + (size_t)u * 256;
        v[u] = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i) : u32x4{0, 0, 0, 0};
    }
    u32x4 acc = v[0];
#pragma unroll
    for (int u = 1; u < kStreamLoads; ++u) acc ^= v[u];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[0] = x;
}

// Zero-fills a workspace of n16 16-byte words and records its byte count in the header,
// followed by its complement (a record is trusted only when the two agree).
__global__ void init_workspace_kernel(uint4 *p, size_t n16, size_t bytes) {
    const uint4 rec = make_uint4((uint32_t)bytes, (uint32_t)(bytes >> 32), ~(uint32_t)bytes, ~(uint32_t)(bytes >> 32));
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = i == kOffWsBytes / 16 ? rec : make_uint4(0, 0, 0, 0);
}

}  // namespace sv

// =======================================================================================
// C ABI
// =======================================================================================
using namespace sv;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A workspace must be zero-filled again after a wait gave up (its epoch is then poisoned)
// or once a call found it poisoned.
bool workspace_needs_init(uint32_t flags, uint32_t epoch) {
    return (flags & (SV_DEVERR_TIMEOUT | SV_DEVERR_POISONED)) != 0u || epoch_poisoned(epoch);
}

int check_logits(const void *p, int dtype, int64_t ld, int V) {
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EUNSUPPORTED;
    if (!p || ld < V) return SV_EINVAL;
    const int64_t esz = dtype == SV_BF16 ? 2 : 4;
    if (!aligned16(p) || (ld * esz) % 16 != 0) return SV_EINVAL;
    return SV_OK;
}

int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SV_OK : SV_EHIP;
}

template <template <int, int> class Launcher, class... Args>
int dispatch_dtypes(int dt, int dd, Args &&...args) {
    if (dt == SV_BF16 && dd == SV_BF16) return Launcher<kDtBF16, kDtBF16>::run(args...);
    if (dt == SV_F32 && dd == SV_F32) return Launcher<kDtF32, kDtF32>::run(args...);
    if (dt == SV_BF16 && dd == SV_F32) return Launcher<kDtBF16, kDtF32>::run(args...);
    return Launcher<kDtF32, kDtBF16>::run(args...);
}

template <int DTT, int DTD>
struct ResidualLauncher {
    static int run(const ResidualArgs &a, unsigned grid, hipStream_t s) {
        hipLaunchKernelGGL((residual_kernel<DTT, DTD>), dim3(grid), dim3(kTeamThreads), 0, s, a);
        return launch_status();
    }
};

const double kLog2e = 1.4426950408889634;

// Bound of a member's wait for its teammates' partials, in 10-ns ticks (sv_set_wait_bound).
int64_t g_wait_ticks = 20000;   // 200 us
const int64_t kFinalizeWaitTicks = 2000000;   // 20 ms beyond it

void fill_team_args(TeamArgs &a, const sv_params *p, const TeamLayout &L, char *ws) {
    a.err = (uint32_t *)(ws + L.off_err);
    a.epoch = (uint32_t *)(ws + L.off_epoch);
    a.gdone = (uint32_t *)(ws + L.off_gdone);
    a.arrive = (uint32_t *)(ws + L.off_arrive);
    a.part = (uint64_t *)(ws + L.off_part);
    a.apart = (uint64_t *)(ws + L.off_apart);
    a.dir = (uint64_t *)(ws + L.off_dir);
    a.acc = (uint64_t *)(ws + L.off_acc);
    a.bonus = (float *)(ws + L.off_bonus);
    a.ld_t = p->ld_t;
    a.ld_d = p->ld_d;
    a.B = p->B;
    a.K = p->K_max;
    a.V = p->V;
    a.S = L.S;
    a.nseg = L.nseg;
    a.nseg_b = L.nseg_b;
    a.c = p->temperature > 0.f ? (float)(kLog2e / (double)p->temperature) : 0.f;
    // c as beta * gamma (beta the nearest bfloat16, rounded to nearest even) for the overlap
    // pass of bfloat16 rows; gamma and 1 / gamma from binary64
    uint32_t cb;
    memcpy(&cb, &a.c, sizeof cb);
    const uint32_t hb = (cb + 0x7fffu + ((cb >> 16) & 1u)) >> 16;
    const uint32_t bbits = hb << 16;
    float beta;
    memcpy(&beta, &bbits, sizeof beta);
    const bool d2 = a.c > 0.f && beta >= 0x1p-100f && beta <= 0x1p100f;
    a.d2_blo = hb;
    a.d2_gamma = d2 ? (float)((double)a.c / (double)beta) : 0.f;
    a.d2_rgamma = d2 ? (float)((double)beta / (double)a.c) : 0.f;
    a.d2_ok = (d2 && isfinite(a.d2_gamma) && a.d2_gamma > 0.f) ? 1 : 0;
    a.seed = p->seed;
    a.step = p->step;
    a.spin_ticks = g_wait_ticks;  // then a member hands its share over (to the finalize)
    // A finalize workgroup waits for members that are still running: longer than any member
    // can take to publish after its own bounded wait.
    a.fin_ticks = g_wait_ticks + kFinalizeWaitTicks;
    a.rows = L.rows;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int32_t B, int32_t K_max, int32_t V) {
    if (B < 0 || K_max < 0 || V <= 0) return 0;
    return team_layout(B, K_max + 1, V).total;   // K_max + 1 slots also cover L_e2e with D = K_max
}

int sv_set_wait_bound(int64_t ns) {
    if (ns < 0) return SV_EINVAL;
    g_wait_ticks = ns / 10;
    return SV_OK;
}

int sv_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || !aligned16(workspace)) return SV_EINVAL;
    const size_t n16 = workspace_bytes / 16;
    if (n16 == 0) return SV_OK;
    const unsigned grid = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(init_workspace_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint4 *)workspace, n16,
                       workspace_bytes);
    return launch_status();
}

}  // extern "C"

static int verify_impl(const sv_params *p, const void *target, const void *draft,
                       const int32_t *draft_tokens, const int32_t *draft_len, bool selected,
                       const int32_t *row_list, int32_t n_rows, float *alpha, uint8_t *accept, float *lse_t, float *lse_d,
                       int32_t *amax_t, int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens,
                       int32_t *n_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!p || p->B < 0 || p->K_max < 0 || p->K_max > SV_K_MAX || p->V <= 0) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (!(p->temperature >= 0.f) || !isfinite(p->temperature)) return SV_EINVAL;
    if (p->B == 0) return SV_OK;
    int st = check_logits(target, p->dtype_t, p->ld_t, p->V);
    if (st) return st;
    if (p->K_max > 0) {
        st = check_logits(draft, p->dtype_d, p->ld_d, p->V);
        if (st) return st;
        if (!draft_tokens || !alpha || !accept) return SV_EINVAL;
    } else if (p->dtype_d != SV_F32 && p->dtype_d != SV_BF16) {
        return SV_EUNSUPPORTED;
    }
    if (!accept_len || !out_tokens || !n_out) return SV_EINVAL;
    const TeamLayout L = team_layout(p->B, p->K_max + 1, p->V, workspace_bytes);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;
    const uint64_t grid64 = (uint64_t)L.rows * (uint64_t)L.S + (uint64_t)p->B;
    if (grid64 > 0x7fffffffull) return SV_EINVAL;

    TeamArgs a{};
    fill_team_args(a, p, L, (char *)workspace);
    a.target = target; a.draft = draft; a.tokens = draft_tokens; a.draft_len = draft_len;
    a.alpha = alpha; a.accept = accept; a.lse_t = lse_t; a.lse_d = lse_d;
    a.amax_t = amax_t; a.amax_d = amax_d;
    a.accept_len = accept_len; a.out_tokens = out_tokens; a.n_out = n_out;
    a.trows = p->K_max + 1;
    a.slots = p->K_max + 1;
    a.want_amax = (amax_t || amax_d) ? 1 : 0;
    a.selected = selected ? 1 : 0;
    a.row_list = row_list;
    a.n_rows = n_rows;
    const int mode = p->temperature == 0.f ? kTeamGreedy : kTeamStoch;
    const hipError_t e = team_launch_stream(a, p->dtype_t, p->dtype_d, mode, (hipStream_t)stream);
    return e == hipSuccess ? SV_OK : SV_EHIP;
}

// ---------------------------------------------------------------------------------------
// The workspace of sv_verify_batch_noalloc: a file-scope device array.  Every device the
// library runs on holds its own copy until the process ends; calls on one device share it.
// ---------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;

struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;   // device address of this device's copy of `scratch`
    int status = SV_EHIP;
    std::atomic<bool> ready{false};   // ptr set and its zero-fill enqueued
};
ScratchSlot g_scratch[kScratchDevices];

// The device address of the current device's copy of `scratch`.  The first call on a
// device takes it with hipGetSymbolAddress (the host-side name is no device address) and
// zero-fills the array with a kernel on `stream`, recording its size (so sv_device_error can
// zero-fill it again); later calls return the kept address.  Nothing is allocated.
int device_scratch(void **out, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SV_EHIP;
    if (dev < 0 || dev >= kScratchDevices) return SV_EUNSUPPORTED;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&] {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return;
        slot.ptr = p;
        slot.status = sv_workspace_init(p, SV_NOALLOC_SCRATCH_BYTES, stream);
        slot.ready.store(slot.status == SV_OK, std::memory_order_release);
    });
    if (slot.status) return slot.status;
    *out = slot.ptr;
    return SV_OK;
}

// The current device's scratch if a call set it up, else nullptr.
void *device_scratch_if_set() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    const ScratchSlot &slot = g_scratch[dev];
    return slot.ready.load(std::memory_order_acquire) ? slot.ptr : nullptr;
}

}  // namespace

extern "C" {

int sv_verify_batch(const sv_params *p, const void *target, const void *draft,
                    const int32_t *draft_tokens, const int32_t *draft_len, float *alpha,
                    uint8_t *accept, float *lse_t, float *lse_d, int32_t *amax_t,
                    int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens, int32_t *n_out,
                    void *workspace, size_t workspace_bytes, void *stream) {
    return verify_impl(p, target, draft, draft_tokens, draft_len, false, nullptr, 0, alpha, accept, lse_t, lse_d, amax_t,
                       amax_d, accept_len, out_tokens, n_out, workspace, workspace_bytes, stream);
}

int sv_verify_batch_noalloc(const sv_params *p, const void *target, const void *draft,
                            const int32_t *draft_tokens, const int32_t *draft_len, float *alpha,
                            uint8_t *accept, float *lse_t, float *lse_d, int32_t *amax_t,
                            int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens, int32_t *n_out,
                            void *stream) {
    if (!p || p->B < 0 || p->K_max < 0 || p->K_max > SV_K_MAX || p->V <= 0) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (sv_workspace_bytes(p->B, p->K_max, p->V) > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_EWORKSPACE;
    void *ws = nullptr;
    const int st = device_scratch(&ws, (hipStream_t)stream);
    if (st) return st;
    return verify_impl(p, target, draft, draft_tokens, draft_len, false, nullptr, 0, alpha, accept, lse_t, lse_d, amax_t,
                       amax_d, accept_len, out_tokens, n_out, ws, SV_NOALLOC_SCRATCH_BYTES, stream);
}

int sv_verify_selected(const sv_params *p, const void *target, const void *draft,
                       const int32_t *draft_tokens, const int32_t *lens, const int32_t *row_list,
                       int32_t n_rows, float *alpha, uint8_t *accept, float *lse_t, float *lse_d,
                       int32_t *amax_t, int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens,
                       int32_t *n_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!p || p->B < 0 || p->K_max < 0) return SV_EINVAL;
    if (n_rows < 0 || (int64_t)n_rows > (int64_t)p->B * p->K_max) return SV_EINVAL;
    if (p->B > 0 && !lens) return SV_EINVAL;
    if (n_rows > 0 && !row_list) return SV_EINVAL;
    return verify_impl(p, target, draft, draft_tokens, lens, true, row_list, n_rows, alpha, accept, lse_t, lse_d,
                       amax_t, amax_d, accept_len, out_tokens, n_out, workspace, workspace_bytes, stream);
}

int sv_accept_len(const uint8_t *accept, const int32_t *draft_len, int32_t B, int32_t K_max,
                  int32_t *accept_len, void *stream) {
    if (B < 0 || K_max < 0) return SV_EINVAL;
    if (B == 0) return SV_OK;   // an empty batch: its (empty) arrays may be NULL
    if (!accept_len || (K_max > 0 && !accept)) return SV_EINVAL;
    hipLaunchKernelGGL(accept_len_kernel, dim3((B + 255) / 256), dim3(256), 0, (hipStream_t)stream, accept,
                       draft_len, B, K_max, accept_len, (uint32_t *)nullptr);
    return launch_status();
}

int sv_residual_sample(const sv_params *p, const void *target, const void *draft,
                       const int32_t *draft_len, const int32_t *accept_len, int32_t *token,
                       void *stream) {
    if (!p || p->B < 0 || p->K_max < 0 || p->K_max > SV_K_MAX || p->V <= 0) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (!(p->temperature >= 0.f) || !isfinite(p->temperature)) return SV_EINVAL;
    if (p->B == 0) return SV_OK;
    int st = check_logits(target, p->dtype_t, p->ld_t, p->V);
    if (st) return st;
    if (p->K_max > 0) {
        st = check_logits(draft, p->dtype_d, p->ld_d, p->V);
        if (st) return st;
    }
    if (!accept_len || !token) return SV_EINVAL;
    ResidualArgs a{};
    a.target = target; a.draft = draft; a.draft_len = draft_len; a.accept_len = accept_len;
    a.out_tokens = token;
    a.ld_t = p->ld_t; a.ld_d = p->ld_d;
    a.K = p->K_max; a.V = p->V;
    const bool greedy = p->temperature == 0.f;
    a.c = greedy ? 0.f : (float)(kLog2e / (double)p->temperature);
    a.seed = p->seed; a.step = p->step;
    return dispatch_dtypes<ResidualLauncher>(p->dtype_t, p->dtype_d, a, (unsigned)p->B, (hipStream_t)stream);
}

int sv_tv_e2e_loss(const sv_params *p, const void *target, const void *draft, float *alpha,
                   float *loss, void *workspace, size_t workspace_bytes, void *stream) {
    if (!p || p->B <= 0 || p->K_max <= 0 || p->V <= 0 || !loss) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (!(p->temperature > 0.f) || !isfinite(p->temperature)) return SV_EINVAL;
    int st = check_logits(target, p->dtype_t, p->ld_t, p->V);
    if (st) return st;
    st = check_logits(draft, p->dtype_d, p->ld_d, p->V);
    if (st) return st;
    const TeamLayout L = team_layout(p->B, p->K_max, p->V, workspace_bytes);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;
    const uint64_t grid64 = (uint64_t)L.rows * (uint64_t)L.S + (uint64_t)p->B;
    if (grid64 > 0x7fffffffull) return SV_EINVAL;
    float *alpha_buf = alpha ? alpha : (float *)((char *)workspace + L.off_alpha);
    TeamArgs a{};
    fill_team_args(a, p, L, (char *)workspace);
    a.target = target; a.draft = draft;
    a.alpha = alpha_buf;
    a.trows = p->K_max;
    a.slots = p->K_max;
    hipError_t e = team_launch_stream(a, p->dtype_t, p->dtype_d, kTeamAlpha, (hipStream_t)stream);
    if (e == hipSuccess) e = team_launch_e2e_alpha(a, p->dtype_t, p->dtype_d, (hipStream_t)stream);
    if (e != hipSuccess) return SV_EHIP;
    hipLaunchKernelGGL(e2e_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, (hipStream_t)stream, alpha_buf, p->B,
                       p->K_max, loss, a.epoch);
    return launch_status();
}

int sv_tv_e2e_backward(const sv_params *p, const void *target, const void *draft, const float *alpha,
                       const float *grad_loss, void *grad, int32_t dtype_g, int64_t ld_g, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (!p || p->B <= 0 || p->K_max <= 0 || p->V <= 0 || !alpha) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (!(p->temperature > 0.f) || !isfinite(p->temperature)) return SV_EINVAL;
    int st = check_logits(target, p->dtype_t, p->ld_t, p->V);
    if (st) return st;
    st = check_logits(draft, p->dtype_d, p->ld_d, p->V);
    if (st) return st;
    st = check_logits(grad, dtype_g, ld_g, p->V);
    if (st) return st;
    const TeamLayout L = team_layout(p->B, p->K_max, p->V, workspace_bytes);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;
    const uint64_t grid64 = (uint64_t)L.rows * (uint64_t)L.S + (uint64_t)p->B;
    if (grid64 > 0x7fffffffull) return SV_EINVAL;
    TeamArgs a{};
    fill_team_args(a, p, L, (char *)workspace);
    a.target = target; a.draft = draft;
    a.trows = p->K_max;
    a.slots = p->K_max;
    GradArgs g{};
    g.grad = grad;
    g.ld_g = ld_g;
    g.alpha = alpha;
    g.grad_loss = grad_loss;
    g.scale = (float *)((char *)workspace + L.off_alpha);
    g.inv_idt = 1.0 / ((double)p->B * (double)p->K_max * (double)p->temperature);
    if (team_launch_grad(a, g, p->dtype_t, p->dtype_d, dtype_g, (hipStream_t)stream) != hipSuccess) return SV_EHIP;
    return launch_status();
}

int sv_sample_drafts(const sv_params *p, const void *draft, int32_t *tokens, float *conf, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (!p || p->B < 0 || p->K_max < 0 || p->V <= 0) return SV_EINVAL;
    if (p->V > SV_V_MAX) return SV_EUNSUPPORTED;
    if (!(p->temperature >= 0.f) || !isfinite(p->temperature)) return SV_EINVAL;
    if (p->B == 0 || p->K_max == 0) return SV_OK;
    const int st = check_logits(draft, p->dtype_d, p->ld_d, p->V);
    if (st) return st;
    if (!tokens || !conf) return SV_EINVAL;
    const TeamLayout L = team_layout(p->B, p->K_max, p->V, workspace_bytes);
    if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SV_EWORKSPACE;
    const uint64_t grid64 = (uint64_t)L.rows * (uint64_t)L.S + (uint64_t)p->B;
    if (grid64 > 0x7fffffffull) return SV_EINVAL;
    TeamArgs a{};
    fill_team_args(a, p, L, (char *)workspace);
    a.draft = draft;
    a.trows = p->K_max;
    a.slots = p->K_max;
    if (team_launch_sample(a, p->dtype_d, tokens, conf, (hipStream_t)stream) != hipSuccess) return SV_EHIP;
    return launch_status();
}

int sv_alloc_verify_budget(const float *conf, const int32_t *draft_len, int32_t B, int32_t K_max,
                           int32_t budget_N, int32_t *lens, int32_t *row_off, int32_t *row_list,
                           void *stream) {
    if (B < 0 || K_max < 0 || budget_N < 0 || !row_off || (B > 0 && !lens)) return SV_EINVAL;
    if ((int64_t)B * K_max > SV_BUDGET_MAX || B > SV_BUDGET_MAX) return SV_EUNSUPPORTED;
    if (B > 0 && K_max > 0 && !conf) return SV_EINVAL;
    hipLaunchKernelGGL(budget_kernel, dim3(1), dim3(kReduceThreads), 0, (hipStream_t)stream, conf, draft_len, B,
                       K_max, budget_N, lens, row_off, row_list, (uint32_t *)nullptr, (const float *)nullptr, 0,
                       (int32_t *)nullptr, (double *)nullptr);
    return launch_status();
}

int sv_dcut_verify_budget(const float *conf, const int32_t *draft_len, int32_t B, int32_t K_max,
                          const float *cost, int32_t n_cost, int32_t *n_chosen, double *utility, int32_t *lens,
                          int32_t *row_off, int32_t *row_list, void *stream) {
    if (B < 0 || K_max < 0 || n_cost < 1 || !cost || !n_chosen || !utility || !row_off || (B > 0 && !lens))
        return SV_EINVAL;
    if ((int64_t)B * K_max > SV_BUDGET_MAX || B > SV_BUDGET_MAX || n_cost > SV_BUDGET_MAX + 1) return SV_EUNSUPPORTED;
    if (B > 0 && K_max > 0 && !conf) return SV_EINVAL;
    hipLaunchKernelGGL(budget_kernel, dim3(1), dim3(kReduceThreads), 0, (hipStream_t)stream, conf, draft_len, B,
                       K_max, 0, lens, row_off, row_list, (uint32_t *)nullptr, cost, n_cost, n_chosen, utility);
    return launch_status();
}

int sv_uniforms(uint64_t seed, const uint64_t *counters, int32_t n, float *out, void *stream) {
    if (n < 0 || (n > 0 && (!counters || !out))) return SV_EINVAL;
    if (n == 0) return SV_OK;
    hipLaunchKernelGGL(uniforms_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, seed, counters, n,
                       out);
    return launch_status();
}

int sv_stream_read(const void *data, size_t bytes, uint32_t *sink, void *stream) {
    if (!data || !sink || !aligned16(data) || bytes % 16 != 0) return SV_EINVAL;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return SV_OK;
    const size_t per = (size_t)256 * kStreamLoads;
    const size_t grid = (n16 + per - 1) / per;
    if (grid > 0x7fffffffull) return SV_EINVAL;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)data, n16, sink);
    return launch_status();
}

int sv_device_error(void *workspace, void *stream, uint32_t *flags) {
    if (!flags) return SV_EINVAL;
    if (!workspace) {   // the current device's sv_verify_batch_noalloc scratch
        workspace = device_scratch_if_set();
        if (!workspace) {
            *flags = 0;
            return SV_OK;
        }
    }
    if (!aligned16(workspace)) return SV_EINVAL;
    uint64_t hdr[kOffArrive / 8] = {};   // err .. recorded byte count
    if (hipMemcpyAsync(hdr, workspace, sizeof hdr, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
        return SV_EHIP;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SV_EHIP;
    const uint32_t v = (uint32_t)hdr[kOffErr / 8];
    // the byte count sv_workspace_init recorded, trusted only next to its complement
    const uint64_t rec = hdr[kOffWsBytes / 8], rec_check = hdr[kOffWsBytes / 8 + 1];
    const size_t recorded = rec_check == ~rec ? (size_t)rec : 0;
    *flags = v;
    if (!v) return SV_OK;
    if (workspace_needs_init(v, (uint32_t)hdr[kOffEpoch / 8]) && recorded >= kOffArrive) {
        // a wait gave up, or the epoch is poisoned: zero-fill the whole workspace again
        // (every kernel of the stream is complete, so no workgroup still writes to it)
        const int st = sv_workspace_init(workspace, recorded, stream);
        if (st) return st;
        if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SV_EHIP;
    } else {
        const uint32_t z = 0;
        if (hipMemcpy(workspace, &z, sizeof z, hipMemcpyHostToDevice) != hipSuccess) return SV_EHIP;
    }
    return SV_EDEVICE;
}

const char *sv_status_string(int status) {
    switch (status) {
        case SV_OK: return "SV_OK";
        case SV_EINVAL: return "SV_EINVAL: invalid argument";
        case SV_EUNSUPPORTED: return "SV_EUNSUPPORTED: unsupported dtype or size";
        case SV_EHIP: return "SV_EHIP: HIP runtime or launch error";
        case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing, misaligned or too small";
        case SV_EDEVICE: return "SV_EDEVICE: device-side precondition violated";
        default: return "unknown status";
    }
}

}  // extern "C"
