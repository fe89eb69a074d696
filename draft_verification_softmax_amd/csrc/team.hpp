// team.hpp -- the fused verification kernel in which a team of workgroups shares one
// (request, draft position) row pair.
//
// Each member workgroup reads its vocabulary chunk of both rows from HBM once and keeps it
// in registers.  Members exchange per-chunk log-sum-exp partials through 64-bit tagged
// words (32-bit payload, 32-bit per-call epoch) written and read with relaxed agent-scope
// atomics, so no cache write-back or invalidation is needed; every member reduces the
// same partials in the same order and gets identical row normalisers, then sums its share
// of min(p, q) from registers.  The member that arrives last at the row counter sums the
// shares, runs the accept test and, when it completes a request, the request's
// first-reject scan and correction/bonus draw.  Every wait is bounded: a member that gives
// up leaves its share to the last arriver, which recomputes it from HBM, so no schedule of
// workgroups can deadlock.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kTeamThreads = 256;             // 4 waves
constexpr int kTeamWaves = kTeamThreads / 64;
constexpr int kTeamE = 32;                    // logits per lane per row held in registers
constexpr int kTeamChunk = kTeamThreads * kTeamE;   // 8192 logits of each row per member
constexpr int kTeamSeg = 64 * kTeamE;               // 2048: one wave's contiguous range
constexpr int kBonusSeg = 512;                       // segment of the single-row bonus draw

enum TeamMode { kTeamStoch = 0, kTeamGreedy = 1, kTeamAlpha = 2 };

struct TeamLayout {
    size_t off_epoch, off_gdone, off_grp, off_rowcnt, off_reqcnt;
    size_t off_part, off_apart, off_dir, off_rec, off_bonus, off_alpha, off_err, total;
    int S, nseg, nseg_b, n_grp;
    int64_t rows;
};

// rows: row slots (B * max(K,1) for verification, I * D for L_e2e); B: requests.
// Counters (which every call returns to zero) sit at the start of the workspace; tagged
// words and per-workgroup scratch sit at its end, so calls of different shapes sharing one
// workspace (always passed with the same size) never overlap a counter with other data.
// ws_bytes == 0 gives the minimal size in `total` (offsets then assume ws_bytes == total).
TeamLayout team_layout(int B, int K, int V, size_t ws_bytes = 0);

struct TeamArgs {
    const void *target, *draft;
    const int32_t *tokens, *draft_len;
    float *alpha;
    uint8_t *accept;
    float *lse_t, *lse_d;
    int32_t *amax_t, *amax_d;
    int32_t *accept_len, *out_tokens, *n_out;
    uint32_t *err, *epoch;
    int32_t *gdone, *grp_cnt, *row_cnt, *req_cnt;
    uint64_t *part;    // [rows][S][8]
    uint64_t *apart;   // [rows][S]
    uint64_t *dir;     // [rows][S * 4]
    uint64_t *rec;     // [rows][4]
    float *bonus;      // [B][2 * nseg_b]
    int64_t ld_t, ld_d;
    int32_t B, K, V, S, nseg, nseg_b;
    int32_t trows;     // target rows per request (K+1 verification, K for L_e2e)
    int32_t n_grp;     // L_e2e: groups of rows counted toward the epoch advance
    float c;           // log2(e) / T
    uint64_t seed, step;
    int32_t want_amax;
    int64_t spin_ticks;     // bounded wait before a member hands its share over (10 ns ticks)
    int64_t spin_ticks_max; // bound on waits that only await stores already issued
};

hipError_t team_launch(const TeamArgs &a, int dtype_t, int dtype_d, int mode, unsigned grid, hipStream_t s);

}  // namespace sv
