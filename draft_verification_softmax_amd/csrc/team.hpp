// team.hpp -- verification kernels in which a team of workgroups shares one (request,
// draft position) row pair.
//
// Stream kernel (the HBM-bound part): member j of a row reads its kTeamChunk-logit chunk of the
// target row and of the drafter row once (16-byte non-temporal loads) and keeps it in
// registers as loaded (bfloat16 pairs), widening on the fly in each pass.  Members
// exchange per-chunk log-sum-exp partials through 64-bit tagged words (32-bit payload,
// 32-bit per-call epoch) written and read with relaxed agent-scope
// atomics, so no cache write-back or invalidation is needed; every member reduces the S
// partials in the same order and gets identical row normalisers, then sums its share of
// min(p, q) and of the residual mass from registers and publishes them.  The member whose
// chunk holds the drafted token runs the accept test and publishes it with the row
// normalisers.  The wait for partials is bounded:
// a member that gives up publishes a hand-over marker instead of its share.  Members have
// no other waits and no atomic read-modify-writes (the finalize's arrival counts are the
// kernel's only ones), so every schedule terminates.
//
// Each request also has a bonus slot: its members read the target row at the request's
// draft length L_r (the row the bonus token is drawn from when every draft is accepted)
// and publish per-wave-range masses against a per-member reference (argmax in greedy
// mode) without waiting.
//
// Finalize (verification: the last B workgroups of the same grid, one per request,
// dispatched after every member): gathers its rows' tagged words as they are published
// (bounded wait), sums the shares in member order, recomputes handed-over shares from HBM,
// and runs the first-reject scan and the correction / bonus draw (one range of the row
// re-read, found by inverse CDF over the published per-range masses), beside the tail of
// the grid rather than after it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "epoch.h"

namespace sv {

constexpr int kTeamThreads = 256;                   // 4 waves
constexpr int kTeamWaves = kTeamThreads / 64;
constexpr int kTeamE = 64;                          // logits per lane per row held in registers
constexpr int kTeamChunk = kTeamThreads * kTeamE;   // logits of each row per member
constexpr int kTeamSeg = 64 * kTeamE;               // one wave's contiguous range
constexpr int kBonusSeg = 512;                      // segment of the single-row bonus draw
constexpr int kXcds = 8;                            // accelerator complex dies of an MI355X
constexpr int kAccWords = 8;                        // tagged words of a row's accept record
constexpr int kArriveSingle = 256;                  // calls of this many units arrive on one counter
constexpr int kArriveSlots = 32;                    // first-level arrival counters of a call
constexpr int kArriveStride = 32;                   // int32 words between them (128 bytes)

// Workspace header (byte offsets, each word on a 64-byte line of its own): device error
// flags, call epoch, second-level arrival counter, the byte count sv_workspace_init recorded
// (uint64; 0 when the workspace was zero-filled some other way), first-level counters.
constexpr size_t kOffErr = 0, kOffEpoch = 64, kOffGdone = 128, kOffWsBytes = 192, kOffArrive = 256;

enum TeamMode { kTeamStoch = 0, kTeamGreedy = 1, kTeamAlpha = 2 };

struct TeamLayout {
    size_t off_err, off_epoch, off_gdone, off_arrive;
    size_t off_part, off_apart, off_dir, off_acc, off_bonus, off_alpha, total;
    int S, nseg, nseg_b;
    int64_t rows;
};

// rows = B * slots row slots: verification uses K + 1 slots per request (positions
// 0..K-1 and the bonus row), L_e2e uses D.
// Counters (which every call returns to zero) sit at the start of the workspace; tagged
// words and per-workgroup scratch sit at its end, so calls of different shapes sharing one
// workspace (always passed with the same size) never overlap a counter with other data.
// ws_bytes == 0 gives the minimal size in `total` (offsets then assume ws_bytes == total).
TeamLayout team_layout(int B, int slots, int V, size_t ws_bytes = 0);

struct TeamArgs {
    const void *target, *draft;
    const int32_t *tokens, *draft_len;
    float *alpha;
    uint8_t *accept;
    float *lse_t, *lse_d;
    int32_t *amax_t, *amax_d;
    int32_t *accept_len, *out_tokens, *n_out;
    uint32_t *err, *epoch;
    uint32_t *gdone;    // second-level arrival counter
    uint32_t *arrive;   // [kArriveSlots][kArriveStride] first-level arrival counters
    uint64_t *part;    // [rows][8][S]: M_t, s_t, M_d, s_d, argmax value/index of both rows;
                       // bonus slots: the member's base-2 reference (stochastic)
    // dir of a bonus slot: per wave range, sum 2^{z c - M_member}
    uint64_t *apart;   // [rows][S]   alpha share of each member (or the hand-over marker)
    uint64_t *dir;     // [rows][4 S] residual mass of each kTeamSeg-logit wave range
    uint64_t *acc;     // [rows][kAccWords] accept flag and the two row normalisers, each as
                       // hi, lo (t.hi, d.hi, t.lo, d.lo), from the member holding the token
    float *bonus;      // [B][2 nseg_b] scratch of the single-row bonus draw
    int64_t ld_t, ld_d;
    int32_t B, K, V, S, nseg, nseg_b;
    int32_t trows;     // target rows per request (K+1 verification, K for L_e2e)
    int32_t slots;     // row slots per request (K+1 verification: the last is the bonus row)
    int64_t rows;      // B * slots
    float c;           // log2(e) / T
    uint64_t seed, step;
    int32_t want_amax;
    int32_t selected;         // 1: the verified rows are the n_rows rows r * K + k of row_list
    const int32_t *row_list;  //    (0: every row k < L_r)
    int32_t n_rows;
    int64_t spin_ticks;  // bounded wait for teammates' partials (10 ns ticks)
    int64_t fin_ticks;   // bounded wait of a finalize workgroup for its request's words
    // c as beta * gamma: beta the nearest bfloat16 (bits in d2_blo), gamma = c / beta and
    // d2_rgamma = beta / c in binary32 (from binary64 on the host); d2_ok = 0 when beta is
    // not a normal bfloat16 or the logits are not bfloat16 (the overlap pass then takes the
    // fma form)
    uint32_t d2_blo;
    float d2_gamma, d2_rgamma;
    int32_t d2_ok;
};

// Grid sizes are derived from a (rows * S + B workgroups at most; the caller checks they fit).
// Verification (kTeamStoch, kTeamGreedy) launches the whole call: members, bonus slots and
// the B finalize workgroups.  kTeamAlpha launches the members of the L_e2e rows only.
hipError_t team_launch_stream(const TeamArgs &a, int dtype_t, int dtype_d, int mode, hipStream_t s);
// L_e2e: alpha per row from the shares (one thread per row).
hipError_t team_launch_e2e_alpha(const TeamArgs &a, int dtype_t, int dtype_d, hipStream_t s);

}  // namespace sv
