/*
 * specverify.h -- C ABI of libspecverify.so: batched speculative-decoding draft
 * verification on AMD Instinct MI355X (gfx950).
 *
 * What is computed comes from the AngelSpec pages ("AngelSpec: Towards Real-World High
 * Performance Inference with Speculative Decoding"):
 *   [ABS]  the English abstract: speculative decoding keeps the target distribution; the
 *          verification budget is a batch-level resource given to high-confidence prefixes.
 *   [TV]   the AngelSpec tutorial page, section "From KL to an end-to-end TV loss": the
 *          single-step acceptance probability of rejection sampling is the overlap
 *          alpha(p,q) = sum_v min(p(v),q(v)) = 1 - TV(p,q); a rejection voids all later
 *          drafts; the L_e2e equation; the greedy (T=0) and T=0.9 results paragraph.
 *   [RT]   the same page, section "Runtime adaptation: verification as a shared pool"
 *          (D-cut): verification compute is pooled across requests and spent on the
 *          prefixes with the highest expected utility.
 * Where the pages are silent the library takes the standard speculative-sampling rule
 * (accept x with probability min(1, p(x)/q(x)); after a rejection draw from
 * norm(max(p - q, 0)); after a fully accepted draft draw a bonus token from p).
 *
 * Conventions (all entry points):
 *   - Every function returns an sv_status code; nothing throws across the ABI.
 *   - Array arguments are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or retains them.  Calls are asynchronous on `stream` (a
 *     hipStream_t; NULL = the null stream) and return once the work is enqueued.
 *   - Host-checkable arguments (sizes, null required pointers, alignment, dtype codes,
 *     temperature) are validated before anything is launched: SV_EINVAL / SV_EUNSUPPORTED,
 *     nothing enqueued.  A failed launch returns SV_EHIP.
 *   - Device-resident preconditions (0 <= token < V, 0 <= draft_len[r] <= K_max, logits
 *     finite or -inf with at least one finite entry per row) cannot be checked without a
 *     synchronisation; kernels guard every memory access against them, treat a violating
 *     position as rejected, and set a flag read back by sv_device_error().
 *   - Logit layout: row-contiguous, row stride ld_* elements; base pointer and the row
 *     stride in bytes must be multiples of 16 bytes; V is arbitrary (1 <= V <= SV_V_MAX).
 *   - Randomness: Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and counter
 *     (request, position, purpose, step); purpose 0 = accept test, 1 = correction/bonus
 *     draw; the uniform is (word0 >> 40) * 2^-24.  Results are a pure function of the
 *     inputs, seed and step: repeated calls give bit-identical outputs.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sv_status {
    SV_OK = 0,
    SV_EINVAL = 1,       /* bad argument (size, null pointer, alignment, range) */
    SV_EUNSUPPORTED = 2, /* valid but unsupported combination (dtype code, V > SV_V_MAX) */
    SV_EHIP = 3,         /* HIP runtime / launch error */
    SV_EWORKSPACE = 4,   /* workspace missing or smaller than sv_workspace_bytes() */
    SV_EDEVICE = 5       /* a device-side precondition was violated (sv_device_error) */
};

enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 };

#define SV_V_MAX (1 << 20)
#define SV_K_MAX 4096
#define SV_BUDGET_MAX 8192 /* max B * K_max for sv_alloc_verify_budget */

/* Device error flags (sv_device_error). */
#define SV_DEVERR_TOKEN 1u     /* a draft token outside [0, V) */
#define SV_DEVERR_DRAFT_LEN 2u /* a draft_len entry outside [0, K_max], or a row list that does not
                                  match its lengths (sv_verify_selected) */
#define SV_DEVERR_TIMEOUT 4u   /* an internal wait for other workgroups' stores of the same call
                                  exceeded its bound (the member wait bound plus 20 ms); the call
                                  recomputed what was missing and left its workspace poisoned
                                  (see sv_workspace_bytes) */
#define SV_DEVERR_POISONED 8u  /* the call found its workspace poisoned and verified (sampled)
                                  nothing: accept_len 0, n_out 0, out_tokens -1, alpha and
                                  accept 0, lse 0, argmax -1 (sampling: token -1, confidence 0) */

typedef struct sv_params {
    int32_t B;          /* requests (or |I| for sv_tv_e2e_loss) */
    int32_t K_max;      /* draft positions per request (or depth D for sv_tv_e2e_loss) */
    int32_t V;          /* vocabulary size */
    int32_t dtype_t;    /* sv_dtype of the target logits */
    int32_t dtype_d;    /* sv_dtype of the drafter logits */
    float temperature;  /* > 0: stochastic verification of softmax(z / T); 0: greedy */
    uint64_t seed;      /* Philox key word 0 */
    uint64_t step;      /* Philox counter word 3 (e.g. the decoding step) */
    int64_t ld_t;       /* row stride of the target logits, elements (>= V) */
    int64_t ld_d;       /* row stride of the drafter logits, elements (>= V) */
} sv_params;

/* Bytes of device workspace needed by sv_verify_batch / sv_tv_e2e_loss for these sizes.
 * The workspace must be zero-filled before its first use (sv_workspace_init); every call
 * leaves it ready for the next one.  One workspace may serve calls of different shapes if
 * it is large enough for each and is always passed with the same workspace_bytes.  Calls
 * that share a workspace must not overlap (same stream, or ordered by events).
 *
 * Poisoning.  Workgroups of one call exchange words tagged with the call's epoch, which the
 * call advances as it ends, once every workgroup that reads the epoch has done so.  When one
 * of the call's bounded waits gives up (SV_DEVERR_TIMEOUT, or SV_DEVERR_DRAFT_LEN for a row
 * that was never streamed) that is no longer known, so the call ends with the epoch
 * poisoned instead: a workgroup still on its way then writes nothing, and every later
 * verification or sampling call on the workspace verifies nothing and raises
 * SV_DEVERR_POISONED (see there for its outputs), so no word of the late workgroup can be
 * taken for one of a later call.  L_e2e and gradient calls have no such late workgroup and
 * run as usual.  Rule: after SV_DEVERR_TIMEOUT or SV_DEVERR_POISONED, zero-fill the workspace
 * again.  sv_device_error() does so itself for a workspace that sv_workspace_init() set up;
 * a workspace zero-filled some other way must be passed to sv_workspace_init().  The tags
 * are 31-bit: after 2^31 - 1 calls on one workspace it is poisoned the same way. */
size_t sv_workspace_bytes(int32_t B, int32_t K_max, int32_t V);

/* Bound, in nanoseconds, of the wait inside a verification, L_e2e or gradient launch for the
 * partial results of the other workgroups that share a row (default 200000).  A workgroup
 * that reaches it hands its share over: a later workgroup (verification) or kernel (L_e2e,
 * gradient) of the same call recomputes it from the logits, so results do not depend on the
 * bound; only time does.  0 makes every
 * workgroup hand over at once unless its partners have already published (for tests of the
 * hand-over path).  Applies to calls issued after it returns; it is process-wide and not
 * synchronised with calls being issued from other host threads.  Errors: SV_EINVAL (ns < 0). */
int sv_set_wait_bound(int64_t ns);

/* Zero-fill a workspace and record workspace_bytes in its header, where sv_device_error()
 * finds it (a fill kernel on `stream`; no host synchronisation). */
int sv_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Fused batched verification [TV] [ABS].
 *   target       [B][K_max+1][ld_t]  logits of the target at draft positions 0..K_max (row
 *                K_max+1 is the bonus row used when every draft is accepted)
 *   draft        [B][K_max][ld_d]    drafter logits at positions 0..K_max-1
 *   draft_tokens [B][K_max] int32    drafted tokens x_{r,k}
 *   draft_len    [B] int32 or NULL   L_r in [0, K_max] (NULL: every request has K_max);
 *                                     only rows k < L_r and bonus row L_r are read
 * Per position k < L_r, with p = softmax(target/T), q = softmax(draft/T):
 *   alpha    [B][K_max] float   sum_v min(p_v, q_v)  (T = 0: [argmax p == argmax q])
 *   accept   [B][K_max] uint8   u_a * q(x) < p(x), u_a = U(seed; r, k, 0, step)
 *                               (T = 0: x == argmax of the target row)
 *   lse_t, lse_d [B][K_max] float or NULL   log sum_v exp(z_v / T) (0 when T = 0)
 *   amax_t, amax_d [B][K_max] int32 or NULL lowest index of the row maximum
 * Entries k >= L_r are written as alpha 0, accept 0, lse 0, amax -1.
 * Per request:
 *   accept_len [B] int32          tau = first rejected position, or L_r
 *   out_tokens [B][K_max+1] int32 x_0..x_{tau-1}, then the correction token (tau < L_r:
 *                                 drawn from norm(max(p_tau - q_tau, 0))) or the bonus
 *                                 token (tau = L_r: drawn from p at row L_r), then -1;
 *                                 the draw is the smallest v whose cumulative weight
 *                                 exceeds u_c * R, u_c = U(seed; r, tau, 1, step);
 *                                 T = 0: the argmax of target row tau
 *   n_out      [B] int32          tau + 1
 * workspace: sv_workspace_bytes(B, K_max, V) bytes, zero-filled before first use. */
int sv_verify_batch(const sv_params *params, const void *target, const void *draft,
                    const int32_t *draft_tokens, const int32_t *draft_len, float *alpha,
                    uint8_t *accept, float *lse_t, float *lse_d, int32_t *amax_t,
                    int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens, int32_t *n_out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sv_verify_batch with the library's own
 * workspace, a file-scope device array of SV_NOALLOC_SCRATCH_BYTES that each device holds
 * from the first such call until the process ends.  Arguments, outputs and results as
 * sv_verify_batch (bit-identical for the same inputs); no workspace argument.  The first
 * call on a device looks up the array's device address and zero-fills it with a kernel on
 * `stream`; no call allocates or frees anything.  Every call on one device shares the array
 * and leaves it ready for the next: calls that overlap on one device (different streams not
 * ordered by events, host threads racing) race on it and give undefined results.  Device
 * error flags: sv_device_error(NULL, ...) on that device.  Errors: SV_EWORKSPACE when
 * sv_workspace_bytes(B, K_max, V) > SV_NOALLOC_SCRATCH_BYTES (nothing enqueued), else as
 * sv_verify_batch. */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
int sv_verify_batch_noalloc(const sv_params *params, const void *target, const void *draft,
                            const int32_t *draft_tokens, const int32_t *draft_len, float *alpha,
                            uint8_t *accept, float *lse_t, float *lse_d, int32_t *amax_t,
                            int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens, int32_t *n_out,
                            void *stream);

/* Verification of the rows a budget allocation selected [RT]: as sv_verify_batch with
 * draft_len = lens, but the work is laid out over the n_rows listed rows only (plus each
 * request's bonus row), so unselected rows cost nothing.  lens [B] and row_list [n_rows]
 * (r * K_max + k, in (r, k) order) are the outputs of one sv_alloc_verify_budget call: row_list
 * must list exactly the rows k < lens[r], and n_rows = sum_r lens[r] = min(budget_N, B * K_max)
 * when that call had no draft_len (the caller knows it without reading the device).  A listed
 * row outside the batch, or a row k < lens[r] left out, sets SV_DEVERR_DRAFT_LEN.
 * Outputs, workspace and errors as sv_verify_batch. */
int sv_verify_selected(const sv_params *params, const void *target, const void *draft,
                       const int32_t *draft_tokens, const int32_t *lens, const int32_t *row_list,
                       int32_t n_rows, float *alpha, uint8_t *accept, float *lse_t, float *lse_d,
                       int32_t *amax_t, int32_t *amax_d, int32_t *accept_len, int32_t *out_tokens,
                       int32_t *n_out, void *workspace, size_t workspace_bytes, void *stream);

/* First-reject prefix length per request [TV]: accept [B][K_max] uint8, draft_len [B] or
 * NULL; accept_len[r] = first k < L_r with accept == 0, else L_r.  B == 0 is a no-op (its
 * arrays may be NULL).  draft_len entries outside [0, K_max] are clamped to that range. */
int sv_accept_len(const uint8_t *accept, const int32_t *draft_len, int32_t B, int32_t K_max,
                  int32_t *accept_len, void *stream);

/* Correction / bonus token per request given its accepted length [TV] [ABS] (for callers
 * with their own accept logic).  [TV]: a draft position is accepted by rejection sampling
 * with probability alpha = sum_v min(p, q), and the first rejection at tau voids every later
 * draft, so one token follows position tau; [ABS]: that token must leave the output
 * distributed as the target's, which the residual draw norm(max(p_tau - q_tau, 0)) after a
 * rejection, and the draw from p at row L_r after a fully accepted draft, do (the standard
 * speculative-sampling rule named above, where the pages give no formula).  Same layout,
 * draw rule and counters as sv_verify_batch: token[r] is out_tokens[r][accept_len[r]] of a
 * verify call with the same arguments, up to the summation order of the draw's total (the
 * two compute their normalisers separately).  Reads target row tau (and drafter row tau
 * when tau < L_r).  accept_len [B] int32 on the device (clamped to [0, L_r]; draft_len
 * entries are clamped to [0, K_max] first); token [B] int32.  Errors: SV_EINVAL,
 * SV_EUNSUPPORTED, SV_EHIP. */
int sv_residual_sample(const sv_params *params, const void *target, const void *draft,
                       const int32_t *draft_len, const int32_t *accept_len, int32_t *token,
                       void *stream);

/* End-to-end TV objective [TV, L_e2e equation]:
 *   loss = 1 - (1 / (|I| D)) sum_i sum_{m<D} prod_{k<=m} alpha_{i,k}
 * params->B = |I|, params->K_max = D, params->temperature > 0 (1 for raw logits).
 * target, draft [|I|][D][ld] (no bonus row: target row (i,k) at (i*D + k) * ld_t).
 * alpha [|I|][D] float or NULL; loss: one float (device).  Deterministic summation order.
 * workspace: sv_workspace_bytes(|I|, D, V) bytes.  |I| and D must be positive (the mean over
 * an empty set is undefined): SV_EINVAL otherwise. */
int sv_tv_e2e_loss(const sv_params *params, const void *target, const void *draft,
                   float *alpha, float *loss, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Gradient of the end-to-end TV objective in the drafter logits, for the training stage that
 * fine-tunes on it [TV, L_e2e equation and the paragraph after it].  The pages do not write
 * the derivative; by the chain rule
 *   grad[i][k][v] = grad_loss * dL_e2e / dz^d_{i,k,v}
 *                 = -grad_loss (w_{i,k} / (|I| D T)) q_v ([q_v < p_v] - sum_{w: q_w < p_w} q_w),
 *   w_{i,k} = sum_{m=k}^{D-1} prod_{j<=m, j!=k} alpha_{i,j},
 * reading the slope of min(p, q) in q as [q < p] (0 at a tie).  The target logits get no
 * gradient (the target model is frozen).
 * params, target, draft: as for sv_tv_e2e_loss.  alpha [|I|][D] float (device): the overlaps
 * of the same inputs, e.g. the alpha output of sv_tv_e2e_loss.  grad_loss: one float (device),
 * or NULL for 1.  grad: [|I|][D] rows of ld_g >= V elements of dtype_g (SV_F32, or SV_BF16
 * rounded to nearest even), 16-byte aligned rows, not overlapping the logits; elements past V
 * are not written.  workspace: sv_workspace_bytes(|I|, D, V) bytes, same rules as
 * sv_tv_e2e_loss.  Errors: SV_EINVAL (sizes, pointers, alignment, T <= 0), SV_EUNSUPPORTED
 * (dtype code, V > SV_V_MAX), SV_EWORKSPACE, SV_EHIP. */
int sv_tv_e2e_backward(const sv_params *params, const void *target, const void *draft,
                       const float *alpha, const float *grad_loss, void *grad, int32_t dtype_g,
                       int64_t ld_g, void *workspace, size_t workspace_bytes, void *stream);

/* Draft tokens and their confidences, the input of the batch-level budget [RT]: the pool
 * ranks prefixes by what the drafter's output distribution says of them.  For each drafter
 * row (r, k < K_max): T > 0: tokens[r][k] ~ q = softmax(z^d / T), drawn by inverse CDF (the
 * smallest x with sum_{j<=x} q_j > u R, R = sum q) at u = U(Philox(seed; r, k, 2, step)), and
 * conf[r][k] = q(x).  T == 0: the first argmax, with conf = its probability at T = 1.
 * params: B, K_max, V, dtype_d, ld_d, temperature >= 0, seed, step (the target fields are
 * unused).  draft [B][K_max] rows as for sv_verify_batch; tokens int32 [B][K_max], conf float
 * [B][K_max] (device).  workspace: sv_workspace_bytes(B, K_max, V) bytes, same rules as
 * sv_verify_batch.  Errors: SV_EINVAL, SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP. */
int sv_sample_drafts(const sv_params *params, const void *draft, int32_t *tokens, float *conf,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Batch-level verification budget [RT] [ABS]: C_{r,k} = prod_{j<=k} conf_{r,j} (binary32,
 * sequential in k); the first min(N, sum_r L_r) candidates (r, k < L_r) in the order
 * (C desc, r asc, k asc) are kept.  conf [B][K_max] float in [0, 1]; draft_len [B] or
 * NULL.  Outputs: lens [B] (selected prefix length per request; pass it as draft_len to
 * sv_verify_batch), row_off [B+1] (exclusive scan of lens), row_list [min(N, sum L)] or
 * NULL (r*K_max + k of each selected row in (r, k) order).  B*K_max <= SV_BUDGET_MAX.
 * B == 0 writes row_off[0] = 0 (lens may then be NULL).  draft_len entries outside
 * [0, K_max] are a caller error; they are clamped to that range (there is no workspace to
 * carry a device flag here). */
int sv_alloc_verify_budget(const float *conf, const int32_t *draft_len, int32_t B,
                           int32_t K_max, int32_t budget_N, int32_t *lens, int32_t *row_off,
                           int32_t *row_list, void *stream);

/* D-cut budget choice [RT]: the total budget is picked from the caller's cost table, then
 * allocated as by sv_alloc_verify_budget.  Reading (the pages give no formula): verifying
 * the best n candidates of the budget order emits in expectation E(n) = B + (sum of their
 * C), one correction/bonus token per request plus the expected accepted drafts.
 *   cost [n_cost] float (device): the caller's measured cost of a step that verifies n
 *                     positions, n = 0..n_cost-1, 1 <= n_cost <= SV_BUDGET_MAX + 1
 *   n_chosen [1] int32 (device): the n maximising E(n) / cost[n] over n <= min(n_cost - 1,
 *                     sum_r L_r) among entries with a finite positive cost (the smallest such
 *                     n on ties; 0 if no entry qualifies)
 *   utility [1] double (device): E(n_chosen)
 *   lens, row_off, row_list: the allocation of sv_alloc_verify_budget with budget_N =
 *                     n_chosen.
 * E is summed in binary64 by a block scan, so on ratios equal to within ~1e-15 relative
 * the choice may differ from a sequential sum's; any such choice is optimal to that
 * precision.  B * K_max <= SV_BUDGET_MAX. */
int sv_dcut_verify_budget(const float *conf, const int32_t *draft_len, int32_t B, int32_t K_max,
                          const float *cost, int32_t n_cost, int32_t *n_chosen, double *utility,
                          int32_t *lens, int32_t *row_off, int32_t *row_list, void *stream);

/* The library's uniforms, for testing the generator: out[i] = U(seed; counters[i][0..3]). */
int sv_uniforms(uint64_t seed, const uint64_t *counters, int32_t n, float *out, void *stream);

/* Measurement aid, not a step of verification: the plain read-only streaming kernel against
 * which the verification kernels' HBM throughput is judged.  Reads every 16-byte word of
 * data[0 .. bytes) once with non-temporal loads, in workgroups of 256 lanes that each take
 * 32 KiB and exit (the verification members' access pattern without their arithmetic).
 * sink: one uint32 of device memory that the kernel writes only for one particular xor of
 * the data (it keeps the loads from being removed).  data 16-byte aligned, bytes a multiple
 * of 16.  Errors: SV_EINVAL, SV_EHIP. */
int sv_stream_read(const void *data, size_t bytes, uint32_t *sink, void *stream);

/* Synchronise `stream`, return the device error flags left in `workspace` (SV_DEVERR_*)
 * in *flags and clear them.  Returns SV_EDEVICE when any flag was set.  When the flags hold
 * SV_DEVERR_TIMEOUT or SV_DEVERR_POISONED, or the epoch is poisoned, and sv_workspace_init()
 * recorded the workspace's size, the whole workspace is zero-filled again (and the stream
 * synchronised) before it returns, so the next call verifies as usual.  workspace NULL:
 * the current device's sv_verify_batch_noalloc array (flags 0 before its first call).
 * Errors: SV_EINVAL (null flags, misaligned workspace), SV_EHIP. */
int sv_device_error(void *workspace, void *stream, uint32_t *flags);

/* Human-readable name of a status code (static storage). */
const char *sv_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
