/*
 * svref.h -- plain CPU oracle for batched speculative-decoding draft verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls
 * this code; only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no source with the GPU library.
 *
 * Everything is computed in double precision, single-threaded, in vocabulary index
 * order, straight from the definitions on the AngelSpec pages:
 *   - overlap alpha(p,q) = sum_v min(p(v), q(v)) = 1 - TV(p,q)
 *       [AngelSpec tutorial, section "From KL to an end-to-end TV loss", overlap equation]
 *   - serial acceptance: a rejection voids every later draft
 *       [same section, paragraph after the overlap equation]
 *   - L_e2e = 1 - (1/(|I| D)) sum_i sum_{m<D} prod_{k<=m} alpha_{i,k}
 *       [same section, L_e2e equation]; its gradient in the draft logits, for the
 *       stage that fine-tunes on it [same section, paragraph after the equation]
 *   - greedy (T=0) and stochastic (T=0.9) decoding modes
 *       [same section, MTP results paragraph]
 *   - verification as a batch-level budget given to high-confidence prefixes, ranked by
 *       what the drafter's distribution says of each prefix
 *       [AngelSpec tutorial, section "Runtime adaptation: verification as a shared pool"]
 *   - the target distribution is left unchanged
 *       [AngelSpec abstract, first sentence]
 *
 * Readings where the pages are silent (accept inequality, residual/bonus token,
 * temperature, tie-break, RNG) are listed with each function below.
 */
#ifndef SVREF_H
#define SVREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVREF_F32 0
#define SVREF_BF16 1

/* Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3", SC'11).  out = bijection_key(ctr). */
void svref_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* Uniform in [0,1) with 24 random bits: (word0 >> 40) * 2^-24 of Philox with
 * key (seed, 0) and counter (c0, c1, c2, c3).  Exactly representable in binary32. */
double svref_uniform(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3);

/* Purposes (counter word 2). */
#define SVREF_PURPOSE_ACCEPT 0
#define SVREF_PURPOSE_CORRECTION 1
#define SVREF_PURPOSE_DRAFT 2

/* Logit element i of a row stored as binary32 or bfloat16, widened to double (exact). */
double svref_logit(const void *row, int dtype, int64_t i);

/* Natural log-normaliser of z/T: L = log sum_v exp(z_v / T).  T > 0. */
double svref_row_lse(const void *row, int dtype, int32_t V, double T);

/* Lowest index among the maxima of z (T-independent). */
int32_t svref_row_argmax(const void *row, int dtype, int32_t V);

/* alpha(p,q) = sum_v min(p_v, q_v) with p = softmax(zt/T), q = softmax(zd/T), T > 0. */
double svref_alpha(const void *trow, int dtype_t, const void *drow, int dtype_d, int32_t V, double T);

typedef struct {
    int32_t B, K_max, V;
    int32_t dtype_t, dtype_d;
    double temperature; /* > 0 stochastic, == 0 greedy */
    uint64_t seed, step;
    int64_t ld_t, ld_d; /* row strides in elements */
} svref_params;

/* Full verification of a batch.  Layout: target row (r,k) at target + (r*(K_max+1)+k)*ld_t
 * for k = 0..K_max; draft row (r,k) at draft + (r*K_max+k)*ld_d for k < K_max.
 * draft_len[r] in [0, K_max] (NULL: all K_max).
 * Outputs ([B][K_max] unless noted; entries k >= L_r get alpha 0, accept 0, lse 0, amax -1):
 *   alpha, accept, lse_t, lse_d (T>0 only; 0 in greedy mode), amax_t, amax_d (may be NULL),
 *   accept_len [B], out_tokens [B][K_max+1] (x_0..x_{tau-1}, token, then -1), n_out [B].
 * Diagnostics (may be NULL): ratio [B][K_max] = p(x)/q(x) (T>0), u_acc [B][K_max],
 *   u_corr [B] = u_c, cdf_target [B] = u_c * R, resid_mass [B] = R.
 * Returns 0 on success, nonzero on bad arguments. */
int svref_verify_batch(const svref_params *p, const void *target, const void *draft,
                       const int32_t *draft_tokens, const int32_t *draft_len,
                       double *alpha, uint8_t *accept, double *lse_t, double *lse_d,
                       int32_t *amax_t, int32_t *amax_d, int32_t *accept_len,
                       int32_t *out_tokens, int32_t *n_out,
                       double *ratio, double *u_acc, double *u_corr, double *cdf_target,
                       double *resid_mass);

/* Cumulative (unnormalised) weight of the correction/bonus distribution of request r
 * at accepted length tau, through token v inclusive: sum_{j<=v} w_j, with
 * w = max(p_tau - q_tau, 0) if tau < L_r else p_{L_r}.  Used to classify near-boundary
 * token draws.  Returns NaN on bad arguments. */
double svref_correction_cdf(const svref_params *p, const void *target, const void *draft,
                            int32_t r, int32_t tau, int32_t L_r, int32_t v);

/* First-reject prefix length per request. */
int svref_accept_len(const uint8_t *accept, const int32_t *draft_len, int32_t B, int32_t K_max,
                     int32_t *accept_len);

/* Correction/bonus token for each request given its accepted length (same counters as
 * svref_verify_batch, so the same token). */
int svref_residual_sample(const svref_params *p, const void *target, const void *draft,
                          const int32_t *draft_len, const int32_t *accept_len, int32_t *token);

/* L_e2e from a given alpha table [I][D]. */
double svref_e2e_from_alpha(const double *alpha, int32_t I, int32_t D);

/* L_e2e from logits: target and draft rows (i,k) at base + (i*D+k)*ld, no bonus row.
 * p->B = |I|, p->K_max = D, temperature > 0.  alpha [I][D] may be NULL. */
int svref_tv_e2e_loss(const svref_params *p, const void *target, const void *draft,
                      double *alpha, double *loss);

/* Gradient of L_e2e with respect to the draft logits z^d (rows as for svref_tv_e2e_loss):
 * grad [I][D][V] = grad_loss * dL_e2e/dz^d, with the slope of min(p, q) in q taken as
 * [q < p] (0 at a tie).  alpha [I][D], loss and log_ratio [I][D][V] = ln p_v - ln q_v may be
 * NULL. */
int svref_tv_e2e_backward(const svref_params *p, const void *target, const void *draft, double grad_loss,
                          double *grad, double *alpha, double *loss, double *log_ratio);

/* Draft tokens and confidences for drafter rows [B][K_max][ld_d] (as svref_verify_batch's
 * draft): T > 0: tokens[r][k] = inverse CDF of q = softmax(z/T) at u = uniform(seed; r, k,
 * DRAFT, step), conf = q(token); T == 0: the argmax (lowest index) and its probability at
 * T = 1.  u_out, R_out ([B][K_max], may be NULL): the draw's u and R = sum q. */
int svref_sample_drafts(const svref_params *p, const void *draft, int32_t *tokens, double *conf,
                        double *u_out, double *R_out);

/* sum_{j<=v} q_j of drafter row (r, k) at temperature T > 0 (v = -1 gives 0). */
double svref_draft_cdf(const svref_params *p, const void *draft, int32_t r, int32_t k, int32_t v);

/* Batch verification budget: C_{r,k} = prod_{j<=k} conf_{r,j} in binary32, sequential;
 * keep the first min(N, sum_r L_r) candidates (r, k < L_r) ordered by (C desc, r asc,
 * k asc).  lens [B], row_off [B+1] exclusive scan, row_list [min(N, sum L)] of
 * r*K_max + k in (r, k) order (may be NULL). */
int svref_alloc_verify_budget(const float *conf, const int32_t *draft_len, int32_t B,
                              int32_t K_max, int32_t budget_N, int32_t *lens, int32_t *row_off,
                              int32_t *row_list);

/* D-cut: the total verification budget chosen from a cost table.  AngelSpec tutorial,
 * section "Runtime adaptation: verification as a shared compute pool": verification is a
 * pool shared across requests, spent on the prefixes with the highest expected benefit,
 * and cut back when the load makes it dear.  Reading (the pages give no formula):
 * verifying the best n candidates of the budget order (C desc, r asc, k asc) emits in
 * expectation E(n) = B + (sum of their C), one correction/bonus token per request plus the
 * expected accepted drafts of a prefix-closed selection; cost[n] (n = 0..n_cost-1) is the
 * caller's measured cost of a step that verifies n positions.  The chosen n maximises
 * E(n) / cost[n] over n <= min(n_cost - 1, sum_r L_r) among entries with a finite
 * positive cost (the smallest such n on ties; 0 when no entry qualifies).  E is summed in
 * binary64 in candidate order.  Outputs *n_chosen, *utility = E(n_chosen) and the
 * allocation of svref_alloc_verify_budget with budget n_chosen. */
int svref_dcut_budget(const float *conf, const int32_t *draft_len, int32_t B, int32_t K_max,
                      const float *cost, int32_t n_cost, int32_t *n_chosen, double *utility,
                      int32_t *lens, int32_t *row_off, int32_t *row_list);

#ifdef __cplusplus
}
#endif
#endif
