/*
 * svref.c -- plain CPU oracle for batched speculative-decoding draft verification.
 *
 * TEST INFRASTRUCTURE ONLY (see svref.h).  Deliberately slow and literal: double
 * precision, one thread, vocabulary index order, every quantity computed straight from
 * its definition.  It shares no code with the GPU library.
 */
#include "svref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon et al., SC'11).  Round: two 64x64->128 products of counter words */
/* 0 and 2 with the published multipliers, then the words are permuted and xored with    */
/* the key; the key is advanced by the published Weyl increments between rounds.        */
/* ------------------------------------------------------------------------------------ */

static const uint64_t PHILOX_MUL_A = 0xD2E7470EE14C6C93ULL;
static const uint64_t PHILOX_MUL_B = 0xCA5A826395121157ULL;
static const uint64_t PHILOX_WEYL_A = 0x9E3779B97F4A7C15ULL;
static const uint64_t PHILOX_WEYL_B = 0xBB67AE8584CAA73BULL;

static void mul_hi_lo(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
    unsigned __int128 prod = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(prod >> 64);
    *lo = (uint64_t)prod;
}

void svref_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_WEYL_A;
            k1 += PHILOX_WEYL_B;
        }
        uint64_t hi_a, lo_a, hi_b, lo_b;
        mul_hi_lo(PHILOX_MUL_A, x0, &hi_a, &lo_a);
        mul_hi_lo(PHILOX_MUL_B, x2, &hi_b, &lo_b);
        uint64_t n0 = hi_b ^ x1 ^ k0;
        uint64_t n1 = lo_b;
        uint64_t n2 = hi_a ^ x3 ^ k1;
        uint64_t n3 = lo_a;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

double svref_uniform(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3) {
    const uint64_t ctr[4] = {c0, c1, c2, c3};
    const uint64_t key[2] = {seed, 0};
    uint64_t out[4];
    svref_philox4x64_10(ctr, key, out);
    return (double)(out[0] >> 40) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------------------------------------ */
/* Rows                                                                                  */
/* ------------------------------------------------------------------------------------ */

double svref_logit(const void *row, int dtype, int64_t i) {
    if (dtype == SVREF_F32) return (double)((const float *)row)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)row)[i] << 16; /* bfloat16 -> binary32 is exact */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Softmax with temperature: p_v = exp(z_v/T - L), L = log sum_v exp(z_v/T).  The pages
 * use p and q as the target and drafter distributions and name T = 0 and T = 0.9; the
 * plain reading is the same T for both, applied to the logits before the softmax. */
double svref_row_lse(const void *row, int dtype, int32_t V, double T) {
    double m = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
        double s = svref_logit(row, dtype, v) / T;
        if (s > m) m = s;
    }
    double S = 0.0;
    for (int32_t v = 0; v < V; ++v) S += exp(svref_logit(row, dtype, v) / T - m);
    return m + log(S);
}

static void row_probs(const void *row, int dtype, int32_t V, double T, double *p) {
    double L = svref_row_lse(row, dtype, V, T);
    for (int32_t v = 0; v < V; ++v) p[v] = exp(svref_logit(row, dtype, v) / T - L);
}

/* Greedy decoding picks the argmax; among equal maxima the lowest index. */
int32_t svref_row_argmax(const void *row, int dtype, int32_t V) {
    int32_t best = 0;
    double bv = svref_logit(row, dtype, 0);
    for (int32_t v = 1; v < V; ++v) {
        double z = svref_logit(row, dtype, v);
        if (z > bv) { bv = z; best = v; }
    }
    return best;
}

/* Overlap equation: alpha(p,q) = sum_v min(p_v, q_v). */
double svref_alpha(const void *trow, int dtype_t, const void *drow, int dtype_d, int32_t V, double T) {
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p || !q) { free(p); free(q); return NAN; }
    row_probs(trow, dtype_t, V, T, p);
    row_probs(drow, dtype_d, V, T, q);
    double a = 0.0;
    for (int32_t v = 0; v < V; ++v) a += (p[v] < q[v]) ? p[v] : q[v];
    free(p);
    free(q);
    return a;
}

/* ------------------------------------------------------------------------------------ */
/* Verification                                                                          */
/* ------------------------------------------------------------------------------------ */

static const void *trow_ptr(const svref_params *p, const void *target, int32_t r, int32_t k) {
    size_t esz = p->dtype_t == SVREF_F32 ? 4 : 2;
    return (const char *)target + ((size_t)r * (size_t)(p->K_max + 1) + (size_t)k) * (size_t)p->ld_t * esz;
}

static const void *drow_ptr(const svref_params *p, const void *draft, int32_t r, int32_t k) {
    size_t esz = p->dtype_d == SVREF_F32 ? 4 : 2;
    return (const char *)draft + ((size_t)r * (size_t)p->K_max + (size_t)k) * (size_t)p->ld_d * esz;
}

static int check_params(const svref_params *p) {
    if (!p || p->B < 0 || p->K_max < 0 || p->V <= 0) return 1;
    if (p->dtype_t != SVREF_F32 && p->dtype_t != SVREF_BF16) return 1;
    if (p->dtype_d != SVREF_F32 && p->dtype_d != SVREF_BF16) return 1;
    if (!(p->temperature >= 0.0) || p->ld_t < p->V || p->ld_d < p->V) return 1;
    return 0;
}

/* Weights of the token drawn after the accepted prefix.  The pages only say the method
 * keeps the target distribution; the one rule that does is standard speculative
 * sampling: after a rejection at tau, draw from norm(max(p_tau - q_tau, 0)); if every
 * draft was accepted (tau = L_r), draw the bonus token from p at row L_r. */
static void correction_weights(const svref_params *p, const void *target, const void *draft,
                               int32_t r, int32_t tau, int32_t L_r, double *w, double *tmp) {
    const int32_t V = p->V;
    const double T = p->temperature;
    row_probs(trow_ptr(p, target, r, tau), p->dtype_t, V, T, w);
    if (tau < L_r) {
        row_probs(drow_ptr(p, draft, r, tau), p->dtype_d, V, T, tmp);
        for (int32_t v = 0; v < V; ++v) {
            double d = w[v] - tmp[v];
            w[v] = d > 0.0 ? d : 0.0;
        }
    }
}

/* Inverse CDF: smallest v with sum_{j<=v} w_j > u * R, R = sum_j w_j.  If rounding runs
 * past the end, the last v with w_v > 0.  Returns -1 when R == 0. */
static int32_t inverse_cdf(const double *w, int32_t V, double u, double *R_out, double *t_out) {
    double R = 0.0;
    for (int32_t v = 0; v < V; ++v) R += w[v];
    double t = u * R;
    if (R_out) *R_out = R;
    if (t_out) *t_out = t;
    if (!(R > 0.0)) return -1;
    double c = 0.0;
    for (int32_t v = 0; v < V; ++v) {
        c += w[v];
        if (c > t) return v;
    }
    for (int32_t v = V - 1; v >= 0; --v)
        if (w[v] > 0.0) return v;
    return -1;
}

static int32_t draw_correction(const svref_params *p, const void *target, const void *draft,
                               int32_t r, int32_t tau, int32_t L_r, double *w, double *tmp,
                               double *u_out, double *t_out, double *R_out) {
    const int32_t V = p->V;
    double u = svref_uniform(p->seed, (uint64_t)r, (uint64_t)tau, SVREF_PURPOSE_CORRECTION, p->step);
    correction_weights(p, target, draft, r, tau, L_r, w, tmp);
    double R, t;
    int32_t tok = inverse_cdf(w, V, u, &R, &t);
    if (tok < 0) { /* p_tau == q_tau exactly: the residual is empty; fall back to p_tau */
        row_probs(trow_ptr(p, target, r, tau), p->dtype_t, V, p->temperature, w);
        tok = inverse_cdf(w, V, u, &R, &t);
    }
    if (u_out) *u_out = u;
    if (t_out) *t_out = t;
    if (R_out) *R_out = R;
    return tok;
}

int svref_verify_batch(const svref_params *p, const void *target, const void *draft,
                       const int32_t *draft_tokens, const int32_t *draft_len,
                       double *alpha, uint8_t *accept, double *lse_t, double *lse_d,
                       int32_t *amax_t, int32_t *amax_d, int32_t *accept_len,
                       int32_t *out_tokens, int32_t *n_out,
                       double *ratio, double *u_acc, double *u_corr, double *cdf_target,
                       double *resid_mass) {
    if (check_params(p) || !target || (p->K_max > 0 && (!draft || !draft_tokens))) return 1;
    if (!alpha || !accept || !accept_len || !out_tokens || !n_out) return 1;
    const int32_t B = p->B, K = p->K_max, V = p->V;
    const double T = p->temperature;
    const int greedy = (T == 0.0);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)V);
    if (!w || !tmp) { free(w); free(tmp); return 1; }

    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K;
        if (L_r < 0 || L_r > K) { free(w); free(tmp); return 1; }
        for (int32_t k = 0; k < K; ++k) {
            const size_t i = (size_t)r * K + k;
            alpha[i] = 0.0;
            accept[i] = 0;
            if (lse_t) lse_t[i] = 0.0;
            if (lse_d) lse_d[i] = 0.0;
            if (amax_t) amax_t[i] = -1;
            if (amax_d) amax_d[i] = -1;
            if (ratio) ratio[i] = NAN;
            if (u_acc) u_acc[i] = NAN;
        }
        for (int32_t k = 0; k < L_r; ++k) {
            const size_t i = (size_t)r * K + k;
            const void *tr = trow_ptr(p, target, r, k);
            const void *dr = drow_ptr(p, draft, r, k);
            const int32_t x = draft_tokens[i];
            if (x < 0 || x >= V) { free(w); free(tmp); return 1; }
            const int32_t at = svref_row_argmax(tr, p->dtype_t, V);
            const int32_t ad = svref_row_argmax(dr, p->dtype_d, V);
            if (amax_t) amax_t[i] = at;
            if (amax_d) amax_d[i] = ad;
            if (greedy) {
                /* T = 0: the softmax is one-hot at the argmax, so the overlap is the
                 * indicator that both argmaxes agree and a draft is accepted iff it is
                 * the target argmax. */
                alpha[i] = (at == ad) ? 1.0 : 0.0;
                accept[i] = (x == at) ? 1 : 0;
            } else {
                const double Lt = svref_row_lse(tr, p->dtype_t, V, T);
                const double Ld = svref_row_lse(dr, p->dtype_d, V, T);
                if (lse_t) lse_t[i] = Lt;
                if (lse_d) lse_d[i] = Ld;
                alpha[i] = svref_alpha(tr, p->dtype_t, dr, p->dtype_d, V, T);
                /* Rejection sampling: accept x with probability min(1, p(x)/q(x)), read as
                 * u * q(x) < p(x) with u uniform in [0,1) keyed by (r, k, accept, step). */
                const double px = exp(svref_logit(tr, p->dtype_t, x) / T - Lt);
                const double qx = exp(svref_logit(dr, p->dtype_d, x) / T - Ld);
                const double u = svref_uniform(p->seed, (uint64_t)r, (uint64_t)k,
                                               SVREF_PURPOSE_ACCEPT, p->step);
                accept[i] = (u * qx < px) ? 1 : 0;
                if (ratio) ratio[i] = px / qx;
                if (u_acc) u_acc[i] = u;
            }
        }
        /* A rejection voids every later draft: tau is the first rejected position. */
        int32_t tau = L_r;
        for (int32_t k = 0; k < L_r; ++k)
            if (!accept[(size_t)r * K + k]) { tau = k; break; }
        accept_len[r] = tau;

        int32_t tok;
        double uc = NAN, tgt = NAN, R = NAN;
        if (greedy) {
            tok = svref_row_argmax(trow_ptr(p, target, r, tau), p->dtype_t, V);
        } else {
            tok = draw_correction(p, target, draft, r, tau, L_r, w, tmp, &uc, &tgt, &R);
        }
        if (u_corr) u_corr[r] = uc;
        if (cdf_target) cdf_target[r] = tgt;
        if (resid_mass) resid_mass[r] = R;
        int32_t *o = out_tokens + (size_t)r * (K + 1);
        for (int32_t j = 0; j <= K; ++j) o[j] = -1;
        for (int32_t j = 0; j < tau; ++j) o[j] = draft_tokens[(size_t)r * K + j];
        o[tau] = tok;
        n_out[r] = tau + 1;
    }
    free(w);
    free(tmp);
    return 0;
}

double svref_correction_cdf(const svref_params *p, const void *target, const void *draft,
                            int32_t r, int32_t tau, int32_t L_r, int32_t v) {
    if (check_params(p) || r < 0 || r >= p->B || L_r < 0 || L_r > p->K_max || tau < 0 ||
        tau > L_r || v < -1 || v >= p->V || !(p->temperature > 0.0))
        return NAN;
    double *w = (double *)malloc(sizeof(double) * (size_t)p->V);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)p->V);
    if (!w || !tmp) { free(w); free(tmp); return NAN; }
    correction_weights(p, target, draft, r, tau, L_r, w, tmp);
    double c = 0.0;
    for (int32_t j = 0; j <= v; ++j) c += w[j];
    free(w);
    free(tmp);
    return c;
}

int svref_accept_len(const uint8_t *accept, const int32_t *draft_len, int32_t B, int32_t K_max,
                     int32_t *accept_len) {
    if (B < 0 || K_max < 0 || !accept_len || (B > 0 && K_max > 0 && !accept)) return 1;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K_max;
        if (L_r < 0 || L_r > K_max) return 1;
        int32_t tau = L_r;
        for (int32_t k = 0; k < L_r; ++k)
            if (!accept[(size_t)r * K_max + k]) { tau = k; break; }
        accept_len[r] = tau;
    }
    return 0;
}

int svref_residual_sample(const svref_params *p, const void *target, const void *draft,
                          const int32_t *draft_len, const int32_t *accept_len, int32_t *token) {
    if (check_params(p) || !target || !accept_len || !token) return 1;
    double *w = (double *)malloc(sizeof(double) * (size_t)p->V);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)p->V);
    if (!w || !tmp) { free(w); free(tmp); return 1; }
    for (int32_t r = 0; r < p->B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : p->K_max;
        const int32_t tau = accept_len[r];
        if (L_r < 0 || L_r > p->K_max || tau < 0 || tau > L_r) { free(w); free(tmp); return 1; }
        if (p->temperature == 0.0)
            token[r] = svref_row_argmax(trow_ptr(p, target, r, tau), p->dtype_t, p->V);
        else
            token[r] = draw_correction(p, target, draft, r, tau, L_r, w, tmp, NULL, NULL, NULL);
    }
    free(w);
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* End-to-end TV objective (L_e2e equation)                                              */
/* ------------------------------------------------------------------------------------ */

double svref_e2e_from_alpha(const double *alpha, int32_t I, int32_t D) {
    if (I <= 0 || D <= 0 || !alpha) return NAN;
    double total = 0.0;
    for (int32_t i = 0; i < I; ++i) {
        for (int32_t m = 0; m < D; ++m) {
            double prod = 1.0;
            for (int32_t k = 0; k <= m; ++k) prod *= alpha[(size_t)i * D + k];
            total += prod;
        }
    }
    return 1.0 - total / ((double)I * (double)D);
}

int svref_tv_e2e_loss(const svref_params *p, const void *target, const void *draft,
                      double *alpha, double *loss) {
    if (check_params(p) || !(p->temperature > 0.0) || p->B <= 0 || p->K_max <= 0 || !target ||
        !draft || !loss)
        return 1;
    const int32_t I = p->B, D = p->K_max;
    const size_t et = p->dtype_t == SVREF_F32 ? 4 : 2, ed = p->dtype_d == SVREF_F32 ? 4 : 2;
    double *a = alpha ? alpha : (double *)malloc(sizeof(double) * (size_t)I * D);
    if (!a) return 1;
    for (int32_t i = 0; i < I; ++i)
        for (int32_t k = 0; k < D; ++k) {
            const size_t row = (size_t)i * D + k;
            a[row] = svref_alpha((const char *)target + row * (size_t)p->ld_t * et, p->dtype_t,
                                 (const char *)draft + row * (size_t)p->ld_d * ed, p->dtype_d,
                                 p->V, p->temperature);
        }
    *loss = svref_e2e_from_alpha(a, I, D);
    if (!alpha) free(a);
    return 0;
}

/* Gradient of L_e2e with respect to the draft logits: what the second training stage
 * descends when it switches to the end-to-end TV objective.  The pages give the loss and
 * the two-stage schedule [AngelSpec tutorial, section "From KL to an end-to-end TV loss",
 * L_e2e equation and the paragraph after it] but not the derivative, so it is written out
 * here by the chain rule, in the plain order of the definition:
 *   dL/dalpha_{i,k} = -(1/(|I| D)) sum_{m=k}^{D-1} prod_{j<=m, j!=k} alpha_{i,j}
 *   dalpha_{i,k}/dz^d_v = (1/T) q_v ([q_v < p_v] - sum_{w: q_w < p_w} q_w)
 * since alpha = sum_w min(p_w, q_w) moves with q_w at slope [q_w < p_w] (at a tie q_w = p_w
 * the one-sided slope 0 is taken) and dq_w/dz^d_v = (1/T) q_w ([w = v] - q_v).  The
 * products over j != k are formed directly, never by dividing by alpha_{i,k}. */
int svref_tv_e2e_backward(const svref_params *p, const void *target, const void *draft, double grad_loss,
                          double *grad, double *alpha, double *loss, double *log_ratio) {
    if (check_params(p) || !(p->temperature > 0.0) || p->B <= 0 || p->K_max <= 0 || !target ||
        !draft || !grad)
        return 1;
    const int32_t I = p->B, D = p->K_max, V = p->V;
    const double T = p->temperature;
    const size_t et = p->dtype_t == SVREF_F32 ? 4 : 2, ed = p->dtype_d == SVREF_F32 ? 4 : 2;
    double *a = alpha ? alpha : (double *)malloc(sizeof(double) * (size_t)I * D);
    double *pp = (double *)malloc(sizeof(double) * (size_t)V);
    double *qq = (double *)malloc(sizeof(double) * (size_t)V);
    if (!a || !pp || !qq) {
        if (!alpha) free(a);
        free(pp);
        free(qq);
        return 1;
    }
    /* the overlaps of every row first: each row's weight needs those of its sequence */
    for (int32_t i = 0; i < I; ++i)
        for (int32_t k = 0; k < D; ++k) {
            const size_t row = (size_t)i * D + k;
            a[row] = svref_alpha((const char *)target + row * (size_t)p->ld_t * et, p->dtype_t,
                                 (const char *)draft + row * (size_t)p->ld_d * ed, p->dtype_d, V, T);
        }
    if (loss) *loss = svref_e2e_from_alpha(a, I, D);
    for (int32_t i = 0; i < I; ++i)
        for (int32_t k = 0; k < D; ++k) {
            const size_t row = (size_t)i * D + k;
            double w = 0.0; /* sum_{m>=k} prod_{j<=m, j!=k} alpha_{i,j} */
            for (int32_t m = k; m < D; ++m) {
                double prod = 1.0;
                for (int32_t j = 0; j <= m; ++j)
                    if (j != k) prod *= a[(size_t)i * D + j];
                w += prod;
            }
            const double dL_dalpha = -w / ((double)I * (double)D);
            const void *trow = (const char *)target + row * (size_t)p->ld_t * et;
            const void *drow = (const char *)draft + row * (size_t)p->ld_d * ed;
            row_probs(trow, p->dtype_t, V, T, pp);
            row_probs(drow, p->dtype_d, V, T, qq);
            double beta = 0.0; /* sum of q over the tokens where q < p */
            for (int32_t v = 0; v < V; ++v)
                if (qq[v] < pp[v]) beta += qq[v];
            for (int32_t v = 0; v < V; ++v) {
                const double slope = (qq[v] < pp[v] ? 1.0 : 0.0) - beta;
                grad[row * (size_t)V + v] = grad_loss * dL_dalpha * qq[v] * slope / T;
            }
            if (log_ratio) {
                const double Lt = svref_row_lse(trow, p->dtype_t, V, T);
                const double Ld = svref_row_lse(drow, p->dtype_d, V, T);
                for (int32_t v = 0; v < V; ++v)
                    log_ratio[row * (size_t)V + v] = (svref_logit(trow, p->dtype_t, v) / T - Lt) -
                                                     (svref_logit(drow, p->dtype_d, v) / T - Ld);
            }
        }
    if (!alpha) free(a);
    free(pp);
    free(qq);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Draft tokens and confidences                                                          */
/* ------------------------------------------------------------------------------------ */

/* The budget step ranks prefixes by an expected utility taken from the drafter's output
 * distribution [AngelSpec tutorial, section "Runtime adaptation: verification as a shared
 * pool", D-cut paragraph]; this is the step that produces what it ranks.  Reading: a
 * drafted token is a sample of q = softmax(z^d / T) and its confidence is q(x).  The draw is
 * the inverse CDF used for every other token here, at u = uniform(seed; r, k, DRAFT, step).
 * T == 0 (greedy drafting): x = argmax, lowest index on ties, and the confidence is the
 * drafter's own probability of it, softmax(z^d)(x) at T = 1 (q at T = 0 would be 1). */
int svref_sample_drafts(const svref_params *p, const void *draft, int32_t *tokens, double *conf,
                        double *u_out, double *R_out) {
    if (check_params(p) || !(p->temperature >= 0.0) || !draft || !tokens || !conf) return 1;
    const int32_t V = p->V;
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    if (!q) return 1;
    for (int32_t r = 0; r < p->B; ++r)
        for (int32_t k = 0; k < p->K_max; ++k) {
            const size_t i = (size_t)r * p->K_max + k;
            const void *drow = drow_ptr(p, draft, r, k);
            int32_t x;
            if (p->temperature > 0.0) {
                row_probs(drow, p->dtype_d, V, p->temperature, q);
                const double u = svref_uniform(p->seed, (uint64_t)r, (uint64_t)k, SVREF_PURPOSE_DRAFT, p->step);
                double R, t;
                x = inverse_cdf(q, V, u, &R, &t);
                if (u_out) u_out[i] = u;
                if (R_out) R_out[i] = R;
            } else {
                x = svref_row_argmax(drow, p->dtype_d, V);
                row_probs(drow, p->dtype_d, V, 1.0, q);
                if (u_out) u_out[i] = 0.0;
                if (R_out) R_out[i] = 1.0;
            }
            if (x < 0) x = 0; /* q == 0 everywhere cannot happen for finite logits */
            tokens[i] = x;
            conf[i] = q[x];
        }
    free(q);
    return 0;
}

/* sum_{j<=v} q_j of drafter row (r, k) at the params' temperature (T > 0). */
double svref_draft_cdf(const svref_params *p, const void *draft, int32_t r, int32_t k, int32_t v) {
    if (check_params(p) || !(p->temperature > 0.0) || r < 0 || r >= p->B || k < 0 || k >= p->K_max || v < -1 ||
        v >= p->V)
        return NAN;
    double *q = (double *)malloc(sizeof(double) * (size_t)p->V);
    if (!q) return NAN;
    row_probs(drow_ptr(p, draft, r, k), p->dtype_d, p->V, p->temperature, q);
    double c = 0.0;
    for (int32_t j = 0; j <= v; ++j) c += q[j];
    free(q);
    return c;
}

/* ------------------------------------------------------------------------------------ */
/* Batch-level verification budget                                                       */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    float c;
    int32_t r, k;
} cand_t;

static int cand_cmp(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->c > y->c) return -1;
    if (x->c < y->c) return 1;
    if (x->r != y->r) return x->r < y->r ? -1 : 1;
    if (x->k != y->k) return x->k < y->k ? -1 : 1;
    return 0;
}

/* The budget goes to the prefixes with the highest expected utility across requests.
 * Reading: the utility of verifying position k of request r is the drafter's cumulative
 * confidence C_{r,k} = prod_{j<=k} c_{r,j} (the probability that the whole prefix
 * survives), a shared pool of N positions is filled in order of C, and each request
 * verifies its selected prefix. */
int svref_alloc_verify_budget(const float *conf, const int32_t *draft_len, int32_t B,
                              int32_t K_max, int32_t budget_N, int32_t *lens, int32_t *row_off,
                              int32_t *row_list) {
    if (B < 0 || K_max < 0 || budget_N < 0 || !lens || !row_off) return 1;
    size_t n = 0;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K_max;
        if (L_r < 0 || L_r > K_max) return 1;
        n += (size_t)L_r;
    }
    cand_t *cand = (cand_t *)malloc(sizeof(cand_t) * (n ? n : 1));
    if (!cand) return 1;
    size_t j = 0;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K_max;
        volatile float C = 1.0f; /* binary32 products, one rounding per step, in k order */
        for (int32_t k = 0; k < L_r; ++k) {
            float c = conf[(size_t)r * K_max + k];
            C = (k == 0) ? c : (float)(C * c);
            cand[j].c = C;
            cand[j].r = r;
            cand[j].k = k;
            ++j;
        }
    }
    qsort(cand, n, sizeof(cand_t), cand_cmp);
    const size_t keep = (size_t)budget_N < n ? (size_t)budget_N : n;
    for (int32_t r = 0; r < B; ++r) lens[r] = 0;
    for (size_t i = 0; i < keep; ++i) lens[cand[i].r]++;
    row_off[0] = 0;
    for (int32_t r = 0; r < B; ++r) row_off[r + 1] = row_off[r] + lens[r];
    if (row_list) {
        /* The selection is prefix-closed when every c <= 1, so request r's rows are
         * k = 0..lens[r]-1. */
        for (int32_t r = 0; r < B; ++r)
            for (int32_t k = 0; k < lens[r]; ++k) row_list[row_off[r] + k] = r * K_max + k;
    }
    free(cand);
    return 0;
}

int svref_dcut_budget(const float *conf, const int32_t *draft_len, int32_t B, int32_t K_max,
                      const float *cost, int32_t n_cost, int32_t *n_chosen, double *utility,
                      int32_t *lens, int32_t *row_off, int32_t *row_list) {
    if (B < 0 || K_max < 0 || n_cost < 1 || !cost || !n_chosen || !utility) return 1;
    size_t n = 0;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K_max;
        if (L_r < 0 || L_r > K_max) return 1;
        n += (size_t)L_r;
    }
    cand_t *cand = (cand_t *)malloc(sizeof(cand_t) * (n ? n : 1));
    if (!cand) return 1;
    size_t j = 0;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t L_r = draft_len ? draft_len[r] : K_max;
        volatile float C = 1.0f;
        for (int32_t k = 0; k < L_r; ++k) {
            float c = conf[(size_t)r * K_max + k];
            C = (k == 0) ? c : (float)(C * c);
            cand[j].c = C;
            cand[j].r = r;
            cand[j].k = k;
            ++j;
        }
    }
    qsort(cand, n, sizeof(cand_t), cand_cmp);
    const size_t nmax = (size_t)(n_cost - 1) < n ? (size_t)(n_cost - 1) : n;
    double P = 0.0;         /* sum of the first m candidates' C, in candidate order */
    double best_ratio = 0.0;
    int32_t best = -1;
    double best_E = (double)B;
    for (size_t m = 0; m <= nmax; ++m) {
        const double E = (double)B + P;
        const double cm = (double)cost[m];
        if (isfinite(cm) && cm > 0.0) {
            const double ratio = E / cm;
            if (best < 0 || ratio > best_ratio) {
                best = (int32_t)m;
                best_ratio = ratio;
                best_E = E;
            }
        }
        if (m < n) P += (double)cand[m].c;
    }
    free(cand);
    if (best < 0) {
        best = 0;
        best_E = (double)B;
    }
    *n_chosen = best;
    *utility = best_E;
    return svref_alloc_verify_budget(conf, draft_len, B, K_max, best, lens, row_off, row_list);
}
