/* Runs the CPU oracle (oracle/svref.c, linked in, built with address and undefined-behaviour
 * sanitizers by the test that compiles this file) on
 *   verify <dir>   the inputs in <dir> (raw little-endian files written by the test):
 *                  params.txt "B K V dtype T seed step", target.bin, draft.bin, tokens.bin,
 *                  draft_len.bin; writes alpha.bin, accept.bin, lse_t.bin, lse_d.bin,
 *                  amax_t.bin, amax_d.bin, accept_len.bin, out_tokens.bin, n_out.bin,
 *                  resid.bin (residual_sample at the verified accepted lengths), e2e.bin
 *                  (L_e2e and its gradient over the drafted rows), samp.bin (sample_drafts)
 *   budget         budget allocations of random confidence tables against a brute force
 *                  (every candidate ranked by (C desc, r, k), the first N kept)
 * Exit status 0 on success; a sanitizer report aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "svref.h"

static void *slurp(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
    void *p = malloc(bytes ? bytes : 1);
    if (fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void spill(const char *dir, const char *name, const void *p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

static int run_verify(const char *dir) {
    char path[4096];
    snprintf(path, sizeof path, "%s/params.txt", dir);
    FILE *f = fopen(path, "r");
    int B, K, V, dt;
    double T;
    unsigned long long seed, step;
    if (!f || fscanf(f, "%d %d %d %d %lf %llu %llu", &B, &K, &V, &dt, &T, &seed, &step) != 7) return 2;
    fclose(f);
    const size_t es = dt == SVREF_BF16 ? 2 : 4;
    void *target = slurp(dir, "target.bin", (size_t)B * (K + 1) * V * es);
    void *draft = slurp(dir, "draft.bin", (size_t)B * K * V * es);
    int32_t *tokens = slurp(dir, "tokens.bin", sizeof(int32_t) * B * K);
    int32_t *dl = slurp(dir, "draft_len.bin", sizeof(int32_t) * B);
    svref_params p = {B, K, V, dt, dt, T, seed, step, V, V};
    const size_t n = (size_t)B * K;
    double *alpha = calloc(n, 8), *lse_t = calloc(n, 8), *lse_d = calloc(n, 8);
    double *ratio = calloc(n, 8), *u_acc = calloc(n, 8), *u_corr = calloc(B, 8), *cdf_t = calloc(B, 8), *rm = calloc(B, 8);
    uint8_t *accept = calloc(n, 1);
    int32_t *amax_t = calloc(n, 4), *amax_d = calloc(n, 4), *al = calloc(B, 4), *ot = calloc((size_t)B * (K + 1), 4);
    int32_t *nout = calloc(B, 4), *resid = calloc(B, 4), *al2 = calloc(B, 4);
    if (svref_verify_batch(&p, target, draft, tokens, dl, alpha, accept, lse_t, lse_d, amax_t, amax_d, al, ot, nout,
                           ratio, u_acc, u_corr, cdf_t, rm))
        return 3;
    if (svref_accept_len(accept, dl, B, K, al2)) return 3;
    if (memcmp(al, al2, sizeof(int32_t) * B)) return 4;
    if (svref_residual_sample(&p, target, draft, dl, al, resid)) return 3;
    for (int r = 0; r < B; ++r) {   /* the CDF at both ends and inside */
        const int tau = al[r], L = dl[r];
        const double lo = svref_correction_cdf(&p, target, draft, r, tau, L, -1);
        const double mid = svref_correction_cdf(&p, target, draft, r, tau, L, V / 2);
        const double hi = svref_correction_cdf(&p, target, draft, r, tau, L, V - 1);
        if (T > 0 && !(lo == 0.0 && mid >= lo && hi >= mid && hi > 0.0)) return 5;
    }
    spill(dir, "alpha.bin", alpha, n * 8);
    spill(dir, "accept.bin", accept, n);
    spill(dir, "lse_t.bin", lse_t, n * 8);
    spill(dir, "lse_d.bin", lse_d, n * 8);
    spill(dir, "amax_t.bin", amax_t, n * 4);
    spill(dir, "amax_d.bin", amax_d, n * 4);
    spill(dir, "accept_len.bin", al, (size_t)B * 4);
    spill(dir, "out_tokens.bin", ot, (size_t)B * (K + 1) * 4);
    spill(dir, "n_out.bin", nout, (size_t)B * 4);
    spill(dir, "resid.bin", resid, (size_t)B * 4);
    if (T > 0 && K > 0) {
        /* L_e2e over the drafted rows: the target's first K rows of each request */
        const size_t rowb = (size_t)V * es;
        char *t2 = malloc((size_t)B * K * rowb);
        for (int r = 0; r < B; ++r) memcpy(t2 + (size_t)r * K * rowb, (char *)target + (size_t)r * (K + 1) * rowb, K * rowb);
        svref_params q = p;
        double loss = 0, loss2 = 0;
        double *a2 = calloc(n, 8), *grad = calloc(n * V, 8), *lr = calloc(n * V, 8);
        if (svref_tv_e2e_loss(&q, t2, draft, a2, &loss)) return 3;
        if (svref_tv_e2e_backward(&q, t2, draft, 1.0, grad, NULL, &loss2, lr)) return 3;
        if (loss != loss2) return 6;
        double e2e[2] = {loss, svref_e2e_from_alpha(a2, B, K)};
        spill(dir, "e2e.bin", e2e, sizeof e2e);
        int32_t *st = calloc(n, 4);
        double *sc = calloc(n, 8), *su = calloc(n, 8), *sR = calloc(n, 8);
        if (svref_sample_drafts(&p, draft, st, sc, su, sR)) return 3;
        spill(dir, "samp.bin", st, n * 4);
        free(t2); free(a2); free(grad); free(lr); free(st); free(sc); free(su); free(sR);
    }
    free(target); free(draft); free(tokens); free(dl);
    free(alpha); free(lse_t); free(lse_d); free(ratio); free(u_acc); free(u_corr); free(cdf_t); free(rm);
    free(accept); free(amax_t); free(amax_d); free(al); free(ot); free(nout); free(resid); free(al2);
    return 0;
}

static unsigned long long lcg = 88172645463325252ull;
static double rnd(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 11) * 0x1.0p-53;
}

static int run_budget(void) {
    for (int trial = 0; trial < 200; ++trial) {
        const int B = 1 + (int)(rnd() * 9), K = 1 + (int)(rnd() * 9);
        /* exact-size heap arrays, so that any access past them is reported */
        float *conf = malloc(sizeof(float) * B * K);
        int32_t *dl = malloc(sizeof(int32_t) * B);
        const int use_dl = rnd() < 0.5;
        for (int i = 0; i < B * K; ++i) conf[i] = rnd() < 0.15 ? 1.0f : (float)rnd();
        int sumL = 0;
        for (int r = 0; r < B; ++r) { dl[r] = use_dl ? (int)(rnd() * (K + 1)) : K; sumL += dl[r]; }
        const int N = (int)(rnd() * (B * K + 3));
        const int n = N < sumL ? N : sumL;
        int32_t *lens = malloc(sizeof(int32_t) * B), *off = malloc(sizeof(int32_t) * (B + 1));
        int32_t *rl = malloc(sizeof(int32_t) * (n > 0 ? n : 1));
        if (svref_alloc_verify_budget(conf, use_dl ? dl : NULL, B, K, N, lens, off, rl)) return 3;
        /* brute force: C by sequential binary32 products; rank every (r, k < L_r) by
         * (C desc, r asc, k asc) with a selection sort; keep the first min(N, sum L) */
        float Cv[100];
        int cand[100], nc = 0, keep[100] = {0};
        for (int r = 0; r < B; ++r) {
            float c = 1.0f;
            for (int k = 0; k < K; ++k) {
                c = c * conf[r * K + k];
                Cv[r * K + k] = c;
                if (k < dl[r]) cand[nc++] = r * K + k;
            }
        }
        for (int s = 0; s < n; ++s) {
            int best = -1;
            for (int i = 0; i < nc; ++i) {
                const int x = cand[i];
                if (keep[x]) continue;
                if (best < 0 || Cv[x] > Cv[best] || (Cv[x] == Cv[best] && x < best)) best = x;
            }
            keep[best] = 1;
        }
        int pos = 0;
        for (int r = 0; r < B; ++r) {
            int cnt = 0;
            if (off[r] != pos) return 7;
            for (int k = 0; k < K; ++k)
                if (keep[r * K + k]) {
                    if (rl[pos++] != r * K + k) return 7;
                    ++cnt;
                }
            if (lens[r] != cnt) return 7;
            for (int k = 0; k < cnt; ++k)   /* the kept rows of a request form a prefix */
                if (!keep[r * K + k]) return 8;
        }
        if (off[B] != n) return 7;
        free(conf); free(dl); free(lens); free(off); free(rl);
    }
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 3 && !strcmp(argv[1], "verify")) return run_verify(argv[2]);
    if (argc == 2 && !strcmp(argv[1], "budget")) return run_budget();
    fprintf(stderr, "usage: %s verify <dir> | budget\n", argv[0]);
    return 2;
}
