"""Element-by-element comparison of GPU verification outputs with the CPU oracle.

Tolerances (from the stated goal for this path):
  * greedy mode: accept flags, accepted lengths, emitted tokens, argmax -- bit-exact;
  * stochastic accept flags: bit-exact unless the oracle's draw lies within 1e-6 of the
    threshold p(x)/q(x); such requests are counted and their tokens are not compared;
  * correction / bonus tokens: bit-exact unless the oracle's CDF target u*R lies within
    1e-6*R of every CDF boundary between the two tokens; counted;
  * alpha, log-normalisers: 1e-5 relative (binary32 accumulation).  alpha is a sum of V
    binary32 exponentials, and the exponential flushes results below the binary32 normal
    range (2^-126) to zero, so alpha also carries an absolute error of at most V * 2^-126;
    that is its only absolute floor (it matters only for overlaps below ~1e-30);
  * the L_e2e gradient: see compare_grad.

Every comparison adds its counts to REPORTS; the test session prints their totals (the
near-threshold counts the goal asks to be reported), and compare_verify fails when they
exceed what the bands can explain (near_accept_max, near_token_max).
"""
import numpy as np

from oracle import svref

ACCEPT_BAND = 1e-6
CDF_BAND = 1e-6
REL_TOL = 1e-5
FLUSH = 2.0 ** -126

REPORTS = []


def near_accept_max(tests):
    """A flag may differ only where the oracle's uniform lies within ACCEPT_BAND of the ratio
    p(x)/q(x): probability 2e-6 per test, so even one is rare; one per call (plus one per 1000
    tests) is allowed before the count itself fails the comparison."""
    return 1 + tests // 1000


def near_token_max(compared):
    """A token may differ only where u R lies within CDF_BAND * R of a boundary between the two
    tokens; the boundary next to the target moves by the binary32 rounding of the weights and
    of the range masses (~1e-7 R), against a spacing of the drawn token's weight (~R / V on
    average).  Up to a tenth of the compared draws (at least two) is allowed."""
    return max(2, compared // 10)


def compare_verify(gpu, ora, target_np, draft_np, dtype, T, check=None, L=None, label=""):
    """gpu/ora: dicts of numpy arrays.  check: request indices to compare (default all).
    Returns a report dict; raises AssertionError on any mismatch outside the bands."""
    B, K = ora["alpha"].shape
    reqs = range(B) if check is None else check
    rep = dict(requests=0, near_accept=0, near_token=0, token_equal=0, accept_tests=0)
    for r in reqs:
        rep["requests"] += 1
        Lr = K if L is None else int(L[r])
        ks = slice(0, Lr)
        # alpha and lse within REL_TOL; unverified tail exactly the fill values
        V = target_np.shape[-1]
        np.testing.assert_allclose(gpu["alpha"][r, ks], ora["alpha"][r, ks], rtol=REL_TOL, atol=V * FLUSH,
                                   err_msg=f"alpha r={r}")
        rep["accept_tests"] += Lr
        assert (gpu["alpha"][r, Lr:] == 0).all() and (gpu["accept"][r, Lr:] == 0).all()
        if T > 0 and gpu.get("lse_t") is not None:
            np.testing.assert_allclose(gpu["lse_t"][r, ks], ora["lse_t"][r, ks], rtol=REL_TOL, err_msg=f"lse_t r={r}")
            np.testing.assert_allclose(gpu["lse_d"][r, ks], ora["lse_d"][r, ks], rtol=REL_TOL, err_msg=f"lse_d r={r}")
        if gpu.get("amax_t") is not None:
            assert (gpu["amax_t"][r, ks] == ora["amax_t"][r, ks]).all(), f"amax_t r={r}"
            assert (gpu["amax_d"][r, ks] == ora["amax_d"][r, ks]).all(), f"amax_d r={r}"
        acc_g, acc_o = gpu["accept"][r, ks], ora["accept"][r, ks]
        if T == 0:
            assert (acc_g == acc_o).all(), f"greedy accept r={r}"
        else:
            diff = np.nonzero(acc_g != acc_o)[0]
            if len(diff):
                margin = np.abs(ora["u_acc"][r, diff] - ora["ratio"][r, diff])
                assert (margin < ACCEPT_BAND).all(), f"accept r={r} k={diff} margin={margin}"
                rep["near_accept"] += 1
                continue
        assert gpu["accept_len"][r] == ora["accept_len"][r], f"tau r={r}"
        assert gpu["n_out"][r] == ora["n_out"][r]
        tau = int(ora["accept_len"][r])
        assert (gpu["out_tokens"][r, :tau] == ora["out_tokens"][r, :tau]).all()
        assert (gpu["out_tokens"][r, tau + 1:] == -1).all()
        tg, to = int(gpu["out_tokens"][r, tau]), int(ora["out_tokens"][r, tau])
        if tg == to:
            rep["token_equal"] += 1
            continue
        assert T > 0, f"greedy token r={r}: gpu {tg} oracle {to}"
        t, R = ora["cdf_target"][r], ora["resid_mass"][r]
        assert 0 <= tg < target_np.shape[-1]
        if tg > to:
            far = svref.correction_cdf(target_np, draft_np, T, dtype, r, tau, Lr, tg - 1)
            gap = far - t
        else:
            far = svref.correction_cdf(target_np, draft_np, T, dtype, r, tau, Lr, tg)
            gap = t - far
        assert 0 <= gap <= CDF_BAND * R, f"token r={r}: gpu {tg} oracle {to}, gap {gap} R {R}"
        rep["near_token"] += 1
    assert rep["near_accept"] <= near_accept_max(rep["accept_tests"]), rep
    compared = rep["requests"] - rep["near_accept"]
    assert rep["near_token"] <= near_token_max(compared), rep
    REPORTS.append(dict(rep, label=label))
    return rep


# ---- gradient of L_e2e in the drafter logits ------------------------------------------
# An element is g = s q ([q < p] - beta).  Its own arithmetic (q = 2^x from one fma, the
# products) is held to GRAD_RTOL relative.  beta is a sum over the whole row; its binary32
# rounding (~1e-7 relative) reaches every element of the row as s q dbeta, bounded by
# GRAD_ROW_ATOL times the row's largest |g|.  Where |ln p - ln q| < TIE_BAND the comparison
# q < p may fall either way in binary32; those elements are counted, checked finite, and not
# compared.  bfloat16 gradients add their rounding (half an ulp, 2^-9 relative).  Below the
# binary32 normal range (2^-126) the kernels' exponential flushes q to zero, so an element is
# also allowed an absolute error of GRAD_FLOOR = 2^-126 times a bound (2^6) on the row scale
# |s| = |grad_loss| w / (|I| D T) of the test cases.
# beta also depends on which side of the tie a token falls: the kernels decide q < p on
# binary32 log-values (errors of a few 1e-6 in ln), so a token with |ln p - ln q| below
# BETA_BAND (about twice that) may be counted in beta or not.  Given ln q, each row's beta is
# allowed to move by the q-mass of those tokens: element v by |s q_v| times that mass, with
# |s q_v| = |g_v| / |[q_v < p_v] - beta|.
GRAD_RTOL = 1e-5
GRAD_ROW_ATOL = 2e-6
GRAD_FLOOR = 2.0 ** -120
TIE_BAND = 1e-4
BETA_BAND = 1e-5


def drafter_log_q(d, T):
    """ln q (binary64) of drafter logits d (a torch tensor [..., V]) at temperature T, for the
    tie band of beta in compare_grad."""
    from scipy.special import log_softmax
    return log_softmax(d.detach().double().cpu().numpy() / T, axis=-1)


def compare_grad(gpu, ora, log_ratio, rtol=GRAD_RTOL, bf16=False, log_q=None):
    """gpu, ora, log_ratio (ln p - ln q), log_q (ln q, optional): [..., V] arrays.  Returns a
    report; raises AssertionError."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(ora, np.float64)
    ties = np.abs(log_ratio) < TIE_BAND
    assert np.isfinite(g).all(), "non-finite gradient"
    row_max = np.abs(o).max(-1, keepdims=True)
    tol = (rtol + (2.0 ** -8 if bf16 else 0.0)) * np.abs(o) + GRAD_ROW_ATOL * row_max + GRAD_FLOOR
    band_rows = 0
    if log_q is not None:
        q = np.exp(np.asarray(log_q, np.float64))
        with np.errstate(invalid="ignore"):
            ind = (log_ratio > 0).astype(np.float64)
            near = np.abs(log_ratio) < BETA_BAND
        beta = (q * ind).sum(-1, keepdims=True)
        band = (q * near).sum(-1, keepdims=True)
        sq = np.abs(o) / np.maximum(np.abs(ind - beta), 1e-300)
        tol = tol + sq * band
        band_rows = int((band > 0).sum())
    bad = (np.abs(g - o) > tol) & ~ties
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"gradient mismatch at {tuple(i)}: gpu {g[tuple(i)]!r} oracle {o[tuple(i)]!r} "
                             f"({int(bad.sum())} elements)")
    normal = ~ties & (np.abs(o) >= 2.0 ** -100)   # relative error where binary32 carries it
    rel = np.abs(g - o)[normal] / np.abs(o)[normal]
    return {"elements": int(o.size), "ties": int(ties.sum()), "below_normal": int((~ties & ~normal).sum()),
            "beta_band_rows": band_rows, "max_rel": float(rel.max()) if rel.size else 0.0}
