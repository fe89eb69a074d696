"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a published generator,
a library routine, a closed form, an invariant of the definitions, a statistical law that
the method must satisfy, or brute force on tiny inputs.
"""
import itertools

import numpy as np
import pytest
from scipy import special, stats

from oracle import svref

RNG = np.random.default_rng(12345)


def _logits(shape, scale=2.0, rng=RNG):
    return (scale * rng.standard_normal(shape)).astype(np.float32)


# ---------------------------------------------------------------------------------------
# Philox4x64-10: known answers from numpy's independent implementation (numpy advances the
# counter once before its first block) and the Random123 zero vector.
# ---------------------------------------------------------------------------------------

def test_philox_zero_vector():
    out = svref.philox4x64_10([0, 0, 0, 0], [0, 0])
    assert [int(x) for x in out] == [0x16554D9ECA36314C, 0xDB20FE9D672D0FDC,
                                     0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]


@pytest.mark.parametrize("trial", range(8))
def test_philox_matches_numpy(trial):
    rng = np.random.default_rng(trial)
    ctr = [int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.int64)]
    key = [int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.int64)]
    bg = np.random.Philox(counter=ctr, key=key)
    want = bg.random_raw(8)
    got0 = svref.philox4x64_10([ctr[0] + 1] + ctr[1:], key)
    got1 = svref.philox4x64_10([ctr[0] + 2] + ctr[1:], key)
    assert list(got0) == list(want[:4])
    assert list(got1) == list(want[4:])


def test_uniform_is_top_24_bits_of_word0():
    for c in [(0, 0, 0, 0), (3, 7, 1, 11), (63, 15, 0, 2**40)]:
        w0 = int(svref.philox4x64_10(list(c), [42, 0])[0])
        u = svref.uniform(42, *c)
        assert u == (w0 >> 40) / 2.0**24
        assert 0.0 <= u < 1.0
        assert np.float32(u) == u  # exactly representable in binary32


# ---------------------------------------------------------------------------------------
# Softmax, argmax, overlap (overlap equation: alpha = sum min(p, q) = 1 - TV)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.5, 0.9, 1.0, 2.0])
def test_lse_matches_scipy(T):
    z = _logits(1000, 3.0)
    assert svref.row_lse(z, "f32", T) == pytest.approx(special.logsumexp(z.astype(np.float64) / T), rel=1e-13)


def test_lse_bf16_widening_is_exact():
    z = _logits(4096, 3.0)
    bits = (z.view(np.uint32) >> 16).astype(np.uint16)  # truncation gives valid bf16 values
    widened = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert svref.row_lse(bits, "bf16", 0.9) == pytest.approx(special.logsumexp(widened / 0.9), rel=1e-13)


def test_lse_with_minus_inf_entries():
    z = _logits(64)
    z[::3] = -np.inf
    assert svref.row_lse(z, "f32", 1.0) == pytest.approx(special.logsumexp(z[np.isfinite(z)].astype(np.float64)), rel=1e-13)


def test_argmax_lowest_index_on_ties():
    rng = np.random.default_rng(7)
    for _ in range(200):
        z = rng.integers(-3, 4, size=50).astype(np.float32)  # many ties
        assert svref.row_argmax(z, "f32") == int(np.argmax(z))  # numpy: first occurrence


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_alpha_plus_tv_is_one(T):
    for _ in range(20):
        zt, zd = _logits(300), _logits(300)
        p = special.softmax(zt.astype(np.float64) / T)
        q = special.softmax(zd.astype(np.float64) / T)
        tv = 0.5 * np.abs(p - q).sum()
        assert svref.alpha(zt, zd, "f32", T) + tv == pytest.approx(1.0, abs=1e-12)


def test_alpha_identity_symmetry_disjoint():
    zt, zd = _logits(500), _logits(500)
    assert svref.alpha(zt, zt, "f32", 0.9) == pytest.approx(1.0, abs=1e-12)
    assert svref.alpha(zt, zd, "f32", 0.9) == pytest.approx(svref.alpha(zd, zt, "f32", 0.9), abs=1e-15)
    a, b = zt.copy(), zd.copy()
    a[:250] = -np.inf
    b[250:] = -np.inf
    assert svref.alpha(a, b, "f32", 1.0) == 0.0


# ---------------------------------------------------------------------------------------
# Verification statistics: serial acceptance gives E[tau] = sum_m prod_{k<=m} alpha_k, and
# rejection sampling with the residual/bonus draw leaves the target distribution intact.
# ---------------------------------------------------------------------------------------

def _mc_batch(B, K, V, T, seed, scale_t=1.5, noise=1.0):
    rng = np.random.default_rng(seed)
    zt = _logits((K + 1, V), scale_t, rng)
    zd = (zt[:K] + noise * rng.standard_normal((K, V))).astype(np.float32)
    q = special.softmax(zd.astype(np.float64) / T, axis=-1)
    # the drafter samples its own tokens: x_{r,k} ~ q_k, independently per request
    toks = np.stack([rng.choice(V, size=B, p=q[k]) for k in range(K)], axis=1).astype(np.int32)
    target = np.broadcast_to(zt, (B, K + 1, V)).copy()
    draft = np.broadcast_to(zd, (B, K, V)).copy()
    return zt, zd, target, draft, toks


@pytest.mark.parametrize("T", [0.9, 1.3])
def test_expected_accept_len_closed_form(T):
    B, K, V = 100_000, 3, 12
    zt, zd, target, draft, toks = _mc_batch(B, K, V, T, seed=11)
    out = svref.verify_batch(target, draft, toks, T, "f32", seed=5, step=3)
    a = np.array([svref.alpha(zt[k], zd[k], "f32", T) for k in range(K)])
    closed = sum(np.prod(a[: m + 1]) for m in range(K))
    tau = out["accept_len"].astype(np.float64)
    se = tau.std() / np.sqrt(B)
    assert abs(tau.mean() - closed) < 4 * se, (tau.mean(), closed, se)
    # per-position acceptance: P(accept_k) = alpha_k, independent of the other positions
    acc = out["accept"].astype(np.float64)
    for k in range(K):
        assert abs(acc[:, k].mean() - a[k]) < 4 * np.sqrt(a[k] * (1 - a[k]) / B)
    # oracle alpha equals the standalone definition
    np.testing.assert_allclose(out["alpha"][0], a, rtol=1e-14)
    # 1 - L_e2e = E[tau] / D: ties the end-to-end objective to the serial acceptance law
    loss, _ = svref.tv_e2e_loss(zt[None, :K].copy(), zd[None].copy(), T, "f32")
    assert abs((1.0 - loss) - tau.mean() / K) < 4 * se / K


def _chi2_ok(counts, probs, min_p=1e-3):
    n = counts.sum()
    exp = probs * n
    keep = exp > 5
    obs = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        obs, e = obs[:-1], e[:-1]
    stat, pval = stats.chisquare(obs, e * obs.sum() / e.sum())
    return pval > min_p, pval


@pytest.mark.parametrize("T", [0.9, 1.0])
def test_emitted_tokens_follow_target(T):
    """Token j of the output, given tau >= j, is distributed as p_j (rows 0..K)."""
    B, K, V = 200_000, 2, 8
    zt, zd, target, draft, toks = _mc_batch(B, K, V, T, seed=21)
    out = svref.verify_batch(target, draft, toks, T, "f32", seed=9, step=1)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    tau, ot = out["accept_len"], out["out_tokens"]
    for j in range(K + 1):
        sel = tau >= j
        counts = np.bincount(ot[sel, j], minlength=V).astype(np.float64)
        ok, pval = _chi2_ok(counts, p[j])
        assert ok, (j, pval)


def test_correction_token_follows_residual():
    """Given a rejection at position 0, the correction is norm(max(p0 - q0, 0))."""
    B, K, V, T = 200_000, 1, 8, 1.0
    zt, zd, target, draft, toks = _mc_batch(B, K, V, T, seed=31, noise=1.5)
    out = svref.verify_batch(target, draft, toks, T, "f32", seed=2, step=0)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    q = special.softmax(zd.astype(np.float64) / T, axis=-1)
    w = np.maximum(p[0] - q[0], 0.0)
    sel = out["accept_len"] == 0
    counts = np.bincount(out["out_tokens"][sel, 0], minlength=V).astype(np.float64)
    assert counts[w == 0].sum() == 0
    ok, pval = _chi2_ok(counts, w / w.sum())
    assert ok, pval


def test_inverse_cdf_is_searchsorted():
    """The draw is the smallest v with sum_{j<=v} w_j > u R (numpy searchsorted, right)."""
    B, K, V, T = 64, 1, 20, 1.0
    zt, zd, target, draft, toks = _mc_batch(B, K, V, T, seed=41)
    out = svref.verify_batch(target, draft, toks, T, "f32", seed=77, step=5, diagnostics=True)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    q = special.softmax(zd.astype(np.float64) / T, axis=-1)
    for r in range(B):
        tau = out["accept_len"][r]
        w = np.maximum(p[0] - q[0], 0) if tau == 0 else p[1]
        u = svref.uniform(77, r, tau, 1, 5)
        assert out["u_corr"][r] == u
        cw = np.cumsum(w)
        assert out["out_tokens"][r, tau] == int(np.searchsorted(cw, u * cw[-1], side="right"))


def _widen_bf16(u16):
    """bfloat16 bit patterns to float64 (the upper half of a binary32), independently of the
    oracle's own widening."""
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.9, 1.7])
def test_correction_cdf_is_cumsum_of_the_draw_weights(dtype, T):
    """svref_correction_cdf (the parity checker's CDF-band test reads it) is the running sum
    of the draw's weights: max(p_tau - q_tau, 0) after a rejection at tau < L_r, p at target
    row L_r for the bonus token (the standard speculative-sampling rule that keeps the target
    distribution).  Checked against scipy's softmax and numpy's cumsum at v = -1 (empty sum),
    0, interior points and V - 1 (the total), for several rows, so a wrong row, wrong weights
    (no clamp, q - p, p alone after a rejection) or an off-by-one in v fails."""
    B, K, V = 3, 4, 257
    rng = np.random.default_rng(71)
    zt = (2.5 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    zt[1, 2, 100:140] = -np.inf   # masked logits (p = 0 there)
    if dtype == "bf16":
        t16 = (zt.view(np.uint32) >> 16).astype(np.uint16)
        d16 = (zd.view(np.uint32) >> 16).astype(np.uint16)
        target, draft = t16, d16
        zt64, zd64 = _widen_bf16(t16), _widen_bf16(d16)
    else:
        target, draft = zt, zd
        zt64, zd64 = zt.astype(np.float64), zd.astype(np.float64)
    p = special.softmax(zt64 / T, axis=-1)
    q = special.softmax(zd64 / T, axis=-1)
    for r, tau, L in [(0, 0, 4), (0, 3, 4), (1, 2, 4), (2, 1, 2), (0, 4, 4), (1, 2, 2), (2, 0, 0)]:
        w = np.maximum(p[r, tau] - q[r, tau], 0.0) if tau < L else p[r, tau]
        cw = np.cumsum(w)
        for v in [-1, 0, 1, 57, 99, 120, 200, V - 2, V - 1]:
            want = 0.0 if v < 0 else cw[v]
            got = svref.correction_cdf(target, draft, T, dtype, r, tau, L, v)
            assert got == pytest.approx(want, rel=1e-12, abs=1e-15), (r, tau, L, v)
    # outside the domain: NaN
    assert np.isnan(svref.correction_cdf(target, draft, T, dtype, 0, 3, 2, 0))     # tau > L_r
    assert np.isnan(svref.correction_cdf(target, draft, T, dtype, 0, 0, 4, V))     # v >= V


def test_correction_cdf_brackets_every_drawn_token():
    """At every request of a verification, the drawn token x is the smallest v whose
    cumulative weight exceeds the draw's target u R: cdf(x - 1) <= u R < cdf(x), with the
    target and total mass the oracle reports (the band the parity checker uses)."""
    B, K, V, T = 40, 3, 300, 0.9
    rng = np.random.default_rng(72)
    zt = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + 1.2 * rng.standard_normal((B, K, V))).astype(np.float32)
    qd = special.softmax(zd.astype(np.float64) / T, axis=-1)
    toks = np.array([[rng.choice(V, p=qd[r, k]) for k in range(K)] for r in range(B)], np.int32)
    out = svref.verify_batch(zt, zd, toks, T, "f32", seed=8, step=2, diagnostics=True)
    p = special.softmax(zt.astype(np.float64) / T, axis=-1)
    q = special.softmax(zd.astype(np.float64) / T, axis=-1)
    for r in range(B):
        tau = int(out["accept_len"][r])
        x = int(out["out_tokens"][r, tau])
        w = np.maximum(p[r, tau] - q[r, tau], 0.0) if tau < K else p[r, tau]
        assert out["resid_mass"][r] == pytest.approx(w.sum(), rel=1e-12)
        t = out["cdf_target"][r]
        lo = svref.correction_cdf(zt, zd, T, "f32", r, tau, K, x - 1)
        hi = svref.correction_cdf(zt, zd, T, "f32", r, tau, K, x)
        assert lo <= t < hi, (r, tau, x, lo, t, hi)


def test_greedy_accept_len_is_argmax_match_prefix():
    rng = np.random.default_rng(5)
    B, K, V = 300, 5, 40
    target = rng.integers(-4, 5, size=(B, K + 1, V)).astype(np.float32)  # ties are frequent
    draft = target[:, :K] + rng.integers(-1, 2, size=(B, K, V)).astype(np.float32)
    toks = np.argmax(draft, axis=-1).astype(np.int32)
    out = svref.verify_batch(target, draft, toks, 0.0, "f32")
    amax_t = np.argmax(target, axis=-1)
    for r in range(B):
        match = toks[r] == amax_t[r, :K]
        tau = K if match.all() else int(np.argmin(match))
        assert out["accept_len"][r] == tau
        assert out["n_out"][r] == tau + 1
        assert list(out["out_tokens"][r, :tau]) == list(toks[r, :tau])
        assert out["out_tokens"][r, tau] == amax_t[r, tau]
        assert (out["out_tokens"][r, tau + 1:] == -1).all()
        np.testing.assert_array_equal(out["alpha"][r], (amax_t[r, :K] == np.argmax(draft[r], -1)).astype(float))


def test_draft_len_masks_positions():
    B, K, V, T = 32, 4, 30, 0.9
    rng = np.random.default_rng(3)
    zt = _logits((B, K + 1, V), 2.0, rng)
    zd = (zt[:, :K] + 0.3 * rng.standard_normal((B, K, V))).astype(np.float32)
    toks = np.argmax(zd, -1).astype(np.int32)
    dl = rng.integers(0, K + 1, size=B).astype(np.int32)
    out = svref.verify_batch(zt, zd, toks, T, "f32", seed=1, draft_len=dl)
    for r in range(B):
        assert out["accept_len"][r] <= dl[r]
        assert (out["alpha"][r, dl[r]:] == 0).all() and (out["accept"][r, dl[r]:] == 0).all()
        assert (out["alpha"][r, :dl[r]] > 0).all()
    # a request with L_r = 0 gets exactly its bonus token, drawn from p at row 0
    assert (out["n_out"][dl == 0] == 1).all()


def test_accept_len_and_residual_sample_agree_with_verify():
    B, K, V, T = 40, 3, 50, 0.9
    rng = np.random.default_rng(8)
    zt = _logits((B, K + 1, V), 2.0, rng)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = np.argmax(zd, -1).astype(np.int32)
    dl = rng.integers(0, K + 1, size=B).astype(np.int32)
    out = svref.verify_batch(zt, zd, toks, T, "f32", seed=4, step=2, draft_len=dl)
    assert (svref.accept_len(out["accept"], dl) == out["accept_len"]).all()
    tok = svref.residual_sample(zt, zd, out["accept_len"], T, "f32", seed=4, step=2, draft_len=dl)
    assert (tok == out["out_tokens"][np.arange(B), out["accept_len"]]).all()


def test_accept_len_first_reject():
    rng = np.random.default_rng(1)
    acc = (rng.random((500, 7)) < 0.7).astype(np.uint8)
    got = svref.accept_len(acc)
    want = np.where(acc.all(1), 7, np.argmin(acc, axis=1))
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------------------------
# End-to-end TV objective: closed forms of the L_e2e equation
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("a,D", [(0.3, 3), (0.75, 5), (0.5, 1), (0.9, 16)])
def test_e2e_constant_alpha(a, D):
    alpha = np.full((17, D), a)
    want = 1.0 - sum(a ** (m + 1) for m in range(D)) / D
    assert svref.e2e_from_alpha(alpha) == pytest.approx(want, abs=1e-14)


def test_e2e_special_cases():
    rng = np.random.default_rng(2)
    a = rng.random((100, 1))
    assert svref.e2e_from_alpha(a) == pytest.approx(1.0 - a.mean(), abs=1e-14)
    assert svref.e2e_from_alpha(np.ones((9, 4))) == 0.0
    assert svref.e2e_from_alpha(np.zeros((9, 4))) == 1.0
    # a rejection at depth 0 voids the rest: alpha_{i,0} = 0 makes row i contribute 0
    b = rng.random((10, 3))
    b[:, 0] = 0.0
    assert svref.e2e_from_alpha(b) == 1.0


# ---------------------------------------------------------------------------------------
# L_e2e gradient in the draft logits: central differences of the forward oracle, a
# two-token closed form, and the shift invariance of the softmax
# ---------------------------------------------------------------------------------------

def _kink_free_case(I, D, V, T, seed, margin=0.05):
    """Logits on a 2^-6 grid with every |ln p - ln q| above `margin`, so that no small
    perturbation of a drafter logit flips a comparison inside min(p, q)."""
    for s in range(seed, seed + 500):
        rng = np.random.default_rng(s)
        t = (np.round(rng.normal(scale=1.5, size=(I, D, V)) * 64) / 64).astype(np.float32)
        d = (np.round(rng.normal(scale=1.5, size=(I, D, V)) * 64) / 64).astype(np.float32)
        lr = svref.tv_e2e_backward(t, d, T, "f32", want_log_ratio=True)[3]
        if np.abs(lr).min() > margin:
            return t, d
    raise AssertionError("no kink-free case found")


@pytest.mark.parametrize("T,seed", [(0.7, 0), (1.3, 100)])
def test_e2e_grad_matches_central_differences(T, seed):
    I, D, V = 2, 3, 6
    t, d = _kink_free_case(I, D, V, T, seed)
    g, _, loss = svref.tv_e2e_backward(t, d, T, "f32", grad_loss=2.5)
    assert loss == pytest.approx(svref.tv_e2e_loss(t, d, T, "f32")[0], abs=1e-15)
    h = 2.0 ** -10   # exact on the 2^-6 grid; moves ln q by < 0.005, far below the margin
    fd = np.zeros_like(g)
    for idx in itertools.product(range(I), range(D), range(V)):
        dp, dm = d.copy(), d.copy()
        dp[idx] += h
        dm[idx] -= h
        fd[idx] = (svref.tv_e2e_loss(t, dp, T, "f32")[0] - svref.tv_e2e_loss(t, dm, T, "f32")[0]) / (2 * h)
    # central differences: error ~ h^2 / 6 times the third derivative
    np.testing.assert_allclose(g, 2.5 * fd, rtol=1e-5, atol=2e-7)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_e2e_grad_two_tokens_closed_form(T):
    # V = 2, one position: L = 1 - alpha = |p_0 - q_0|, so dL/dz^d_0 = sign(q_0 - p_0) q_0 q_1 / T
    rng = np.random.default_rng(7)
    for _ in range(20):
        t = rng.normal(size=(1, 1, 2)).astype(np.float32)
        d = rng.normal(size=(1, 1, 2)).astype(np.float32)
        p = special.softmax(t[0, 0].astype(np.float64) / T)
        q = special.softmax(d[0, 0].astype(np.float64) / T)
        g, a, loss = svref.tv_e2e_backward(t, d, T, "f32")
        assert loss == pytest.approx(abs(p[0] - q[0]), abs=1e-15)
        want = np.sign(q[0] - p[0]) * q[0] * q[1] / T
        assert g[0, 0, 0] == pytest.approx(want, rel=1e-12, abs=1e-300)
        assert g[0, 0, 1] == pytest.approx(-want, rel=1e-12, abs=1e-300)


def test_e2e_grad_rows_sum_to_zero():
    # adding a constant to a drafter row leaves q, hence the loss, unchanged
    t = _logits((3, 4, 1000))
    d = _logits((3, 4, 1000))
    g, _, _ = svref.tv_e2e_backward(t, d, 0.9, "f32")
    assert np.abs(g.sum(-1)).max() <= 1e-14 * np.abs(g).sum(-1).max()
    assert np.abs(g).max() > 0


def test_e2e_grad_zero_weight_after_a_certain_reject():
    # alpha_{i,0} = 0 (disjoint supports) gives positions k >= 1 of that sequence zero weight
    V = 8
    t = np.full((1, 3, V), -np.inf, np.float32)
    d = np.full((1, 3, V), -np.inf, np.float32)
    t[0, 0, :4] = _logits(4)
    d[0, 0, 4:] = _logits(4)
    t[0, 1:] = _logits((2, V))
    d[0, 1:] = _logits((2, V))
    g, a, _ = svref.tv_e2e_backward(t, d, 1.0, "f32")
    assert a[0, 0] == 0.0
    assert np.all(g[0, 1:] == 0.0)


# ---------------------------------------------------------------------------------------
# Draft tokens and confidences: the draw follows q, the confidence is q(x), the draw is a
# searchsorted inverse CDF keyed by the DRAFT counter, greedy takes the first maximum
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.7, 1.0])
def test_draft_tokens_follow_q(T):
    """Rows of identical logits draw independent uniforms (r, k differ): counts follow q."""
    B, K, V = 50_000, 2, 6
    z = _logits(V, rng=np.random.default_rng(31))
    d = np.broadcast_to(z, (B, K, V)).astype(np.float32).copy()
    tok, conf, _, _ = svref.sample_drafts(d, T, "f32", seed=4, step=2)
    q = special.softmax(z.astype(np.float64) / T)
    for k in range(K):
        counts = np.bincount(tok[:, k], minlength=V).astype(np.float64)
        ok, pval = _chi2_ok(counts, q)
        assert ok, (k, pval)
    np.testing.assert_allclose(conf, q[tok], rtol=1e-14)


@pytest.mark.parametrize("T", [0.0, 0.5, 1.3])
def test_draft_confidence_is_softmax_of_token(T):
    d = _logits((3, 4, 50), rng=np.random.default_rng(32))
    tok, conf, _, _ = svref.sample_drafts(d, T, "f32", seed=1, step=0)
    q = special.softmax(d.astype(np.float64) / (T if T > 0 else 1.0), axis=-1)
    want = np.take_along_axis(q, tok[..., None].astype(np.int64), -1)[..., 0]
    np.testing.assert_allclose(conf, want, rtol=1e-13)
    if T == 0:
        np.testing.assert_array_equal(tok, d.argmax(-1))


def test_draft_draw_is_searchsorted_on_the_draft_counter():
    B, K, V, T, seed, step = 8, 5, 40, 0.9, 123, 7
    d = _logits((B, K, V), rng=np.random.default_rng(33))
    tok, _, u, R = svref.sample_drafts(d, T, "f32", seed=seed, step=step)
    q = special.softmax(d.astype(np.float64) / T, axis=-1)
    for r in range(B):
        for k in range(K):
            assert u[r, k] == svref.uniform(seed, r, k, 2, step)      # purpose word 2
            assert u[r, k] != svref.uniform(seed, r, k, 1, step)
            cq = np.cumsum(q[r, k])
            assert R[r, k] == pytest.approx(1.0, abs=1e-12)
            assert tok[r, k] == int(np.searchsorted(cq, u[r, k] * R[r, k], side="right"))
            assert svref.draft_cdf(d, T, "f32", r, k, int(tok[r, k])) == pytest.approx(cq[tok[r, k]], abs=1e-13)


def test_draft_greedy_ties_take_lowest_index():
    d = np.zeros((1, 2, 9), np.float32)
    d[0, 0, [2, 5, 7]] = 3.0
    d[0, 1, [8, 1]] = -1.0
    d[0, 1, 4] = -1.0
    d[0, 1] -= 5.0
    d[0, 1, [1, 4, 8]] = 0.5
    tok, conf, _, _ = svref.sample_drafts(d, 0.0, "f32")
    assert tok.tolist() == [[2, 1]]
    q0 = special.softmax(d[0, 0].astype(np.float64))
    assert conf[0, 0] == pytest.approx(q0[2], rel=1e-14)


# ---------------------------------------------------------------------------------------
# Batch-level budget: the greedy selection is the best prefix allocation (brute force)
# ---------------------------------------------------------------------------------------

def _brute_best(C, N):
    B, K = C.shape
    total = min(N, B * K)
    best = -1.0
    for lens in itertools.product(range(K + 1), repeat=B):
        if sum(lens) != total:
            continue
        s = sum(float(C[r, :lens[r]].astype(np.float64).sum()) for r in range(B))
        best = max(best, s)
    return best


@pytest.mark.parametrize("trial", range(25))
def test_budget_matches_brute_force(trial):
    rng = np.random.default_rng(100 + trial)
    B, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    conf = rng.beta(5, 2, size=(B, K)).astype(np.float32)
    C = np.multiply.accumulate(conf, axis=1, dtype=np.float32)  # sequential binary32
    for N in range(0, B * K + 2):
        lens, off, rl = svref.alloc_verify_budget(conf, N)
        assert lens.sum() == min(N, B * K)
        assert (np.diff(off) == lens).all() and off[0] == 0
        got = sum(float(C[r, :lens[r]].astype(np.float64).sum()) for r in range(B))
        assert got == pytest.approx(_brute_best(C, N), abs=1e-6)
        # prefix-closed: every selected (r,k) has all k' < k selected
        want_rows = [r * K + k for r in range(B) for k in range(lens[r])]
        assert list(rl) == want_rows


def test_budget_edges_and_ties():
    conf = np.array([[0.5, 1.0, 0.5], [0.5, 0.5, 1.0]], np.float32)
    # C = [[.5,.5,.25],[.5,.25,.25]]; ties broken by request then position
    lens, off, _ = svref.alloc_verify_budget(conf, 3)
    assert list(lens) == [2, 1]
    lens, off, _ = svref.alloc_verify_budget(conf, 4)
    assert list(lens) == [3, 1]
    lens, _, _ = svref.alloc_verify_budget(conf, 0)
    assert list(lens) == [0, 0]
    lens, _, rl = svref.alloc_verify_budget(conf, 100)
    assert list(lens) == [3, 3] and len(rl) == 6
    dl = np.array([1, 3], np.int32)
    lens, _, _ = svref.alloc_verify_budget(conf, 100, draft_len=dl)
    assert list(lens) == [1, 3]


def test_budget_binary32_cumprod_is_sequential():
    conf = np.array([[0.9999999, 0.3333333, 0.7777777, 0.1234567, 0.999]], np.float32)
    C = np.float32(conf[0, 0])
    seq = [C]
    for c in conf[0, 1:]:
        C = np.float32(C * c)
        seq.append(C)
    # with N = k+1 exactly the first k+1 are chosen; compare against a second request
    # whose single confidence equals the k-th product bit for bit (tie -> lower r wins)
    for k in range(5):
        conf2 = np.zeros((2, 5), np.float32)
        conf2[0] = conf[0]
        conf2[1, 0] = seq[k]
        dl = np.array([5, 1], np.int32)
        lens, _, _ = svref.alloc_verify_budget(conf2, k + 1, draft_len=dl)
        assert list(lens) == [k + 1, 0]
        lens, _, _ = svref.alloc_verify_budget(conf2, k + 2, draft_len=dl)
        assert list(lens) == [k + 1, 1] or k == 4


# ---- D-cut budget choice from a cost table -------------------------------------------

def test_dcut_hand_example():
    # C = [[.9, .72, .36], [.6, .54, .486]]; E(n) = 2 + best n products; cost 1 + 0.2 n:
    # E/cost = 2, 2.417, 2.586, 2.6375, 2.644, 2.623, 2.548 -> n = 4
    conf = np.array([[0.9, 0.8, 0.5], [0.6, 0.9, 0.9]], np.float32)
    cost = np.array([1.0, 1.2, 1.4, 1.6, 1.8, 2.0, 2.2], np.float32)
    n, E, lens, off, rl = svref.dcut_budget(conf, cost)
    assert n == 4
    assert E == pytest.approx(2 + 0.9 + 0.72 + 0.6 + 0.54, abs=1e-6)
    assert list(lens) == [2, 2] and list(rl) == [0, 1, 3, 4]


@pytest.mark.parametrize("trial", range(20))
def test_dcut_matches_brute_force(trial):
    rng = np.random.default_rng(300 + trial)
    B, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.beta(5, 2, size=(B, K)).astype(np.float32)
    C = np.multiply.accumulate(conf, axis=1, dtype=np.float32)
    n_cost = int(rng.integers(1, B * K + 3))
    cost = (1.0 + rng.random(n_cost) * 3).astype(np.float32)
    cost[rng.random(n_cost) < 0.15] = [0.0, -1.0, np.inf, np.nan][trial % 4]   # never chosen
    best, best_ratio, best_E = None, None, None
    for n in range(0, min(n_cost - 1, B * K) + 1):
        if not (np.isfinite(cost[n]) and cost[n] > 0):
            continue
        E = B + _brute_best(C, n)
        ratio = E / float(cost[n])
        if best is None or ratio > best_ratio * (1 + 1e-12):
            best, best_ratio, best_E = n, ratio, E
    if best is None:
        best, best_E = 0, float(B)
    n, E, lens, off, rl = svref.dcut_budget(conf, cost)
    assert n == best
    assert E == pytest.approx(best_E, abs=1e-9)
    want_lens, _, _ = svref.alloc_verify_budget(conf, n)
    assert np.array_equal(lens, want_lens)


def test_dcut_special_cases():
    conf = np.full((3, 4), 0.9, np.float32)
    # a flat cost: every extra position adds expected tokens for free -> verify everything
    n, E, lens, _, _ = svref.dcut_budget(conf, np.ones(100, np.float32))
    assert n == 12 and list(lens) == [4, 4, 4]
    # a table shorter than the candidates caps the choice
    n, _, _, _, _ = svref.dcut_budget(conf, np.ones(6, np.float32))
    assert n == 5
    # cost growing faster than any gain: verify nothing (B tokens from the bonus rows)
    n, E, lens, _, _ = svref.dcut_budget(conf, np.array([1.0] + [100.0] * 12, np.float32))
    assert n == 0 and E == 3.0 and list(lens) == [0, 0, 0]
    # no usable entry at all
    n, E, _, _, _ = svref.dcut_budget(conf, np.array([0.0, np.nan, -2.0], np.float32))
    assert n == 0 and E == 3.0
    # draft_len bounds the candidates
    n, _, lens, _, _ = svref.dcut_budget(conf, np.ones(100, np.float32), draft_len=np.array([1, 0, 2], np.int32))
    assert n == 3 and list(lens) == [1, 0, 2]
