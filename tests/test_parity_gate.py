"""The verification comparison (tests/parity.py) that every GPU parity test goes through,
pinned on the CPU: the oracle's own outputs pass it, each planted mistake fails it, and the
near-threshold bands admit what they are stated to admit and nothing wider."""
import copy

import numpy as np
import pytest

import parity
from oracle import svref
from parity import ACCEPT_BAND, CDF_BAND, compare_verify

OUT_KEYS = ("alpha", "accept", "lse_t", "lse_d", "amax_t", "amax_d", "accept_len", "out_tokens", "n_out")


@pytest.fixture(autouse=True)
def _keep_session_report():
    """These comparisons are synthetic: their counts stay out of the session's parity report."""
    n = len(parity.REPORTS)
    yield
    del parity.REPORTS[n:]


def _case(T, seed=5, B=8, K=5, V=300, draft_len=None):
    rng = np.random.default_rng(seed)
    t = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d = (t[:, :K] + 0.7 * rng.standard_normal((B, K, V))).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[:, 0] = np.argmax(d[:, 0], -1)   # some early accepts
    o = svref.verify_batch(t, d, x, T, "f32", seed=seed, draft_len=draft_len, diagnostics=True)
    gpu = {k: o[k].copy() for k in OUT_KEYS}
    return t, d, o, gpu


def _rejected(o):
    """A request that rejected a draft (its emitted token is a correction)."""
    r = [i for i in range(o["accept_len"].shape[0]) if o["accept_len"][i] < o["alpha"].shape[1]]
    assert r
    return r[0]


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_oracle_outputs_pass(T):
    t, d, o, gpu = _case(T)
    rep = compare_verify(gpu, o, t, d, "f32", T)
    assert rep["requests"] == 8 and rep["token_equal"] == 8
    assert rep["near_accept"] == 0 and rep["near_token"] == 0


def _mutations(o):
    r = _rejected(o)
    tau = int(o["accept_len"][r])
    V = 300

    def alpha(g):
        g["alpha"][r, 0] *= 1 + 1e-4

    def lse(g):
        g["lse_t"][r, 1] *= 1 + 1e-4

    def amax(g):
        g["amax_d"][r, 2] = (g["amax_d"][r, 2] + 1) % V

    def accept_far(g):
        # a flag whose draw lies far from its threshold
        k = int(np.argmax(np.abs(o["u_acc"][r] - o["ratio"][r])))
        g["accept"][r, k] ^= 1

    def n_out(g):
        g["n_out"][r] += 1

    def tail(g):
        g["out_tokens"][r, tau + 1] = 0   # past the emitted tokens: must stay -1

    def prefix(g):
        if tau > 0:
            g["out_tokens"][r, 0] = (g["out_tokens"][r, 0] + 1) % V
        else:
            g["accept_len"][r] += 1

    def token_far(g):
        # a correction token half the vocabulary away from the oracle's along the CDF
        g["out_tokens"][r, tau] = (int(g["out_tokens"][r, tau]) + V // 2) % V

    return dict(alpha=alpha, lse=lse, amax=amax, accept_far=accept_far, n_out=n_out, tail=tail,
                prefix=prefix, token_far=token_far)


@pytest.mark.parametrize("name", ["alpha", "lse", "amax", "accept_far", "n_out", "tail", "prefix",
                                  "token_far"])
def test_planted_mistake_fails(name):
    t, d, o, gpu = _case(0.9)
    _mutations(o)[name](gpu)
    with pytest.raises(AssertionError):
        compare_verify(gpu, o, t, d, "f32", 0.9)


def test_greedy_token_must_match():
    t, d, o, gpu = _case(0.0)
    r = _rejected(o)
    tau = int(o["accept_len"][r])
    gpu["out_tokens"][r, tau] = (gpu["out_tokens"][r, tau] + 1) % 300
    with pytest.raises(AssertionError):
        compare_verify(gpu, o, t, d, "f32", 0.0)


def test_unverified_tail_must_hold_the_fill_values():
    L = np.array([5, 3, 0, 5, 2, 5, 1, 4], np.int32)
    t, d, o, gpu = _case(0.9, draft_len=L)
    compare_verify(gpu, o, t, d, "f32", 0.9, L=L)
    bad = copy.deepcopy(gpu)
    bad["alpha"][1, 4] = 0.5   # request 1 verifies 3 positions
    with pytest.raises(AssertionError):
        compare_verify(bad, o, t, d, "f32", 0.9, L=L)


@pytest.mark.parametrize("margin,admitted", [(0.5 * ACCEPT_BAND, True), (2.0 * ACCEPT_BAND, False)])
def test_accept_band(margin, admitted):
    """A flipped flag passes only where the oracle's uniform lies within ACCEPT_BAND of p/q:
    the oracle's diagnostic uniform is moved next to the ratio by hand."""
    t, d, o, gpu = _case(0.9)
    r = _rejected(o)
    k = 0
    o = copy.deepcopy(o)
    o["u_acc"][r, k] = o["ratio"][r, k] - margin
    gpu["accept"][r, k] ^= 1
    if admitted:
        rep = compare_verify(gpu, o, t, d, "f32", 0.9)
        assert rep["near_accept"] == 1
    else:
        with pytest.raises(AssertionError):
            compare_verify(gpu, o, t, d, "f32", 0.9)


@pytest.mark.parametrize("margin,admitted", [(0.5 * CDF_BAND, True), (2.0 * CDF_BAND, False)])
def test_cdf_band(margin, admitted):
    """The next token passes only where the oracle's CDF target u R lies within CDF_BAND * R
    below the boundary between the two tokens: the target is moved there by hand (the drawn
    token stays the oracle's, its weight being larger than the move)."""
    t, d, o, gpu = _case(0.9)
    r = _rejected(o)
    tau = int(o["accept_len"][r])
    to = int(o["out_tokens"][r, tau])
    R = o["resid_mass"][r]
    hi = svref.correction_cdf(t, d, 0.9, "f32", r, tau, 5, to)
    lo = svref.correction_cdf(t, d, 0.9, "f32", r, tau, 5, to - 1) if to > 0 else 0.0
    assert hi - lo > 2.0 * CDF_BAND * R and to + 1 < t.shape[-1]
    o = copy.deepcopy(o)
    o["cdf_target"][r] = hi - margin * R
    gpu["out_tokens"][r, tau] = to + 1
    if admitted:
        rep = compare_verify(gpu, o, t, d, "f32", 0.9)
        assert rep["near_token"] == 1
    else:
        with pytest.raises(AssertionError):
            compare_verify(gpu, o, t, d, "f32", 0.9)
