"""The gradient comparison's allowance for beta (tests/parity.py), on oracle gradients with beta
moved by hand: a token within BETA_BAND of a tie may be counted on either side, one outside
it may not."""
import numpy as np
import pytest
import torch

from oracle import svref
from parity import BETA_BAND, TIE_BAND, compare_grad, drafter_log_q


def _row_with_near_tie(delta, seed=3, V=2000, T=1.0):
    """Target and drafter rows (binary32, [1][1][V]) whose token `v` has ln p - ln q close to
    delta: d_v is set from the two normalisers, which it moves only slightly, three times."""
    g = torch.Generator().manual_seed(seed)
    t = 3.0 * torch.randn((1, 1, V), generator=g, dtype=torch.float64)
    d = t + 0.3 * torch.randn((1, 1, V), generator=g, dtype=torch.float64)
    v = int(torch.argsort(t.flatten(), descending=True)[V // 20])   # q_v of about 1e-3
    for _ in range(3):
        lse_t = torch.logsumexp(t / T, -1)
        lse_d = torch.logsumexp(d / T, -1)
        d[0, 0, v] = t[0, 0, v] - T * (lse_t - lse_d)[0, 0] - T * delta
    return t.float(), d.float(), v, T


def _moved(og, log_q, lr, v):
    """The oracle gradient with token v counted on the other side of the tie in beta:
    g_w = s q_w ([q_w < p_w] - beta) with beta -/+ q_v, and token v's own indicator flipped."""
    q = np.exp(log_q)
    ind = (lr > 0).astype(np.float64)
    beta = (q * ind).sum(-1, keepdims=True)
    sq = og / (ind - beta)                   # s q_w, signed
    sign = 1.0 if ind[..., v] else -1.0      # v leaves (or joins) the set q < p
    beta2 = beta - sign * q[..., v:v + 1]
    ind2 = ind.copy()
    ind2[..., v] = 1.0 - ind2[..., v]
    return sq * (ind2 - beta2)


@pytest.mark.parametrize("delta", [3e-6, -3e-6])
def test_beta_band_admits_a_near_tie(delta):
    t, d, v, T = _row_with_near_tie(delta)
    og, _, _, lr = svref.tv_e2e_backward(t.numpy(), d.numpy(), T, "f32", want_log_ratio=True)
    assert 0 < abs(lr[0, 0, v]) < BETA_BAND
    assert (np.abs(lr) < 10 * BETA_BAND).sum() == 1   # no other token near a tie
    log_q = drafter_log_q(d, T)
    g = _moved(og, log_q, lr, v)
    with pytest.raises(AssertionError):
        compare_grad(g, og, lr)                      # without ln q: the row moves beyond 1e-5
    rep = compare_grad(g, og, lr, log_q=log_q)
    assert rep["beta_band_rows"] == 1


def test_beta_band_rejects_a_token_outside_it():
    """Between BETA_BAND and the elementwise tie band: token v's own element is not compared,
    but beta may not move by its q."""
    t, d, v, T = _row_with_near_tie(5e-5)
    og, _, _, lr = svref.tv_e2e_backward(t.numpy(), d.numpy(), T, "f32", want_log_ratio=True)
    assert 2 * BETA_BAND < abs(lr[0, 0, v]) < TIE_BAND
    log_q = drafter_log_q(d, T)
    with pytest.raises(AssertionError):
        compare_grad(_moved(og, log_q, lr, v), og, lr, log_q=log_q)
