"""The hand-over paths: with the in-kernel wait bound at 0 every workgroup that does not find
its teammates' partials at once hands its share over, and the later kernels of the call
recompute it from the logits.  Results must match the oracle exactly as on the normal path
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import svref
from parity import compare_grad, compare_verify, drafter_log_q

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture()
def sv():
    import draft_verification_softmax_amd as m
    m.sv_set_wait_bound(0)
    try:
        yield m
    finally:
        m.sv_set_wait_bound(200000)


def _verify_case(sv, T, selected=False, name="mtp", B=None):
    v = workloads.make_verify_inputs(name, device="cpu", T=T, B=B)
    t, d, x = v.target.to(DEV), v.draft.to(DEV), v.draft_tokens.to(DEV)
    B, K = v.draft_tokens.shape
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, t.shape[-1])
    dl = None
    if selected:
        conf = torch.linspace(0.99, 0.5, B * K, device=DEV).reshape(B, K).contiguous()
        lens, _, rl = sv.sv_alloc_verify_budget(conf, 20)
        out = sv.sv_verify_selected(t, d, x, T, lens, rl, 20, seed=v.seed, workspace=buf)
        dl = lens.cpu().numpy()
    else:
        out = sv.sv_verify_batch(t, d, x, T, seed=v.seed, workspace=buf, want_amax=True)
    torch.cuda.synchronize()
    g = {k: (None if w is None else w.cpu().numpy()) for k, w in out.items()}
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    o = svref.verify_batch(tn, dn, v.draft_tokens.numpy(), T, "bf16", seed=v.seed,
                           draft_len=dl, diagnostics=True)
    rep = compare_verify(g, o, tn, dn, "bf16", T, L=dl)
    assert sv.sv_device_error(buf) == 0
    return rep


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_verify_with_every_share_handed_over(sv, T):
    _say(f"hand-over verify MTP T={T}")
    _say(f"report {_verify_case(sv, T)}")


def test_verify_large_grid_with_every_share_handed_over(sv):
    # 8 requests x 16 drafts: 1096 workgroups, more than fit on the device at once at three
    # per compute unit, so the variant without kept terms runs (the MTP case above runs the
    # other one at T = 0.9)
    _say("hand-over verify DFly B=8 T=0.9")
    _say(f"report {_verify_case(sv, 0.9, name='dfly', B=8)}")


def test_selected_verify_with_every_share_handed_over(sv):
    _say("hand-over selected verify")
    _say(f"report {_verify_case(sv, 0.9, selected=True)}")


def test_e2e_forward_and_backward_with_every_share_handed_over(sv):
    g_ = torch.Generator().manual_seed(4)
    I, D, V, T = 4, 3, 50000, 1.0
    t = (3.0 * torch.randn((I, D, V), generator=g_)).to(torch.bfloat16)
    d = (t.float() + torch.randn((I, D, V), generator=g_)).to(torch.bfloat16)
    og, oa, oloss, lr = svref.tv_e2e_backward(workloads.to_oracle(t), workloads.to_oracle(d), T, "bf16",
                                              want_log_ratio=True)
    t, d = t.to(DEV), d.to(DEV)
    _say("hand-over L_e2e forward and backward")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    g = sv.sv_tv_e2e_backward(t, d, alpha, T, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    assert abs(loss.item() - oloss) <= 1e-5 * abs(oloss)
    _say(f"report {compare_grad(g.cpu().numpy(), og, lr, rtol=D * 1e-5, log_q=drafter_log_q(d, T))}")
