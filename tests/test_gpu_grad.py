"""Gradient of L_e2e in the drafter logits: GPU path vs the CPU oracle, through the C ABI
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import svref
from parity import compare_grad, drafter_log_q

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    import draft_verification_softmax_amd as m
    return m


def _odt(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def _padded(x):
    """x on the GPU in rows of a 16-byte-aligned stride (the ABI's row alignment)."""
    V = x.shape[-1]
    ld = (V + 7) // 8 * 8
    buf = torch.zeros(x.shape[:-1] + (ld,), dtype=x.dtype, device=DEV)
    buf[..., :V] = x.to(DEV)
    return buf[..., :V]


def _inputs(I, D, V, dt_t=torch.bfloat16, dt_d=torch.bfloat16, seed=11, scale=3.0):
    """Drafter rows near the target rows (the shape of a trained drafter's logits)."""
    g = torch.Generator().manual_seed(seed)
    t = scale * torch.randn((I, D, V), generator=g)
    d = t + torch.randn((I, D, V), generator=g)
    return _padded(t.to(dt_t)), _padded(d.to(dt_d))


def _oracle(t, d, T, grad_loss=1.0):
    # mixed dtypes: the oracle takes one dtype code for both, so widen both to float32
    # (bfloat16 -> float32 is exact)
    if t.dtype != d.dtype:
        t, d = t.float(), d.float()
    g, a, loss, lr = svref.tv_e2e_backward(workloads.to_oracle(t), workloads.to_oracle(d), T, _odt(t),
                                           grad_loss=grad_loss, want_log_ratio=True)
    return g, a, loss, lr


@pytest.mark.parametrize("dt,gdt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                    (torch.float32, torch.float32)])
def test_backward_matches_oracle(sv, dt, gdt):
    """Oracle alpha in, so the comparison covers the gradient kernels alone: 3 x 3 rows of
    20000 tokens (two members per row, the second ragged)."""
    I, D, V, T = 3, 3, 20000, 1.0
    t, d = _inputs(I, D, V, dt, dt)
    og, oa, _, lr = _oracle(t, d, T)
    _say(f"backward I={I} D={D} V={V} logits {dt} grad {gdt}")
    alpha = torch.as_tensor(oa, dtype=torch.float32, device=DEV)
    g = sv.sv_tv_e2e_backward(t, d, alpha, T, grad_dtype=gdt)
    torch.cuda.synchronize()
    rep = compare_grad(g.float().cpu().numpy(), og, lr, bf16=gdt == torch.bfloat16,
                       log_q=drafter_log_q(d, T))
    _say(f"report {rep}")


def test_backward_after_gpu_forward(sv):
    """The forward's own alpha in: its 1e-5 relative error reaches each row's weight through
    at most D - 1 factors, so the bound is D * 1e-5."""
    I, D, V, T = 4, 4, 33000, 0.8
    t, d = _inputs(I, D, V, torch.float32, torch.float32, seed=3)
    og, oa, oloss, lr = _oracle(t, d, T)
    _say(f"forward + backward I={I} D={D} V={V}")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    g = sv.sv_tv_e2e_backward(t, d, alpha, T, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    rep = compare_grad(g.cpu().numpy(), og, lr, rtol=D * 1e-5, log_q=drafter_log_q(d, T))
    _say(f"report {rep}")
    # rows of the gradient sum to zero (a constant added to a drafter row changes nothing)
    gs = g.double().sum(-1).abs().cpu().numpy()
    ga = g.double().abs().sum(-1).cpu().numpy()
    assert (gs <= 1e-5 * ga).all()


@pytest.mark.parametrize("V", [1, 7, 4097, 16384, 16385, 1 << 20])
def test_backward_edge_vocabularies(sv, V):
    """Tiny, ragged, exactly one member, one member plus one token, and SV_V_MAX (64 members
    a row); mixed logit dtypes and depth 1 and 5."""
    for I, D in [(2, 1), (1, 5)]:
        t, d = _inputs(I, D, V, torch.bfloat16, torch.float32, seed=V + D)
        og, oa, _, lr = _oracle(t, d, 1.3)
        _say(f"backward edge V={V} I={I} D={D}")
        alpha = torch.as_tensor(oa, dtype=torch.float32, device=DEV)
        g = sv.sv_tv_e2e_backward(t, d, alpha, 1.3, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        compare_grad(g.cpu().numpy(), og, lr, log_q=drafter_log_q(d, 1.3))


@pytest.mark.parametrize("D", [16, 512, 4096])
def test_e2e_deep_blocks(sv, D):
    """Depth 16 (a DFly block), 512 and SV_K_MAX = 4096, with drafter rows close to the target
    (alpha about 0.97..0.9998), so the running products stay in binary32's normal range to the
    end of the block (about 1e-20 at depth 4096).  Forward: alpha within 1e-5, and L_e2e within
    the bound that a relative error of 1e-5 per alpha carries through the products (term m
    has m + 1 factors).  Backward, from the oracle's alpha (its plain weights cost O(D^3), so
    up to depth 512): the gradient of every row."""
    I, V, T = 2, 2000, 1.0
    g = torch.Generator().manual_seed(D)
    t = 3.0 * torch.randn((I, D, V), generator=g)
    d = t + 0.03 * torch.randn((I, D, V), generator=g)
    t, d = _padded(t), _padded(d)
    _say(f"e2e deep I={I} D={D} V={V}")
    ol, oa = svref.tv_e2e_loss(workloads.to_oracle(t), workloads.to_oracle(d), T, "f32")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    torch.cuda.synchronize()
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    P = np.cumprod(oa, axis=1)
    bound = (P * (np.arange(D) + 1) * 1e-5).sum() / (I * D) + 2.0 ** -24
    assert abs(loss.item() - ol) <= bound, (loss.item(), ol, bound)
    if D > 512:
        return
    og, _, _, lr = _oracle(t, d, T)
    gg = sv.sv_tv_e2e_backward(t, d, torch.as_tensor(oa, dtype=torch.float32, device=DEV), T,
                               grad_dtype=torch.float32)
    torch.cuda.synchronize()
    rep = compare_grad(gg.cpu().numpy(), og, lr, log_q=drafter_log_q(d, T))
    _say(f"report {rep}")


def test_e2e_rows_beyond_2gib(sv):
    """L_e2e forward and backward on 1100 x 2 rows of a 2 MiB + 16 byte stride (bfloat16
    logits and gradient, 4.6 GB per tensor): rows past the first 1024 lie beyond 2^31 bytes,
    in the logits and in the gradient."""
    I, D, V, T = 1100, 2, 1000, 1.0
    ld = (1 << 20) + 8
    g = torch.Generator().manual_seed(ld)
    t0 = (3.0 * torch.randn((I, D, V), generator=g)).to(torch.bfloat16)
    d0 = (t0.float() + torch.randn((I, D, V), generator=g)).to(torch.bfloat16)

    def big(x):
        buf = torch.empty((I, D, ld), dtype=x.dtype, device=DEV)
        buf[..., :V] = x.to(DEV)
        return buf[..., :V]
    t, d = big(t0), big(d0)
    _say(f"e2e rows beyond 2 GiB I={I} D={D} V={V} ld={ld}")
    og, oa, oloss, lr = _oracle(t, d, T)
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    grad = torch.empty((I, D, ld), dtype=torch.bfloat16, device=DEV)[..., :V]
    gg = sv.sv_tv_e2e_backward(t, d, alpha, T, grad=grad)
    torch.cuda.synchronize()
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    assert abs(loss.item() - oloss) <= 1e-5 * abs(oloss)
    rep = compare_grad(gg.float().cpu().numpy(), og, lr, rtol=D * 1e-5, bf16=True, log_q=drafter_log_q(d, T))
    _say(f"report {rep}")


def test_backward_grad_loss_and_padded_rows(sv):
    """A device grad_loss scales the result; rows with a stride above V keep their padding."""
    I, D, V, T = 2, 3, 3000, 1.0
    t, d = _inputs(I, D, V, torch.float32, torch.float32, seed=8)
    og, oa, _, lr = _oracle(t, d, T, grad_loss=-2.5)
    alpha = torch.as_tensor(oa, dtype=torch.float32, device=DEV)
    gl = torch.tensor([-2.5], dtype=torch.float32, device=DEV)
    buf = torch.full((I, D, V + 16), 7.0, dtype=torch.float32, device=DEV)
    _say("backward grad_loss and padded rows")
    g = sv.sv_tv_e2e_backward(t, d, alpha, T, grad_loss=gl, grad=buf[:, :, :V])
    torch.cuda.synchronize()
    compare_grad(g.cpu().numpy(), og, lr, log_q=drafter_log_q(d, T))
    assert (buf[:, :, V:] == 7.0).all()


def test_backward_workspace_reuse(sv):
    """One workspace across forward, backward and verification calls of different shapes:
    every call must see only its own tagged words."""
    ws = sv.Workspace(DEV)
    buf = ws.get(6, 4, 40000)
    for it, (I, D, V) in enumerate([(3, 2, 40000), (6, 4, 9000), (2, 3, 40000)]):
        t, d = _inputs(I, D, V, torch.bfloat16, torch.bfloat16, seed=100 + it)
        og, oa, _, lr = _oracle(t, d, 1.0)
        _say(f"workspace reuse call {it}: I={I} D={D} V={V}")
        loss, alpha = sv.sv_tv_e2e_loss(t, d, 1.0, workspace=buf)
        g = sv.sv_tv_e2e_backward(t, d, alpha, 1.0, grad_dtype=torch.float32, workspace=buf)
        v = workloads.make_verify_inputs("tiny", device="cpu", T=1.0)
        sv.sv_verify_batch(v.target.to(DEV), v.draft.to(DEV), v.draft_tokens.to(DEV), 1.0, workspace=buf)
        torch.cuda.synchronize()
        compare_grad(g.cpu().numpy(), og, lr, rtol=D * 1e-5, log_q=drafter_log_q(d, 1.0))
    assert sv.sv_device_error(buf) == 0


def test_backward_low_temperature(sv):
    """T = 0.02: base-2 normalisers of several hundred (kept as hi + lo); most of q lies below
    the binary32 normal range, where the floor of the comparison applies."""
    I, D, V, T = 3, 4, 40000, 0.02
    t, d = _inputs(I, D, V, torch.bfloat16, torch.bfloat16, seed=12)
    og, oa, oloss, lr = _oracle(t, d, T)
    _say(f"backward low temperature I={I} D={D} V={V} T={T}")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    g = sv.sv_tv_e2e_backward(t, d, alpha, T, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    rep = compare_grad(g.cpu().numpy(), og, lr, rtol=D * 1e-5, log_q=drafter_log_q(d, T))
    _say(f"report {rep}")


def test_backward_full_size_sampled(sv):
    """|I| = 8192, D = 3, V = 131072, bfloat16 logits and gradient (the benchmarked launch),
    forward alpha from the GPU; 64 sequences spread over the launch (first, last, every 128th)
    recomputed by the oracle, whose per-sequence gradient scales by 1/|I| in the full batch
    (L_e2e averages over sequences)."""
    t, d, T = workloads.make_e2e_inputs(device=DEV)
    I, D, V = t.shape
    _say(f"backward full I={I} D={D} V={V}")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    g = sv.sv_tv_e2e_backward(t, d, alpha, T)
    torch.cuda.synchronize()
    assert g.dtype == torch.bfloat16
    idx = sorted(set([0, 1, 8191] + list(range(64, 8192, 128))))[:64]
    assert len(idx) == 64
    worst = 0.0
    for i in idx:
        og, oa, _, lr = _oracle(t[i:i + 1], d[i:i + 1], T)
        np.testing.assert_allclose(alpha[i].cpu().numpy(), oa[0], rtol=1e-5)
        rep = compare_grad(g[i:i + 1].float().cpu().numpy(), og / I, lr, rtol=D * 1e-5, bf16=True,
                           log_q=drafter_log_q(d[i:i + 1], T))
        worst = max(worst, rep["max_rel"])
    _say(f"64 sequences compared, largest relative error {worst:.3g}")
    assert torch.isfinite(g).all()
