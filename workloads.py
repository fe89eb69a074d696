"""Seeded synthetic inputs for batched draft verification.

This module only draws data: Gaussian logits, spikes, per-request noise scales, Beta
confidences and the drafter's own token choice.  It holds none of the verification
arithmetic; the GPU path and the CPU oracle both consume exactly the tensors made here.

Workloads (shapes and value distributions follow the AngelSpec pages' settings: MTP depth
3, DFly blocks of 16, concurrency 4-64, a ~128k vocabulary, T in {0, 0.9}):

  tiny   B=1,  K=3,  V=1000,   fp32, target ~ N(0, 2^2), draft = target + N(0, 1^2)
  mtp    B=16, K=3,  V=131072, bf16, target ~ N(0, 3^2), draft = target + N(0, 1.5^2)
  dfly   B=64, K=16, V=131072, bf16, target ~ N(0, 3^2) plus +12 at one uniform token per
         row (the draft inherits it), draft = target + N(0, s_r^2), s_r ~ U(0.3, 2.0)
  budget dfly logits plus confidences conf[64][16] ~ Beta(5, 2), budget N = 256
  e2e    I=8192, D=3, V=131072, bf16, target ~ N(0, 3^2), draft = target + N(0, 1^2), T=1

Draft tokens are the drafter's choice: a sample x ~ softmax(z_d / T) drawn with the
Gumbel-max trick (argmax of z_d / T + Gumbel noise) for T > 0, the first argmax of z_d for
T = 0.  Logits are drawn in float32 and rounded to bfloat16 (round-to-nearest-even) before
the tokens are drawn, so tokens are drawn from the distribution the verifier sees.
"""
from dataclasses import dataclass
from typing import Optional

import torch

VERIFY_CONFIGS = {
    # name: (B, K, V, dtype, target_sigma, draft_sigma or None (per-request), spike, seed)
    "tiny": (1, 3, 1000, torch.float32, 2.0, 1.0, 0.0, 0),
    "mtp": (16, 3, 131072, torch.bfloat16, 3.0, 1.5, 0.0, 2),
    "dfly": (64, 16, 131072, torch.bfloat16, 3.0, None, 12.0, 3),
}
DEFAULT_T = {"tiny": 1.0, "mtp": 0.9, "dfly": 0.9, "budget": 0.9, "e2e": 1.0}


@dataclass
class VerifyInputs:
    target: torch.Tensor        # [B][K+1][V]
    draft: torch.Tensor         # [B][K][V]
    draft_tokens: torch.Tensor  # [B][K] int32
    T: float
    seed: int                   # Philox key used by the verifier
    name: str


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _draft_tokens(draft: torch.Tensor, T: float, g: torch.Generator) -> torch.Tensor:
    """The drafter's token per row: Gumbel-max sample of softmax(z/T), or argmax at T=0."""
    B, K, V = draft.shape
    out = torch.empty((B, K), dtype=torch.int32, device=draft.device)
    for r in range(B):
        z = draft[r].float()
        if T > 0:
            u = torch.rand(z.shape, generator=g, device=z.device).clamp_(min=1e-20)
            z = z / T - torch.log(-torch.log(u))
        out[r] = torch.argmax(z, dim=-1).to(torch.int32)
    return out


def make_verify_inputs(name: str, device="cpu", T: Optional[float] = None,
                       seed: Optional[int] = None, B: Optional[int] = None,
                       K: Optional[int] = None, V: Optional[int] = None) -> VerifyInputs:
    """Inputs of one verify workload; B, K, V may be overridden to make smaller cases of
    the same distribution."""
    B0, K0, V0, dtype, ts, ds, spike, s0 = VERIFY_CONFIGS[name]
    B, K, V = B or B0, K if K is not None else K0, V or V0
    seed = s0 if seed is None else seed
    T = DEFAULT_T[name] if T is None else T
    g = _gen(device, seed)
    target = torch.empty((B, K + 1, V), dtype=dtype, device=device)
    draft = torch.empty((B, K, V), dtype=dtype, device=device)
    if ds is None:
        sig = 0.3 + 1.7 * torch.rand((B,), generator=g, device=device)
    else:
        sig = torch.full((B,), ds, device=device)
    for r in range(B):
        t = ts * torch.randn((K + 1, V), generator=g, device=device)
        if spike:
            pos = torch.randint(0, V, (K + 1,), generator=g, device=device)
            t[torch.arange(K + 1, device=device), pos] += spike
        d = t[:K] + sig[r] * torch.randn((K, V), generator=g, device=device)
        target[r] = t.to(dtype)
        draft[r] = d.to(dtype)
    toks = _draft_tokens(draft, T, g)
    return VerifyInputs(target, draft, toks, float(T), seed, name)


def make_budget_conf(device="cpu", B=64, K=16, seed=4) -> torch.Tensor:
    """Drafter confidences in (0,1), Beta(5, 2), float32 [B][K]."""
    g = _gen(device, seed)
    # Beta(5,2) as X/(X+Y) with X ~ Gamma(5), Y ~ Gamma(2); Gamma(n) = -sum log(U) for
    # integer n (sum of n unit exponentials).
    u = torch.rand((B, K, 7), generator=g, device=device, dtype=torch.float64).clamp_(min=1e-300)
    e = -torch.log(u)
    x = e[..., :5].sum(-1)
    y = e[..., 5:].sum(-1)
    return (x / (x + y)).to(torch.float32)


def make_budget_inputs(device="cpu", T=None, seed=4):
    """The ragged-verify workload: dfly-shaped logits plus confidences."""
    v = make_verify_inputs("dfly", device=device, T=DEFAULT_T["budget"] if T is None else T, seed=seed)
    conf = make_budget_conf(device=device, B=v.target.shape[0], K=v.draft.shape[1], seed=seed + 1000)
    return v, conf, 256


def make_e2e_inputs(device="cpu", I=8192, D=3, V=131072, seed=5, chunk=512):
    """target, draft [I][D][V] bf16 for the end-to-end TV objective."""
    g = _gen(device, seed)
    target = torch.empty((I, D, V), dtype=torch.bfloat16, device=device)
    draft = torch.empty((I, D, V), dtype=torch.bfloat16, device=device)
    for i0 in range(0, I, chunk):
        n = min(chunk, I - i0)
        t = 3.0 * torch.randn((n, D, V), generator=g, device=device)
        d = t + torch.randn((n, D, V), generator=g, device=device)
        target[i0:i0 + n] = t.to(torch.bfloat16)
        draft[i0:i0 + n] = d.to(torch.bfloat16)
    return target, draft, DEFAULT_T["e2e"]


def to_oracle(x: torch.Tensor):
    """Host numpy view for the oracle: float32 stays float32, bfloat16 becomes its uint16
    bit pattern."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float32:
        return x.numpy()
    return x.numpy()
