"""Draft tokens and confidences: GPU path vs the CPU oracle, through the C ABI (needs an
MI355X)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import svref
from parity import CDF_BAND, REL_TOL

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    import draft_verification_softmax_amd as m
    return m


def _padded(x):
    V = x.shape[-1]
    ld = (V + 7) // 8 * 8
    buf = torch.zeros(x.shape[:-1] + (ld,), dtype=x.dtype, device=DEV)
    buf[..., :V] = x.to(DEV)
    return buf[..., :V]


def _drafts(B, K, V, dt=torch.bfloat16, seed=21, scale=3.0):
    g = torch.Generator().manual_seed(seed)
    return _padded((scale * torch.randn((B, K, V), generator=g)).to(dt))


def _compare(sv_tok, sv_conf, d, T, seed, step):
    """Tokens bit-exact unless the oracle's target u R lies within CDF_BAND * R of a CDF
    boundary between the two tokens; confidences 1e-5 relative (of the token drawn)."""
    dn = workloads.to_oracle(d)
    dt = "bf16" if d.dtype == torch.bfloat16 else "f32"
    tok, conf, u, R = svref.sample_drafts(dn, T, dt, seed=seed, step=step)
    g_tok = sv_tok.cpu().numpy()
    g_conf = sv_conf.cpu().numpy().astype(np.float64)
    B, K = tok.shape
    near = 0
    for r in range(B):
        for k in range(K):
            tg, to = int(g_tok[r, k]), int(tok[r, k])
            if tg == to:
                assert abs(g_conf[r, k] - conf[r, k]) <= REL_TOL * conf[r, k], (r, k, g_conf[r, k], conf[r, k])
                continue
            assert T > 0, f"greedy token ({r},{k}): gpu {tg} oracle {to}"
            assert 0 <= tg < d.shape[-1]
            t = u[r, k] * R[r, k]
            if tg > to:
                gap = svref.draft_cdf(dn, T, dt, r, k, tg - 1) - t
            else:
                gap = t - svref.draft_cdf(dn, T, dt, r, k, tg)
            assert 0 <= gap <= CDF_BAND * R[r, k], f"token ({r},{k}): gpu {tg} oracle {to}, gap {gap}"
            qg = svref.draft_cdf(dn, T, dt, r, k, tg) - svref.draft_cdf(dn, T, dt, r, k, tg - 1)
            assert abs(g_conf[r, k] - qg) <= REL_TOL * qg
            near += 1
    return {"rows": B * K, "near_boundary": near}


@pytest.mark.parametrize("T", [0.02, 0.3, 0.9, 1.5, 25.0])
def test_sample_matches_oracle(sv, T):
    """T = 0.02 puts the base-2 normalisers near 700 (kept as hi + lo) and q near one-hot;
    T = 25 makes q nearly flat."""
    d = _drafts(4, 5, 50000)
    _say(f"sample B=4 K=5 V=50000 T={T}")
    tok, conf = sv.sv_sample_drafts(d, T, seed=17, step=3)
    torch.cuda.synchronize()
    _say(f"report {_compare(tok, conf, d, T, 17, 3)}")


def test_sample_greedy(sv):
    d = _drafts(3, 4, 40000, dt=torch.float32, seed=5)
    d[1, 2, 7] = d[1, 2].max() + 1.0   # a clear maximum
    d[2, 0, [100, 30000]] = d[2, 0].max() + 2.0   # a tie: the lower index
    _say("sample greedy")
    tok, conf = sv.sv_sample_drafts(d, 0.0)
    torch.cuda.synchronize()
    assert tok[1, 2].item() == 7 and tok[2, 0].item() == 100
    _compare(tok, conf, d, 0.0, 0, 0)


@pytest.mark.parametrize("V", [1, 7, 4097, 16384, 16385])
def test_sample_edge_vocabularies(sv, V):
    for T in [0.0, 1.0]:
        d = _drafts(3, 2, V, dt=torch.float32, seed=V)
        _say(f"sample edge V={V} T={T}")
        tok, conf = sv.sv_sample_drafts(d, T, seed=2, step=V)
        torch.cuda.synchronize()
        _compare(tok, conf, d, T, 2, V)


def test_sample_masked_logits(sv):
    """-inf entries are never drawn and carry no mass."""
    d = _drafts(2, 3, 20000, dt=torch.float32, seed=9)
    d[:, :, ::3] = -float("inf")
    _say("sample masked")
    tok, conf = sv.sv_sample_drafts(d, 0.8, seed=1)
    torch.cuda.synchronize()
    assert (tok.cpu() % 3 != 0).all()
    _compare(tok, conf, d, 0.8, 1, 0)


def test_sample_full_dfly_batch(sv):
    """B = 64 requests x 16 drafter rows of V = 131072 bfloat16 logits (the benchmarked launch),
    every row against the oracle, two steps in a row on one workspace."""
    d = _drafts(64, 16, 131072, seed=77)
    ws = sv.Workspace(DEV)
    for step in [0, 1]:
        _say(f"sample full DFly step {step}")
        tok, conf = sv.sv_sample_drafts(d, 0.9, seed=123, step=step, workspace=ws)
        torch.cuda.synchronize()
        _say(f"report {_compare(tok, conf, d, 0.9, 123, step)}")


def test_sample_rows_beyond_2gib(sv):
    """2 x 1100 drafter rows of a 2 MiB + 16 byte stride (4.6 GB): rows past the first 1024
    lie beyond 2^31 bytes."""
    B, K, V = 2, 1100, 1000
    ld = (1 << 20) + 8
    g = torch.Generator().manual_seed(ld)
    x = (3.0 * torch.randn((B, K, V), generator=g)).to(torch.bfloat16)
    buf = torch.empty((B, K, ld), dtype=torch.bfloat16, device=DEV)
    buf[..., :V] = x.to(DEV)
    d = buf[..., :V]
    for T in (0.9, 0.0):
        _say(f"sample rows beyond 2 GiB T={T}")
        tok, conf = sv.sv_sample_drafts(d, T, seed=5, step=1)
        torch.cuda.synchronize()
        _say(f"report {_compare(tok, conf, d, T, 5, 1)}")


def test_sample_largest_vocabulary(sv):
    """V = SV_V_MAX = 2^20: 64 members a row, so a finalize wave gathers S + 4S = 320 words
    (greedy: 4S = 256), the most it holds."""
    d = _drafts(2, 3, 1 << 20, seed=20)
    for T in (0.9, 0.0):
        _say(f"sample V=2^20 T={T}")
        tok, conf = sv.sv_sample_drafts(d, T, seed=3, step=2)
        torch.cuda.synchronize()
        _say(f"report {_compare(tok, conf, d, T, 3, 2)}")
