"""GPU path vs the CPU oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import svref
from parity import CDF_BAND, compare_verify, near_token_max

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def sv():
    import draft_verification_softmax_amd as m
    return m


def _np(out):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def _oracle_dtype(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def _run_pair(sv, v, T, draft_len=None, check=None, want_amax=True, seed=None, step=0):
    seed = v.seed if seed is None else seed
    label = (f"{v.name} B={v.target.shape[0]} K={v.draft.shape[1]} V={v.target.shape[2]} T={T} "
             f"ragged={draft_len is not None} amax={want_amax}")
    _say(label)
    dl_dev = None if draft_len is None else torch.as_tensor(draft_len, dtype=torch.int32, device=DEV)
    out = sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=seed, step=step,
                             draft_len=dl_dev, want_amax=want_amax)
    torch.cuda.synchronize()
    g = _np(out)
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    dt = _oracle_dtype(v.target)
    B, K = v.draft_tokens.shape
    dl = np.full(B, K, np.int32) if draft_len is None else np.asarray(draft_len, np.int32).copy()
    if check is not None:  # oracle only on sampled requests: others get L_r = 0
        mask = np.zeros(B, bool)
        mask[list(check)] = True
        dl[~mask] = 0
    o = svref.verify_batch(tn, dn, v.draft_tokens.cpu().numpy(), T, dt, seed=seed, step=step,
                           draft_len=dl, diagnostics=True)
    rep = compare_verify(g, o, tn, dn, dt, T, check=check, L=dl if draft_len is not None else None, label=label)
    _say(f"report {rep}")
    return g, o, rep


def _move(v):
    return workloads.VerifyInputs(v.target.to(DEV), v.draft.to(DEV), v.draft_tokens.to(DEV), v.T, v.seed, v.name)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_tiny(sv, T):
    v = _move(workloads.make_verify_inputs("tiny", device="cpu", T=T))
    g, o, rep = _run_pair(sv, v, T)
    assert rep["requests"] == 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [0.9, 0.0, 1.7])
def test_ragged_vocab_several_tiles(sv, dtype, T):
    """V not a multiple of the 8-logit vector nor of the 4096-logit tile, padded rows."""
    B, K, V, ld = 6, 5, 9001, 9008
    g = torch.Generator(device=DEV).manual_seed(17)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tt = torch.full((B, K + 1, ld), float("nan"), device=DEV, dtype=tdt)
    dd = torch.full((B, K, ld), float("nan"), device=DEV, dtype=tdt)
    t = 2.5 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    d = t[:, :K] + 0.7 * torch.randn((B, K, V), generator=g, device=DEV)
    tt[..., :V] = t.to(tdt)
    dd[..., :V] = d.to(tdt)
    toks = torch.argmax(d, -1).to(torch.int32)
    toks[:, 1] = torch.randint(0, V, (B,), generator=g, device=DEV, dtype=torch.int32)
    _say(f"ragged-vocab {dtype} T={T}")
    out = sv.sv_verify_batch(tt[..., :V], dd[..., :V], toks, T, seed=3, step=1, want_amax=True)
    torch.cuda.synchronize()
    gpu = _np(out)
    # the oracle gets the same padded rows (it reads only V of every ld)
    tn = workloads.to_oracle(tt[..., :V].contiguous())
    dn = workloads.to_oracle(dd[..., :V].contiguous())
    o = svref.verify_batch(tn, dn, toks.cpu().numpy(), T, dtype, seed=3, step=1, diagnostics=True)
    rep = compare_verify(gpu, o, tn, dn, dtype, T, label=f"ragged vocab 9001 {dtype} T={T}")
    _say(f"report {rep}")


@pytest.mark.parametrize("T,want_amax", [(0.9, False), (0.9, True), (0.0, True)])
def test_mtp_full(sv, T, want_amax):
    """The MTP workload (16 x 3 x 131072): its grid fits on the device at once, so the
    kept-term instance runs; without argmax outputs its pass 1 takes the first-logit reference
    (the configuration a caller gets by default), with them the exact maxima."""
    v = _move(workloads.make_verify_inputs("mtp", device="cpu", T=T))
    _run_pair(sv, v, T, want_amax=want_amax)


@pytest.mark.parametrize("T,want_amax", [(0.9, False), (0.9, True), (0.0, True)])
def test_dfly_full(sv, T, want_amax):
    """Every request of the DFly workload (64 x 16 x 131072, the measured configuration:
    T = 0.9 without argmax outputs is the call the benchmark times) against the oracle."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=T)
    _run_pair(sv, v, T, want_amax=want_amax)


def test_dfly_ragged_lengths(sv):
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=12)
    rng = np.random.default_rng(0)
    dl = rng.integers(0, 17, size=12).astype(np.int32)
    dl[0], dl[1], dl[2] = 0, 16, 1
    _run_pair(sv, v, 0.9, draft_len=dl)


def test_determinism(sv):
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=16)
    _say("determinism")
    a = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=1, want_amax=True))
    b = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=1, want_amax=True))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_uniforms_match_oracle(sv):
    rng = np.random.default_rng(1)
    ctr = rng.integers(0, 2**62, size=(257, 4), dtype=np.int64)
    ctr[:4] = [[0, 0, 0, 0], [1, 2, 0, 3], [63, 15, 1, 0], [7, 7, 7, 7]]
    _say("uniforms")
    u = sv.sv_uniforms(11, torch.as_tensor(ctr, device=DEV)).cpu().numpy()
    want = np.array([svref.uniform(11, *[int(x) for x in c]) for c in ctr])
    assert np.array_equal(u.astype(np.float64), want)


def test_accept_len_matches_oracle(sv):
    """sv_accept_len against the oracle's first-reject scan on random accept arrays, with and
    without draft lengths (including 0, K and entries past L_r that must be ignored)."""
    rng = np.random.default_rng(3)
    for trial, (B, K) in enumerate([(1, 1), (7, 3), (64, 16), (300, 5), (5, 0), (33, 64)]):
        acc = (rng.random((B, K)) < [0.5, 0.9, 0.7, 0.3, 0.5, 0.95][trial]).astype(np.uint8)
        dl = rng.integers(0, K + 1, size=B).astype(np.int32)
        if B > 2:
            dl[0], dl[1] = 0, K
        _say(f"accept_len B={B} K={K}")
        acc_d = torch.as_tensor(acc, device=DEV)
        got = sv.sv_accept_len(acc_d).cpu().numpy()
        assert np.array_equal(got, svref.accept_len(acc)), trial
        got = sv.sv_accept_len(acc_d, torch.as_tensor(dl, device=DEV)).cpu().numpy()
        assert np.array_equal(got, svref.accept_len(acc, draft_len=dl)), trial
        if B > 2:   # lengths outside [0, K] are clamped
            dl2 = dl.copy()
            dl2[0], dl2[1] = -4, K + 3
            got = sv.sv_accept_len(acc_d, torch.as_tensor(dl2, device=DEV)).cpu().numpy()
            assert np.array_equal(got, svref.accept_len(acc, draft_len=np.clip(dl2, 0, K))), trial


def _token_in_band(tn, dn, T, dtype, r, tau, L, tg, to, seed, step):
    """The oracle's CDF at the GPU token brackets the draw's target within CDF_BAND * R (the
    same test compare_verify applies to the fused call's tokens)."""
    w_t = svref.uniform(seed, r, tau, 1, step)
    R = svref.correction_cdf(tn, dn, T, dtype, r, tau, L, tn.shape[-1] - 1)
    t = w_t * R
    if tg > to:
        gap = svref.correction_cdf(tn, dn, T, dtype, r, tau, L, tg - 1) - t
    else:
        gap = t - svref.correction_cdf(tn, dn, T, dtype, r, tau, L, tg)
    return 0 <= gap <= CDF_BAND * R


def test_accept_len_and_residual_sample(sv):
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=8)
    _say("accept_len + residual_sample")
    dl = torch.tensor([16, 3, 0, 7, 16, 1, 9, 12], dtype=torch.int32, device=DEV)
    out = sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=v.seed, step=4, draft_len=dl)
    al = sv.sv_accept_len(out["accept"], dl)
    assert torch.equal(al, out["accept_len"])
    assert np.array_equal(al.cpu().numpy(), svref.accept_len(out["accept"].cpu().numpy(), draft_len=dl.cpu().numpy()))
    tok = sv.sv_residual_sample(v.target, v.draft, out["accept_len"], 0.9, seed=v.seed, step=4, draft_len=dl)
    want = out["out_tokens"].gather(1, out["accept_len"].long()[:, None])[:, 0]
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    dln = dl.cpu().numpy()
    # the stand-alone draw and the fused one sum their normalisers separately: equal tokens,
    # or (counted) both equal to the oracle's or within its CDF band
    tok_np, want_np, al_np = tok.cpu().numpy(), want.cpu().numpy(), al.cpu().numpy()
    otok0 = svref.residual_sample(tn, dn, al_np, 0.9, "bf16", seed=v.seed, step=4, draft_len=dln)
    differ = 0
    for r in range(8):
        if tok_np[r] != want_np[r]:
            differ += 1
            for g in (int(tok_np[r]), int(want_np[r])):
                assert g == otok0[r] or _token_in_band(tn, dn, 0.9, "bf16", r, int(al_np[r]), int(dln[r]), g,
                                                       int(otok0[r]), v.seed, 4), (r, g, otok0[r])
    _say(f"residual_sample vs fused: {differ} of 8 differ")
    assert differ <= near_token_max(8)
    # oracle on forced accepted lengths (including 0 and L_r): equal, or within the CDF band
    near = 0
    for seed, step, forced in [(2, 0, [0, 3, 0, 2, 16, 1, 5, 12]), (9, 3, [15, 2, 0, 7, 0, 0, 8, 11]),
                               (v.seed, 1, [16, 1, 0, 6, 3, 1, 9, 0])]:
        forced = np.array(forced, np.int32)
        tok2 = sv.sv_residual_sample(v.target, v.draft, torch.as_tensor(forced, device=DEV), 0.9, seed=seed,
                                     step=step, draft_len=dl).cpu().numpy()
        otok = svref.residual_sample(tn, dn, forced, 0.9, "bf16", seed=seed, step=step, draft_len=dln)
        for r in range(8):
            if tok2[r] != otok[r]:
                assert _token_in_band(tn, dn, 0.9, "bf16", r, int(forced[r]), int(dln[r]), int(tok2[r]),
                                      int(otok[r]), seed, step), (seed, r, tok2[r], otok[r])
                near += 1
    _say(f"residual_sample near_token {near} of 24")
    assert near <= near_token_max(24)
    # greedy: argmax of target row tau
    tok3 = sv.sv_residual_sample(v.target, v.draft, torch.as_tensor(forced, device=DEV), 0.0,
                                 draft_len=dl).cpu().numpy()
    otok3 = svref.residual_sample(tn, dn, forced, 0.0, "bf16", draft_len=dl.cpu().numpy())
    assert np.array_equal(tok3, otok3)


def test_budget_matches_oracle(sv):
    conf = workloads.make_budget_conf(device="cpu")
    for N in [0, 1, 7, 256, 1023, 1024, 5000]:
        _say(f"budget N={N}")
        lens, off, rl = sv.sv_alloc_verify_budget(conf.to(DEV), N)
        torch.cuda.synchronize()
        ol, oo, orl = svref.alloc_verify_budget(conf.numpy(), N)
        assert np.array_equal(lens.cpu().numpy(), ol)
        assert np.array_equal(off.cpu().numpy(), oo)
        assert np.array_equal(rl.cpu().numpy()[: len(orl)], orl)
    rng = np.random.default_rng(9)
    for trial in range(20):
        B, K = int(rng.integers(1, 90)), int(rng.integers(1, 90))
        if B * K > 8192:
            continue
        c = rng.beta(2, 2, size=(B, K)).astype(np.float32)
        c[rng.random((B, K)) < 0.1] = 1.0   # ties
        dl = rng.integers(0, K + 1, size=B).astype(np.int32)
        N = int(rng.integers(0, B * K + 3))
        lens, off, rl = sv.sv_alloc_verify_budget(torch.as_tensor(c, device=DEV), N,
                                                  draft_len=torch.as_tensor(dl, device=DEV))
        ol, oo, orl = svref.alloc_verify_budget(c, N, draft_len=dl)
        assert np.array_equal(lens.cpu().numpy(), ol), trial
        assert np.array_equal(off.cpu().numpy(), oo), trial
        assert np.array_equal(rl.cpu().numpy()[: len(orl)], orl), trial


@pytest.mark.parametrize("B,K,value,N", [(64, 16, 1.0, 300), (64, 128, 1.0, 4097), (128, 64, 0.5, 1000),
                                         (128, 64, 0.5, 8191)])
def test_budget_all_equal_confidences(sv, B, K, value, N):
    """Equal confidences: every request's cumulative products are the same sequence, so keys
    tie in C across requests (all of them at C = 1) and the allocation is decided by the
    (r, k) order alone; the selection has to run through the keys' low digits.  Up to the
    8192-candidate maximum."""
    c = np.full((B, K), value, np.float32)
    _say(f"budget equal conf B={B} K={K} c={value} N={N}")
    lens, off, rl = sv.sv_alloc_verify_budget(torch.as_tensor(c, device=DEV), N)
    torch.cuda.synchronize()
    ol, oo, orl = svref.alloc_verify_budget(c, N)
    assert np.array_equal(lens.cpu().numpy(), ol)
    assert np.array_equal(off.cpu().numpy(), oo)
    assert np.array_equal(rl.cpu().numpy()[: len(orl)], orl)


def test_budget_then_ragged_verify(sv):
    v, conf, N = workloads.make_budget_inputs(device=DEV)
    lens, off, _ = sv.sv_alloc_verify_budget(conf, N)
    ol, _, _ = svref.alloc_verify_budget(conf.cpu().numpy(), N)
    assert np.array_equal(lens.cpu().numpy(), ol)
    # ragged verify on the GPU, the oracle on every request with its selected length
    _say("budget ragged verify")
    out = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, v.T, seed=v.seed, draft_len=lens,
                                 want_amax=True))
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    o = svref.verify_batch(tn, dn, v.draft_tokens.cpu().numpy(), v.T, "bf16", seed=v.seed, draft_len=ol,
                           diagnostics=True)
    rep = compare_verify(out, o, tn, dn, "bf16", v.T, L=ol, label="budget 256 of 64x16, ragged verify")
    _say(f"report {rep}")


def test_budget_clamps_draft_lengths(sv):
    """draft_len entries outside [0, K_max] (a caller error) allocate as the clamped lengths,
    for the plain budget and the D-cut choice; the clamped allocation equals the oracle's."""
    rng = np.random.default_rng(8)
    B, K = 6, 5
    conf = rng.beta(5, 2, size=(B, K)).astype(np.float32)
    bad = np.array([9, -2, 3, 5, 0, 7], np.int32)
    ok = np.clip(bad, 0, K).astype(np.int32)
    cost = (40.0 + 0.05 * np.arange(B * K + 1)).astype(np.float32)
    cd = torch.as_tensor(conf, device=DEV)
    _say("budget with draft lengths out of range")
    for N in (0, 7, 30):
        got = [x.cpu().numpy() for x in sv.sv_alloc_verify_budget(cd, N, torch.as_tensor(bad, device=DEV))]
        want = [x.cpu().numpy() for x in sv.sv_alloc_verify_budget(cd, N, torch.as_tensor(ok, device=DEV))]
        ol, oo, orl = svref.alloc_verify_budget(conf, N, draft_len=ok)
        n = int(oo[-1])
        for g_, w_ in zip(got[:2], want[:2]):
            assert np.array_equal(g_, w_)
        assert np.array_equal(got[0], ol) and np.array_equal(got[1], oo)
        assert np.array_equal(got[2][:n], want[2][:n]) and np.array_equal(got[2][:n], orl)
    got = [x.cpu().numpy() for x in sv.sv_dcut_verify_budget(cd, torch.as_tensor(cost, device=DEV),
                                                              torch.as_tensor(bad, device=DEV))]
    on, ou, ol, oo, _ = svref.dcut_budget(conf, cost, draft_len=ok)
    assert int(got[0][0]) == on and abs(float(got[1][0]) - ou) <= 1e-12 * abs(ou)
    assert np.array_equal(got[2], ol) and np.array_equal(got[3], oo)


def test_budget_selected_verify(sv):
    """sv_verify_selected over the allocation's row list equals sv_verify_batch with
    draft_len = lens (same kernels, same member order), and the oracle on sampled requests."""
    v, conf, N = workloads.make_budget_inputs(device=DEV)
    B, K = conf.shape
    lens, off, rl = sv.sv_alloc_verify_budget(conf, N)
    n_rows = min(N, B * K)
    assert int(off[-1].item()) == n_rows
    ws = sv.Workspace(DEV)
    for T in (v.T, 0.0):
        _say(f"budget selected verify T={T}")
        sel = _np(sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, T, lens, rl, n_rows, seed=v.seed,
                                        want_amax=True, workspace=ws))
        bat = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=v.seed, draft_len=lens,
                                     want_amax=True, workspace=ws))
        for key in bat:
            if bat[key] is not None:
                assert np.array_equal(sel[key], bat[key]), key
    assert sv.sv_device_error(ws.get(B, K, v.target.shape[2])) == 0
    ol = lens.cpu().numpy()
    tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
    o = svref.verify_batch(tn, dn, v.draft_tokens.cpu().numpy(), v.T, "bf16", seed=v.seed, draft_len=ol,
                           diagnostics=True)
    for want_amax in (False, True):
        sel = _np(sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, v.T, lens, rl, n_rows, seed=v.seed,
                                        want_amax=want_amax))
        rep = compare_verify(sel, o, tn, dn, "bf16", v.T, L=ol, label=f"budget selected verify amax={want_amax}")
        _say(f"report {rep}")


def test_selected_verify_small_ragged_vocab(sv):
    """Random small batches, vocabulary 9001 in rows padded to 9008 (a ragged last chunk),
    budget allocation then sv_verify_selected, against the oracle on every request."""
    rng = np.random.default_rng(11)
    V, ld = 9001, 9008
    for trial in range(4):
        B, K = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        T = [0.9, 0.0, 1.3, 0.9][trial]
        g = torch.Generator(device=DEV).manual_seed(60 + trial)
        tt = torch.full((B, K + 1, ld), float("nan"), device=DEV, dtype=torch.bfloat16)
        dd = torch.full((B, K, ld), float("nan"), device=DEV, dtype=torch.bfloat16)
        t = 2.5 * torch.randn((B, K + 1, V), generator=g, device=DEV)
        d = t[:, :K] + 0.7 * torch.randn((B, K, V), generator=g, device=DEV)
        tt[..., :V] = t.to(torch.bfloat16)
        dd[..., :V] = d.to(torch.bfloat16)
        toks = torch.argmax(d, -1).to(torch.int32)
        toks[:, 0] = torch.randint(0, V, (B,), generator=g, device=DEV, dtype=torch.int32)
        conf = torch.as_tensor(rng.beta(5, 2, size=(B, K)).astype(np.float32), device=DEV)
        N = int(rng.integers(0, B * K + 2))
        lens, off, rl = sv.sv_alloc_verify_budget(conf, N)
        n_rows = min(N, B * K)
        _say(f"selected small trial {trial} B={B} K={K} N={N} T={T}")
        ws = sv.Workspace(DEV)
        out = _np(sv.sv_verify_selected(tt[..., :V], dd[..., :V], toks, T, lens, rl, n_rows, seed=5, step=trial,
                                        want_amax=True, workspace=ws))
        assert sv.sv_device_error(ws.get(B, K, V)) == 0
        tn = workloads.to_oracle(tt[..., :V].contiguous())
        dn = workloads.to_oracle(dd[..., :V].contiguous())
        dl = lens.cpu().numpy()
        o = svref.verify_batch(tn, dn, toks.cpu().numpy(), T, "bf16", seed=5, step=trial, draft_len=dl,
                               diagnostics=True)
        compare_verify(out, o, tn, dn, "bf16", T, L=dl, label=f"selected small trial {trial} T={T}")


def _dcut_ratios(conf, cost, draft_len=None):
    """E(n) / cost[n] for every n, E summed in candidate order (binary64, sequential)."""
    B, K = conf.shape
    C = np.multiply.accumulate(conf, axis=1, dtype=np.float32)
    L = np.full(B, K) if draft_len is None else draft_len
    cand = [(-float(C[r, k]), r, k) for r in range(B) for k in range(L[r])]
    cand.sort()
    P = np.concatenate([[0.0], np.cumsum([-c for c, _, _ in cand])])
    nmax = min(len(cost) - 1, len(cand))
    out = {}
    for n in range(nmax + 1):
        if np.isfinite(cost[n]) and cost[n] > 0:
            out[n] = (B + P[n]) / float(cost[n])
    return out


def test_dcut_matches_oracle(sv):
    rng = np.random.default_rng(21)
    cases = [(64, 16, 40.0 + 0.05 * np.arange(1025)), (64, 16, 1.0 + 0.002 * np.arange(1025) ** 1.3)]
    # candidate counts at and between powers of two: the sort pads to one (one key per thread
    # up to 1024 candidates, exchanges in LDS beyond)
    for B, K in [(16, 16), (16, 17), (20, 20), (30, 30), (32, 32), (40, 40)]:
        cases.append((B, K, 1.0 + 0.01 * np.arange(B * K + 1)))
    for trial in range(30):
        B, K = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        if B * K > 8192:
            continue
        n_cost = int(rng.integers(1, B * K + 3))
        cost = (1.0 + np.sort(rng.random(n_cost)) * float(rng.integers(1, 5))).astype(np.float64)
        if trial % 3 == 0:
            cost[rng.random(n_cost) < 0.2] = [0.0, np.nan, -1.0][trial % 2]
        cases.append((B, K, cost))
    for i, (B, K, cost) in enumerate(cases):
        conf = rng.beta(5, 2, size=(B, K)).astype(np.float32)
        if i % 4 == 1:
            conf[rng.random((B, K)) < 0.2] = 1.0   # ties in C
        dl = rng.integers(0, K + 1, size=B).astype(np.int32) if i % 5 == 2 else None
        cost = np.asarray(cost, np.float32)
        _say(f"dcut case {i} B={B} K={K} n_cost={len(cost)}")
        n_dev, u_dev, lens, off, rl = sv.sv_dcut_verify_budget(
            torch.as_tensor(conf, device=DEV), torch.as_tensor(cost, device=DEV),
            draft_len=None if dl is None else torch.as_tensor(dl, device=DEV))
        torch.cuda.synchronize()
        n_gpu, u_gpu = int(n_dev.item()), float(u_dev.item())
        n_or, u_or, _, _, _ = svref.dcut_budget(conf, cost, draft_len=dl)
        if n_gpu != n_or:
            # only a tie within rounding of the two summation orders may differ
            r = _dcut_ratios(conf, cost, dl)
            assert n_gpu in r and abs(r[n_gpu] - r[n_or]) <= 1e-12 * abs(r[n_or]), (i, n_gpu, n_or)
        else:
            assert abs(u_gpu - u_or) <= 1e-12 * abs(u_or), (i, u_gpu, u_or)
        want_lens, want_off, want_rl = svref.alloc_verify_budget(conf, n_gpu, draft_len=dl)
        assert np.array_equal(lens.cpu().numpy(), want_lens), i
        assert np.array_equal(off.cpu().numpy(), want_off), i
        assert np.array_equal(rl.cpu().numpy()[: len(want_rl)], want_rl), i


def test_e2e_small(sv):
    t, d, T = workloads.make_e2e_inputs(device=DEV, I=48, D=3)
    _say("e2e small")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    torch.cuda.synchronize()
    ol, oa = svref.tv_e2e_loss(workloads.to_oracle(t), workloads.to_oracle(d), T, "bf16")
    np.testing.assert_allclose(alpha.cpu().numpy(), oa, rtol=1e-5)
    assert abs(loss.item() - ol) <= 1e-5 * abs(ol)


def test_e2e_full_sampled(sv):
    t, d, T = workloads.make_e2e_inputs(device=DEV)
    _say("e2e full 8192x3")
    loss, alpha = sv.sv_tv_e2e_loss(t, d, T)
    torch.cuda.synchronize()
    a = alpha.cpu().numpy().astype(np.float64)
    # 256 sequences spread over the launch (first, last and every 32nd), each against the oracle
    idx = sorted(set([0, 1, 8191] + list(range(5, 8192, 32))))[:256]
    assert len(idx) == 256
    _, oa = svref.tv_e2e_loss(workloads.to_oracle(t[idx]), workloads.to_oracle(d[idx]), T, "bf16")
    np.testing.assert_allclose(a[idx], oa, rtol=1e-5, atol=t.shape[2] * 2.0 ** -126)
    # the reduction is the L_e2e equation applied to the returned alpha table
    want = 1.0 - np.cumprod(a, axis=1).sum() / a.size
    assert abs(loss.item() - want) <= 1e-6
    assert 0.0 < loss.item() < 1.0


def test_device_error_flag_for_bad_token(sv):
    v = _move(workloads.make_verify_inputs("tiny", device="cpu", T=1.0))
    toks = v.draft_tokens.clone()
    toks[0, 1] = 5000  # outside [0, V): the kernel guards the read and rejects
    ws = sv.Workspace(DEV)
    buf = ws.get(1, 3, 1000)
    _say("device error flag")
    out = sv.sv_verify_batch(v.target, v.draft, toks, 1.0, workspace=buf)
    flags = sv.sv_device_error(buf)
    assert flags & 1
    assert out["accept"][0, 1].item() == 0
    assert sv.sv_device_error(buf) == 0


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_draft_len_out_of_range_is_clamped_and_flagged(sv, T):
    """draft_len entries outside [0, K_max] (K_max + 5, -3) verify as K_max and 0, the same
    outputs as a call with the clamped lengths, and raise SV_DEVERR_DRAFT_LEN."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=T, B=4, K=6, V=20000, seed=5)
    ws = sv.Workspace(DEV)
    _say(f"draft_len out of range T={T}")
    bad = torch.tensor([11, -3, 2, 6], dtype=torch.int32, device=DEV)
    ok = torch.tensor([6, 0, 2, 6], dtype=torch.int32, device=DEV)
    a = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=3, draft_len=bad, want_amax=True,
                               workspace=ws))
    assert sv.sv_device_error(ws.buf) == sv.SV_DEVERR_DRAFT_LEN
    b = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=3, draft_len=ok, want_amax=True,
                               workspace=ws))
    assert sv.sv_device_error(ws.buf) == 0
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_selected_with_zero_budget(sv, T):
    """A budget of 0 selects no row: every request gets its bonus token from target row 0,
    the same as dense verification with every draft length 0 (the grid holds only the bonus
    slots and the finalize workgroups)."""
    v, conf, _ = workloads.make_budget_inputs(device=DEV, T=T)
    B, K = conf.shape
    lens, off, rl = sv.sv_alloc_verify_budget(conf, 0)
    assert int(lens.sum().item()) == 0 and int(off[-1].item()) == 0
    _say(f"selected verify with no rows, T={T}")
    sel = _np(sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, T, lens, rl, 0, seed=v.seed, want_amax=True))
    bat = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=v.seed, draft_len=lens, want_amax=True))
    for key in bat:
        if bat[key] is not None:
            assert np.array_equal(sel[key], bat[key]), key
    assert (sel["accept_len"] == 0).all() and (sel["n_out"] == 1).all()
    assert ((sel["out_tokens"][:, 0] >= 0) & (sel["out_tokens"][:, 0] < v.target.shape[2])).all()


def _keep_limit():
    # workgroups of a verification grid that runs with the kept binary32 terms: three per CU
    return 3 * torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("want_amax", [False, True])
@pytest.mark.parametrize("T", [0.9, 0.3])
def test_both_stream_variants_on_one_batch(sv, T, want_amax):
    """The same requests in a grid that fits on the device at once (kept terms) and in a larger
    one (terms recomputed): both against the oracle, and equal to each other where the result
    is discrete."""
    big = workloads.make_verify_inputs("mtp", device="cpu", T=T, B=40)
    B, K = big.draft_tokens.shape
    S = (big.target.shape[-1] + 16383) // 16384
    n_small, n_big = 16, B
    assert (n_small * K + n_small) * S + n_small <= _keep_limit() < (n_big * K + n_big) * S + n_big
    t, d, x = big.target.to(DEV), big.draft.to(DEV), big.draft_tokens.to(DEV)
    _say(f"both variants T={T}: B={n_big} and its first {n_small} requests")
    full = _np(sv.sv_verify_batch(t, d, x, T, seed=big.seed, want_amax=want_amax))
    part = _np(sv.sv_verify_batch(t[:n_small].contiguous(), d[:n_small].contiguous(), x[:n_small].contiguous(), T,
                                  seed=big.seed, want_amax=want_amax))
    tn, dn = workloads.to_oracle(big.target), workloads.to_oracle(big.draft)
    o = svref.verify_batch(tn, dn, big.draft_tokens.numpy(), T, "bf16", seed=big.seed, diagnostics=True)
    compare_verify(full, o, tn, dn, "bf16", T, label=f"both variants, large grid T={T} amax={want_amax}")
    os_ = svref.verify_batch(tn[:n_small], dn[:n_small], big.draft_tokens.numpy()[:n_small], T, "bf16",
                             seed=big.seed, diagnostics=True)
    compare_verify(part, os_, tn[:n_small], dn[:n_small], "bf16", T,
                   label=f"both variants, small grid T={T} amax={want_amax}")
    np.testing.assert_allclose(part["alpha"], full["alpha"][:n_small], rtol=1e-5)
    if want_amax:
        for key in ("amax_t", "amax_d"):
            assert np.array_equal(part[key], full[key][:n_small])


@pytest.mark.parametrize("tdt,ddt,T,want_amax", [("f32", "f32", 0.9, False), ("f32", "f32", 1.7, True),
                                                  ("bf16", "f32", 0.9, True), ("f32", "bf16", 0.9, False)])
def test_fp32_and_mixed_logits_large_grid(sv, tdt, ddt, T, want_amax):
    """binary32 and mixed-dtype logits in a grid above the kept-term threshold (64 x 16 rows of
    a ragged vocabulary 9001 in rows padded to 9008), so the 96-register instances run; the
    small fp32 cases elsewhere run the kept-term ones."""
    B, K, V, ld = 64, 16, 9001, 9008
    assert (B * K + B) * 1 + B > _keep_limit()
    g = torch.Generator(device=DEV).manual_seed(23)
    tt_ = torch.bfloat16 if tdt == "bf16" else torch.float32
    dt_ = torch.bfloat16 if ddt == "bf16" else torch.float32
    tt = torch.full((B, K + 1, ld), float("nan"), device=DEV, dtype=tt_)
    dd = torch.full((B, K, ld), float("nan"), device=DEV, dtype=dt_)
    t = 2.5 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    d = t[:, :K] + 0.8 * torch.randn((B, K, V), generator=g, device=DEV)
    tt[..., :V] = t.to(tt_)
    dd[..., :V] = d.to(dt_)
    toks = torch.argmax(d, -1).to(torch.int32)
    toks[:, 2] = torch.randint(0, V, (B,), generator=g, device=DEV, dtype=torch.int32)
    _say(f"large-grid {tdt}/{ddt} T={T} amax={want_amax}")
    out = _np(sv.sv_verify_batch(tt[..., :V], dd[..., :V], toks, T, seed=4, step=2, want_amax=want_amax))
    # bfloat16 values are exact in binary32: the oracle takes both rows as binary32
    tn = tt[..., :V].float().cpu().numpy()
    dn = dd[..., :V].float().cpu().numpy()
    o = svref.verify_batch(tn, dn, toks.cpu().numpy(), T, "f32", seed=4, step=2, diagnostics=True)
    _say(f"report {compare_verify(out, o, tn, dn, 'f32', T, label=f'large grid {tdt}/{ddt} T={T}')}")


def test_graph_replay_matches_eager(sv):
    """One verification call captured in a HIP graph and replayed: the call epoch lives on the
    device, so every replay tags its words afresh.  Each replay (outputs cleared first) equals
    the eager call, with other eager calls on the same workspace and synchronizations between
    the replays."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=8)
    B, K, V = 8, 16, v.target.shape[2]
    ref = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=5, step=3, want_amax=True))
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, V)
    out = sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=5, step=3, workspace=buf, want_amax=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.9, seed=5, step=3, workspace=buf, out=out,
                           want_amax=True)
    torch.cuda.synchronize()
    for rep in range(4):
        _say(f"graph replay {rep}")
        for t in out.values():
            if t is not None:
                t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = _np(out)
        for key in ref:
            if ref[key] is not None:
                assert np.array_equal(got[key], ref[key]), (rep, key)
        # eager work on the same workspace between the replays
        sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, 0.0 if rep % 2 else 0.9, seed=9, step=rep + 10,
                           workspace=buf)
        torch.cuda.synchronize()
    assert sv.sv_device_error(buf) == 0


def test_selected_row_left_out_is_flagged(sv):
    """A row list that leaves out a row its lengths include: that row is never streamed, so
    the request's finalize workgroup waits out its bound (about 20 ms per wait, two waits)
    and flags the call.  The next call on the same workspace is unaffected."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=4, K=4, V=20000)
    B, K = 4, 4
    lens = torch.tensor([3, 1, 4, 2], dtype=torch.int32, device=DEV)
    full = [r * K + k for r in range(B) for k in range(int(lens[r]))]
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, 20000)
    left = [f for f in full if f != 2 * K + 1]   # request 2 loses its row 1
    rl = torch.tensor(left, dtype=torch.int32, device=DEV)
    _say("selected verify, one row left out")
    sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, 0.9, lens, rl, len(left), seed=3, workspace=buf)
    flags = sv.sv_device_error(buf)
    assert flags & 2, flags
    rl = torch.tensor(full, dtype=torch.int32, device=DEV)
    _say("selected verify, full list, same workspace")
    a = _np(sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, 0.9, lens, rl, len(full), seed=3,
                                  want_amax=True, workspace=buf))
    b = _np(sv.sv_verify_selected(v.target, v.draft, v.draft_tokens, 0.9, lens, rl, len(full), seed=3,
                                  want_amax=True))
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k
    assert sv.sv_device_error(buf) == 0


def test_workspace_reuse_across_calls_and_modes(sv):
    """One workspace, many calls (the per-call epoch advances inside the kernel): every
    call equals the same call on a fresh workspace."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=6)
    t2, d2, _ = workloads.make_e2e_inputs(device=DEV, I=5, D=3, V=131072, seed=8)
    ws = sv.Workspace(DEV)
    buf = ws.get(64, 16, 131072)
    plan = [(0.9, None, 0), (0.0, None, 1), (0.9, [3, 0, 16, 1, 7, 2], 2), ("e2e", None, 0), (1.3, None, 3),
            ("sample", 0.9, 6), (0.9, [16, 16, 0, 0, 5, 9], 4), ("sample", 0.0, 7), (0.0, [2, 0, 1, 16, 16, 3], 5),
            ("e2e", None, 0), (0.9, None, 0)]
    for i, (T, dl, step) in enumerate(plan):
        _say(f"reuse call {i}: T={T} dl={dl}")
        if T == "e2e":
            l1, a1 = sv.sv_tv_e2e_loss(t2, d2, 1.0, workspace=buf)
            l2, a2 = sv.sv_tv_e2e_loss(t2, d2, 1.0)
            assert torch.equal(a1, a2) and torch.equal(l1, l2)
            continue
        if T == "sample":   # the draft sampler on the same workspace (its own one-kernel call)
            x1, c1 = sv.sv_sample_drafts(v.draft, dl, seed=7, step=step, workspace=buf)
            x2, c2 = sv.sv_sample_drafts(v.draft, dl, seed=7, step=step)
            assert torch.equal(x1, x2) and torch.equal(c1, c2)
            continue
        dlt = None if dl is None else torch.tensor(dl, dtype=torch.int32, device=DEV)
        a = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=7, step=step, draft_len=dlt,
                                   workspace=buf, want_amax=True))
        b = _np(sv.sv_verify_batch(v.target, v.draft, v.draft_tokens, T, seed=7, step=step, draft_len=dlt,
                                   want_amax=True))
        for k in a:
            assert np.array_equal(a[k], b[k]), (i, k)
    assert sv.sv_device_error(buf) == 0


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_all_accepted_bonus_token(sv, T):
    """Drafter logits equal to the target's: every draft is accepted (u < p/q = 1) and the
    bonus token is drawn from the target row at L_r, for dense and ragged lengths."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=T, B=6)
    draft = v.target[:, :-1].contiguous()
    z = draft.float()
    if T > 0:
        g = torch.Generator(device=DEV).manual_seed(5)
        u = torch.rand(z.shape, generator=g, device=DEV).clamp_(min=1e-20)
        z = z / T - torch.log(-torch.log(u))
    toks = torch.argmax(z, -1).to(torch.int32)
    w = workloads.VerifyInputs(v.target, draft, toks, T, v.seed, "dfly-all-accepted")
    g_, o, rep = _run_pair(sv, w, T)
    assert (o["accept_len"] == 16).all()
    dl = np.array([16, 0, 5, 1, 16, 9], np.int32)
    g2, o2, rep2 = _run_pair(sv, w, T, draft_len=dl)
    assert (o2["accept_len"] == dl).all()


# ---- edge cases ----------------------------------------------------------------------

def _custom(t, d, toks, T, name, seed=13):
    return workloads.VerifyInputs(t.contiguous(), d.contiguous(), toks.to(torch.int32).contiguous(), T, seed, name)


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_no_drafts_only_bonus(sv, T):
    """K_max = 0: nothing to verify, every request emits its bonus token from target row 0."""
    g = torch.Generator(device=DEV).manual_seed(31)
    B, V = 5, 3000
    t = (2.0 * torch.randn((B, 1, V), generator=g, device=DEV)).to(torch.bfloat16)
    d = torch.empty((B, 0, V), dtype=torch.bfloat16, device=DEV)
    toks = torch.empty((B, 0), dtype=torch.int32, device=DEV)
    _, o, _ = _run_pair(sv, _custom(t, d, toks, T, "K=0"), T)
    assert (o["accept_len"] == 0).all()
    # the stand-alone draw with no drafts: the bonus token from target row 0
    tok = sv.sv_residual_sample(t, d, torch.zeros((B,), dtype=torch.int32, device=DEV), T, seed=13).cpu().numpy()
    tn, dn = workloads.to_oracle(t), workloads.to_oracle(d)
    otok = svref.residual_sample(tn, dn, np.zeros(B, np.int32), T, "bf16", seed=13)
    assert np.array_equal(otok, o["out_tokens"][:, 0])
    for r in range(B):
        assert tok[r] == otok[r] or (T > 0 and _token_in_band(tn, dn, T, "bf16", r, 0, 0, int(tok[r]), int(otok[r]),
                                                              13, 0)), (r, tok[r], otok[r])


@pytest.mark.parametrize("V", [1, 7, 8, 4095, 4097])
def test_tiny_and_boundary_vocabularies(sv, V):
    """A single token, fewer logits than one 8-wide load, and sizes around a wave range."""
    g = torch.Generator(device=DEV).manual_seed(V)
    B, K = 3, 4
    ld = (V + 7) // 8 * 8
    tt = torch.full((B, K + 1, ld), float("nan"), device=DEV, dtype=torch.float32)
    dd = torch.full((B, K, ld), float("nan"), device=DEV, dtype=torch.float32)
    tt[..., :V] = 1.5 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    dd[..., :V] = tt[:, :K, :V] + 0.8 * torch.randn((B, K, V), generator=g, device=DEV)
    toks = torch.randint(0, V, (B, K), generator=g, device=DEV, dtype=torch.int32)
    for T in (1.0, 0.0):
        _say(f"vocab V={V} T={T}")
        out = _np(sv.sv_verify_batch(tt[..., :V], dd[..., :V], toks, T, seed=2, want_amax=True))
        tn, dn = workloads.to_oracle(tt[..., :V].contiguous()), workloads.to_oracle(dd[..., :V].contiguous())
        o = svref.verify_batch(tn, dn, toks.cpu().numpy(), T, "f32", seed=2, diagnostics=True)
        compare_verify(out, o, tn, dn, "f32", T, label=f"vocab V={V} T={T}")
        if V == 1:
            assert (o["accept_len"] == K).all() and np.allclose(o["alpha"], 1.0)


def test_largest_vocabulary(sv):
    """V = SV_V_MAX (2^20): 64 members per row."""
    g = torch.Generator(device=DEV).manual_seed(77)
    B, K, V = 2, 2, 1 << 20
    t = (3.0 * torch.randn((B, K + 1, V), generator=g, device=DEV)).to(torch.bfloat16)
    d = (t[:, :K].float() + torch.randn((B, K, V), generator=g, device=DEV)).to(torch.bfloat16)
    toks = torch.argmax(d.float(), -1).to(torch.int32)
    toks[:, 1] = torch.randint(0, V, (B,), generator=g, device=DEV, dtype=torch.int32)
    tn, dn = workloads.to_oracle(t), workloads.to_oracle(d)
    for T in (0.9, 0.0):
        _, o, _ = _run_pair(sv, _custom(t, d, toks, T, "V=2^20"), T)
        # the stand-alone draw at every accepted length 0..K (a correction, or the bonus at K)
        for tau in range(K + 1):
            al = np.full(B, tau, np.int32)
            tok = sv.sv_residual_sample(t, d, torch.as_tensor(al, device=DEV), T, seed=13).cpu().numpy()
            otok = svref.residual_sample(tn, dn, al, T, "bf16", seed=13)
            for r in range(B):
                assert tok[r] == otok[r] or (T > 0 and _token_in_band(tn, dn, T, "bf16", r, tau, K, int(tok[r]),
                                                                      int(otok[r]), 13, 0)), (T, tau, r)


@pytest.mark.parametrize("K", [300, 4096])
@pytest.mark.parametrize("T,want_amax", [(0.9, False), (0.9, True), (0.0, True)])
def test_longest_drafts(sv, K, T, want_amax):
    """Draft blocks of 300 and SV_K_MAX = 4096 positions with long accepted prefixes: the
    finalize stages its rows in several batches and, past 255 positions, computes the draw's
    uniform for the scanned tau on demand.  Request 0 has a certain reject at 3/4 of its block
    (the target masks the drafted token there), request 1 accepts every draft (bonus row K),
    request 2 follows the target up to position 260 and an independent drafter after it."""
    g = torch.Generator(device=DEV).manual_seed(K + int(10 * T))
    B, V = 3, 2000
    t = (2.0 * torch.randn((B, K + 1, V), generator=g, device=DEV)).to(torch.bfloat16)
    d = t[:, :K].clone()
    d[2, 260:] = (2.0 * torch.randn((K - 260, V), generator=g, device=DEV)).to(torch.bfloat16)
    z = d.float()
    if T > 0:
        u = torch.rand(z.shape, generator=g, device=DEV).clamp_(min=1e-20)
        z = z / T - torch.log(-torch.log(u))
    toks = torch.argmax(z, -1).to(torch.int32)
    k0 = 3 * K // 4
    t[0, k0, toks[0, k0]] = float("-inf")
    w = _custom(t, d, toks, T, f"long drafts K={K}", seed=K)
    _, o, _ = _run_pair(sv, w, T, want_amax=want_amax)
    assert o["accept_len"][0] == k0 and o["accept_len"][1] == K and o["accept_len"][2] >= 260
    dl = np.array([K, K - 37, 290], np.int32)
    _, o2, _ = _run_pair(sv, w, T, draft_len=dl, want_amax=want_amax)
    assert o2["accept_len"][0] == k0 and o2["accept_len"][1] == K - 37 and o2["accept_len"][2] >= 260


BIG_LD = (1 << 20) + 8   # a row stride of 2 MiB + 16 bytes (bfloat16): row 1024 starts past 2^31 bytes


def _big_stride(x):
    """x [..., V] copied into rows of stride BIG_LD on the GPU (padding left uninitialised,
    never read): rows past the first 1024 sit beyond 2^31 bytes from the start."""
    buf = torch.empty(x.shape[:-1] + (BIG_LD,), dtype=x.dtype, device=DEV)
    buf[..., :x.shape[-1]] = x.to(DEV)
    return buf[..., :x.shape[-1]]


@pytest.mark.parametrize("T,want_amax", [(0.9, False), (0.9, True), (0.0, True)])
def test_rows_beyond_2gib(sv, T, want_amax):
    """Row offsets past 2^31 bytes (3 requests x 700 drafts in rows of a 2 MiB stride, 4.4 GB
    per tensor): every row address is 64-bit.  Request 1 accepts up to a certain reject at
    position 600 (row 1301, beyond 2 GiB: its residual draw reads there); request 2 accepts
    every draft (its bonus row 2102); dense and ragged lengths."""
    g = torch.Generator().manual_seed(1 << 20)
    B, K, V = 3, 700, 1000
    t = (2.0 * torch.randn((B, K + 1, V), generator=g)).to(torch.bfloat16)
    d = (t[:, :K].float() + 0.5 * torch.randn((B, K, V), generator=g)).to(torch.bfloat16)
    d[1, :600] = t[1, :600]
    d[2] = t[2, :K]
    z = d.float()
    if T > 0:
        u = torch.rand(z.shape, generator=g).clamp_(min=1e-20)
        z = z / T - torch.log(-torch.log(u))
    toks = torch.argmax(z, -1).to(torch.int32)
    t[1, 600, toks[1, 600]] = float("-inf")
    w = workloads.VerifyInputs(_big_stride(t), _big_stride(d), toks.to(DEV), T, 9, "rows beyond 2 GiB")
    assert w.target.stride(1) == BIG_LD and (B * (K + 1) - 1) * BIG_LD * 2 > (1 << 31)
    _, o, _ = _run_pair(sv, w, T, want_amax=want_amax)
    assert o["accept_len"][1] == 600 and o["accept_len"][2] == K
    dl = np.array([K, 650, K - 1], np.int32)
    _, o2, _ = _run_pair(sv, w, T, draft_len=dl, want_amax=want_amax)
    assert o2["accept_len"][1] == 600 and o2["accept_len"][2] == K - 1
    # the stand-alone draw at the oracle's accepted lengths reads the same far rows
    if not want_amax:
        tn, dn = workloads.to_oracle(w.target), workloads.to_oracle(w.draft)
        al = o2["accept_len"].astype(np.int32)
        tok = sv.sv_residual_sample(w.target, w.draft, torch.as_tensor(al, device=DEV), T, seed=9,
                                    draft_len=torch.as_tensor(dl, device=DEV)).cpu().numpy()
        otok = svref.residual_sample(tn, dn, al, T, "bf16", seed=9, draft_len=dl)
        for r in range(B):
            assert tok[r] == otok[r] or _token_in_band(tn, dn, T, "bf16", r, int(al[r]), int(dl[r]), int(tok[r]),
                                                       int(otok[r]), 9, 0), (r, tok[r], otok[r])


def test_two_streams_at_once(sv):
    """Verification calls issued together on two streams, each with its own workspace, eight
    rounds (where the device runs the two grids at once they compete for the CUs; a team
    member that cannot get a slot is covered by the bounded wait and its hand-over): both
    match the oracle and neither workspace reports a device error."""
    va = workloads.make_verify_inputs("dfly", device=DEV, T=0.9, B=24, seed=101)
    vb = workloads.make_verify_inputs("mtp", device=DEV, T=0.9, B=40, seed=202)
    wa, wb = sv.Workspace(DEV), sv.Workspace(DEV)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for it in range(8):
        _say(f"two streams, round {it}")
        with torch.cuda.stream(sa):
            oa = sv.sv_verify_batch(va.target, va.draft, va.draft_tokens, 0.9, seed=va.seed, step=it, workspace=wa,
                                    stream=sa)
        with torch.cuda.stream(sb):
            ob = sv.sv_verify_batch(vb.target, vb.draft, vb.draft_tokens, 0.9, seed=vb.seed, step=it, workspace=wb,
                                    stream=sb)
        outs.append((it, oa, ob))
    torch.cuda.synchronize()
    assert sv.sv_device_error(wa.buf) == 0 and sv.sv_device_error(wb.buf) == 0
    for v, k in ((va, 1), (vb, 2)):
        tn, dn = workloads.to_oracle(v.target), workloads.to_oracle(v.draft)
        for it in (0, 7):
            o = svref.verify_batch(tn, dn, v.draft_tokens.cpu().numpy(), 0.9, "bf16", seed=v.seed, step=it,
                                   diagnostics=True)
            compare_verify(_np(outs[it][k]), o, tn, dn, "bf16", 0.9, label=f"two streams {v.name} step {it}")


def test_stream_read_covers_every_word(sv):
    """The read-only streaming reference reads every 16-byte word: a single word holding its
    sink value (the rest zero) reaches the sink wherever it sits, including the ragged last
    workgroup; an all-zero buffer leaves the sink untouched."""
    marker = 0x9E3779B9
    n16 = 2048 * 3 + 5                        # three full workgroups of 2048 words and five more
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    sv.sv_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 0
    for word in (0, 1, 255, 256, 2047, 2048, 4100, n16 - 5, n16 - 1):
        for comp in (0, 3):
            _say(f"stream_read word {word} component {comp}")
            buf.zero_()
            sink.zero_()
            buf[4 * word + comp] = marker - (1 << 32)   # the same 32 bits as a signed int32
            sv.sv_stream_read(buf, sink)
            torch.cuda.synchronize()
            assert int(sink[0].item()) & 0xFFFFFFFF == marker, (word, comp)


def test_empty_batches(sv):
    """Empty batches through every entry point: no requests (B = 0), no draft positions
    (K = 0) for the budget and the sampler, no counters.  Verification returns empty outputs;
    the budget and the D-cut choice equal the oracle's (row_off = [0] for no requests); an
    L_e2e over an empty set is refused (its mean is undefined)."""
    V = 1000
    t = torch.zeros((0, 4, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((0, 3, V), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((0, 3), dtype=torch.int32, device=DEV)
    ws = sv.Workspace(DEV)
    for T in (0.9, 0.0):
        _say(f"empty verify T={T}")
        outs = [sv.sv_verify_batch(t, d, x, T, want_amax=True, workspace=ws),
                sv.sv_verify_batch_noalloc(t, d, x, T, want_amax=True),
                sv.sv_verify_selected(t, d, x, T, torch.zeros((0,), dtype=torch.int32, device=DEV), None, 0,
                                      want_amax=True, workspace=ws)]
        for o in outs:
            assert o["alpha"].shape == (0, 3) and o["out_tokens"].shape == (0, 4) and o["n_out"].shape == (0,)
    torch.cuda.synchronize()
    assert sv.sv_device_error(ws.get(0, 3, V)) == 0
    _say("empty accept_len, residual_sample, sample_drafts, uniforms")
    assert sv.sv_accept_len(torch.zeros((0, 3), dtype=torch.uint8, device=DEV)).shape == (0,)
    assert sv.sv_residual_sample(t, d, torch.zeros((0,), dtype=torch.int32, device=DEV), 0.9).shape == (0,)
    for dd in (d, torch.zeros((2, 0, V), dtype=torch.bfloat16, device=DEV)):
        tok, conf = sv.sv_sample_drafts(dd, 0.9)
        assert tok.shape == dd.shape[:2] and conf.shape == dd.shape[:2]
    assert sv.sv_uniforms(1, torch.zeros((0, 4), dtype=torch.int64, device=DEV)).shape == (0,)
    cost = (40.0 + 0.05 * np.arange(9)).astype(np.float32)
    for shape in [(0, 4), (3, 0)]:
        _say(f"empty budget {shape}")
        conf = np.zeros(shape, np.float32)
        lens, off, _ = sv.sv_alloc_verify_budget(torch.as_tensor(conf, device=DEV), 10)
        ol, oo, _ = svref.alloc_verify_budget(conf, 10)
        assert np.array_equal(lens.cpu().numpy(), ol) and np.array_equal(off.cpu().numpy(), oo)
        n, u, lens, off, _ = sv.sv_dcut_verify_budget(torch.as_tensor(conf, device=DEV), torch.as_tensor(cost, device=DEV))
        on, ou, ol, oo, _ = svref.dcut_budget(conf, cost)
        assert int(n.item()) == on and float(u.item()) == ou
        assert np.array_equal(lens.cpu().numpy(), ol) and np.array_equal(off.cpu().numpy(), oo)
    with pytest.raises(sv.SVError):
        sv.sv_tv_e2e_loss(torch.zeros((0, 3, V), dtype=torch.bfloat16, device=DEV),
                          torch.zeros((0, 3, V), dtype=torch.bfloat16, device=DEV), 1.0)


@pytest.mark.parametrize("T,want_amax", [(0.9, False), (0.9, True), (0.0, True)])
def test_largest_vocabulary_full_block(sv, T, want_amax):
    """V = 2^20 (64 members a row) with blocks of 16: a row then carries 256 directory words
    and the finalize stages its rows in batches of 12 (6 with argmax outputs), so a block
    takes two or three batches at the largest team.  Request 3 drafts with the target's own
    logits (every draft accepted, its bonus drawn from the 64-member bonus slot)."""
    v = workloads.make_verify_inputs("dfly", device=DEV, T=T, B=4, V=1 << 20, seed=77)
    d = v.draft.clone()
    d[3] = v.target[3, :-1]
    toks = v.draft_tokens.clone()
    z = d[3].float()
    if T > 0:
        g = torch.Generator(device=DEV).manual_seed(78)
        u = torch.rand(z.shape, generator=g, device=DEV).clamp_(min=1e-20)
        z = z / T - torch.log(-torch.log(u))
    toks[3] = torch.argmax(z, -1).to(torch.int32)
    w = workloads.VerifyInputs(v.target, d, toks, T, v.seed, "V=2^20 block 16")
    _, o, _ = _run_pair(sv, w, T, want_amax=want_amax)
    assert o["accept_len"][3] == 16


def _grid(B, K, V):
    """Workgroups of a dense verification grid: members of every row and bonus slot, then the
    finalize workgroups."""
    return (B * K + B) * ((V + 16383) // 16384) + B


@pytest.mark.parametrize("want_amax", [False, True])
@pytest.mark.parametrize("B", [4, 64])
def test_masked_logits(sv, B, want_amax):
    """-inf logits (masked vocabulary): p or q is exactly 0 there; drafted tokens inside the
    target's mask are always rejected, and no emitted token is a masked one.  B = 4 runs the
    kept-term instance, B = 64 (832 workgroups) the other; in both, the drafter's wave range
    [8192, 12288) starts with 512 masked logits, so the wave's first logit is -inf, its
    provisional reference is -inf and the exact-maximum fallback runs.  That holds without
    argmax outputs (want_amax False), where pass 1 takes the provisional first-logit reference;
    with them, pass 1 takes the exact maxima and no fallback is needed."""
    g = torch.Generator(device=DEV).manual_seed(5)
    K, V = 5, 20000
    assert (_grid(B, K, V) > _keep_limit()) == (B == 64)
    t = 2.0 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    d = t[:, :K] + torch.randn((B, K, V), generator=g, device=DEV)
    t[..., 5000:9000] = float("-inf")
    d[..., 8000:12000] = float("-inf")
    t[:, :, 15000] = float("-inf")
    t, d = t.to(torch.bfloat16), d.to(torch.bfloat16)
    toks = torch.randint(0, V, (B, K), generator=g, device=DEV, dtype=torch.int32)
    toks[:, 0] = 6000            # masked in the target only: p = 0 -> reject
    toks[:, 2] = 8500            # masked in both
    for T in (0.9, 0.0):
        gg, o, _ = _run_pair(sv, _custom(t, d, toks, T, "masked"), T, want_amax=want_amax or T == 0)
        emitted = [gg["out_tokens"][r, gg["accept_len"][r]] for r in range(B)]
        assert all(not (5000 <= x < 9000) and x != 15000 for x in emitted)
        if T > 0:
            assert (gg["accept"][:, 0] == 0).all()


@pytest.mark.parametrize("low", [-3.0, -25.0])
@pytest.mark.parametrize("B", [4, 64])
def test_low_reference_logit(sv, B, low):
    """Every wave range (4096 logits) starts with a logit below the rest of its row, and that
    first logit is the provisional pass-1 reference of its wave.  The wave maxima lie near 6
    (1.5 sigma times ~4), so at T = 0.3 (c = 4.81) -3 leaves the lane sums near 2^45, inside
    range with the largest terms' exponents near 45, and -25 takes them past 2^64, so each wave
    falls back to its exact maximum; at T = 0.9 (c = 1.60) both stay in range, -25 with sums
    near 2^50.  B = 4 runs the kept-term instance, B = 64 the other."""
    g = torch.Generator(device=DEV).manual_seed(11)
    K, V = 4, 40000
    assert (_grid(B, K, V) > _keep_limit()) == (B == 64)
    t = 1.5 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    d = t[:, :K] + 0.5 * torch.randn((B, K, V), generator=g, device=DEV)
    t[..., ::4096] = low
    d[..., ::4096] = low
    t, d = t.to(torch.bfloat16), d.to(torch.bfloat16)
    toks = torch.randint(0, V, (B, K), generator=g, device=DEV, dtype=torch.int32)
    for T in (0.3, 0.9):
        _run_pair(sv, _custom(t, d, toks, T, f"low first logit {low}"), T, want_amax=False)


@pytest.mark.parametrize("want_amax", [False, True])
@pytest.mark.parametrize("T,B", [(0.005, 4), (0.02, 4), (25.0, 4), (0.005, 48), (0.02, 48)])
def test_extreme_temperatures(sv, T, B, want_amax):
    """Very low temperatures (base-2 normalisers of several hundred to a few thousand, past
    what one binary32 value holds to 1e-5, and sums far from the provisional reference: the
    exact-maximum fallback when pass 1 takes the provisional first-logit reference, i.e. without
    argmax outputs) and a very high one (nearly uniform rows).  B = 4 runs the kept-term
    instance, B = 48 (816 workgroups) the other."""
    assert (_grid(B, 3, 50000) > _keep_limit()) == (B == 48)
    v = _move(workloads.make_verify_inputs("mtp", device="cpu", T=T, B=B, K=3, V=50000))
    _run_pair(sv, v, T, want_amax=want_amax)


def test_argmax_ties_lowest_index(sv):
    """Greedy: equal maxima in a row resolve to the lowest index on both sides."""
    g = torch.Generator(device=DEV).manual_seed(3)
    B, K, V = 3, 4, 40000
    t = torch.randn((B, K + 1, V), generator=g, device=DEV)
    d = t[:, :K].clone()
    for r in range(B):
        for k in range(K + 1):
            t[r, k, [777 + 5000 * k, 39999, 20000]] = 9.0      # three-way tie
        for k in range(K):
            d[r, k, [300, 31000]] = 9.0
    t, d = t.to(torch.bfloat16), d.to(torch.bfloat16)
    toks = torch.full((B, K), 777, dtype=torch.int32, device=DEV)
    gg, o, _ = _run_pair(sv, _custom(t, d, toks, 0.0, "ties"), 0.0)
    assert (gg["amax_t"][:, 0] == 777).all() and (gg["amax_d"] == 300).all()


def test_many_requests_short_drafts(sv):
    """B = 300 requests of one draft each (grid mapping over many requests)."""
    v = _move(workloads.make_verify_inputs("mtp", device="cpu", T=0.9, B=300, K=1, V=5000))
    for T in (0.9, 0.0):
        _run_pair(sv, v, T)
