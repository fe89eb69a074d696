"""sv_verify_batch_noalloc (the entry point whose workspace is the library's own per-device
array) against sv_verify_batch on a workspace of its own: bit-identical outputs on two calls
in a row, the second with a smaller input; inputs beyond the array's size rejected with
nothing launched."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sv():
    import draft_verification_softmax_amd as m
    return m


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _case(name, B, K, V, seed, T, ragged):
    v = workloads.make_verify_inputs(name, device="cpu", T=T, B=B, K=K, V=V, seed=seed)
    t, d, x = v.target.to(DEV), v.draft.to(DEV), v.draft_tokens.to(DEV)
    dl = None
    if ragged:
        g = torch.Generator().manual_seed(seed)
        dl = torch.randint(0, K + 1, (B,), generator=g, dtype=torch.int32).to(DEV)
    return t, d, x, dl


def _np(out):
    return {k: (None if v is None else v.cpu().numpy().copy()) for k, v in out.items()}


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_noalloc_matches_verify_batch_on_two_calls(sv, T):
    cases = [("dfly", 24, 16, 131072, 51, True),   # larger first: 24 x 17 rows of 131072
             ("mtp", 5, 3, 40000, 52, False)]       # then a smaller one, different shape
    for name, B, K, V, seed, ragged in cases:
        _say(f"noalloc vs verify_batch {name} B={B} K={K} V={V} T={T} ragged={ragged}")
        t, d, x, dl = _case(name, B, K, V, seed, T, ragged)
        kw = dict(seed=seed, step=3, draft_len=dl, want_amax=True)
        want = _np(sv.sv_verify_batch(t, d, x, T, workspace=sv.Workspace(DEV), **kw))
        got = _np(sv.sv_verify_batch_noalloc(t, d, x, T, **kw))
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=f"{name} {k}")
        assert sv.sv_device_error(None) == 0


def test_noalloc_rejects_inputs_beyond_its_array(sv):
    B, K, V = 8192, 15, 16   # 21.6 MiB of workspace > 16 MiB
    assert sv.sv_workspace_bytes(B, K, V) > sv.SV_NOALLOC_SCRATCH_BYTES
    _say(f"noalloc rejects B={B} K={K} V={V}")
    t = torch.zeros((B, K + 1, V), dtype=torch.float32, device=DEV)
    d = torch.zeros((B, K, V), dtype=torch.float32, device=DEV)
    x = torch.zeros((B, K), dtype=torch.int32, device=DEV)
    out = dict(alpha=torch.full((B, K), 7.0, device=DEV), accept=torch.full((B, K), 7, dtype=torch.uint8, device=DEV),
               lse_t=None, lse_d=None, amax_t=None, amax_d=None,
               accept_len=torch.full((B,), 7, dtype=torch.int32, device=DEV),
               out_tokens=torch.full((B, K + 1), 7, dtype=torch.int32, device=DEV),
               n_out=torch.full((B,), 7, dtype=torch.int32, device=DEV))
    with pytest.raises(sv.SVError) as e:
        sv.sv_verify_batch_noalloc(t, d, x, 1.0, out=out)
    assert "SV_EWORKSPACE" in str(e.value)
    torch.cuda.synchronize()
    assert (out["alpha"] == 7.0).all() and (out["n_out"] == 7).all()   # nothing launched
