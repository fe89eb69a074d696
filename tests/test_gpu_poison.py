"""A poisoned workspace (the state a call leaves after one of its bounded waits gave up),
forced from the host by writing the epoch word, never by provoking a timeout: verification
and sampling then verify (sample) nothing and raise SV_DEVERR_POISONED; sv_device_error
zero-fills the workspace again, after which results are those of a clean workspace; L_e2e
runs as usual on it."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPOCH_WORD = 64 // 4          # the epoch: byte 64 of the workspace header, as int32 words
POISONED_EPOCH = -(2**31) + 5   # 0x80000005: poison bit and tag bits


@pytest.fixture(scope="module")
def sv():
    import draft_verification_softmax_amd as m
    return m


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _poison(buf):
    buf.view(torch.int32)[EPOCH_WORD] = POISONED_EPOCH
    torch.cuda.synchronize()


def _epoch(buf):
    torch.cuda.synchronize()
    return int(buf.view(torch.int32)[EPOCH_WORD].item()) & 0xffffffff


def _np(out):
    return {k: (None if v is None else v.cpu().numpy().copy()) for k, v in out.items()}


def _inputs():
    v = workloads.make_verify_inputs("dfly", device="cpu", B=5, K=4, V=40000, seed=41)
    return v.target.to(DEV), v.draft.to(DEV), v.draft_tokens.to(DEV)


@pytest.mark.parametrize("T", [0.9, 0.0])
def test_poisoned_workspace_verifies_nothing_until_reinitialised(sv, T):
    _say(f"poisoned verify T={T}")
    t, d, x = _inputs()
    B, K = x.shape
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, t.shape[2])
    kw = dict(seed=3, step=1, want_amax=True, workspace=ws)
    clean = _np(sv.sv_verify_batch(t, d, x, T, **kw))
    assert sv.sv_device_error(buf) == 0
    assert clean["n_out"].min() >= 1

    _poison(buf)
    got = _np(sv.sv_verify_batch(t, d, x, T, **kw))
    assert (got["accept_len"] == 0).all() and (got["n_out"] == 0).all()
    assert (got["out_tokens"] == -1).all()
    assert (got["alpha"] == 0).all() and (got["accept"] == 0).all()
    assert (got["lse_t"] == 0).all() and (got["lse_d"] == 0).all()
    assert (got["amax_t"] == -1).all() and (got["amax_d"] == -1).all()
    assert _epoch(buf) == POISONED_EPOCH & 0xffffffff   # a poisoned call leaves the epoch alone
    flags = sv.sv_device_error(buf)
    assert flags == sv.SV_DEVERR_POISONED
    assert _epoch(buf) == 0   # zero-filled again

    again = _np(sv.sv_verify_batch(t, d, x, T, **kw))
    assert sv.sv_device_error(buf) == 0
    for k in clean:
        np.testing.assert_array_equal(again[k], clean[k], err_msg=k)


def test_poison_stays_until_init_for_a_workspace_zeroed_elsewhere(sv):
    """A workspace zero-filled by the caller (no recorded size): sv_device_error clears the
    flag only, the next call is poisoned again, sv_workspace_init recovers."""
    _say("poisoned verify, caller-zeroed workspace")
    t, d, x = _inputs()
    B, K = x.shape
    buf = torch.zeros(sv.sv_workspace_bytes(B, K, t.shape[2]), dtype=torch.uint8, device=DEV)
    clean = _np(sv.sv_verify_batch(t, d, x, 0.9, seed=3, workspace=buf))
    assert sv.sv_device_error(buf) == 0
    _poison(buf)
    for _ in range(2):
        got = _np(sv.sv_verify_batch(t, d, x, 0.9, seed=3, workspace=buf))
        assert (got["n_out"] == 0).all()
        assert sv.sv_device_error(buf) == sv.SV_DEVERR_POISONED
    sv.sv_workspace_init(buf)
    again = _np(sv.sv_verify_batch(t, d, x, 0.9, seed=3, workspace=buf))
    assert sv.sv_device_error(buf) == 0
    for k in clean:
        np.testing.assert_array_equal(again[k], clean[k], err_msg=k)


@pytest.mark.parametrize("T", [0.8, 0.0])
def test_poisoned_workspace_samples_nothing(sv, T):
    _say(f"poisoned sampling T={T}")
    _, d, _ = _inputs()
    B, K, V = d.shape
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, V)
    tok0, conf0 = sv.sv_sample_drafts(d, T, seed=9, workspace=ws)
    tok0, conf0 = tok0.cpu(), conf0.cpu()
    assert sv.sv_device_error(buf) == 0
    _poison(buf)
    tok, conf = sv.sv_sample_drafts(d, T, seed=9, workspace=ws)
    assert (tok.cpu() == -1).all() and (conf.cpu() == 0).all()
    assert sv.sv_device_error(buf) == sv.SV_DEVERR_POISONED
    tok, conf = sv.sv_sample_drafts(d, T, seed=9, workspace=ws)
    assert sv.sv_device_error(buf) == 0
    assert torch.equal(tok.cpu(), tok0) and torch.equal(conf.cpu(), conf0)


def test_e2e_runs_on_a_poisoned_workspace(sv):
    """L_e2e and its gradient have no workgroup that reads the epoch after it advances: they
    run as usual on a poisoned workspace and leave the poison for the next verification."""
    _say("L_e2e on a poisoned workspace")
    t, d, _ = _inputs()
    t, d = t[:, :4].contiguous(), d.contiguous()
    I, D, V = d.shape
    ws = sv.Workspace(DEV)
    buf = ws.get(I, D, V)
    loss0, alpha0 = sv.sv_tv_e2e_loss(t, d, 1.0, workspace=ws)
    g0 = sv.sv_tv_e2e_backward(t, d, alpha0, 1.0, grad_dtype=torch.float32, workspace=ws)
    loss0, alpha0, g0 = loss0.cpu(), alpha0.cpu(), g0.cpu()
    assert sv.sv_device_error(buf) == 0
    _poison(buf)
    loss, alpha = sv.sv_tv_e2e_loss(t, d, 1.0, workspace=ws)
    g = sv.sv_tv_e2e_backward(t, d, alpha, 1.0, grad_dtype=torch.float32, workspace=ws)
    assert torch.equal(loss.cpu(), loss0) and torch.equal(alpha.cpu(), alpha0) and torch.equal(g.cpu(), g0)
    assert sv.sv_device_error(buf) == 0
    assert _epoch(buf) & 0x80000000   # still poisoned
    sv.sv_workspace_init(buf)
    assert _epoch(buf) == 0


def test_size_record_without_its_complement_is_not_trusted(sv):
    """sv_device_error zero-fills again only a workspace whose recorded byte count sits next
    to its complement: with the complement overwritten it clears the flag and leaves the
    workspace poisoned, as for a workspace zeroed by the caller."""
    _say("poisoned verify, damaged size record")
    t, d, x = _inputs()
    B, K = x.shape
    ws = sv.Workspace(DEV)
    buf = ws.get(B, K, t.shape[2])
    _poison(buf)
    buf.view(torch.int32)[200 // 4] = 12345   # the complement's low word (bytes 200..203)
    torch.cuda.synchronize()
    got = _np(sv.sv_verify_batch(t, d, x, 0.9, seed=3, workspace=ws))
    assert (got["n_out"] == 0).all()
    assert sv.sv_device_error(buf) == sv.SV_DEVERR_POISONED
    assert _epoch(buf) == POISONED_EPOCH & 0xffffffff   # not zero-filled
    sv.sv_workspace_init(buf)
    again = _np(sv.sv_verify_batch(t, d, x, 0.9, seed=3, workspace=ws))
    assert sv.sv_device_error(buf) == 0 and (again["n_out"] >= 1).all()
