"""The C-ABI library loads, exports every entry point its header declares, and rejects
bad host-side arguments before launching anything (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def svlib():
    import draft_verification_softmax_amd as sv
    return sv.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["sv_verify_batch", "sv_accept_len", "sv_residual_sample", "sv_tv_e2e_loss", "sv_tv_e2e_backward",
              "sv_alloc_verify_budget", "sv_workspace_bytes", "sv_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(svlib):
    raw = C.CDLL(os.path.join(ROOT, "draft_verification_softmax_amd", "libspecverify.so"))
    for n in _declared():
        assert hasattr(raw, n), n


def test_status_strings(svlib):
    for code in range(6):
        s = svlib.sv_status_string(code).decode()
        assert s.startswith("SV_")
    assert svlib.sv_status_string(99).decode() == "unknown status"


def test_workspace_bytes(svlib):
    assert svlib.sv_workspace_bytes(-1, 3, 10) == 0
    assert svlib.sv_workspace_bytes(1, 3, 0) == 0
    a = svlib.sv_workspace_bytes(64, 16, 131072)
    b = svlib.sv_workspace_bytes(64, 16, 1000)
    assert a > b > 0 and a % 256 == 0


def test_host_validation_rejects_without_launch(svlib):
    from draft_verification_softmax_amd.binding import Params
    EINVAL, EUNSUP, EWS = 1, 2, 4
    nul = None
    args17 = lambda prm, t=nul: (C.byref(prm), t, nul, nul, nul, nul, nul, nul, nul, nul, nul, nul, nul, nul, nul, 0, nul)
    # negative sizes
    assert svlib.sv_verify_batch(*args17(Params(-1, 3, 100, 0, 0, 1.0, 0, 0, 100, 100))) == EINVAL
    # more draft positions than SV_K_MAX
    assert svlib.sv_verify_batch(*args17(Params(1, 4097, 100, 0, 0, 1.0, 0, 0, 100, 100))) == EINVAL
    # V too large
    assert svlib.sv_verify_batch(*args17(Params(1, 3, (1 << 20) + 1, 0, 0, 1.0, 0, 0, (1 << 20) + 8, (1 << 20) + 8))) == EUNSUP
    # negative / NaN temperature
    assert svlib.sv_verify_batch(*args17(Params(1, 3, 100, 0, 0, -1.0, 0, 0, 100, 100))) == EINVAL
    assert svlib.sv_verify_batch(*args17(Params(1, 3, 100, 0, 0, float("nan"), 0, 0, 100, 100))) == EINVAL
    # null target
    assert svlib.sv_verify_batch(*args17(Params(1, 3, 100, 0, 0, 1.0, 0, 0, 100, 100))) == EINVAL
    # misaligned target pointer / stride (pointer values are never dereferenced on the host)
    fake = C.c_void_p(0x1000)
    odd = C.c_void_p(0x1002)
    assert svlib.sv_verify_batch(*args17(Params(1, 0, 100, 1, 1, 1.0, 0, 0, 100, 100), odd)) == EINVAL
    assert svlib.sv_verify_batch(*args17(Params(1, 0, 100, 1, 1, 1.0, 0, 0, 101, 104), fake)) == EINVAL
    # bad dtype code
    assert svlib.sv_verify_batch(*args17(Params(1, 0, 100, 7, 1, 1.0, 0, 0, 104, 104), fake)) == EUNSUP
    # missing workspace (everything else valid, K = 0)
    prm = Params(1, 0, 96, 1, 1, 1.0, 0, 0, 96, 96)
    a = [C.byref(prm), fake, nul, nul, nul, nul, nul, nul, nul, nul, nul, fake, fake, fake, nul, 0, nul]
    assert svlib.sv_verify_batch(*a) == EWS
    # budget limits
    assert svlib.sv_alloc_verify_budget(fake, nul, 100, 100, 10, fake, fake, nul, nul) == EUNSUP
    assert svlib.sv_alloc_verify_budget(fake, nul, 4, 4, -1, fake, fake, nul, nul) == EINVAL
    # e2e needs T > 0
    assert svlib.sv_tv_e2e_loss(C.byref(Params(2, 3, 96, 1, 1, 0.0, 0, 0, 96, 96)), fake, fake, nul, fake, fake, 1 << 30, nul) == EINVAL
    # uniforms: negative count
    assert svlib.sv_uniforms(0, nul, -1, nul, nul) == EINVAL
    # B = 0 is a no-op
    assert svlib.sv_verify_batch(*args17(Params(0, 3, 100, 0, 0, 1.0, 0, 0, 100, 100))) == 0
    # an empty batch's arrays may be NULL (an empty tensor's address is 0)
    assert svlib.sv_accept_len(nul, nul, 0, 3, nul, nul) == 0
    assert svlib.sv_accept_len(nul, nul, 2, 3, nul, nul) == EINVAL
    # L_e2e over an empty set is undefined
    assert svlib.sv_tv_e2e_loss(C.byref(Params(0, 3, 96, 1, 1, 1.0, 0, 0, 96, 96)), fake, fake, nul, fake, fake, 1 << 30, nul) == EINVAL


def test_verify_selected_host_validation(svlib):
    from draft_verification_softmax_amd.binding import Params
    EINVAL, EWS = 1, 4
    nul = None
    fake = C.c_void_p(0x1000)
    prm = Params(2, 3, 96, 1, 1, 1.0, 0, 0, 96, 96)

    def call(lens, rows, n, ws=nul):
        return svlib.sv_verify_selected(C.byref(prm), fake, fake, fake, lens, rows, n, fake, fake, nul, nul, nul,
                                        nul, fake, fake, fake, ws, 0, nul)
    assert call(fake, fake, -1) == EINVAL          # negative row count
    assert call(fake, fake, 2 * 3 + 1) == EINVAL   # more rows than the batch has
    assert call(nul, fake, 2) == EINVAL            # no lengths
    assert call(fake, nul, 2) == EINVAL            # rows without a list
    assert call(fake, nul, 0) == EWS               # zero rows is valid; then the workspace is missing
    assert call(fake, fake, 6) == EWS


def test_dcut_host_validation(svlib):
    EINVAL, EUNSUP = 1, 2
    nul = None
    fake = C.c_void_p(0x1000)
    ok = [fake, nul, 4, 4, fake, 17, fake, fake, fake, fake, nul, nul]
    bad_ncost = list(ok); bad_ncost[5] = 0
    assert svlib.sv_dcut_verify_budget(*bad_ncost) == EINVAL
    no_cost = list(ok); no_cost[4] = nul
    assert svlib.sv_dcut_verify_budget(*no_cost) == EINVAL
    no_out = list(ok); no_out[6] = nul
    assert svlib.sv_dcut_verify_budget(*no_out) == EINVAL
    big = list(ok); big[2], big[3] = 100, 100
    assert svlib.sv_dcut_verify_budget(*big) == EUNSUP
    long_table = list(ok); long_table[5] = 8194
    assert svlib.sv_dcut_verify_budget(*long_table) == EUNSUP


def test_e2e_backward_host_validation(svlib):
    from draft_verification_softmax_amd.binding import Params
    EINVAL, EUNSUP, EWS = 1, 2, 4
    nul = None
    fake = C.c_void_p(0x1000)
    odd = C.c_void_p(0x1004)

    def call(prm, alpha=fake, grad=fake, dg=1, ld_g=96, ws=nul, wsb=0):
        return svlib.sv_tv_e2e_backward(C.byref(prm), fake, fake, alpha, nul, grad, dg, ld_g, ws, wsb, nul)
    ok = Params(2, 3, 96, 1, 1, 1.0, 0, 0, 96, 96)
    assert call(Params(2, 3, 96, 1, 1, 0.0, 0, 0, 96, 96)) == EINVAL     # T = 0
    assert call(Params(0, 3, 96, 1, 1, 1.0, 0, 0, 96, 96)) == EINVAL     # |I| = 0
    assert call(ok, alpha=nul) == EINVAL                                  # no alpha
    assert call(ok, grad=nul) == EINVAL                                   # no gradient
    assert call(ok, grad=odd) == EINVAL                                   # misaligned gradient rows
    assert call(ok, ld_g=100) == EINVAL                                   # stride not 16-byte aligned
    assert call(ok, ld_g=90) == EINVAL                                    # stride below V
    assert call(ok, dg=5) == EUNSUP                                       # gradient dtype code
    assert call(ok) == EWS                                                # everything valid but the workspace


def test_sample_drafts_host_validation(svlib):
    from draft_verification_softmax_amd.binding import Params
    EINVAL, EUNSUP, EWS = 1, 2, 4
    nul = None
    fake = C.c_void_p(0x1000)

    def call(prm, draft=fake, tok=fake, conf=fake):
        return svlib.sv_sample_drafts(C.byref(prm), draft, tok, conf, nul, 0, nul)
    assert call(Params(2, 3, 96, 1, 1, -1.0, 0, 0, 96, 96)) == EINVAL             # T < 0
    assert call(Params(2, 3, 96, 1, 1, float("inf"), 0, 0, 96, 96)) == EINVAL     # T infinite
    assert call(Params(2, 3, (1 << 20) + 8, 1, 1, 1.0, 0, 0, 96, (1 << 20) + 8)) == EUNSUP
    assert call(Params(2, 3, 96, 1, 1, 1.0, 0, 0, 96, 90)) == EINVAL              # stride below V
    assert call(Params(2, 3, 96, 1, 1, 1.0, 0, 0, 96, 96), tok=nul) == EINVAL
    assert call(Params(2, 3, 96, 1, 1, 1.0, 0, 0, 96, 96), conf=nul) == EINVAL
    assert call(Params(0, 3, 96, 1, 1, 1.0, 0, 0, 96, 96)) == 0                   # nothing to draw
    assert call(Params(2, 3, 96, 1, 1, 0.0, 0, 0, 96, 96)) == EWS                 # greedy, no workspace


def test_wait_bound_validation(svlib):
    assert svlib.sv_set_wait_bound(-1) == 1
    assert svlib.sv_set_wait_bound(0) == 0
    assert svlib.sv_set_wait_bound(200000) == 0   # back to the default
