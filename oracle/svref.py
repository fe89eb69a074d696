"""ctypes front end of the plain-C oracle (``libsvref.so``) -- TEST INFRASTRUCTURE ONLY.

Arrays are numpy host arrays: logits as float32 (dtype ``"f32"``) or as uint16 bfloat16
bit patterns (dtype ``"bf16"``).  All results are float64 / int32 / uint8 numpy arrays.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        u64, i32, i64, dbl, vp = C.c_uint64, C.c_int32, C.c_int64, C.c_double, C.c_void_p
        L.svref_philox4x64_10.argtypes = [vp, vp, vp]
        L.svref_uniform.argtypes = [u64, u64, u64, u64, u64]
        L.svref_uniform.restype = dbl
        L.svref_row_lse.argtypes = [vp, C.c_int, i32, dbl]
        L.svref_row_lse.restype = dbl
        L.svref_row_argmax.argtypes = [vp, C.c_int, i32]
        L.svref_row_argmax.restype = i32
        L.svref_alpha.argtypes = [vp, C.c_int, vp, C.c_int, i32, dbl]
        L.svref_alpha.restype = dbl
        L.svref_verify_batch.argtypes = [C.POINTER(Params)] + [vp] * 17
        L.svref_verify_batch.restype = C.c_int
        L.svref_correction_cdf.argtypes = [C.POINTER(Params), vp, vp, i32, i32, i32, i32]
        L.svref_correction_cdf.restype = dbl
        L.svref_accept_len.argtypes = [vp, vp, i32, i32, vp]
        L.svref_residual_sample.argtypes = [C.POINTER(Params), vp, vp, vp, vp, vp]
        L.svref_e2e_from_alpha.argtypes = [vp, i32, i32]
        L.svref_e2e_from_alpha.restype = dbl
        L.svref_tv_e2e_loss.argtypes = [C.POINTER(Params), vp, vp, vp, vp]
        L.svref_tv_e2e_backward.argtypes = [C.POINTER(Params), vp, vp, dbl, vp, vp, vp, vp]
        L.svref_sample_drafts.argtypes = [C.POINTER(Params), vp, vp, vp, vp, vp]
        L.svref_draft_cdf.argtypes = [C.POINTER(Params), vp, i32, i32, i32]
        L.svref_draft_cdf.restype = dbl
        L.svref_alloc_verify_budget.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.svref_dcut_budget.argtypes = [vp, vp, i32, i32, vp, i32, C.POINTER(C.c_int32), C.POINTER(C.c_double), vp, vp, vp]
        _lib = L
    return _lib


class Params(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("K_max", C.c_int32), ("V", C.c_int32),
        ("dtype_t", C.c_int32), ("dtype_d", C.c_int32),
        ("temperature", C.c_double),
        ("seed", C.c_uint64), ("step", C.c_uint64),
        ("ld_t", C.c_int64), ("ld_d", C.c_int64),
    ]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _logits(a, dtype):
    want = np.float32 if dtype == "f32" else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"logits for dtype {dtype} must be {want}, got {a.dtype}")
    return a


def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().svref_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, c0, c1, c2, c3):
    return lib().svref_uniform(seed, c0, c1, c2, c3)


def row_lse(row, dtype, T):
    row = _logits(row, dtype)
    return lib().svref_row_lse(_ptr(row), _DT[dtype], row.shape[-1], float(T))


def row_argmax(row, dtype):
    row = _logits(row, dtype)
    return lib().svref_row_argmax(_ptr(row), _DT[dtype], row.shape[-1])


def alpha(trow, drow, dtype, T):
    trow, drow = _logits(trow, dtype), _logits(drow, dtype)
    return lib().svref_alpha(_ptr(trow), _DT[dtype], _ptr(drow), _DT[dtype], trow.shape[-1], float(T))


def make_params(B, K, V, dtype, T, seed=0, step=0, ld=None):
    return Params(B, K, V, _DT[dtype], _DT[dtype], float(T), seed, step, ld or V, ld or V)


def verify_batch(target, draft, draft_tokens, T, dtype, seed=0, step=0, draft_len=None,
                 diagnostics=False):
    """target [B][K+1][V], draft [B][K][V], draft_tokens [B][K] int32."""
    target, draft = _logits(target, dtype), _logits(draft, dtype)
    B, K1, V = target.shape
    K = K1 - 1
    assert draft.shape == (B, K, V)
    xt = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    dl = None if draft_len is None else np.ascontiguousarray(draft_len, dtype=np.int32)
    prm = make_params(B, K, V, dtype, T, seed, step)
    out = dict(
        alpha=np.zeros((B, K)), accept=np.zeros((B, K), np.uint8),
        lse_t=np.zeros((B, K)), lse_d=np.zeros((B, K)),
        amax_t=np.zeros((B, K), np.int32), amax_d=np.zeros((B, K), np.int32),
        accept_len=np.zeros(B, np.int32), out_tokens=np.zeros((B, K + 1), np.int32),
        n_out=np.zeros(B, np.int32),
    )
    diag = dict(ratio=np.zeros((B, K)), u_acc=np.zeros((B, K)), u_corr=np.zeros(B),
                cdf_target=np.zeros(B), resid_mass=np.zeros(B)) if diagnostics else {}
    rc = lib().svref_verify_batch(
        C.byref(prm), _ptr(target), _ptr(draft), _ptr(xt), _ptr(dl),
        _ptr(out["alpha"]), _ptr(out["accept"]), _ptr(out["lse_t"]), _ptr(out["lse_d"]),
        _ptr(out["amax_t"]), _ptr(out["amax_d"]), _ptr(out["accept_len"]),
        _ptr(out["out_tokens"]), _ptr(out["n_out"]),
        _ptr(diag.get("ratio")), _ptr(diag.get("u_acc")), _ptr(diag.get("u_corr")),
        _ptr(diag.get("cdf_target")), _ptr(diag.get("resid_mass")))
    if rc != 0:
        raise ValueError("svref_verify_batch rejected its arguments")
    out.update(diag)
    return out


def correction_cdf(target, draft, T, dtype, r, tau, L_r, v):
    target, draft = _logits(target, dtype), _logits(draft, dtype)
    B, K1, V = target.shape
    prm = make_params(B, K1 - 1, V, dtype, T)
    return lib().svref_correction_cdf(C.byref(prm), _ptr(target), _ptr(draft), r, tau, L_r, v)


def accept_len(accept, draft_len=None):
    acc = np.ascontiguousarray(accept, dtype=np.uint8)
    B, K = acc.shape
    dl = None if draft_len is None else np.ascontiguousarray(draft_len, dtype=np.int32)
    out = np.zeros(B, np.int32)
    if lib().svref_accept_len(_ptr(acc), _ptr(dl), B, K, _ptr(out)) != 0:
        raise ValueError("svref_accept_len rejected its arguments")
    return out


def residual_sample(target, draft, accept_len_, T, dtype, seed=0, step=0, draft_len=None):
    target, draft = _logits(target, dtype), _logits(draft, dtype)
    B, K1, V = target.shape
    prm = make_params(B, K1 - 1, V, dtype, T, seed, step)
    al = np.ascontiguousarray(accept_len_, dtype=np.int32)
    dl = None if draft_len is None else np.ascontiguousarray(draft_len, dtype=np.int32)
    tok = np.zeros(B, np.int32)
    if lib().svref_residual_sample(C.byref(prm), _ptr(target), _ptr(draft), _ptr(dl), _ptr(al), _ptr(tok)) != 0:
        raise ValueError("svref_residual_sample rejected its arguments")
    return tok


def e2e_from_alpha(alpha_):
    a = np.ascontiguousarray(alpha_, dtype=np.float64)
    I, D = a.shape
    return lib().svref_e2e_from_alpha(_ptr(a), I, D)


def tv_e2e_loss(target, draft, T, dtype):
    """target, draft [I][D][V]; returns (loss, alpha[I][D])."""
    target, draft = _logits(target, dtype), _logits(draft, dtype)
    I, D, V = target.shape
    assert draft.shape == (I, D, V)
    prm = make_params(I, D, V, dtype, T)
    a = np.zeros((I, D))
    loss = np.zeros(1)
    if lib().svref_tv_e2e_loss(C.byref(prm), _ptr(target), _ptr(draft), _ptr(a), _ptr(loss)) != 0:
        raise ValueError("svref_tv_e2e_loss rejected its arguments")
    return float(loss[0]), a


def tv_e2e_backward(target, draft, T, dtype, grad_loss=1.0, want_log_ratio=False):
    """target, draft [I][D][V]; returns (grad [I][D][V], alpha [I][D], loss) and, if asked,
    log_ratio [I][D][V] = ln p - ln q."""
    target, draft = _logits(target, dtype), _logits(draft, dtype)
    I, D, V = target.shape
    assert draft.shape == (I, D, V)
    prm = make_params(I, D, V, dtype, T)
    g = np.zeros((I, D, V))
    a = np.zeros((I, D))
    loss = np.zeros(1)
    lr = np.zeros((I, D, V)) if want_log_ratio else None
    if lib().svref_tv_e2e_backward(C.byref(prm), _ptr(target), _ptr(draft), float(grad_loss), _ptr(g), _ptr(a),
                                   _ptr(loss), _ptr(lr)) != 0:
        raise ValueError("svref_tv_e2e_backward rejected its arguments")
    return (g, a, float(loss[0]), lr) if want_log_ratio else (g, a, float(loss[0]))


def sample_drafts(draft, T, dtype, seed=0, step=0):
    """draft [B][K][V]; returns (tokens [B][K] int32, conf [B][K], u [B][K], R [B][K])."""
    draft = _logits(draft, dtype)
    B, K, V = draft.shape
    prm = make_params(B, K, V, dtype, T, seed, step)
    tok = np.zeros((B, K), np.int32)
    conf, u, R = np.zeros((B, K)), np.zeros((B, K)), np.zeros((B, K))
    if lib().svref_sample_drafts(C.byref(prm), _ptr(draft), _ptr(tok), _ptr(conf), _ptr(u), _ptr(R)) != 0:
        raise ValueError("svref_sample_drafts rejected its arguments")
    return tok, conf, u, R


def draft_cdf(draft, T, dtype, r, k, v):
    draft = _logits(draft, dtype)
    B, K, V = draft.shape
    prm = make_params(B, K, V, dtype, T)
    return lib().svref_draft_cdf(C.byref(prm), _ptr(draft), r, k, v)


def dcut_budget(conf, cost, draft_len=None):
    """D-cut budget choice: returns (n_chosen, utility, lens, row_off, row_list)."""
    c = np.ascontiguousarray(conf, dtype=np.float32)
    B, K = c.shape
    dl = None if draft_len is None else np.ascontiguousarray(draft_len, dtype=np.int32)
    cs = np.ascontiguousarray(cost, dtype=np.float32)
    lens = np.zeros(B, np.int32)
    off = np.zeros(B + 1, np.int32)
    rl = np.zeros(max(B * K, 1), np.int32)
    nc = C.c_int32(0)
    ut = C.c_double(0.0)
    if lib().svref_dcut_budget(_ptr(c), _ptr(dl), B, K, _ptr(cs), len(cs), C.byref(nc), C.byref(ut), _ptr(lens),
                               _ptr(off), _ptr(rl)) != 0:
        raise ValueError("svref_dcut_budget rejected its arguments")
    return int(nc.value), float(ut.value), lens, off, rl[: int(off[-1])]


def alloc_verify_budget(conf, budget_N, draft_len=None):
    c = np.ascontiguousarray(conf, dtype=np.float32)
    B, K = c.shape
    dl = None if draft_len is None else np.ascontiguousarray(draft_len, dtype=np.int32)
    lens = np.zeros(B, np.int32)
    off = np.zeros(B + 1, np.int32)
    n = int(min(budget_N, (K * B) if dl is None else int(dl.sum())))
    rl = np.zeros(max(n, 1), np.int32)
    if lib().svref_alloc_verify_budget(_ptr(c), _ptr(dl), B, K, int(budget_N), _ptr(lens), _ptr(off), _ptr(rl)) != 0:
        raise ValueError("svref_alloc_verify_budget rejected its arguments")
    return lens, off, rl[:n]
