"""ctypes binding of libspecverify.so: argument marshalling only.

Tensors must live on the GPU; their ``data_ptr()`` and the launch stream (default
``torch.cuda.current_stream()``) are handed to the C entry points unchanged.  Output tensors
are allocated here with torch (device memory plumbing) when the caller does not pass them,
and calls without a workspace share one per (device, launch stream).  ``PreparedVerify``
marshals a verification call once for repeated launches.
"""
import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_NOALLOC_SCRATCH_BYTES = 16 << 20   # the per-device array of sv_verify_batch_noalloc

# device error flags (sv_device_error)
SV_DEVERR_TOKEN, SV_DEVERR_DRAFT_LEN, SV_DEVERR_TIMEOUT, SV_DEVERR_POISONED = 1, 2, 4, 8
_STATUS = {0: "SV_OK", 1: "SV_EINVAL", 2: "SV_EUNSUPPORTED", 3: "SV_EHIP", 4: "SV_EWORKSPACE", 5: "SV_EDEVICE"}

EXPORTS = [
    "sv_workspace_bytes", "sv_workspace_init", "sv_verify_batch", "sv_verify_batch_noalloc", "sv_verify_selected", "sv_accept_len",
    "sv_residual_sample", "sv_tv_e2e_loss", "sv_tv_e2e_backward", "sv_sample_drafts", "sv_alloc_verify_budget",
    "sv_dcut_verify_budget", "sv_uniforms", "sv_device_error", "sv_status_string", "sv_set_wait_bound",
    "sv_stream_read",
]


class SVError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.sv_status_string(code).decode() if _lib is not None else _STATUS.get(code, str(code))
        super().__init__(f"{fn}: {msg}")


class Params(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("K_max", C.c_int32), ("V", C.c_int32),
        ("dtype_t", C.c_int32), ("dtype_d", C.c_int32),
        ("temperature", C.c_float),
        ("seed", C.c_uint64), ("step", C.c_uint64),
        ("ld_t", C.c_int64), ("ld_d", C.c_int64),
    ]


_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python draft_verification_softmax_amd/build.py` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        vp, i32, u64, sz = C.c_void_p, C.c_int32, C.c_uint64, C.c_size_t
        P = C.POINTER(Params)
        L.sv_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_workspace_bytes.restype = sz
        L.sv_workspace_init.argtypes = [vp, sz, vp]
        L.sv_verify_batch.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sv_verify_batch_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sv_verify_selected.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sv_accept_len.argtypes = [vp, vp, i32, i32, vp, vp]
        L.sv_residual_sample.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.sv_tv_e2e_loss.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.sv_tv_e2e_backward.argtypes = [P, vp, vp, vp, vp, vp, i32, C.c_int64, vp, sz, vp]
        L.sv_sample_drafts.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.sv_alloc_verify_budget.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
        L.sv_dcut_verify_budget.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        L.sv_uniforms.argtypes = [u64, vp, i32, vp, vp]
        L.sv_device_error.argtypes = [vp, vp, C.POINTER(C.c_uint32)]
        L.sv_set_wait_bound.argtypes = [C.c_int64]
        L.sv_stream_read.argtypes = [vp, sz, vp, vp]
        L.sv_status_string.argtypes = [C.c_int]
        L.sv_status_string.restype = C.c_char_p
        for name in EXPORTS:
            if name not in ("sv_workspace_bytes", "sv_status_string"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def sv_set_wait_bound(ns: int):
    """Bound (ns) of the in-kernel wait for teammates' partials; 0 forces every hand-over."""
    _check("sv_set_wait_bound", lib().sv_set_wait_bound(int(ns)))


def sv_status_string(code: int) -> str:
    return lib().sv_status_string(code).decode()


def _check(fn, code):
    if code != 0:
        raise SVError(fn, code)


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libspecverify must be on the GPU")
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError(f"unsupported logit dtype {t.dtype}")


def sv_workspace_bytes(B, K_max, V) -> int:
    return int(lib().sv_workspace_bytes(B, K_max, V))


def sv_workspace_init(ws: torch.Tensor, stream=None):
    _check("sv_workspace_init", lib().sv_workspace_init(_p(ws), ws.numel() * ws.element_size(), _stream(stream)))


class Workspace:
    """A zero-initialised device workspace that grows on demand."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, B, K_max, V, stream=None):
        need = sv_workspace_bytes(B, K_max, V)
        if self.buf is None or self.buf.numel() < need:
            self.buf = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            fs = _foreign(stream)
            if fs is not None:   # allocated on the current stream, used on the launch stream
                self.buf.record_stream(fs)
            sv_workspace_init(self.buf, stream)
        return self.buf


_default_ws = {}


def default_workspace(device=None, stream=None) -> Workspace:
    """The workspace of calls that pass none: one per (device, launch stream), kept for the
    life of the process, so such calls do not allocate and zero a workspace each time and
    their device error flags stay readable (sv_device_error(default_workspace().buf))."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (s.device.index, s.cuda_stream)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(s.device)
    return ws


def _foreign(stream):
    """The launch stream when it is not its device's current stream, else None.  Tensors
    allocated here come from the current stream's pool; when another stream runs the kernel
    that uses them they are recorded on it, so the caching allocator does not hand their
    memory to a new tensor while that kernel may still use it."""
    if stream is None:
        return None
    return None if torch.cuda.current_stream(stream.device).cuda_stream == stream.cuda_stream else stream


def _ws_for(workspace, dev, B, K, V, stream):
    if isinstance(workspace, torch.Tensor):
        return workspace
    return (workspace or default_workspace(dev, stream)).get(B, K, V, stream)


def _record(fs, *tensors):
    if fs is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(fs)


def _rows_ld(t):
    if t.stride(-1) != 1:
        raise ValueError("logit rows must be contiguous")
    return t.stride(-2) if t.dim() >= 2 else t.shape[-1]


def _check_rows(t, rows_per_item):
    """The ABI addresses row (i, k) at (i * rows_per_item + k) * ld: rows must be packed."""
    if t is None or t.numel() == 0:
        return
    ld = _rows_ld(t)
    if t.stride(1) != ld or t.stride(0) != rows_per_item * ld:
        raise ValueError("logit rows must be packed [B][rows][ld] with a common row stride")


def _params(B, K, V, target, draft, T, seed, step):
    ld_t = _rows_ld(target)
    ld_d = _rows_ld(draft) if draft is not None and draft.numel() else V
    dd = _dtype_code(draft) if draft is not None else _dtype_code(target)
    return Params(B, K, V, _dtype_code(target), dd, float(T), seed, step, ld_t, ld_d)


def sv_verify_batch(target, draft, draft_tokens, T, seed=0, step=0, draft_len=None,
                    want_lse=True, want_amax=False, workspace=None, out=None, stream=None):
    """target [B][K+1][V], draft [B][K][V], draft_tokens [B][K] int32 (all on the GPU).
    Returns a dict of device tensors (alpha, accept, lse_t, lse_d, amax_t, amax_d,
    accept_len, out_tokens, n_out)."""
    return _verify(target, draft, draft_tokens, T, seed, step, draft_len, None, 0, want_lse, want_amax, workspace,
                   out, stream)


def sv_verify_batch_noalloc(target, draft, draft_tokens, T, seed=0, step=0, draft_len=None, want_lse=True,
                            want_amax=False, out=None, stream=None):
    """sv_verify_batch on the library's own per-device scratch array (no workspace; the C
    entry point allocates nothing).  Outputs are allocated here unless `out` (a dict as
    returned by sv_verify_batch) is given."""
    fn, args, _, out, _ = _prepare_verify(target, draft, draft_tokens, T, seed, step, draft_len, None, 0, want_lse,
                                          want_amax, None, out, stream, noalloc=True)
    _check("sv_verify_batch_noalloc", fn(*args))
    return out


def sv_verify_selected(target, draft, draft_tokens, T, lens, row_list, n_rows, seed=0, step=0, want_lse=True,
                       want_amax=False, workspace=None, out=None, stream=None):
    """Verification of the rows one sv_alloc_verify_budget call selected: lens [B] and
    row_list are its outputs, n_rows their number (host int).  Same outputs as
    sv_verify_batch(draft_len=lens)."""
    if lens is None or lens.dtype != torch.int32:
        raise ValueError("lens must be int32 [B]")
    n_rows = int(n_rows)
    if n_rows > 0 and (row_list is None or row_list.dtype != torch.int32 or row_list.numel() < n_rows):
        raise ValueError("row_list must be int32 with at least n_rows entries")
    return _verify(target, draft, draft_tokens, T, seed, step, lens, row_list, n_rows, want_lse, want_amax,
                   workspace, out, stream, selected=True)


def _prepare_verify(target, draft, draft_tokens, T, seed, step, draft_len, row_list, n_rows, want_lse, want_amax,
                    workspace, out, stream, selected=False, noalloc=False):
    """Checks shapes and marshals one verification call: returns (entry point, argument
    tuple, the Params it points to, outputs, the workspace or None for the no-allocation
    entry point)."""
    B, K1, V = target.shape
    K = K1 - 1
    if draft.shape != (B, K, V) or draft_tokens.shape != (B, K):
        raise ValueError("shape mismatch between target, draft and draft_tokens")
    if draft_tokens.dtype != torch.int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32")
    if draft_len is not None and (draft_len.dtype != torch.int32 or draft_len.shape != (B,)):
        raise ValueError("draft_len must be int32 [B]")
    _check_rows(target, K + 1)
    _check_rows(draft, K)
    dev = target.device
    fs = _foreign(stream)
    if out is None:
        out = dict(
            alpha=torch.empty((B, K), dtype=torch.float32, device=dev),
            accept=torch.empty((B, K), dtype=torch.uint8, device=dev),
            lse_t=torch.empty((B, K), dtype=torch.float32, device=dev) if want_lse else None,
            lse_d=torch.empty((B, K), dtype=torch.float32, device=dev) if want_lse else None,
            amax_t=torch.empty((B, K), dtype=torch.int32, device=dev) if want_amax else None,
            amax_d=torch.empty((B, K), dtype=torch.int32, device=dev) if want_amax else None,
            accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
            out_tokens=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            n_out=torch.empty((B,), dtype=torch.int32, device=dev),
        )
        _record(fs, *out.values())
    ws = None if noalloc else _ws_for(workspace, dev, B, K, V, stream)
    prm = _params(B, K, V, target, draft, T, seed, step)
    outs = (_p(out["alpha"]), _p(out["accept"]), _p(out["lse_t"]), _p(out["lse_d"]), _p(out["amax_t"]),
            _p(out["amax_d"]), _p(out["accept_len"]), _p(out["out_tokens"]), _p(out["n_out"]))
    if noalloc:
        fn = lib().sv_verify_batch_noalloc
        args = (C.byref(prm), _p(target), _p(draft), _p(draft_tokens), _p(draft_len), *outs, _stream(stream))
    elif selected:
        fn = lib().sv_verify_selected
        args = (C.byref(prm), _p(target), _p(draft), _p(draft_tokens), _p(draft_len), _p(row_list), n_rows, *outs,
                _p(ws), ws.numel(), _stream(stream))
    else:
        fn = lib().sv_verify_batch
        args = (C.byref(prm), _p(target), _p(draft), _p(draft_tokens), _p(draft_len), *outs, _p(ws), ws.numel(),
                _stream(stream))
    return fn, args, prm, out, ws


def _verify(target, draft, draft_tokens, T, seed, step, draft_len, row_list, n_rows, want_lse, want_amax, workspace,
            out, stream, selected=False):
    fn, args, _, out, _ = _prepare_verify(target, draft, draft_tokens, T, seed, step, draft_len, row_list, n_rows,
                                          want_lse, want_amax, workspace, out, stream, selected)
    _check("sv_verify_selected" if selected else "sv_verify_batch", fn(*args))
    return out


class PreparedVerify:
    """One verification call (sv_verify_batch, or sv_verify_selected when row_list is given)
    marshalled once for repeated launches on the same buffers, as a decoding loop issues
    them: launch(step) writes the generator's step counter (and optionally the seed) into the
    stored parameters and calls the entry point with the stored arguments.  The tensors
    passed here (inputs, outputs, workspace) must stay alive and in place while it is used;
    the launch stream is fixed here (default: the current stream)."""

    def __init__(self, target, draft, draft_tokens, T, seed=0, draft_len=None, row_list=None, n_rows=None,
                 want_lse=True, want_amax=False, workspace=None, out=None, stream=None):
        selected = row_list is not None
        if selected:
            if draft_len is None or draft_len.dtype != torch.int32:
                raise ValueError("a selected-row call needs lens (draft_len) as int32 [B]")
            if row_list.dtype != torch.int32 or n_rows is None or row_list.numel() < int(n_rows):
                raise ValueError("row_list must be int32 with at least n_rows entries")
        self.stream = torch.cuda.current_stream(target.device) if stream is None else stream
        self._fn, self._args, self._prm, self.out, self.workspace = _prepare_verify(
            target, draft, draft_tokens, T, seed, 0, draft_len, row_list, int(n_rows or 0), want_lse, want_amax,
            workspace, out, self.stream, selected)
        self._keep = (target, draft, draft_tokens, draft_len, row_list)
        self._name = "sv_verify_selected" if selected else "sv_verify_batch"

    def launch(self, step, seed=None):
        self._prm.step = step
        if seed is not None:
            self._prm.seed = seed
        rc = self._fn(*self._args)
        if rc:
            raise SVError(self._name, rc)
        return self.out


def sv_accept_len(accept, draft_len=None, out=None, stream=None):
    B, K = accept.shape
    out = torch.empty((B,), dtype=torch.int32, device=accept.device) if out is None else out
    _record(_foreign(stream), out)
    _check("sv_accept_len", lib().sv_accept_len(_p(accept), _p(draft_len), B, K, _p(out), _stream(stream)))
    return out


def sv_residual_sample(target, draft, accept_len, T, seed=0, step=0, draft_len=None, out=None, stream=None):
    B, K1, V = target.shape
    K = K1 - 1
    _check_rows(target, K + 1)
    _check_rows(draft, K)
    out = torch.empty((B,), dtype=torch.int32, device=target.device) if out is None else out
    _record(_foreign(stream), out)
    prm = _params(B, K, V, target, draft, T, seed, step)
    _check("sv_residual_sample", lib().sv_residual_sample(
        C.byref(prm), _p(target), _p(draft), _p(draft_len), _p(accept_len), _p(out), _stream(stream)))
    return out


def sv_tv_e2e_loss(target, draft, T=1.0, alpha=None, workspace=None, stream=None):
    """target, draft [I][D][V]; returns (loss [1] float32, alpha [I][D] float32)."""
    I, D, V = target.shape
    if draft.shape != (I, D, V):
        raise ValueError("target and draft must have the same shape")
    _check_rows(target, D)
    _check_rows(draft, D)
    dev = target.device
    alpha = torch.empty((I, D), dtype=torch.float32, device=dev) if alpha is None else alpha
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    _record(_foreign(stream), alpha, loss)
    ws = _ws_for(workspace, dev, I, D, V, stream)
    prm = _params(I, D, V, target, draft, T, 0, 0)
    _check("sv_tv_e2e_loss", lib().sv_tv_e2e_loss(C.byref(prm), _p(target), _p(draft), _p(alpha), _p(loss),
                                                  _p(ws), ws.numel(), _stream(stream)))
    return loss, alpha


def sv_tv_e2e_backward(target, draft, alpha, T=1.0, grad_loss=None, grad_dtype=None, grad=None, workspace=None,
                       stream=None):
    """Gradient of L_e2e in the drafter logits.  target, draft [I][D][V]; alpha [I][D] float32
    (the overlaps of the same inputs, e.g. from sv_tv_e2e_loss); grad_loss: float32 [1] on the
    GPU or None (1).  Returns grad [I][D][V] of grad_dtype (default: the drafter's dtype)."""
    I, D, V = target.shape
    if draft.shape != (I, D, V):
        raise ValueError("target and draft must have the same shape")
    if alpha.shape != (I, D) or alpha.dtype != torch.float32 or not alpha.is_contiguous():
        raise ValueError("alpha must be a contiguous float32 [I][D] tensor")
    _check_rows(target, D)
    _check_rows(draft, D)
    dev = target.device
    if grad is None:   # rows padded to a 16-byte stride
        ld = (V + 7) // 8 * 8
        grad = torch.empty((I, D, ld), dtype=grad_dtype or draft.dtype, device=dev)[:, :, :V]
    elif grad.shape != (I, D, V):
        raise ValueError("grad must be [I][D][V]")
    _check_rows(grad, D)
    _record(_foreign(stream), grad)
    ws = _ws_for(workspace, dev, I, D, V, stream)
    prm = _params(I, D, V, target, draft, T, 0, 0)
    _check("sv_tv_e2e_backward", lib().sv_tv_e2e_backward(
        C.byref(prm), _p(target), _p(draft), _p(alpha), _p(grad_loss), _p(grad), _dtype_code(grad), _rows_ld(grad),
        _p(ws), ws.numel(), _stream(stream)))
    return grad


def sv_sample_drafts(draft, T, seed=0, step=0, workspace=None, stream=None):
    """draft [B][K][V] (GPU).  Returns (tokens [B][K] int32, conf [B][K] float32): a sample of
    softmax(draft / T) per row and its probability (T = 0: the argmax and its probability at
    T = 1)."""
    B, K, V = draft.shape
    dev = draft.device
    tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    conf = torch.empty((B, K), dtype=torch.float32, device=dev)
    if B == 0 or K == 0:
        return tokens, conf
    _check_rows(draft, K)
    _record(_foreign(stream), tokens, conf)
    ws = _ws_for(workspace, dev, B, K, V, stream)
    prm = Params(B, K, V, _dtype_code(draft), _dtype_code(draft), float(T), seed, step, _rows_ld(draft), _rows_ld(draft))
    _check("sv_sample_drafts", lib().sv_sample_drafts(C.byref(prm), _p(draft), _p(tokens), _p(conf), _p(ws),
                                                      ws.numel(), _stream(stream)))
    return tokens, conf


def sv_alloc_verify_budget(conf, budget_N, draft_len=None, want_row_list=True, out=None, stream=None):
    """conf [B][K] float32 in [0,1]; returns (lens [B], row_off [B+1], row_list [N'] or None),
    written into `out` (such a tuple from an earlier call of at least this budget) if given."""
    B, K = conf.shape
    dev = conf.device
    n = min(int(budget_N), B * K)  # upper bound on the selected count
    if out is not None:
        lens, row_off, row_list = out
        if lens.shape != (B,) or row_off.shape != (B + 1,) or (row_list is not None and row_list.numel() < max(n, 1)):
            raise ValueError("out does not fit this allocation")
    else:
        lens = torch.empty((B,), dtype=torch.int32, device=dev)
        row_off = torch.empty((B + 1,), dtype=torch.int32, device=dev)
        row_list = torch.empty((max(n, 1),), dtype=torch.int32, device=dev) if want_row_list else None
        _record(_foreign(stream), lens, row_off, row_list)
    _check("sv_alloc_verify_budget", lib().sv_alloc_verify_budget(
        _p(conf), _p(draft_len), B, K, int(budget_N), _p(lens), _p(row_off), _p(row_list), _stream(stream)))
    return lens, row_off, row_list


def sv_dcut_verify_budget(conf, cost, draft_len=None, want_row_list=True, stream=None):
    """conf [B][K] float32, cost [n_cost] float32 (both on the GPU).  Returns (n_chosen [1]
    int32, utility [1] float64, lens [B], row_off [B+1], row_list [B*K] or None), all device
    tensors; row_list holds row_off[B] valid entries."""
    B, K = conf.shape
    dev = conf.device
    if cost.dtype != torch.float32 or cost.dim() != 1 or not cost.is_contiguous():
        raise ValueError("cost must be a contiguous float32 vector")
    n_chosen = torch.empty((1,), dtype=torch.int32, device=dev)
    utility = torch.empty((1,), dtype=torch.float64, device=dev)
    lens = torch.empty((B,), dtype=torch.int32, device=dev)
    row_off = torch.empty((B + 1,), dtype=torch.int32, device=dev)
    row_list = torch.empty((max(B * K, 1),), dtype=torch.int32, device=dev) if want_row_list else None
    _record(_foreign(stream), n_chosen, utility, lens, row_off, row_list)
    _check("sv_dcut_verify_budget", lib().sv_dcut_verify_budget(
        _p(conf), _p(draft_len), B, K, _p(cost), cost.numel(), _p(n_chosen), _p(utility), _p(lens), _p(row_off),
        _p(row_list), _stream(stream)))
    return n_chosen, utility, lens, row_off, row_list


def sv_uniforms(seed, counters, stream=None):
    """counters [n][4] uint64 (torch int64 on the GPU); returns float32 [n]."""
    n = counters.shape[0]
    out = torch.empty((n,), dtype=torch.float32, device=counters.device)
    _record(_foreign(stream), out)
    _check("sv_uniforms", lib().sv_uniforms(C.c_uint64(seed), _p(counters), n, _p(out), _stream(stream)))
    return out


def sv_stream_read(data: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read every byte of `data` once (the read-only streaming reference); sink: a device
    tensor of at least 4 bytes."""
    _check("sv_stream_read", lib().sv_stream_read(_p(data), data.numel() * data.element_size(), _p(sink),
                                                  _stream(stream)))


def sv_device_error(ws, stream=None) -> int:
    """Synchronises the stream and returns (and clears) the workspace's SV_DEVERR_* flags.
    After SV_DEVERR_TIMEOUT or SV_DEVERR_POISONED the library zero-fills the workspace again
    (one that sv_workspace_init set up, as Workspace does), so the next call verifies.
    ws None: the current device's sv_verify_batch_noalloc array."""
    flags = C.c_uint32(0)
    rc = lib().sv_device_error(_p(ws), _stream(stream), C.byref(flags))
    if rc not in (0, 5):
        raise SVError("sv_device_error", rc)
    return int(flags.value)
