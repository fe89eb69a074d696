"""MI355X-native batched speculative-decoding draft verification.

A thin binding over ``libspecverify.so`` (C ABI, ``include/specverify.h``).  Each
``sv_*`` function marshals torch tensors to device pointers and the current HIP stream and
calls the entry point of the same name; every step of the computation runs in the HIP
kernels.  There is no CPU fallback: importing this package loads the library and raises
ImportError when it has not been built.
"""
from .binding import (  # noqa: F401
    LIB_PATH, SV_BF16, SV_DEVERR_DRAFT_LEN, SV_DEVERR_POISONED, SV_DEVERR_TIMEOUT, SV_DEVERR_TOKEN, SV_F32,
    SV_NOALLOC_SCRATCH_BYTES, PreparedVerify, SVError, Workspace, default_workspace, lib, sv_accept_len, sv_alloc_verify_budget, sv_dcut_verify_budget,
    sv_device_error, sv_residual_sample, sv_sample_drafts, sv_set_wait_bound, sv_status_string, sv_tv_e2e_backward,
    sv_stream_read, sv_tv_e2e_loss, sv_uniforms, sv_verify_batch, sv_verify_batch_noalloc, sv_verify_selected, sv_workspace_bytes,
    sv_workspace_init,
)

lib()  # fail loudly now if the HIP library is missing
