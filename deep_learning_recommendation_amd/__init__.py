"""DLRM hot path for one AMD Instinct MI355X (gfx950).

``libdlrm.so`` (C ABI, ``include/dlrm.h``) holds every kernel; ``_lib``
binds it with ctypes and ``pipeline`` orders the calls of a forward pass and
a training step.  There is no CPU fallback: without the built library every
entry point raises.
"""
from ._lib import (DLRM_ACT_NONE, DLRM_ACT_RELU, DLRM_BF16, DLRM_F32, DLRM_I8, DLRMError, EXPORTS,  # noqa: F401
                   LIB_PATH,
                   device_pointer_array, dlrm_abi_version, dlrm_bce_grad, dlrm_check_indices,
                   dlrm_embbag_bwd_sgd, dlrm_embbag_bwd_sgd_apply, dlrm_embbag_bwd_sgd_noalloc, dlrm_embbag_bwd_sgd_prepare,
                   dlrm_embbag_bwd_sgd_workspace_size, dlrm_embbag_fwd, dlrm_embbag_fwd_lp,
                   dlrm_embbag_interact_fwd, dlrm_embbag_interact_fwd_lp,
                   dlrm_interact_bwd, dlrm_interact_fwd, dlrm_linear_fwd,
                   dlrm_mlp_bwd, dlrm_mlp_bwd_workspace_size, dlrm_mlp_fwd, dlrm_mlp_workspace_size, lib)
