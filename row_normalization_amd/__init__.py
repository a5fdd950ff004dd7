"""Fused RMSNorm and LayerNorm forward/backward for the AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/rmsnorm.h`` and ``include/layernorm.h`` (``librmsnorm.so``, built in-tree by
``row_normalization_amd.build``).  This package only marshals arguments to it;
there is no CPU or PyTorch fallback.
"""
from ._lib import (
    LIB_PATH,
    RMSNormError,
    header_functions,
    layernorm_bwd,
    layernorm_bwd_rows,
    layernorm_bwd_workspace_bytes,
    layernorm_dwdb_reduce,
    layernorm_fwd,
    lib,
    rmsnorm_bwd,
    rmsnorm_bwd_rows,
    rmsnorm_bwd_workspace_bytes,
    rmsnorm_dgamma_reduce,
    rmsnorm_fwd,
    rmsnorm_status_string,
)
from .autograd import CALLS, LayerNorm, LayerNormFunction, RMSNorm, RMSNormFunction, layernorm, rmsnorm

__all__ = [
    "LIB_PATH",
    "RMSNormError",
    "header_functions",
    "lib",
    "rmsnorm_fwd",
    "rmsnorm_bwd",
    "rmsnorm_bwd_rows",
    "rmsnorm_dgamma_reduce",
    "rmsnorm_bwd_workspace_bytes",
    "rmsnorm_status_string",
    "rmsnorm",
    "RMSNorm",
    "RMSNormFunction",
    "CALLS",
    "layernorm_fwd",
    "layernorm_bwd",
    "layernorm_bwd_rows",
    "layernorm_dwdb_reduce",
    "layernorm_bwd_workspace_bytes",
    "layernorm",
    "LayerNorm",
    "LayerNormFunction",
]
