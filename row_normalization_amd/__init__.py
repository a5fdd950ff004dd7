"""Fused RMSNorm and LayerNorm forward/backward, and the RoPE and SwiGLU
elementwise ops, for the AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/*.h`` (``librmsnorm.so``, built in-tree by
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
    rope_bwd,
    rope_fwd,
    swiglu_bwd,
    swiglu_fwd,
    rmsnorm_bwd,
    rmsnorm_bwd_noalloc,
    rmsnorm_bwd_rows,
    rmsnorm_bwd_workspace_bytes,
    rmsnorm_dgamma_reduce,
    rmsnorm_fwd,
    rmsnorm_status_string,
)
from .autograd import (CALLS, LayerNorm, LayerNormFunction, RMSNorm, RMSNormFunction, RoPEFunction, SwiGLUFunction,
                       layernorm, rmsnorm, rope_embedding, swiglu)

__all__ = [
    "LIB_PATH",
    "RMSNormError",
    "header_functions",
    "lib",
    "rmsnorm_fwd",
    "rmsnorm_bwd",
    "rmsnorm_bwd_noalloc",
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
    "rope_fwd",
    "rope_bwd",
    "rope_embedding",
    "RoPEFunction",
    "swiglu_fwd",
    "swiglu_bwd",
    "swiglu",
    "SwiGLUFunction",
]
