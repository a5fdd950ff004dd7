"""ctypes binding of ``librmsnorm.so`` (the C ABI in ``include/rmsnorm.h``,
``include/layernorm.h``, ``include/rope.h`` and ``include/swiglu.h``).

Argument marshalling only: tensors are turned into device pointers, shapes,
row strides, a dtype code and the current HIP stream, and the C status is
turned into an exception.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library has not been built, or a tensor
is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librmsnorm.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADERS = tuple(os.path.join(INCLUDE, h) for h in ("rmsnorm.h", "layernorm.h", "rope.h", "swiglu.h"))

F32, BF16, F16 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
GEMMA, ROUND_NORMED = 1, 2  # bits of the C ABI's flags argument

STATUS = {
    0: "RMSNORM_OK", -1: "RMSNORM_E_NULL", -2: "RMSNORM_E_SHAPE", -3: "RMSNORM_E_STRIDE", -4: "RMSNORM_E_ALIGN",
    -5: "RMSNORM_E_DTYPE", -6: "RMSNORM_E_EPS", -7: "RMSNORM_E_ALIAS", -8: "RMSNORM_E_WORKSPACE",
    -9: "RMSNORM_E_FLAG", -10: "RMSNORM_E_HIP", -11: "RMSNORM_E_SCRATCH",
}

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p

_SIGNATURES = {
    "rmsnorm_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_float, ctypes.c_int,
                                   ctypes.c_int, _c_p]),
    "rmsnorm_bwd_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "rmsnorm_bwd_rows": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_i64, _c_i64, _c_i64,
                                        ctypes.c_int, ctypes.c_int, ctypes.POINTER(_c_i64), _c_p]),
    "rmsnorm_dgamma_reduce": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "rmsnorm_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_i64, _c_i64, _c_i64,
                                   ctypes.c_int, ctypes.c_int, _c_p]),
    "rmsnorm_bwd_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                           ctypes.c_int, _c_p]),
    "rmsnorm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "layernorm_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_float,
                                     ctypes.c_int, _c_p]),
    "layernorm_bwd_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "layernorm_bwd_rows": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_i64, _c_i64,
                                          _c_i64, ctypes.c_int, ctypes.POINTER(_c_i64), _c_p]),
    "layernorm_dwdb_reduce": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "layernorm_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_i64,
                                     _c_i64, _c_i64, ctypes.c_int, _c_p]),
    "rope_fwd": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_i64, ctypes.c_int,
                                _c_p]),
    "rope_bwd": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_i64, ctypes.c_int,
                                _c_p]),
    "swiglu_fwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_p]),
    "swiglu_bwd": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_p]),
}

_lib = None


class RMSNormError(RuntimeError):
    """A HIP launch failure reported by the library."""


def header_functions() -> list[str]:
    """Names of the functions the headers under ``include/`` declare."""
    names = []
    for h in HEADERS:
        with open(h) as f:
            text = f.read()
        names += re.findall(r"^(?:int|const char\*)\s+((?:rmsnorm|layernorm|rope|swiglu)_\w+)\s*\(", text, flags=re.M)
    return names


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m row_normalization_amd.build` "
                               "(there is no fallback implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def rmsnorm_status_string(status: int) -> str:
    return lib().rmsnorm_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status == 0:
        return
    msg = f"{what}: {STATUS.get(status, status)} ({rmsnorm_status_string(status)})"
    if status == -10:
        raise RMSNormError(msg)
    raise ValueError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}; the library takes float32, bfloat16 or float16")
    return _DTYPES[t.dtype]


def _gpu(*ts: torch.Tensor):
    """The one GPU every given tensor is on.  Raises for a CPU tensor (there is
    no CPU path) and for tensors on different GPUs (a kernel launched on one
    device cannot use another device's pointers)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("the RMSNorm library takes GPU tensors only (no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors of a call must be on one GPU (found {dev} and {t.device})")
    return dev


def _rows(t: torch.Tensor, name: str) -> tuple[int, int, int]:
    """(M, N, row_stride) of a 2-D view whose rows are contiguous."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, N]")
    M, N = t.shape
    if N > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows (stride(1) == 1)")
    return M, N, t.stride(0) if M > 1 else max(N, t.stride(0))


def _same_layout(ref: torch.Tensor, other: torch.Tensor, name: str, stride: int) -> None:
    if other.shape != ref.shape or other.dtype != ref.dtype:
        raise ValueError(f"{name} must match x in shape and dtype")
    if other.shape[0] > 1 and other.stride(0) != stride:
        raise ValueError(f"{name} must share x's row stride ({stride})")
    if other.shape[1] > 1 and other.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")


def _vec(t, n: int, dtype, name: str) -> None:
    """A per-column (or per-row) vector: n elements of `dtype`, adjacent in memory."""
    if t.dtype != dtype or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of {n} elements")


def _scratch_bytes(t, name: str, need_elems: int = 0) -> int:
    """Bytes of a contiguous scratch tensor (at least `need_elems` fp32 elements)."""
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if need_elems and (t.dtype != torch.float32 or t.numel() < need_elems):
        raise ValueError(f"{name} must be float32 with at least {need_elems} elements")
    return t.numel() * t.element_size()


def _stream(stream, dev) -> int:
    """The HIP stream to launch on: the given one, else the current stream of
    the tensors' device."""
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _flags(gemma: bool, round_normed: bool = False) -> int:
    return (GEMMA if gemma else 0) | (ROUND_NORMED if round_normed else 0)


def rmsnorm_fwd(x, gamma, y, rstd, eps: float = 1e-6, gemma: bool = False, round_normed: bool = False,
                stream=None) -> None:
    """y = x * r * w and rstd = r (w = gamma, or 1 + gamma with ``gemma``), on the GPU.

    ``round_normed`` rounds x * r to the I/O dtype before the weight multiply
    (the Hugging Face order); by default y is rounded once."""
    dev = _gpu(x, gamma, y, rstd)
    M, N, stride = _rows(x, "x")
    _same_layout(x, y, "y", stride)
    _vec(gamma, N, x.dtype, "gamma")
    _vec(rstd, M, torch.float32, "rstd")
    with torch.cuda.device(dev):
        st = lib().rmsnorm_fwd(_ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), M, N, stride, float(eps), _dtype_code(x),
                               _flags(gemma, round_normed), _stream(stream, dev))
    _check(st, "rmsnorm_fwd")


def rmsnorm_bwd_workspace_bytes(M: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DTYPES.get(dtype, -1)
    out = ctypes.c_size_t(0)
    _check(lib().rmsnorm_bwd_workspace_bytes(int(M), int(N), int(code), ctypes.byref(out)),
           "rmsnorm_bwd_workspace_bytes")
    return int(out.value)


def _bwd_checks(x, gamma, dy, rstd, dx):
    _gpu(x, gamma, dy, rstd, dx)
    M, N, stride = _rows(x, "x")
    _same_layout(x, dy, "dy", stride)
    _same_layout(x, dx, "dx", stride)
    _vec(gamma, N, x.dtype, "gamma")
    _vec(rstd, M, torch.float32, "rstd")
    return M, N, stride


def rmsnorm_bwd_rows(x, gamma, dy, rstd, dx, workspace, gemma: bool = False, stream=None) -> int:
    """dx (may be dy itself) and per-workgroup dgamma partial rows; returns the partial-row count."""
    M, N, stride = _bwd_checks(x, gamma, dy, rstd, dx)
    dev = _gpu(x, workspace)
    wbytes = _scratch_bytes(workspace, "workspace")
    rows = _c_i64(0)
    with torch.cuda.device(dev):
        st = lib().rmsnorm_bwd_rows(_ptr(x), _ptr(gamma), _ptr(dy), _ptr(rstd), _ptr(dx), _ptr(workspace),
                                    wbytes, M, N, stride, _dtype_code(x),
                                    _flags(gemma), ctypes.byref(rows), _stream(stream, dev))
    _check(st, "rmsnorm_bwd_rows")
    return int(rows.value)


def rmsnorm_dgamma_reduce(partials, rows: int, N: int, dgamma, stream=None) -> None:
    """dgamma[j] = sum of the first ``rows`` rows of the [rows, N] fp32 partials."""
    dev = _gpu(partials, dgamma)
    _vec(dgamma, N, torch.float32, "dgamma")
    if rows > 0:
        _scratch_bytes(partials, "partials", int(rows) * int(N))
    with torch.cuda.device(dev):
        st = lib().rmsnorm_dgamma_reduce(_ptr(partials), int(rows), int(N), _ptr(dgamma), _stream(stream, dev))
    _check(st, "rmsnorm_dgamma_reduce")


def rmsnorm_bwd(x, gamma, dy, rstd, dx, dgamma, workspace, gemma: bool = False, stream=None) -> None:
    """Full backward: dx (may be dy itself) and dgamma (fp32, overwritten)."""
    M, N, stride = _bwd_checks(x, gamma, dy, rstd, dx)
    dev = _gpu(x, dgamma, workspace)
    _vec(dgamma, N, torch.float32, "dgamma")
    wbytes = _scratch_bytes(workspace, "workspace")
    with torch.cuda.device(dev):
        st = lib().rmsnorm_bwd(_ptr(x), _ptr(gamma), _ptr(dy), _ptr(rstd), _ptr(dx), _ptr(dgamma), _ptr(workspace),
                               wbytes, M, N, stride, _dtype_code(x), _flags(gemma), _stream(stream, dev))
    _check(st, "rmsnorm_bwd")


def rmsnorm_bwd_noalloc(x, gamma, dy, rstd, dx, dgamma, gemma: bool = False, stream=None) -> None:
    """The full backward with the library's static scratch in place of a
    workspace (no device allocation; calls on one GPU must not overlap)."""
    M, N, stride = _bwd_checks(x, gamma, dy, rstd, dx)
    dev = _gpu(x, dgamma)
    _vec(dgamma, N, torch.float32, "dgamma")
    with torch.cuda.device(dev):
        st = lib().rmsnorm_bwd_noalloc(_ptr(x), _ptr(gamma), _ptr(dy), _ptr(rstd), _ptr(dx), _ptr(dgamma), M, N,
                                       stride, _dtype_code(x), _flags(gemma), _stream(stream, dev))
    _check(st, "rmsnorm_bwd_noalloc")


# ---------------------------------------------------------------------------
# LayerNorm (include/layernorm.h)
# ---------------------------------------------------------------------------

def _vec_f32(t, n: int, name: str) -> None:
    if t.dtype != torch.float32 or t.numel() != n or (n > 1 and t.stride(-1) != 1) or t.dim() != 1:
        raise ValueError(f"{name} must be a contiguous 1-D float32 tensor of {n} elements")


def layernorm_fwd(x, weight, bias, y, mean, rstd, eps: float = 1e-5, stream=None) -> None:
    """y = (x - mean) * rstd * weight + bias, and the per-row mean and rstd, on the GPU."""
    dev = _gpu(x, weight, bias, y, mean, rstd)
    M, N, stride = _rows(x, "x")
    _same_layout(x, y, "y", stride)
    _vec(weight, N, x.dtype, "weight")
    _vec(bias, N, x.dtype, "bias")
    _vec_f32(mean, M, "mean")
    _vec_f32(rstd, M, "rstd")
    with torch.cuda.device(dev):
        st = lib().layernorm_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(y), _ptr(mean), _ptr(rstd), M, N, stride,
                                 float(eps), _dtype_code(x), _stream(stream, dev))
    _check(st, "layernorm_fwd")


def layernorm_bwd_workspace_bytes(M: int, N: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DTYPES.get(dtype, -1)
    out = ctypes.c_size_t(0)
    _check(lib().layernorm_bwd_workspace_bytes(int(M), int(N), int(code), ctypes.byref(out)),
           "layernorm_bwd_workspace_bytes")
    return int(out.value)


def _ln_bwd_checks(x, weight, dy, mean, rstd, dx):
    _gpu(x, weight, dy, mean, rstd, dx)
    M, N, stride = _rows(x, "x")
    _same_layout(x, dy, "dy", stride)
    _same_layout(x, dx, "dx", stride)
    _vec(weight, N, x.dtype, "weight")
    _vec_f32(mean, M, "mean")
    _vec_f32(rstd, M, "rstd")
    return M, N, stride


def layernorm_bwd_rows(x, weight, dy, mean, rstd, dx, workspace, stream=None) -> int:
    """dx (may be dy itself) and per-workgroup dw / db partial rows; returns P, the
    partial-row count (dw partials in rows [0, P), db partials in rows [P, 2P))."""
    M, N, stride = _ln_bwd_checks(x, weight, dy, mean, rstd, dx)
    dev = _gpu(x, workspace)
    wbytes = _scratch_bytes(workspace, "workspace")
    rows = _c_i64(0)
    with torch.cuda.device(dev):
        st = lib().layernorm_bwd_rows(_ptr(x), _ptr(weight), _ptr(dy), _ptr(mean), _ptr(rstd), _ptr(dx),
                                      _ptr(workspace), wbytes, M, N, stride, _dtype_code(x),
                                      ctypes.byref(rows), _stream(stream, dev))
    _check(st, "layernorm_bwd_rows")
    return int(rows.value)


def layernorm_dwdb_reduce(partials, rows: int, N: int, dw, db, stream=None) -> None:
    """dw[j] = sum of partials[p, j] over p < rows; db[j] = sum of partials[rows + p, j]."""
    dev = _gpu(partials, dw, db)
    _vec_f32(dw, N, "dw")
    _vec_f32(db, N, "db")
    if rows > 0:
        _scratch_bytes(partials, "partials", 2 * int(rows) * int(N))
    with torch.cuda.device(dev):
        st = lib().layernorm_dwdb_reduce(_ptr(partials), int(rows), int(N), _ptr(dw), _ptr(db), _stream(stream, dev))
    _check(st, "layernorm_dwdb_reduce")


def layernorm_bwd(x, weight, dy, mean, rstd, dx, dw, db, workspace, stream=None) -> None:
    """Full LayerNorm backward: dx (may be dy itself), dw and db (fp32, overwritten)."""
    M, N, stride = _ln_bwd_checks(x, weight, dy, mean, rstd, dx)
    dev = _gpu(x, dw, db, workspace)
    _vec_f32(dw, N, "dw")
    _vec_f32(db, N, "db")
    wbytes = _scratch_bytes(workspace, "workspace")
    with torch.cuda.device(dev):
        st = lib().layernorm_bwd(_ptr(x), _ptr(weight), _ptr(dy), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dw),
                                 _ptr(db), _ptr(workspace), wbytes, M, N, stride, _dtype_code(x), _stream(stream, dev))
    _check(st, "layernorm_bwd")


# ---------------------------------------------------------------------------
# RoPE (include/rope.h) and SwiGLU (include/swiglu.h)
# ---------------------------------------------------------------------------

def _rope_args(q, cos, sin, positions, seq_len):
    dev = _gpu(q, cos, sin, positions)
    if q.dim() != 3:
        raise ValueError("q must be 3-D [tokens, heads, head_dim]")
    T, H, D = q.shape
    if D > 1 and q.stride(2) != 1 or H > 1 and q.stride(1) != D:
        raise ValueError("the heads of a token must be contiguous ([.., heads, head_dim] dense per token)")
    stride = q.stride(0) if T > 1 else H * D
    for t, name in ((cos, "cos"), (sin, "sin")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != D // 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [table_rows, head_dim/2] table")
    if cos.shape != sin.shape:
        raise ValueError("cos and sin must have the same shape")
    if positions is not None and (positions.dtype != torch.int32 or positions.numel() != T or
                                  not positions.is_contiguous()):
        raise ValueError("positions must be a contiguous int32 tensor of one entry per token")
    seq = int(seq_len) if seq_len is not None else cos.shape[0]
    return T, H, D, stride, cos.shape[0], seq, dev


def rope_fwd(q, cos, sin, positions=None, seq_len=None, stream=None) -> None:
    """Rotates q [tokens, heads, head_dim] in place (pairs are the two head halves)."""
    T, H, D, stride, rows, seq, dev = _rope_args(q, cos, sin, positions, seq_len)
    with torch.cuda.device(dev):
        st = lib().rope_fwd(_ptr(q), T, H, D, stride, _ptr(cos), _ptr(sin), rows, _ptr(positions), seq,
                            _dtype_code(q), _stream(stream, dev))
    _check(st, "rope_fwd")


def rope_bwd(dq, cos, sin, positions=None, seq_len=None, stream=None) -> None:
    """The inverse rotation (sin negated) of the gradient dq, in place."""
    T, H, D, stride, rows, seq, dev = _rope_args(dq, cos, sin, positions, seq_len)
    with torch.cuda.device(dev):
        st = lib().rope_bwd(_ptr(dq), T, H, D, stride, _ptr(cos), _ptr(sin), rows, _ptr(positions), seq,
                            _dtype_code(dq), _stream(stream, dev))
    _check(st, "rope_bwd")


def _elementwise_layout(ref, others, names):
    M, N, stride = _rows(ref, names[0])
    for t, name in zip(others, names[1:]):
        _same_layout(ref, t, name, stride)
    return M, N, stride


def swiglu_fwd(e, g, h, stream=None) -> None:
    """h = T(T(silu(e)) * g) over [M, N] (h may be e or g itself)."""
    dev = _gpu(e, g, h)
    M, N, stride = _elementwise_layout(e, (g, h), ("e", "g", "h"))
    with torch.cuda.device(dev):
        st = lib().swiglu_fwd(_ptr(e), _ptr(g), _ptr(h), M, N, stride, _dtype_code(e), _stream(stream, dev))
    _check(st, "swiglu_fwd")


def swiglu_bwd(dh, e, g, h, df, de, stream=None) -> None:
    """h (recomputed), df = dh * T(f) and de = dh * g * silu'(e); each output may be one of the inputs."""
    dev = _gpu(dh, e, g, h, df, de)
    M, N, stride = _elementwise_layout(e, (dh, g, h, df, de), ("e", "dh", "g", "h", "df", "de"))
    with torch.cuda.device(dev):
        st = lib().swiglu_bwd(_ptr(dh), _ptr(e), _ptr(g), _ptr(h), _ptr(df), _ptr(de), M, N, stride, _dtype_code(e),
                              _stream(stream, dev))
    _check(st, "swiglu_bwd")
