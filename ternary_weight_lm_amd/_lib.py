"""ctypes binding of libbitlinear.so: the C entry points under the same
names, with torch tensors turned into device pointers and the current HIP
stream.  Argument marshalling only; every step of the layer runs in the HIP
kernels behind these calls.  A missing library is an error, never a
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "bitlinear.h")

BL_F32, BL_F16, BL_BF16 = 0, 1, 2
BL_PATH_AUTO, BL_PATH_FUSED, BL_PATH_SKINNY, BL_PATH_MFMA = 0, 1, 2, 3

STATUS = {
    0: "BL_OK", -1: "BL_ERR_NULL", -2: "BL_ERR_DTYPE", -3: "BL_ERR_SHAPE",
    -4: "BL_ERR_ALIGN", -5: "BL_ERR_WORKSPACE", -6: "BL_ERR_EPS",
    -7: "BL_ERR_HIP", -8: "BL_ERR_UNSUPPORTED", -9: "BL_ERR_PATH",
}

DTYPE_CODE = {torch.float32: BL_F32, torch.float16: BL_F16, torch.bfloat16: BL_BF16}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}


class BitLinearError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({message})")
        self.status = status


_lib = None

P = ctypes.c_void_p


class BlContractCall(ctypes.Structure):
    """struct bl_contract_call of bitlinear.h"""
    _fields_ = [("xq", ctypes.c_void_p), ("s", ctypes.c_void_p), ("rowsum", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64)]


class BlCall(ctypes.Structure):
    """struct bl_call of bitlinear.h"""
    _fields_ = [("x", ctypes.c_void_p), ("gain", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64)]


I64 = ctypes.c_int64
SZ = ctypes.c_size_t
I = ctypes.c_int
F = ctypes.c_float

SIGNATURES = {
    "bitlinear_packed_bytes": ([I64, I64], SZ),
    "bitlinear_pack_workspace_bytes": ([I64, I64], SZ),
    "bitlinear_pack_weights": ([P, I64, I64, P, P, P, SZ, P], I),
    "bitlinear_workspace_bytes": ([I64, I64, I64], SZ),
    "bitlinear_forward": ([P, I, I64, I64, P, P, P, I64, P, I, F, P, SZ, P], I),
    "bitlinear_forward_path": ([P, I, I64, I64, P, P, P, I64, P, I, F, P, SZ, I, P], I),
    "bitlinear_forward_grouped": ([P, I, I, I, F, P], I),
    "bitlinear_status_string": ([I], ctypes.c_char_p),
    "bitlinear_select_path": ([I64, I64], I),
    "bitlinear_grouped_workspace_bytes": ([P, I, I], SZ),
    "bitlinear_contract_grouped": ([P, I, I, P], I),
    "bitlinear_forward_grouped_ws": ([P, I, I, I, F, P, SZ, P], I),
    "bitlinear_act_quant": ([P, I, P, I64, I64, F, P, P, P, P], I),
    "bitlinear_gemm_i32": ([P, P, I64, I64, P, I64, P, I, P], I),
    "bitlinear_contract": ([P, P, P, I64, I64, P, P, I64, P, I, I, P], I),
    "bitlinear_pack_glu_weights": ([P, I64, I64, P, P, P, SZ, P], I),
    "bitlinear_forward_glu": ([P, I, I64, I64, P, P, P, I64, P, I, F, P, SZ, I, P], I),
    "bitlinear_unpack_weights": ([P, I64, I64, P, P], I),
}


def lib() -> ctypes.CDLL:
    """Load libbitlinear.so (built by ternary_weight_lm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m ternary_weight_lm_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        msg = lib().bitlinear_status_string(status).decode()
        raise BitLinearError(fn, status, msg)


# --------------------------------------------------------- same-name calls

def bitlinear_packed_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes(N, K))


def bitlinear_pack_workspace_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_pack_workspace_bytes(N, K))


def bitlinear_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().bitlinear_workspace_bytes(M, K, N))


def bitlinear_select_path(M: int, K: int) -> int:
    p = int(lib().bitlinear_select_path(M, K))
    _check("bitlinear_select_path", min(p, 0))
    return p


def bitlinear_status_string(status: int) -> str:
    return lib().bitlinear_status_string(status).decode()


def bitlinear_pack_weights(W, packed, beta, ws, stream=None):
    N, K = W.shape
    _check("bitlinear_pack_weights", lib().bitlinear_pack_weights(
        _ptr(W), N, K, _ptr(packed), _ptr(beta), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward(x, gain, packed, beta, N, y, ws, eps=1e-8, stream=None):
    M, K = x.shape
    _check("bitlinear_forward", lib().bitlinear_forward(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), N,
        _ptr(y), DTYPE_CODE[y.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward_path(x, gain, packed, beta, N, y, ws, path, eps=1e-8, stream=None):
    M, K = x.shape
    _check("bitlinear_forward_path", lib().bitlinear_forward_path(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), N,
        _ptr(y), DTYPE_CODE[y.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        path, _stream(stream)))


def bitlinear_pack_glu_weights(W, packed, beta, ws, stream=None):
    """W: gate_proj [2F, K] fp32 (rows 0..F-1 SiLU-gated, F..2F-1 multiplied)."""
    N2, K = W.shape
    _check("bitlinear_pack_glu_weights", lib().bitlinear_pack_glu_weights(
        _ptr(W), N2 // 2, K, _ptr(packed), _ptr(beta), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward_glu(x, gain, packed, beta, F, h, ws, path=BL_PATH_AUTO, eps=1e-8,
                          stream=None):
    M, K = x.shape
    _check("bitlinear_forward_glu", lib().bitlinear_forward_glu(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), F,
        _ptr(h), DTYPE_CODE[h.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        path, _stream(stream)))


def make_calls(items):
    """ctypes array of bl_call from (x, gain, packed, beta, y) tensor tuples."""
    arr = (BlCall * len(items))()
    for i, (x, gain, packed, beta, y) in enumerate(items):
        M, K = x.shape
        arr[i] = BlCall(_ptr(x), _ptr(gain), _ptr(packed), _ptr(beta), _ptr(y), M, K,
                        y.shape[1])
    return arr


def bitlinear_forward_grouped(calls, x_dtype, y_dtype, eps=1e-8, stream=None):
    """calls: a make_calls() array (kept by the caller, e.g. for graph capture)
    or a list of (x, gain, packed, beta, y) tuples."""
    if not isinstance(calls, ctypes.Array):
        calls = make_calls(calls)
    _check("bitlinear_forward_grouped", lib().bitlinear_forward_grouped(
        ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[x_dtype],
        DTYPE_CODE[y_dtype], eps, _stream(stream)))


def bitlinear_grouped_workspace_bytes(calls, x_dtype) -> int:
    """calls: a make_calls() array or a list of (x, gain, packed, beta, y)."""
    if not isinstance(calls, ctypes.Array):
        calls = make_calls(calls)
    return int(lib().bitlinear_grouped_workspace_bytes(
        ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[x_dtype]))


def bitlinear_forward_grouped_ws(calls, x_dtype, y_dtype, ws, eps=1e-8, stream=None):
    """calls: a make_calls() array (kept by the caller, e.g. for graph capture)
    or a list of (x, gain, packed, beta, y) tuples; ws: a device tensor of at
    least bitlinear_grouped_workspace_bytes(calls, x_dtype) bytes, or None."""
    if not isinstance(calls, ctypes.Array):
        calls = make_calls(calls)
    _check("bitlinear_forward_grouped_ws", lib().bitlinear_forward_grouped_ws(
        ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[x_dtype],
        DTYPE_CODE[y_dtype], eps, _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def bitlinear_act_quant(x, gain, xq, s, rowsum, eps=1e-8, stream=None):
    M, K = x.shape
    _check("bitlinear_act_quant", lib().bitlinear_act_quant(
        _ptr(x), DTYPE_CODE[x.dtype], _ptr(gain), M, K, eps, _ptr(xq), _ptr(s),
        _ptr(rowsum), _stream(stream)))


def bitlinear_gemm_i32(xq, rowsum, packed, N, acc, path=BL_PATH_AUTO, stream=None):
    M, K = xq.shape
    _check("bitlinear_gemm_i32", lib().bitlinear_gemm_i32(
        _ptr(xq), _ptr(rowsum), M, K, _ptr(packed), N, _ptr(acc), path, _stream(stream)))


def bitlinear_contract(xq, s, rowsum, packed, beta, N, y, path=BL_PATH_AUTO, stream=None):
    M, K = xq.shape
    _check("bitlinear_contract", lib().bitlinear_contract(
        _ptr(xq), _ptr(s), _ptr(rowsum), M, K, _ptr(packed), _ptr(beta), N, _ptr(y),
        DTYPE_CODE[y.dtype], path, _stream(stream)))


def make_contract_calls(items):
    """ctypes array of bl_contract_call from (xq, s, rowsum, packed, beta, y)
    tensor tuples."""
    arr = (BlContractCall * len(items))()
    for i, (xq, s, rowsum, packed, beta, y) in enumerate(items):
        M, K = xq.shape
        arr[i] = BlContractCall(_ptr(xq), _ptr(s), _ptr(rowsum), _ptr(packed), _ptr(beta),
                                _ptr(y), M, K, y.shape[1])
    return arr


def bitlinear_contract_grouped(calls, y_dtype, stream=None):
    """calls: a make_contract_calls() array or a list of tuples for it."""
    if not isinstance(calls, ctypes.Array):
        calls = make_contract_calls(calls)
    _check("bitlinear_contract_grouped", lib().bitlinear_contract_grouped(
        ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[y_dtype], _stream(stream)))


def bitlinear_unpack_weights(packed, N, K, Wq, stream=None):
    _check("bitlinear_unpack_weights", lib().bitlinear_unpack_weights(
        _ptr(packed), N, K, _ptr(Wq), _stream(stream)))
