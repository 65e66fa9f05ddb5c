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
    -7: "BL_ERR_HIP", -8: "BL_ERR_UNSUPPORTED", -9: "BL_ERR_PATH", -10: "BL_ERR_SCRATCH",
    -11: "BL_ERR_TIMEOUT",
}
BL_ERR_TIMEOUT = -11

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


class BlChainCall(ctypes.Structure):
    """struct bl_chain_call of bitlinear.h"""
    _fields_ = [("x", ctypes.c_void_p), ("gain", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("y", ctypes.c_void_p), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64), ("glu", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class BlChain(ctypes.Structure):
    """struct bl_chain of bitlinear.h (a planned chain)"""
    _fields_ = [("ws", ctypes.c_void_p), ("M", ctypes.c_int64), ("items", ctypes.c_int64),
                ("kmax", ctypes.c_int64), ("grid", ctypes.c_int64), ("lds", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("ncalls", ctypes.c_int32)]


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
    "bitlinear_contract_grouped_path": ([P, I, I, I, P], I),
    "bitlinear_forward_grouped_ws": ([P, I, I, I, F, P, SZ, P], I),
    "bitlinear_act_quant": ([P, I, P, I64, I64, F, P, P, P, P], I),
    "bitlinear_gemm_i32": ([P, P, I64, I64, P, I64, P, I, P], I),
    "bitlinear_contract": ([P, P, P, I64, I64, P, P, I64, P, I, I, P], I),
    "bitlinear_contract_glu": ([P, P, P, I64, I64, P, P, I64, P, I, I, P], I),
    "bitlinear_pack_glu_weights": ([P, I64, I64, P, P, P, SZ, P], I),
    "bitlinear_forward_glu": ([P, I, I64, I64, P, P, P, I64, P, I, F, P, SZ, I, P], I),
    "bitlinear_unpack_weights": ([P, I64, I64, P, P], I),
    "bitlinear_noalloc_max_scratch_bytes": ([], SZ),
    "bitlinear_test_fail_launches": ([I], None),
    "bitlinear_set_decode_contraction": ([I], I),
    "bitlinear_get_decode_contraction": ([], I),
    "bitlinear_rmsnorm_swish_gate": ([P, P, P, I, I64, I64, F, P, P], I),
    "bitlinear_forward_gated": ([P, P, P, F, I, I64, I64, P, P, P, I64, P, I, F, P, SZ, P], I),
    "bitlinear_chain_workspace_bytes": ([P, I, I64], SZ),
    "bitlinear_chain_plan": ([P, I, I64, I, F, P, SZ, P, P], I),
    "bitlinear_chain_run": ([P, P], I),
    "bitlinear_chain_run_ex": ([P, ctypes.c_uint32, P], I),
    "bitlinear_chain_status": ([P, P], I),
    "bitlinear_forward_noalloc": ([P, I, I64, I64, P, P, P, I64, P, I, F, P], I),
    "bitlinear_mlgru_workspace_bytes": ([I64, I64, I64], SZ),
    "bitlinear_mlgru_scan": ([P, P, I, I64, I64, I64, P, P, P, P, SZ, P], I),
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


def _need(t, name, dtype=None, numel=None, dims=None):
    """Host-side size / dtype check of a tensor handed to the C ABI: the ABI
    sees only pointers, so a tensor smaller than the call implies would let
    the kernels read or write past its allocation.  Runs before any pointer
    is taken."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, (tuple, list, set)) else t.dtype == dtype
        if not ok:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimension(s), has shape {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


def _nbytes(t):
    return t.numel() * t.element_size()


FLOATS = (torch.float32, torch.float16, torch.bfloat16)


def _check_layer_io(x, gain, packed, beta, N, y, n_out):
    """x [M, K] (any float dtype), gain [K] (x's dtype), packed >= N K / 4
    bytes, beta fp32 [>= 1], y [M, n_out] float."""
    _need(x, "x", FLOATS, dims=2)
    M, K = x.shape
    _need(gain, "gain", x.dtype, numel=K)
    _need(packed, "packed", numel=1)
    if _nbytes(packed) < N * K // 4:
        raise ValueError(f"packed holds {_nbytes(packed)} bytes, an [{N}, {K}] matrix needs "
                         f"{N * K // 4}")
    _need(beta, "beta", torch.float32, numel=1)
    _need(y, "y", FLOATS, numel=M * n_out)
    return M, K


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


def _check_pack(W, packed, beta, ws, rows):
    _need(W, "W", torch.float32, dims=2)
    N, K = W.shape
    _need(packed, "packed", numel=1)
    if _nbytes(packed) < rows * K // 4:
        raise ValueError(f"packed holds {_nbytes(packed)} bytes, needs {rows * K // 4}")
    _need(beta, "beta", torch.float32, numel=1)
    _need(ws, "ws", numel=1)
    return N, K


def bitlinear_pack_weights(W, packed, beta, ws, stream=None):
    N, K = _check_pack(W, packed, beta, ws, W.shape[0] if W is not None and W.dim() == 2 else 0)
    _check("bitlinear_pack_weights", lib().bitlinear_pack_weights(
        _ptr(W), N, K, _ptr(packed), _ptr(beta), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward(x, gain, packed, beta, N, y, ws, eps=1e-8, stream=None):
    M, K = _check_layer_io(x, gain, packed, beta, N, y, N)
    _need(ws, "ws", numel=1)
    _check("bitlinear_forward", lib().bitlinear_forward(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), N,
        _ptr(y), DTYPE_CODE[y.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward_path(x, gain, packed, beta, N, y, ws, path, eps=1e-8, stream=None):
    M, K = _check_layer_io(x, gain, packed, beta, N, y, N)
    _need(ws, "ws", numel=1)
    _check("bitlinear_forward_path", lib().bitlinear_forward_path(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), N,
        _ptr(y), DTYPE_CODE[y.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        path, _stream(stream)))


def bitlinear_test_fail_launches(n: int):
    """Test hook: the next n kernel launches of the library fail with
    BL_ERR_HIP without launching (0 clears)."""
    lib().bitlinear_test_fail_launches(int(n))


BL_DECODE_AUTO, BL_DECODE_MFMA, BL_DECODE_VALU = 0, 1, 2


def bitlinear_set_decode_contraction(unit: int):
    """Matrix cores (BL_DECODE_MFMA) or vector ALU (BL_DECODE_VALU) for the
    decode kernels' 1- and 2-token contractions; BL_DECODE_AUTO restores the
    library's choice.  Outputs are identical either way."""
    _check("bitlinear_set_decode_contraction", lib().bitlinear_set_decode_contraction(int(unit)))


def bitlinear_get_decode_contraction() -> int:
    return int(lib().bitlinear_get_decode_contraction())


def bitlinear_noalloc_max_scratch_bytes() -> int:
    return int(lib().bitlinear_noalloc_max_scratch_bytes())


def bitlinear_forward_noalloc(x, gain, packed, beta, N, y, eps=1e-8, stream=None):
    """bitlinear_forward with the library's static scratch instead of a
    workspace (no device allocation anywhere in the call)."""
    M, K = _check_layer_io(x, gain, packed, beta, N, y, N)
    _check("bitlinear_forward_noalloc", lib().bitlinear_forward_noalloc(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), N,
        _ptr(y), DTYPE_CODE[y.dtype], eps, _stream(stream)))


def bitlinear_pack_glu_weights(W, packed, beta, ws, stream=None):
    """W: gate_proj [2F, K] fp32 (rows 0..F-1 SiLU-gated, F..2F-1 multiplied)."""
    N2, K = _check_pack(W, packed, beta, ws, W.shape[0] if W is not None and W.dim() == 2 else 0)
    _check("bitlinear_pack_glu_weights", lib().bitlinear_pack_glu_weights(
        _ptr(W), N2 // 2, K, _ptr(packed), _ptr(beta), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def bitlinear_forward_glu(x, gain, packed, beta, F, h, ws, path=BL_PATH_AUTO, eps=1e-8,
                          stream=None):
    M, K = _check_layer_io(x, gain, packed, beta, 2 * F, h, F)
    _need(ws, "ws", numel=1)
    _check("bitlinear_forward_glu", lib().bitlinear_forward_glu(
        _ptr(x), DTYPE_CODE[x.dtype], M, K, _ptr(gain), _ptr(packed), _ptr(beta), F,
        _ptr(h), DTYPE_CODE[h.dtype], eps, _ptr(ws), ws.numel() * ws.element_size(),
        path, _stream(stream)))


def make_calls(items):
    """ctypes array of bl_call from (x, gain, packed, beta, y) tensor tuples."""
    arr = (BlCall * len(items))()
    for i, (x, gain, packed, beta, y) in enumerate(items):
        _need(y, "y", FLOATS, dims=2)
        M, K = _check_layer_io(x, gain, packed, beta, y.shape[1], y, y.shape[1])
        if y.shape[0] != M:
            raise ValueError(f"y has {y.shape[0]} rows, x has {M}")
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
    _need(x, "x", FLOATS, dims=2)
    M, K = x.shape
    _need(gain, "gain", x.dtype, numel=K)
    _need(xq, "xq", torch.int8, numel=M * K)
    _need(s, "s", torch.float32, numel=M)
    _need(rowsum, "rowsum", torch.int32, numel=M)
    _check("bitlinear_act_quant", lib().bitlinear_act_quant(
        _ptr(x), DTYPE_CODE[x.dtype], _ptr(gain), M, K, eps, _ptr(xq), _ptr(s),
        _ptr(rowsum), _stream(stream)))


def _check_codes(xq, rowsum, packed, N, s=None, beta=None):
    _need(xq, "xq", torch.int8, dims=2)
    M, K = xq.shape
    _need(rowsum, "rowsum", torch.int32, numel=M)
    _need(packed, "packed", numel=1)
    if _nbytes(packed) < N * K // 4:
        raise ValueError(f"packed holds {_nbytes(packed)} bytes, an [{N}, {K}] matrix needs "
                         f"{N * K // 4}")
    if s is not None or beta is not None:
        _need(s, "s", torch.float32, numel=M)
        _need(beta, "beta", torch.float32, numel=1)
    return M, K


def bitlinear_gemm_i32(xq, rowsum, packed, N, acc, path=BL_PATH_AUTO, stream=None):
    M, K = _check_codes(xq, rowsum, packed, N)
    _need(acc, "acc", torch.int32, numel=M * N)
    _check("bitlinear_gemm_i32", lib().bitlinear_gemm_i32(
        _ptr(xq), _ptr(rowsum), M, K, _ptr(packed), N, _ptr(acc), path, _stream(stream)))


def bitlinear_contract(xq, s, rowsum, packed, beta, N, y, path=BL_PATH_AUTO, stream=None):
    M, K = _check_codes(xq, rowsum, packed, N, s, beta)
    _need(y, "y", FLOATS, numel=M * N)
    _check("bitlinear_contract", lib().bitlinear_contract(
        _ptr(xq), _ptr(s), _ptr(rowsum), M, K, _ptr(packed), _ptr(beta), N, _ptr(y),
        DTYPE_CODE[y.dtype], path, _stream(stream)))


def bitlinear_contract_glu(xq, s, rowsum, packed, beta, F, h, path=BL_PATH_AUTO, stream=None):
    M, K = _check_codes(xq, rowsum, packed, 2 * F, s, beta)
    _need(h, "h", FLOATS, numel=M * F)
    _check("bitlinear_contract_glu", lib().bitlinear_contract_glu(
        _ptr(xq), _ptr(s), _ptr(rowsum), M, K, _ptr(packed), _ptr(beta), F, _ptr(h),
        DTYPE_CODE[h.dtype], path, _stream(stream)))


def make_contract_calls(items):
    """ctypes array of bl_contract_call from (xq, s, rowsum, packed, beta, y)
    tensor tuples."""
    arr = (BlContractCall * len(items))()
    for i, (xq, s, rowsum, packed, beta, y) in enumerate(items):
        _need(y, "y", FLOATS, dims=2)
        M, K = _check_codes(xq, rowsum, packed, y.shape[1], s, beta)
        if y.shape[0] != M:
            raise ValueError(f"y has {y.shape[0]} rows, xq has {M}")
        arr[i] = BlContractCall(_ptr(xq), _ptr(s), _ptr(rowsum), _ptr(packed), _ptr(beta),
                                _ptr(y), M, K, y.shape[1])
    return arr


def bitlinear_contract_grouped(calls, y_dtype, path=BL_PATH_MFMA, stream=None):
    """calls: a make_contract_calls() array or a list of tuples for it.
    path BL_PATH_MFMA calls bitlinear_contract_grouped, any other path
    bitlinear_contract_grouped_path."""
    if not isinstance(calls, ctypes.Array):
        calls = make_contract_calls(calls)
    if path == BL_PATH_MFMA:
        _check("bitlinear_contract_grouped", lib().bitlinear_contract_grouped(
            ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[y_dtype], _stream(stream)))
    else:
        _check("bitlinear_contract_grouped_path", lib().bitlinear_contract_grouped_path(
            ctypes.cast(calls, ctypes.c_void_p), len(calls), DTYPE_CODE[y_dtype], path,
            _stream(stream)))


def bitlinear_unpack_weights(packed, N, K, Wq, stream=None):
    _need(packed, "packed", numel=1)
    if _nbytes(packed) < N * K // 4:
        raise ValueError(f"packed holds {_nbytes(packed)} bytes, an [{N}, {K}] matrix needs "
                         f"{N * K // 4}")
    _need(Wq, "Wq", torch.int8, numel=N * K)
    _check("bitlinear_unpack_weights", lib().bitlinear_unpack_weights(
        _ptr(packed), N, K, _ptr(Wq), _stream(stream)))


# ------------------------------------------------------------ chained decode

def make_chain_calls(items):
    """ctypes array of bl_chain_call from (x, gain, packed, beta, y, glu)
    tuples: x [M, K] and y [M, n_out] 16-bit; N = n_out, or 2 n_out when glu.
    A call whose x is an earlier call's y reads that call's output."""
    arr = (BlChainCall * len(items))()
    for i, (x, gain, packed, beta, y, glu) in enumerate(items):
        _need(y, "y", (torch.float16, torch.bfloat16), dims=2)
        N = 2 * y.shape[1] if glu else y.shape[1]
        M, K = _check_layer_io(x, gain, packed, beta, N, y, y.shape[1])
        if y.shape[0] != M:
            raise ValueError(f"y has {y.shape[0]} rows, x has {M}")
        arr[i] = BlChainCall(_ptr(x), _ptr(gain), _ptr(packed), _ptr(beta), _ptr(y), K, N,
                             1 if glu else 0, 0)
    return arr


def bitlinear_chain_workspace_bytes(calls, M: int) -> int:
    return int(lib().bitlinear_chain_workspace_bytes(ctypes.cast(calls, ctypes.c_void_p),
                                                     len(calls), M))


def bitlinear_chain_plan(calls, M, dtype, ws, eps=1e-8, stream=None) -> BlChain:
    """Plan a chain (calls: a make_chain_calls() array) into the workspace
    tensor ws; returns the plan (keep ws alive as long as the plan)."""
    _need(ws, "ws", numel=1)
    plan = BlChain()
    _check("bitlinear_chain_plan", lib().bitlinear_chain_plan(
        ctypes.cast(calls, ctypes.c_void_p), len(calls), M, DTYPE_CODE[dtype], eps, _ptr(ws),
        _nbytes(ws), ctypes.byref(plan), _stream(stream)))
    return plan


def bitlinear_chain_run(plan: BlChain, stream=None):
    _check("bitlinear_chain_run", lib().bitlinear_chain_run(ctypes.byref(plan), _stream(stream)))


def bitlinear_chain_run_ex(plan: BlChain, wait_us: int, stream=None):
    _check("bitlinear_chain_run_ex", lib().bitlinear_chain_run_ex(
        ctypes.byref(plan), int(wait_us), _stream(stream)))


def bitlinear_chain_status(plan: BlChain, stream=None) -> int:
    """BL_OK (0) or BL_ERR_TIMEOUT after synchronizing the stream (clears the
    error word); any other failure raises."""
    st = int(lib().bitlinear_chain_status(ctypes.byref(plan), _stream(stream)))
    if st not in (0, BL_ERR_TIMEOUT):
        _check("bitlinear_chain_status", st)
    return st


# ------------------------------------------------------ swish gate (o_proj)

def bitlinear_rmsnorm_swish_gate(o, g, w, z, eps=1e-6, stream=None):
    """z = ((o * r) * w) * silu(g), r = 1/sqrt(mean(o^2) + eps), per row."""
    _need(o, "o", FLOATS, dims=2)
    M, K = o.shape
    _need(g, "g", o.dtype, numel=M * K)
    _need(w, "w", o.dtype, numel=K)
    _need(z, "z", o.dtype, numel=M * K)
    _check("bitlinear_rmsnorm_swish_gate", lib().bitlinear_rmsnorm_swish_gate(
        _ptr(o), _ptr(g), _ptr(w), DTYPE_CODE[o.dtype], M, K, eps, _ptr(z), _stream(stream)))


def bitlinear_mlgru_workspace_bytes(B, T, D):
    return int(lib().bitlinear_mlgru_workspace_bytes(B, T, D))


def bitlinear_mlgru_scan(i, f, h, h0=None, hT=None, ws=None, stream=None):
    """h [B,T,D] = the MLGRU recurrence over i, f [B,T,D] (or [T,D] for one
    sequence): h_t = a h_{t-1} + (1 - a) i_t, a = sigmoid(f_t), from h0
    (fp32 [B,D], zeros when None); hT (fp32 [B,D]) receives the last state.
    ws: scratch of bitlinear_mlgru_workspace_bytes(B, T, D) bytes (allocated
    here when None and needed)."""
    _need(i, "i", FLOATS)
    if i.dim() == 2:
        B, (T, D) = 1, i.shape
    elif i.dim() == 3:
        B, T, D = i.shape
    else:
        raise ValueError(f"i must be [T, D] or [B, T, D], got {tuple(i.shape)}")
    _need(f, "f", i.dtype, numel=B * T * D)
    _need(h, "h", i.dtype, numel=B * T * D)
    if h0 is not None:
        _need(h0, "h0", torch.float32, numel=B * D)
    if hT is not None:
        _need(hT, "hT", torch.float32, numel=B * D)
    need = bitlinear_mlgru_workspace_bytes(B, T, D)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=i.device)
    if ws is not None:
        _need(ws, "ws", numel=1)
    _check("bitlinear_mlgru_scan", lib().bitlinear_mlgru_scan(
        _ptr(i), _ptr(f), DTYPE_CODE[i.dtype], B, T, D, _ptr(h0), _ptr(h), _ptr(hT), _ptr(ws),
        _nbytes(ws) if ws is not None else 0, _stream(stream)))


def bitlinear_forward_gated(o, g, gate_w, gain, packed, beta, N, y, ws, gate_eps=1e-6, eps=1e-8,
                            stream=None):
    """y = FusedBitLinear(z) with z = the swish gate of (o, g) (o_proj with
    the gate as its prologue)."""
    M, K = _check_layer_io(o, gain, packed, beta, N, y, N)
    _need(g, "g", o.dtype, numel=M * K)
    _need(gate_w, "gate_w", o.dtype, numel=K)
    _need(ws, "ws", numel=1)
    _check("bitlinear_forward_gated", lib().bitlinear_forward_gated(
        _ptr(o), _ptr(g), _ptr(gate_w), gate_eps, DTYPE_CODE[o.dtype], M, K, _ptr(gain),
        _ptr(packed), _ptr(beta), N, _ptr(y), DTYPE_CODE[y.dtype], eps, _ptr(ws), _nbytes(ws),
        _stream(stream)))
