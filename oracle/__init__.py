"""ctypes front end of the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py.  The library package never imports it.

Every function takes and returns numpy arrays; the arithmetic is all in the
C file, whose header lists the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (plain gcc)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    """The compiled oracle; ORACLE_LIB names another build of oracle.c to load
    instead (the sanitizer run of the pin suite uses it)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("ORACLE_LIB")
        if alt:
            _lib = load(alt)
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"oracle library {_LIB_PATH} is not built; run "
                "__graft_entry__.build() (or oracle.build()) first")
        _lib = load(_LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Open a compiled oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    L.oracle_matmul_i64.argtypes = [P, P, I64, I64, I64, P]
    L.oracle_matmul_i64.restype = None
    L.oracle_abs_sum.argtypes = [P, I64]
    L.oracle_abs_sum.restype = ctypes.c_double
    L.oracle_weight_scale.argtypes = [P, I64, I64]
    L.oracle_weight_scale.restype = F
    L.oracle_ternarize.argtypes = [P, I64, F, P]
    L.oracle_ternarize.restype = None
    L.oracle_packed_bytes.argtypes = [I64, I64]
    L.oracle_packed_bytes.restype = I64
    L.oracle_pack.argtypes = [P, I64, I64, P]
    L.oracle_pack.restype = ctypes.c_int
    L.oracle_unpack.argtypes = [P, I64, I64, P]
    L.oracle_unpack.restype = ctypes.c_int
    L.oracle_pack_weights.argtypes = [P, I64, I64, P, P, P]
    L.oracle_pack_weights.restype = ctypes.c_int
    L.oracle_rmsnorm.argtypes = [P, P, I64, I64, F, P, P]
    L.oracle_rmsnorm.restype = None
    L.oracle_act_quant.argtypes = [P, I64, I64, P, P, P]
    L.oracle_act_quant.restype = None
    L.oracle_contract.argtypes = [P, P, I64, I64, I64, P]
    L.oracle_contract.restype = ctypes.c_int
    L.oracle_epilogue.argtypes = [P, P, F, I64, I64, P]
    L.oracle_epilogue.restype = None
    L.oracle_forward.argtypes = [P, P, I64, I64, P, F, I64, F, P, P, P, P, P]
    L.oracle_silu.restype = ctypes.c_double
    L.oracle_silu.argtypes = [ctypes.c_double]
    L.oracle_rmsnorm_swish_gate.argtypes = [P, P, P, I64, I64, ctypes.c_double, P]
    L.oracle_rmsnorm_swish_gate.restype = None
    L.oracle_glu.restype = None
    L.oracle_glu.argtypes = [P, I64, I64, P]
    L.oracle_glu_rows.restype = ctypes.c_int
    L.oracle_glu_rows.argtypes = [I64, P]
    L.oracle_forward.restype = ctypes.c_int
    L.oracle_mlgru_scan.argtypes = [P, P, I64, I64, I64, P, P, P]
    L.oracle_mlgru_scan.restype = None
    return L


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- wrappers

def matmul_i64(A, B) -> np.ndarray:
    A = _c(A, np.int64)
    B = _c(B, np.int64)
    m, k = A.shape
    k2, n = B.shape
    assert k == k2
    C = np.empty((m, n), np.int64)
    lib().oracle_matmul_i64(_p(A), _p(B), m, k, n, _p(C))
    return C


def abs_sum(W) -> float:
    W = _c(W, np.float32)
    return float(lib().oracle_abs_sum(_p(W), W.size))


def weight_scale(W) -> np.float32:
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(lib().oracle_weight_scale(_p(W), N, K))


def ternarize(W, beta) -> np.ndarray:
    W = _c(W, np.float32)
    Wq = np.empty(W.shape, np.int8)
    lib().oracle_ternarize(_p(W), W.size, np.float32(beta), _p(Wq))
    return Wq


def pack(Wq) -> np.ndarray:
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    out = np.empty(N * K // 4, np.uint8)
    rc = lib().oracle_pack(_p(Wq), N, K, _p(out))
    if rc != 0:
        raise ValueError("oracle_pack rejected the input")
    return out


def unpack(packed, N: int, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    assert packed.size == N * K // 4
    Wq = np.empty((N, K), np.int8)
    rc = lib().oracle_unpack(_p(packed), N, K, _p(Wq))
    if rc != 0:
        raise ValueError("oracle_unpack rejected the input")
    return Wq


def pack_weights(W):
    """Returns (packed uint8 [N*K/4], beta float32, Wq int8 [N,K])."""
    W = _c(W, np.float32)
    N, K = W.shape
    packed = np.empty(N * K // 4, np.uint8)
    Wq = np.empty((N, K), np.int8)
    beta = np.zeros(1, np.float32)
    rc = lib().oracle_pack_weights(_p(W), N, K, _p(packed), _p(beta), _p(Wq))
    if rc != 0:
        raise ValueError("oracle_pack_weights rejected the input")
    return packed, np.float32(beta[0]), Wq


def rmsnorm(x, g, eps=1e-8):
    """Returns (xn float32 [M,K], r float32 [M])."""
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(g, np.float32)
    M, K = x.shape
    xn = np.empty((M, K), np.float32)
    r = np.empty(M, np.float32)
    lib().oracle_rmsnorm(_p(x), _p(g), M, K, np.float32(eps), _p(xn), _p(r))
    return xn, r


def act_quant(xn):
    """Returns (xq int8 [M,K], s float32 [M], v float32 [M,K])."""
    xn = _c(np.atleast_2d(xn), np.float32)
    M, K = xn.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    v = np.empty((M, K), np.float32)
    lib().oracle_act_quant(_p(xn), M, K, _p(xq), _p(s), _p(v))
    return xq, s, v


def contract(xq, Wq) -> np.ndarray:
    xq = _c(np.atleast_2d(xq), np.int8)
    Wq = _c(np.atleast_2d(Wq), np.int8)
    M, K = xq.shape
    N, K2 = Wq.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    rc = lib().oracle_contract(_p(xq), _p(Wq), M, N, K, _p(acc))
    if rc != 0:
        raise OverflowError("oracle_contract: sum outside int32")
    return acc


def epilogue(acc, s, beta) -> np.ndarray:
    acc = _c(np.atleast_2d(acc), np.int32)
    s = _c(s, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    lib().oracle_epilogue(_p(acc), _p(s), np.float32(beta), M, N, _p(y))
    return y


def forward(x, g, Wq, beta, eps=1e-8):
    """Whole FusedBitLinear forward.  Returns dict with y (fp64 [M,N]),
    xq, s, v, acc."""
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(g, np.float32)
    Wq = _c(Wq, np.int8)
    M, K = x.shape
    N = Wq.shape[0]
    y = np.empty((M, N), np.float64)
    xq = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    v = np.empty((M, K), np.float32)
    acc = np.empty((M, N), np.int32)
    rc = lib().oracle_forward(_p(x), _p(g), M, K, _p(Wq), np.float32(beta), N,
                              np.float32(eps), _p(y), _p(xq), _p(s), _p(v),
                              _p(acc))
    if rc != 0:
        raise RuntimeError("oracle_forward failed")
    return {"y": y, "xq": xq, "s": s, "v": v, "acc": acc}


# ------------------------------------------------------------------ GLU MLP

def silu(a: float) -> float:
    return float(lib().oracle_silu(float(a)))


def glu(y) -> np.ndarray:
    """h [M,F] = silu(y[:, :F]) * y[:, F:] for the gate_proj output y [M,2F]."""
    y = _c(np.atleast_2d(y), np.float64)
    M, F2 = y.shape
    assert F2 % 2 == 0
    F = F2 // 2
    h = np.empty((M, F), np.float64)
    lib().oracle_glu(_p(y), M, F, _p(h))
    return h


def glu_rows(F: int) -> np.ndarray:
    """Source row of every packed row of a [2F, K] gate_proj in GLU order."""
    src = np.empty(2 * F, np.int64)
    if lib().oracle_glu_rows(F, _p(src)) != 0:
        raise ValueError("F must be a positive multiple of 16")
    return src


def pack_glu_weights(W):
    """gate_proj W [2F,K] -> (packed in GLU row order, beta, Wq [2F,K] in
    the original row order).  beta is the per-tensor scale of all 2F rows."""
    W = _c(W, np.float32)
    src = glu_rows(W.shape[0] // 2)
    packed, beta, Wq_perm = pack_weights(W[src])
    Wq = np.empty_like(Wq_perm)
    Wq[src] = Wq_perm
    return packed, beta, Wq


def forward_glu(x, g, Wq, beta, eps=1e-8):
    """gate_proj FusedBitLinear (Wq [2F,K], original row order) followed by
    the GLU gate.  Returns the forward() dict plus h (fp64 [M,F])."""
    out = forward(x, g, Wq, beta, eps)
    out["h"] = glu(out["y"])
    return out


# ------------------------------------------- FusedRMSNormSwishGate (reading)

def rmsnorm_swish_gate(o, g, w, eps=1e-6) -> np.ndarray:
    """z [M,K] (fp64) = (o * r) * w * silu(g), r = 1/sqrt(mean(o^2) + eps):
    the reading of FusedRMSNormSwishGate (oracle.c)."""
    o = _c(np.atleast_2d(o), np.float32)
    g = _c(np.atleast_2d(g), np.float32)
    w = _c(w, np.float32)
    M, K = o.shape
    assert g.shape == (M, K) and w.shape == (K,)
    z = np.empty((M, K), np.float64)
    lib().oracle_rmsnorm_swish_gate(_p(o), _p(g), _p(w), M, K, float(eps), _p(z))
    return z


def mlgru_scan(i, f, h0=None):
    """h [B,T,D] (fp64), hT [B,D] (fp64): the reading of the MLGRU recurrence
    (oracle.c): h_t = a h_{t-1} + (1 - a) i_t, a = sigmoid(f_t), h_{-1} = h0
    (zeros when None).  i, f [B,T,D] (or [T,D] for one sequence), widened
    exactly to fp32."""
    i = np.asarray(i)
    squeeze = i.ndim == 2
    i = _c(i[None] if squeeze else i, np.float32)
    f = np.asarray(f)
    f = _c(f[None] if squeeze else f, np.float32)
    B, T, D = i.shape
    assert f.shape == (B, T, D)
    h = np.empty((B, T, D), np.float64)
    hT = np.empty((B, D), np.float64)
    h0p = None
    if h0 is not None:
        h0 = _c(np.asarray(h0).reshape(B, D), np.float64)
        h0p = _p(h0)
    lib().oracle_mlgru_scan(_p(i), _p(f), B, T, D, h0p, _p(h), _p(hT))
    return (h[0], hT[0]) if squeeze else (h, hT)
