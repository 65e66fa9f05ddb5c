"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/bitlinear.h declares, answers the size queries with
their closed forms, and rejects every malformed call with the documented
status before launching anything (so made-up pointers are never touched).
"""
import ctypes
import os
import re

import pytest

import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import _lib

OK, NULL, DTYPE, SHAPE, ALIGN, WS, EPS, HIP, UNSUP, PATH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9

# made-up, 16-byte aligned device addresses: validation fails before any use
A = 0x7F0000001000
B = 0x7F0000002000
C = 0x7F0000003000
D = 0x7F0000004000
E = 0x7F0000005000
Y = 0x7F0000006000
WSP = 0x7F0000100000


def declared_functions():
    text = open(_lib.HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tw.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_size_queries_closed_forms():
    L = tw.lib()
    for N, K in [(32, 128), (1024, 1024), (11264, 2048), (2048, 5632), (2560, 7040)]:
        assert L.bitlinear_packed_bytes(N, K) == N * K // 4
        assert L.bitlinear_pack_workspace_bytes(N, K) > 0
    for bad in [(16, 128), (32, 64), (33, 128), (32, 130), (0, 128), (32, 0),
                (32, 65536 + 128), ((1 << 20) + 32, 128)]:
        assert L.bitlinear_packed_bytes(*bad) == 0
        assert L.bitlinear_pack_workspace_bytes(*bad) == 0

    def al(v):
        return (v + 255) // 256 * 256
    for M, K, N in [(1, 1024, 1024), (16, 1024, 1024), (4096, 2048, 11264), (3, 7040, 2560)]:
        assert L.bitlinear_workspace_bytes(M, K, N) == al(M * K) + 2 * al(4 * M)
    assert L.bitlinear_workspace_bytes(-1, 128, 32) == 0
    assert L.bitlinear_workspace_bytes((1 << 24) + 1, 128, 32) == 0
    assert L.bitlinear_workspace_bytes(0, 128, 32) == 2 * 0 + 0


def test_select_path_rule():
    L = tw.lib()
    assert L.bitlinear_select_path(1, 1024) == 1
    assert L.bitlinear_select_path(4, 7040) == 1
    assert L.bitlinear_select_path(4, 16384) == 2     # fused needs K <= 8192
    assert L.bitlinear_select_path(5, 1024) == 1     # row mode of the decode kernel
    assert L.bitlinear_select_path(8, 4096) == 1
    assert L.bitlinear_select_path(8, 4224) == 2     # row mode needs K <= 4096
    assert L.bitlinear_select_path(9, 1024) == 1     # two rows per wave
    assert L.bitlinear_select_path(16, 1024) == 1
    assert L.bitlinear_select_path(10, 4096) == 1    # 10 * 4112 bytes of codes fit
    assert L.bitlinear_select_path(12, 4096) == 2    # 12 * 4112 do not
    assert L.bitlinear_select_path(16, 2688) == 1
    assert L.bitlinear_select_path(16, 2816) == 2
    assert L.bitlinear_select_path(17, 1024) == 2
    assert L.bitlinear_select_path(64, 7040) == 2
    assert L.bitlinear_select_path(65, 1024) == 3
    assert L.bitlinear_select_path(4096, 2048) == 3
    assert L.bitlinear_select_path(0, 1024) == SHAPE
    assert L.bitlinear_select_path(1, 1000) == SHAPE


def test_status_strings():
    L = tw.lib()
    for code in (OK, NULL, DTYPE, SHAPE, ALIGN, WS, EPS, HIP, UNSUP, PATH, 12345):
        s = L.bitlinear_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


def fwd(x=A, xdt=1, M=4, K=1024, g=B, pk=C, beta=D, N=1024, y=Y, ydt=1, eps=1e-8,
        ws=WSP, wsb=None, path=0):
    L = tw.lib()
    if wsb is None:
        wsb = L.bitlinear_workspace_bytes(M, K, N) if M >= 0 else 0
    return L.bitlinear_forward_path(x, xdt, M, K, g, pk, beta, N, y, ydt, eps, ws, wsb, path, None)


def test_forward_validation_order_and_codes():
    assert fwd(xdt=3) == DTYPE
    assert fwd(ydt=-1) == DTYPE
    assert fwd(K=1000) == SHAPE
    assert fwd(K=0) == SHAPE
    assert fwd(N=48) == SHAPE
    assert fwd(M=-1) == SHAPE
    assert fwd(M=(1 << 24) + 1) == SHAPE
    assert fwd(K=65536 + 128) == SHAPE
    assert fwd(eps=0.0) == EPS
    assert fwd(eps=-1e-8) == EPS
    assert fwd(eps=float("nan")) == EPS
    assert fwd(eps=float("inf")) == EPS
    assert fwd(path=7) == PATH
    assert fwd(path=-1) == PATH
    # empty batch: a valid no-op, even with no buffers at all
    assert fwd(M=0, x=None, y=None, ws=None, wsb=0) == OK
    for kw in ("x", "g", "pk", "beta", "y"):
        assert fwd(**{kw: None}) == NULL, kw
    assert fwd(ws=None) == WS
    assert fwd(wsb=100) == WS
    for kw in ("x", "g", "pk", "y", "ws"):
        assert fwd(**{kw: {"x": A, "g": B, "pk": C, "y": Y, "ws": WSP}[kw] + 8}) == ALIGN, kw
    assert fwd(beta=D + 2) == ALIGN
    # path limits
    assert fwd(M=17, path=1) == SHAPE
    assert fwd(M=65, path=2) == SHAPE
    assert fwd(M=16, K=8192, path=1) == SHAPE   # fused LDS budget exceeded
    assert fwd(M=1, K=8320, path=1) == SHAPE    # fused K limit


def test_forward_default_entry_point_validates_the_same_way():
    L = tw.lib()
    ws = L.bitlinear_workspace_bytes(4, 1024, 1024)
    assert L.bitlinear_forward(A, 1, 4, 1000, B, C, D, 1024, Y, 1, 1e-8, WSP, ws, None) == SHAPE
    assert L.bitlinear_forward(A, 1, 4, 1024, B, C, D, 1024, Y, 1, 0.0, WSP, ws, None) == EPS
    assert L.bitlinear_forward(None, 1, 4, 1024, B, C, D, 1024, Y, 1, 1e-8, WSP, ws, None) == NULL
    assert L.bitlinear_forward(A, 1, 0, 1024, B, C, D, 1024, Y, 1, 1e-8, None, 0, None) == OK


def test_pack_validation():
    L = tw.lib()
    wsb = L.bitlinear_pack_workspace_bytes(64, 256)
    assert L.bitlinear_pack_weights(A, 48, 256, C, D, WSP, wsb, None) == SHAPE
    assert L.bitlinear_pack_weights(A, 64, 200, C, D, WSP, wsb, None) == SHAPE
    assert L.bitlinear_pack_weights(None, 64, 256, C, D, WSP, wsb, None) == NULL
    assert L.bitlinear_pack_weights(A, 64, 256, None, D, WSP, wsb, None) == NULL
    assert L.bitlinear_pack_weights(A, 64, 256, C, None, WSP, wsb, None) == NULL
    assert L.bitlinear_pack_weights(A, 64, 256, C, D, None, wsb, None) == WS
    assert L.bitlinear_pack_weights(A, 64, 256, C, D, WSP, wsb - 1, None) == WS
    assert L.bitlinear_pack_weights(A + 4, 64, 256, C, D, WSP, wsb, None) == ALIGN
    assert L.bitlinear_pack_weights(A, 64, 256, C + 4, D, WSP, wsb, None) == ALIGN
    assert L.bitlinear_pack_weights(A, 64, 256, C, D + 1, WSP, wsb, None) == ALIGN


def test_stage_entry_points_validation():
    L = tw.lib()
    assert L.bitlinear_act_quant(A, 5, B, 4, 1024, 1e-8, C, D, E, None) == DTYPE
    assert L.bitlinear_act_quant(A, 1, B, 4, 1000, 1e-8, C, D, E, None) == SHAPE
    assert L.bitlinear_act_quant(A, 1, B, 4, 1024, 0.0, C, D, E, None) == EPS
    assert L.bitlinear_act_quant(A, 1, B, 4, 1024, 1e-8, None, D, E, None) == NULL
    assert L.bitlinear_act_quant(A, 1, B, 4, 1024, 1e-8, C + 8, D, E, None) == ALIGN
    assert L.bitlinear_act_quant(A, 1, B, 0, 1024, 1e-8, None, None, None, None) == OK
    assert L.bitlinear_gemm_i32(A, B, 4, 1024, C, 1000, D, 0, None) == SHAPE
    assert L.bitlinear_gemm_i32(A, B, 4, 1024, C, 1024, D, 1, None) == PATH
    assert L.bitlinear_gemm_i32(A, B, 65, 1024, C, 1024, D, 2, None) == SHAPE
    assert L.bitlinear_gemm_i32(None, B, 4, 1024, C, 1024, D, 0, None) == NULL
    assert L.bitlinear_gemm_i32(A, B + 2, 4, 1024, C, 1024, D, 0, None) == ALIGN
    assert L.bitlinear_contract(A, B, E, 4, 1024, C, D, 1024, Y, 7, 0, None) == DTYPE
    assert L.bitlinear_contract(A, B, E, 4, 1024, C, D, 1000, Y, 1, 0, None) == SHAPE
    assert L.bitlinear_contract(A, B, E, 4, 1024, C, D, 1024, Y, 1, 1, None) == PATH
    assert L.bitlinear_contract(A, B, E, 65, 1024, C, D, 1024, Y, 1, 2, None) == SHAPE
    assert L.bitlinear_contract(A, None, E, 4, 1024, C, D, 1024, Y, 1, 0, None) == NULL
    assert L.bitlinear_contract(A, B, E, 4, 1024, C, D, 1024, Y + 4, 1, 0, None) == ALIGN
    assert L.bitlinear_contract(A, B, E, 0, 1024, C, D, 1024, None, 1, 0, None) == OK
    assert L.bitlinear_unpack_weights(C, 32, 100, D, None) == SHAPE
    assert L.bitlinear_unpack_weights(None, 32, 128, D, None) == NULL
    assert L.bitlinear_unpack_weights(C, 32, 128, D + 8, None) == ALIGN


def test_grouped_validation():
    from ternary_weight_lm_amd._lib import BlCall
    L = tw.lib()

    def grp(calls, xdt=1, ydt=1, eps=1e-8, n=None):
        arr = (BlCall * max(1, len(calls)))(*calls)
        return L.bitlinear_forward_grouped(ctypes.cast(arr, ctypes.c_void_p),
                                           len(calls) if n is None else n, xdt, ydt, eps, None)
    good = BlCall(A, B, C, D, Y, 1, 1024, 1024)
    assert grp([good], xdt=9) == DTYPE
    assert grp([good], eps=0.0) == EPS
    assert grp([good], n=-1) == SHAPE
    assert grp([good], n=5000) == SHAPE
    assert L.bitlinear_forward_grouped(None, 2, 1, 1, 1e-8, None) == NULL
    assert L.bitlinear_forward_grouped(None, 0, 1, 1, 1e-8, None) == OK
    assert grp([good, BlCall(A, B, C, D, Y, 1, 1000, 1024)]) == SHAPE
    assert grp([good, BlCall(A, B, C, D, Y, 17, 1024, 1024)]) == SHAPE   # not fused-eligible
    assert grp([good, BlCall(A, B, C, D, Y, 16, 8192, 1024)]) == SHAPE   # LDS budget
    assert grp([good, BlCall(A, None, C, D, Y, 1, 1024, 1024)]) == NULL
    assert grp([good, BlCall(A, B, C + 8, D, Y, 1, 1024, 1024)]) == ALIGN
    assert grp([good, BlCall(A, B, C, D + 2, Y, 1, 1024, 1024)]) == ALIGN
    # empty calls are skipped: nothing to launch
    assert grp([BlCall(None, None, None, None, None, 0, 1024, 1024)] * 3) == OK


def test_grouped_ws_plan_and_validation():
    """The workspace query follows the run rule (up to three consecutive
    MFMA-path calls of one shape share a launch pair and need one workspace
    each; runs reuse it), and every malformed group is rejected first."""
    from ternary_weight_lm_amd._lib import BlCall
    L = tw.lib()

    def arr(calls):
        return (BlCall * max(1, len(calls)))(*calls)

    def need(calls, xdt=2):
        return L.bitlinear_grouped_workspace_bytes(ctypes.cast(arr(calls), ctypes.c_void_p),
                                                   len(calls), xdt)

    def grp(calls, ws=WSP, ws_bytes=1 << 40, xdt=2, ydt=2, eps=1e-8, n=None):
        return L.bitlinear_forward_grouped_ws(ctypes.cast(arr(calls), ctypes.c_void_p),
                                              len(calls) if n is None else n, xdt, ydt, eps,
                                              ws, ws_bytes, None)

    def wsb(M, K, N):
        return L.bitlinear_workspace_bytes(M, K, N)
    big = BlCall(A, B, C, D, Y, 4096, 2048, 2048)
    other = BlCall(A, B, C, D, Y, 4096, 2048, 11264)
    dec = BlCall(A, B, C, D, Y, 1, 1024, 1024)
    sk = BlCall(A, B, C, D, Y, 20, 512, 160)
    assert need([dec, dec, dec]) == 0                        # fused calls need none
    assert need([big]) == wsb(4096, 2048, 2048)
    assert need([big, big, big]) == 3 * wsb(4096, 2048, 2048)
    assert need([big, big, big, big]) == 3 * wsb(4096, 2048, 2048)   # runs of at most 3
    assert need([big, other, big]) == max(wsb(4096, 2048, 2048), wsb(4096, 2048, 11264))
    assert need([sk, dec]) == wsb(20, 512, 160)              # skinny path: its own workspace
    assert need([sk, sk, sk]) == 3 * wsb(20, 512, 160)      # skinny run: one act-quant launch
    assert need([sk, big]) == wsb(4096, 2048, 2048)
    assert need([big, BlCall(A, B, C, D, Y, 4096, 1000, 2048)]) == 0   # invalid group
    assert need([big], xdt=7) == 0
    assert grp([big], xdt=9) == DTYPE
    assert grp([big], ydt=9) == DTYPE
    assert grp([big], eps=float("nan")) == EPS
    assert grp([big], n=-1) == SHAPE
    assert grp([big], n=5000) == SHAPE
    assert L.bitlinear_forward_grouped_ws(None, 2, 2, 2, 1e-8, WSP, 1 << 40, None) == NULL
    assert L.bitlinear_forward_grouped_ws(None, 0, 2, 2, 1e-8, None, 0, None) == OK
    assert grp([big, BlCall(A, B, C, D, Y, 4096, 2048, 100)]) == SHAPE
    assert grp([big, BlCall(A, None, C, D, Y, 4096, 2048, 2048)]) == NULL
    assert grp([big, BlCall(A, B, C, D, Y + 4, 4096, 2048, 2048)]) == ALIGN
    assert grp([big, big], ws=None) == WS
    assert grp([big, big], ws_bytes=2 * wsb(4096, 2048, 2048) - 1) == WS
    assert grp([big], ws=WSP + 8) == ALIGN
    assert grp([BlCall(None, None, None, None, None, 0, 1024, 1024)] * 3, ws=None, ws_bytes=0) == OK


def test_contract_grouped_validation():
    from ternary_weight_lm_amd._lib import BlContractCall
    L = tw.lib()

    def grp(calls, ydt=2, n=None):
        arr = (BlContractCall * max(1, len(calls)))(*calls)
        return L.bitlinear_contract_grouped(ctypes.cast(arr, ctypes.c_void_p),
                                            len(calls) if n is None else n, ydt, None)
    good = BlContractCall(A, B, C, D, E, Y, 4096, 2048, 2048)
    assert grp([good], ydt=9) == DTYPE
    assert grp([good], n=-1) == SHAPE
    assert grp([good], n=5000) == SHAPE
    assert L.bitlinear_contract_grouped(None, 2, 2, None) == NULL
    assert L.bitlinear_contract_grouped(None, 0, 2, None) == OK
    assert grp([good, BlContractCall(A, B, C, D, E, Y, 4096, 2000, 2048)]) == SHAPE
    assert grp([good, BlContractCall(A, None, C, D, E, Y, 4096, 2048, 2048)]) == NULL
    assert grp([good, BlContractCall(A + 4, B, C, D, E, Y, 4096, 2048, 2048)]) == ALIGN
    assert grp([good, BlContractCall(A, B + 2, C, D, E, Y, 4096, 2048, 2048)]) == ALIGN
    assert grp([BlContractCall(None, None, None, None, None, None, 0, 2048, 2048)] * 3) == OK


def test_contract_grouped_path_validation():
    """The path-taking grouped contraction: unknown paths and BL_PATH_FUSED
    are refused, BL_PATH_SKINNY refuses any call of more than 64 rows, and
    everything bitlinear_contract_grouped checks is still checked -- all
    before a launch (no GPU here)."""
    from ternary_weight_lm_amd._lib import BlContractCall
    L = tw.lib()
    PATH = -9

    def grp(calls, path, ydt=2):
        arr = (BlContractCall * max(1, len(calls)))(*calls)
        return L.bitlinear_contract_grouped_path(ctypes.cast(arr, ctypes.c_void_p), len(calls),
                                                 ydt, path, None)
    small = BlContractCall(A, B, C, D, E, Y, 64, 2560, 2560)
    big = BlContractCall(A, B, C, D, E, Y, 65, 2560, 2560)
    assert grp([small], 7) == PATH
    assert grp([small], tw.BL_PATH_FUSED) == PATH
    assert grp([small], -1) == PATH
    assert grp([small, big], tw.BL_PATH_SKINNY) == SHAPE
    assert grp([small], tw.BL_PATH_SKINNY, ydt=9) == DTYPE
    assert grp([small, BlContractCall(A, None, C, D, E, Y, 64, 2560, 2560)], tw.BL_PATH_AUTO) == NULL
    assert grp([small, BlContractCall(A + 4, B, C, D, E, Y, 64, 2560, 2560)],
               tw.BL_PATH_SKINNY) == ALIGN
    assert grp([BlContractCall(None, None, None, None, None, None, 0, 2560, 2560)] * 3,
               tw.BL_PATH_SKINNY) == OK
    assert L.bitlinear_contract_grouped_path(None, 0, 2, tw.BL_PATH_AUTO, None) == OK
    assert L.bitlinear_contract_grouped_path(None, 1, 2, tw.BL_PATH_AUTO, None) == NULL


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        _lib._ptr(x)


def test_missing_library_is_an_error(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError):
        _lib.lib()


def test_glu_entry_points_validation():
    L = tw.lib()
    ws = L.bitlinear_pack_workspace_bytes(64, 256)
    assert L.bitlinear_pack_glu_weights(A, 24, 256, C, D, WSP, ws, None) == SHAPE   # F % 16
    assert L.bitlinear_pack_glu_weights(A, 0, 256, C, D, WSP, ws, None) == SHAPE
    assert L.bitlinear_pack_glu_weights(A, 32, 200, C, D, WSP, ws, None) == SHAPE   # K % 128
    assert L.bitlinear_pack_glu_weights(None, 32, 256, C, D, WSP, ws, None) == NULL
    assert L.bitlinear_pack_glu_weights(A, 32, 256, C, D, WSP, 8, None) == WS
    assert L.bitlinear_pack_glu_weights(A + 4, 32, 256, C, D, WSP, ws, None) == ALIGN
    wsf = L.bitlinear_workspace_bytes(4, 1024, 2 * 48)
    glu = L.bitlinear_forward_glu
    assert glu(A, 1, 4, 1024, B, C, D, 40, Y, 1, 1e-8, WSP, wsf, 0, None) == SHAPE  # F % 16
    assert glu(A, 1, 4, 1000, B, C, D, 48, Y, 1, 1e-8, WSP, wsf, 0, None) == SHAPE
    assert glu(A, 9, 4, 1024, B, C, D, 48, Y, 1, 1e-8, WSP, wsf, 0, None) == DTYPE
    assert glu(A, 1, 4, 1024, B, C, D, 48, Y, 1, 0.0, WSP, wsf, 0, None) == EPS
    assert glu(A, 1, 4, 1024, B, None, D, 48, Y, 1, 1e-8, WSP, wsf, 0, None) == NULL
    assert glu(A, 1, 4, 1024, B, C, D, 48, Y, 1, 1e-8, WSP, 16, 0, None) == WS
    assert glu(A, 1, 4, 1024, B, C, D, 48, Y + 2, 1, 1e-8, WSP, wsf, 0, None) == ALIGN
    assert glu(A, 1, 4, 1024, B, C, D, 48, Y, 1, 1e-8, WSP, wsf, 7, None) == PATH
    assert glu(A, 1, 65, 1024, B, C, D, 48, Y, 1, 1e-8, WSP,
               L.bitlinear_workspace_bytes(65, 1024, 96), 2, None) == SHAPE
    assert glu(A, 1, 0, 1024, B, C, D, 48, None, 1, 1e-8, None, 0, 0, None) == OK


def test_contract_glu_validation():
    L = tw.lib()
    cg = L.bitlinear_contract_glu
    assert cg(A, B, C, 8, 1024, D, E, 48, Y, 9, 0, None) == DTYPE
    assert cg(A, B, C, 8, 1024, D, E, 40, Y, 1, 0, None) == SHAPE      # F % 16
    assert cg(A, B, C, 8, 1000, D, E, 48, Y, 1, 0, None) == SHAPE      # K % 128
    assert cg(A, B, C, 8, 1024, D, E, 48, Y, 1, 1, None) == PATH       # fused is not a contraction path
    assert cg(A, B, C, 65, 1024, D, E, 48, Y, 1, 2, None) == SHAPE     # skinny is M <= 64
    assert cg(A, None, C, 8, 1024, D, E, 48, Y, 1, 0, None) == NULL
    assert cg(A, B, C, 8, 1024, D, E, 48, Y + 8, 1, 0, None) == ALIGN
    assert cg(A, B + 2, C, 8, 1024, D, E, 48, Y, 1, 0, None) == ALIGN
    assert cg(None, None, None, 0, 1024, None, None, 48, None, 1, 0, None) == OK


def test_binding_checks_sizes_before_pointers():
    """The binding checks dtype and element counts of every tensor against
    the call's shape before it takes a pointer (the C ABI cannot see sizes):
    mis-sized host tensors are refused for their size, well-sized ones get as
    far as the device check."""
    import torch
    f16, i8, i32, f32 = torch.float16, torch.int8, torch.int32, torch.float32
    M, K, N = 4, 256, 64
    x = torch.zeros(M, K, dtype=f16)
    g = torch.zeros(K, dtype=f16)
    pk = torch.zeros(N * K // 4, dtype=torch.uint8)
    beta = torch.zeros(1, dtype=f32)
    y = torch.zeros(M, N, dtype=f16)
    ws = torch.zeros(1024, dtype=torch.uint8)

    def refused(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    # well-sized: reaches the pointer check
    refused(tw.bitlinear_forward, x, g, pk, beta, N, y, ws, match="GPU")
    refused(tw.bitlinear_forward, x, g[:K - 8], pk, beta, N, y, ws, match="gain")
    refused(tw.bitlinear_forward, x, g.float(), pk, beta, N, y, ws, match="gain")
    refused(tw.bitlinear_forward, x, g, pk[:100], beta, N, y, ws, match="packed")
    refused(tw.bitlinear_forward, x, g, pk, beta.half(), N, y, ws, match="beta")
    refused(tw.bitlinear_forward, x, g, pk, beta, N, y[:, :N - 1].contiguous(), ws, match="y")
    refused(tw.bitlinear_forward, x.view(-1), g, pk, beta, N, y, ws, match="x")
    refused(tw.bitlinear_forward_path, x, g, pk, beta, N, y[:2], ws, 0, match="y")
    F = N // 2
    h = torch.zeros(M, F, dtype=f16)
    refused(tw.bitlinear_forward_glu, x, g, pk, beta, F, h, ws, match="GPU")
    refused(tw.bitlinear_forward_glu, x, g, pk, beta, F, h[:3], ws, match="h|y")
    refused(tw.bitlinear_forward_glu, x, g, pk[:N * K // 8], beta, F, h, ws, match="packed")
    xq = torch.zeros(M, K, dtype=i8)
    s = torch.zeros(M, dtype=f32)
    rs = torch.zeros(M, dtype=i32)
    refused(tw.bitlinear_act_quant, x, g, xq, s, rs, match="GPU")
    refused(tw.bitlinear_act_quant, x, g, xq[:3], s, rs, match="xq")
    refused(tw.bitlinear_act_quant, x, g, xq, s[:3], rs, match="s ")
    refused(tw.bitlinear_act_quant, x, g, xq, s, rs.float(), match="rowsum")
    acc = torch.zeros(M, N, dtype=i32)
    refused(tw.bitlinear_gemm_i32, xq, rs, pk, N, acc, match="GPU")
    refused(tw.bitlinear_gemm_i32, xq, rs, pk, N, acc[:2], match="acc")
    refused(tw.bitlinear_gemm_i32, xq, rs, pk, 2 * N, acc, match="packed")
    refused(tw.bitlinear_contract, xq, s, rs, pk, beta, N, y, match="GPU")
    refused(tw.bitlinear_contract, xq, s[:1], rs, pk, beta, N, y, match="s ")
    refused(tw.bitlinear_contract_glu, xq, s, rs, pk, beta, F, h, match="GPU")
    refused(tw.bitlinear_contract_glu, xq, s, rs, pk, beta, F, h[:1], match="h")
    refused(tw.make_calls, [(x, g, pk, beta, y)], match="GPU")
    refused(tw.make_calls, [(x, g, pk, beta, y[:2])], match="y")
    refused(tw.make_contract_calls, [(xq, s, rs, pk, beta, y)], match="GPU")
    refused(tw.make_contract_calls, [(xq, s, rs, pk[:8], beta, y)], match="packed")
    Wf = torch.zeros(N, K, dtype=f32)
    refused(tw.bitlinear_pack_weights, Wf, pk, beta, ws, match="GPU")
    refused(tw.bitlinear_pack_weights, Wf.half(), pk, beta, ws, match="W")
    refused(tw.bitlinear_pack_weights, Wf, pk[:N * K // 8], beta, ws, match="packed")
    Wq = torch.zeros(N, K, dtype=i8)
    refused(tw.bitlinear_unpack_weights, pk, N, K, Wq, match="GPU")
    refused(tw.bitlinear_unpack_weights, pk, N, K, Wq[:2], match="Wq")


def test_noalloc_validation():
    """The no-allocation forward validates like bitlinear_forward and rejects
    a request beyond its static scratch before touching any device."""
    L = tw.lib()
    cap = L.bitlinear_noalloc_max_scratch_bytes()
    assert cap == 32 << 20
    na = L.bitlinear_forward_noalloc
    assert na(A, 9, 4, 1024, B, C, D, 1024, Y, 1, 1e-8, None) == DTYPE
    assert na(A, 1, 4, 1000, B, C, D, 1024, Y, 1, 1e-8, None) == SHAPE
    assert na(A, 1, 4, 1024, B, C, D, 1024, Y, 1, -1.0, None) == EPS
    assert na(A, 1, 4, 1024, None, C, D, 1024, Y, 1, 1e-8, None) == NULL
    assert na(A + 8, 1, 4, 1024, B, C, D, 1024, Y, 1, 1e-8, None) == ALIGN
    assert na(None, 1, 0, 1024, None, None, None, 1024, None, 1, 1e-8, None) == OK
    K = 8192
    assert na(A, 1, cap // K + 1, K, B, C, D, 1024, Y, 1, 1e-8, None) == -10
    assert L.bitlinear_status_string(-10).decode().startswith("request needs more")


def test_chain_plan_validation():
    """Chain planning: validation and dependency analysis are host-only, so
    every rejection comes back before any HIP call (made-up pointers)."""
    from ternary_weight_lm_amd._lib import BlChainCall, BlChain
    L = tw.lib()
    X0, G, PK, BE = 0x7F0000010000, 0x7F0000020000, 0x7F0000030000, 0x7F0000040000
    Y1, Y2, Y3 = 0x7F0000050000, 0x7F0000060000, 0x7F0000070000

    def arr(calls):
        a = (BlChainCall * len(calls))(*calls)
        return ctypes.cast(a, ctypes.c_void_p), len(calls), a

    good = [BlChainCall(X0, G, PK, BE, Y1, 1024, 1024, 0, 0),      # reads the chain input
            BlChainCall(Y1, G, PK, BE, Y2, 1024, 2048, 1, 0),      # reads call 0; GLU -> 1024 wide
            BlChainCall(Y2, G, PK, BE, Y3, 1024, 512, 0, 0)]       # reads call 1's h
    p, n, keep = arr(good)
    ws = L.bitlinear_chain_workspace_bytes(p, n, 1)
    # header, 3 descriptors, item0 table, done counters, tagged outputs of calls 0 and 1
    assert ws == 256 + 512 + 256 + 256 + 1024 * 4 + 1024 * 4
    assert L.bitlinear_chain_workspace_bytes(p, n, 4) == 256 + 512 + 256 + 256 + 2 * 4 * 4096
    plan = BlChain()
    pl = L.bitlinear_chain_plan
    WSD = 0x7F0001000000
    assert pl(p, n, 1, 2, 1e-8, WSD, ws - 1, ctypes.byref(plan), None) == WS
    assert pl(p, n, 1, 2, 1e-8, WSD + 16, ws, ctypes.byref(plan), None) == ALIGN
    assert pl(p, n, 1, 0, 1e-8, WSD, ws, ctypes.byref(plan), None) == UNSUP    # fp32 chains
    assert pl(p, n, 1, 7, 1e-8, WSD, ws, ctypes.byref(plan), None) == DTYPE
    assert pl(p, n, 5, 2, 1e-8, WSD, ws, ctypes.byref(plan), None) == SHAPE    # M <= 4
    assert pl(p, n, 0, 2, 1e-8, WSD, ws, ctypes.byref(plan), None) == SHAPE
    assert pl(p, n, 1, 2, 0.0, WSD, ws, ctypes.byref(plan), None) == EPS
    assert pl(p, n, 1, 2, 1e-8, WSD, ws, None, None) == NULL
    assert pl(p, 0, 1, 2, 1e-8, WSD, ws, ctypes.byref(plan), None) == SHAPE
    assert pl(None, 3, 1, 2, 1e-8, WSD, ws, ctypes.byref(plan), None) == NULL

    def one(bad):
        q, m, k = arr(bad)
        return pl(q, m, 1, 2, 1e-8, WSD, 1 << 30, ctypes.byref(plan), None)

    assert one([good[0], BlChainCall(Y1, G, PK, BE, Y2, 2048, 1024, 0, 0)]) == SHAPE   # width
    assert one([BlChainCall(X0, G, PK, BE, Y1, 9216, 1024, 0, 0)]) == SHAPE           # K > 8192
    assert one([BlChainCall(X0, G, PK, BE, Y1, 1024, 1056, 1, 0)]) == SHAPE           # GLU N % 64
    assert one([BlChainCall(X0, G, PK, BE, Y1, 1024, 1024, 2, 0)]) == SHAPE
    assert one([BlChainCall(X0, None, PK, BE, Y1, 1024, 1024, 0, 0)]) == NULL
    assert one([BlChainCall(X0 + 8, G, PK, BE, Y1, 1024, 1024, 0, 0)]) == ALIGN
    # a plain input that a call of the chain writes (here: the later call's y)
    assert one([BlChainCall(X0, G, PK, BE, Y1, 1024, 1024, 0, 0),
                BlChainCall(Y3, G, PK, BE, X0 + 512, 1024, 1024, 0, 0)]) == UNSUP
    # the status entry points need a plan
    assert L.bitlinear_chain_run(None, None) == NULL
    assert L.bitlinear_chain_status(None, None) == NULL
    assert L.bitlinear_chain_run_ex(ctypes.byref(BlChain()), 0, None) == NULL
    assert L.bitlinear_status_string(-11).decode().startswith("a chained launch")


def test_decode_contraction_setting():
    """bitlinear_set_decode_contraction accepts the three units, refuses any
    other value with BL_ERR_PATH and leaves the setting unchanged then."""
    L = tw.lib()
    try:
        for u in (tw.BL_DECODE_VALU, tw.BL_DECODE_MFMA, tw.BL_DECODE_AUTO):
            assert L.bitlinear_set_decode_contraction(u) == OK
            assert L.bitlinear_get_decode_contraction() == u
        assert L.bitlinear_set_decode_contraction(tw.BL_DECODE_VALU) == OK
        for bad in (-1, 3, 99):
            assert L.bitlinear_set_decode_contraction(bad) == -9
            assert L.bitlinear_get_decode_contraction() == tw.BL_DECODE_VALU
    finally:
        L.bitlinear_set_decode_contraction(tw.BL_DECODE_AUTO)


def test_forced_launch_failure_reaches_the_caller():
    """The launch-failure hook: a valid call whose launch is forced to fail
    returns BL_ERR_HIP from every kind of entry point (no GPU involved: the
    forced launch never happens), and a rejected call does not consume it."""
    from ternary_weight_lm_amd._lib import BlCall
    L = tw.lib()
    try:
        L.bitlinear_test_fail_launches(1)
        assert fwd(M=0) == OK                      # nothing to launch: not consumed
        assert fwd(eps=0.0) == EPS                 # rejected: not consumed
        assert fwd() == HIP                        # consumed here
        L.bitlinear_test_fail_launches(3)
        assert L.bitlinear_pack_weights(A, 64, 256, C, D, WSP,
                                        L.bitlinear_pack_workspace_bytes(64, 256), None) == HIP
        assert L.bitlinear_forward_path(A, 1, 300, 1024, B, C, D, 1024, Y, 1, 1e-8, WSP,
                                        L.bitlinear_workspace_bytes(300, 1024, 1024), 3, None) == HIP
        calls = (BlCall * 3)(*[BlCall(A, B, C, D, Y, 4096, 2048, 2048)] * 3)
        gws = L.bitlinear_grouped_workspace_bytes(ctypes.cast(calls, ctypes.c_void_p), 3, 2)
        assert L.bitlinear_forward_grouped_ws(ctypes.cast(calls, ctypes.c_void_p), 3, 2, 2, 1e-8,
                                              WSP, gws, None) == HIP
    finally:
        L.bitlinear_test_fail_launches(0)


def test_gate_entry_points_validation():
    L = tw.lib()
    gt = L.bitlinear_rmsnorm_swish_gate
    assert gt(A, B, C, 9, 4, 1024, 1e-6, Y, None) == DTYPE
    assert gt(A, B, C, 2, 4, 1000, 1e-6, Y, None) == SHAPE
    assert gt(A, B, C, 2, 4, 8192, 1e-6, Y, None) == UNSUP      # K > 4096
    assert gt(A, B, C, 2, 4, 1024, 0.0, Y, None) == EPS
    assert gt(A, None, C, 2, 4, 1024, 1e-6, Y, None) == NULL
    assert gt(A, B, C + 4, 2, 4, 1024, 1e-6, Y, None) == ALIGN
    assert gt(None, None, None, 2, 0, 1024, 1e-6, None, None) == OK
    fg = L.bitlinear_forward_gated
    wsb = L.bitlinear_workspace_bytes(4, 1024, 512)
    args = lambda **k: dict(dict(o=A, g=B, w=C, ge=1e-6, xdt=2, M=4, K=1024, gain=D, pk=E, beta=D,
                                 N=512, y=Y, ydt=2, eps=1e-8, ws=WSP, wsb=wsb), **k)

    def call(**k):
        a = args(**k)
        return fg(a["o"], a["g"], a["w"], a["ge"], a["xdt"], a["M"], a["K"], a["gain"], a["pk"],
                  a["beta"], a["N"], a["y"], a["ydt"], a["eps"], a["ws"], a["wsb"], None)

    assert call(xdt=5) == DTYPE
    assert call(N=100) == SHAPE
    assert call(K=8192, wsb=1 << 20) == UNSUP
    assert call(ge=-1.0) == EPS
    assert call(eps=float("nan")) == EPS
    assert call(g=None) == NULL
    assert call(wsb=16) == WS
    assert call(o=A + 2) == ALIGN
    assert call(M=0, o=None, g=None) == OK


def test_mlgru_workspace_closed_form():
    L = tw.lib()
    # 2 B C D floats with C = ceil(T / L) chunks, L = 16 for 33..1023 steps,
    # else 32; none for one chunk (up to 32 steps)
    assert L.bitlinear_mlgru_workspace_bytes(1, 32, 2560) == 0
    assert L.bitlinear_mlgru_workspace_bytes(1, 33, 2560) == 2 * 1 * 3 * 2560 * 4
    assert L.bitlinear_mlgru_workspace_bytes(2, 1023, 64) == 2 * 2 * 64 * 64 * 4
    assert L.bitlinear_mlgru_workspace_bytes(2, 1024, 64) == 2 * 2 * 32 * 64 * 4
    assert L.bitlinear_mlgru_workspace_bytes(4, 4095, 2048) == 2 * 4 * 128 * 2048 * 4
    assert L.bitlinear_mlgru_workspace_bytes(4, 8192, 2048) == 2 * 4 * 256 * 2048 * 4
    assert L.bitlinear_mlgru_workspace_bytes(1, 100, 12) == 0       # D % 8 != 0: invalid
    assert L.bitlinear_mlgru_workspace_bytes(-1, 100, 16) == 0


def test_mlgru_scan_validation():
    L = tw.lib()
    sc = L.bitlinear_mlgru_scan
    wsb = L.bitlinear_mlgru_workspace_bytes(2, 300, 64)

    def call(i=A, f=B, dt=2, Bn=2, T=300, Dn=64, h0=None, h=Y, hT=None, ws=WSP, wsb=wsb):
        return sc(i, f, dt, Bn, T, Dn, h0, h, hT, ws, wsb, None)

    assert call(dt=7) == DTYPE
    assert call(Dn=60) == SHAPE                   # D % 8 != 0
    assert call(Bn=70000) == SHAPE
    assert call(T=(1 << 20) + 1) == SHAPE
    assert call(Dn=-8) == SHAPE
    assert call(f=None) == NULL
    assert call(h=None) == NULL
    assert call(i=A + 8) == ALIGN
    assert call(ws=None) == WS
    assert call(wsb=wsb - 1) == WS
    assert call(ws=WSP + 4) == ALIGN
    assert call(T=0, i=None, f=None, h=None) == OK    # empty: nothing touched
    assert call(Bn=0, i=None, f=None, h=None) == OK
    assert call(Dn=0, i=None, f=None, h=None) == OK
