"""GPU tests of the decode kernels' two contraction units
(bitlinear_set_decode_contraction): at 1 token (split mode) and 2 tokens
(row mode) the contraction runs on the matrix cores or on the vector ALU
(v_dot4_i32_i8 on the unpacked codes).

Bars: the two units give the same output bits on every call -- single
projections, grouped i/f/g triples (one launch for the three), the GLU
gate_proj, every K capacity of the kernels and all three activation dtypes
-- and the VALU unit's outputs are within the oracle's tolerance (y: the
FusedBitLinear bar; h: 1e-3 + r |h|).  Outputs guarded; the setting is
restored after each test."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, Guarded, check_xq, check_y, gpu_act_quant, say, y_to_np
from tests.test_gpu_glu import check_h

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def restore_unit():
    yield
    tw.bitlinear_set_decode_contraction(tw.BL_DECODE_AUTO)


def _operands(seed, M, N, K, dt, glu=False):
    x = synth.make_x(seed, 0, 0, M, K, dt, outlier_p=0.01)
    g = synth.make_gain(seed, 0, 1, K, dt)
    W = synth.make_w(seed, 0, 2, N, K, zero_row_frac=0.05)
    packed, beta = (tw.pack_glu if glu else tw.pack)(W.to(DEV))
    return x, g, W, packed, beta


def _forward(unit, x, g, packed, beta, N, ydt, glu):
    tw.bitlinear_set_decode_contraction(unit)
    M, K = x.shape
    out = Guarded((M, N // 2 if glu else N), synth.DTYPES[ydt], fill=float("nan"))
    ws = torch.empty(max(16, tw.bitlinear_workspace_bytes(M, K, N)), dtype=torch.uint8, device=DEV)
    if glu:
        tw.bitlinear_forward_glu(x.to(DEV), g.to(DEV), packed, beta, N // 2, out.t, ws,
                                 path=tw.BL_PATH_FUSED)
    else:
        tw.bitlinear_forward_path(x.to(DEV), g.to(DEV), packed, beta, N, out.t, ws, tw.BL_PATH_FUSED)
    torch.cuda.synchronize()
    out.check("out")
    return out.t


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


# (M, N, K, activation dtype, output dtype, GLU): M = 1 takes the split mode
# (every K capacity 1024 KC, KC = 1, 2, 3, 4, 6, 8), M = 2 the row mode
# (K <= 4096); the 2.7B shapes: o_proj 2560 -> 2560, gate_proj 2560 -> 2 x
# 7040 with the GLU gate, down_proj 7040 -> 2560.
CASES = [(1, 1024, 1024, "bf16", "bf16", False), (1, 2560, 2560, "bf16", "bf16", False),
         (1, 2 * 7040, 2560, "bf16", "bf16", True), (1, 2560, 7040, "bf16", "bf16", False),
         (1, 96, 3968, "fp16", "fp32", False), (1, 160, 6144, "fp32", "fp32", False),
         (1, 512, 8192, "bf16", "fp16", False), (1, 2 * 1536, 1024, "fp16", "fp16", True),
         (2, 1024, 1024, "bf16", "bf16", False), (2, 2560, 2560, "bf16", "bf16", False),
         (2, 2 * 1536, 2048, "bf16", "bf16", True), (2, 160, 3968, "fp32", "fp32", False),
         (2, 96, 4096, "fp16", "bf16", False)]


@pytest.mark.parametrize("M,N,K,xdt,ydt,glu", CASES)
def test_valu_matches_mfma_and_oracle(M, N, K, xdt, ydt, glu):
    say(f"decode units M={M} N={N} K={K} {xdt}->{ydt} glu={glu}")
    x, g, W, packed, beta = _operands(400 + M + K // 128, M, N, K, xdt, glu)
    y_m = _forward(tw.BL_DECODE_MFMA, x, g, packed, beta, N, ydt, glu)
    y_v = _forward(tw.BL_DECODE_VALU, x, g, packed, beta, N, ydt, glu)
    assert torch.equal(_bits(y_m), _bits(y_v))
    o_packed, o_beta, o_Wq = (oracle.pack_glu_weights if glu else oracle.pack_weights)(W.numpy())
    assert np.array_equal(packed.cpu().numpy(), o_packed)
    ref = oracle.forward(synth.widen(x), synth.widen(g), o_Wq, o_beta)
    xq, s, _ = gpu_act_quant(x.to(DEV), g.to(DEV))
    check_xq(xq, s, ref)
    if glu:
        check_h(y_to_np(y_v), ref, N // 2, ydt, o_Wq, o_beta, xq, s)
    else:
        check_y(y_to_np(y_v), ref, ydt, Wq=o_Wq, beta=o_beta, xq_gpu=xq, s_gpu=s)


@pytest.mark.parametrize("M,N,K", [(1, 2560, 2560), (2, 2560, 2560), (1, 1024, 2048),
                                   (2, 2048, 4096)])
def test_valu_grouped_triple(M, N, K):
    """i/f/g as one grouped launch (decode3 / rows3 kernels): the three
    outputs bit-identical under both units and to single calls."""
    say(f"decode units grouped M={M} N={N} K={K}")
    ops = [_operands(600 + j, M, N, K, "bf16") for j in range(3)]
    outs = {}
    for unit in (tw.BL_DECODE_MFMA, tw.BL_DECODE_VALU):
        tw.bitlinear_set_decode_contraction(unit)
        ys = [Guarded((M, N), torch.bfloat16, fill=float("nan")) for _ in range(3)]
        tw.bitlinear_forward_grouped([(x.to(DEV), g.to(DEV), p, b, y.t)
                                      for (x, g, _, p, b), y in zip(ops, ys)],
                                     torch.bfloat16, torch.bfloat16)
        torch.cuda.synchronize()
        for y in ys:
            y.check("y")
        outs[unit] = [y.t.clone() for y in ys]
    for j, (x, g, _, p, b) in enumerate(ops):
        single = _forward(tw.BL_DECODE_MFMA, x, g, p, b, N, "bf16", False)
        assert torch.equal(_bits(outs[tw.BL_DECODE_MFMA][j]), _bits(single)), j
        assert torch.equal(_bits(outs[tw.BL_DECODE_VALU][j]), _bits(single)), j


def test_unit_setting_round_trip():
    for u in (tw.BL_DECODE_VALU, tw.BL_DECODE_MFMA, tw.BL_DECODE_AUTO):
        tw.bitlinear_set_decode_contraction(u)
        assert tw.bitlinear_get_decode_contraction() == u
