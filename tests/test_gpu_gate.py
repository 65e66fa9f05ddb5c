"""GPU parity of FusedRMSNormSwishGate (the reading of the module's name:
z = RMSNorm(o) * w * swish(g)) and of o_proj with the gate as its prologue.

Bars: z (a floating-point output rounded to the activation dtype) within the
output tolerance 1e-3 + r |z| of the oracle's fp64 z; the gated forward's
codes, scales and y bit-identical to running the gate and then
bitlinear_forward on the stored z, and y within the usual tolerance of the
oracle's FusedBitLinear on that z ("given identical input": the GPU's z
feeds the oracle's projection).  Outputs guarded."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import (ATOL, DEV, RTOL, Guarded, check_pack, check_xq, check_y,
                          gpu_act_quant, say, y_to_np)

pytestmark = pytest.mark.gpu
GATE_EPS = 1e-6


def _gate_inputs(seed, M, K, dt):
    o = synth.make_x(seed, 0, 0, M, K, dt, outlier_p=0.01)
    g = synth.make_x(seed, 0, 1, M, K, dt) * 2
    w = synth.make_gain(seed, 0, 2, K, dt)
    if M >= 3:
        o[1] = 0          # an all-zero mixer row: z = 0
        g[2] = 0          # a closed gate: z = 0
    return o, g.to(synth.DTYPES[dt]), w


def _check_z(z_gpu, z_ref, dt):
    tol = ATOL + RTOL[dt] * np.abs(z_ref)
    err = np.abs(z_gpu - z_ref)
    assert np.all(err <= tol), f"max |dz| {err.max()} (tol {tol[np.argmax(err - tol)]})"


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K", [(1, 128), (5, 1024), (64, 2560), (300, 4096), (33, 3072)])
def test_gate_matches_oracle(dt, M, K):
    say(f"gate {dt} M={M} K={K}")
    o, g, w = _gate_inputs(40 + M + K, M, K, dt)
    z = Guarded((M, K), synth.DTYPES[dt])
    tw.bitlinear_rmsnorm_swish_gate(o.to(DEV), g.to(DEV), w.to(DEV), z.t, eps=GATE_EPS)
    z.check("z")
    ref = oracle.rmsnorm_swish_gate(synth.widen(o), synth.widen(g), synth.widen(w), eps=GATE_EPS)
    _check_z(y_to_np(z.t), ref, dt)
    if M >= 3:
        assert np.all(y_to_np(z.t)[1:3] == 0.0)


# 1..8 rows of 16-bit activations take one launch (the decode kernel's row
# mode with the gate in front; every K capacity 1024 KC, KC = 1..4, 1 and 8
# rows); more rows or fp32 the gated act-quant launch and the contraction.
@pytest.mark.parametrize("M,K,N,dt", [(1, 2560, 2560, "bf16"), (4, 1024, 1024, "fp16"),
                                      (8, 4096, 512, "bf16"), (3, 2048, 160, "fp16"),
                                      (5, 128, 96, "bf16"), (8, 2560, 2560, "fp16"),
                                      (40, 2048, 512, "bf16"), (300, 2560, 2560, "bf16"),
                                      (130, 1024, 160, "fp32"), (2, 1024, 1024, "fp32")])
def test_gated_forward(M, K, N, dt):
    """o_proj with the gate as its prologue: bit-identical to gate then
    bitlinear_forward, and y within tolerance of the oracle on the GPU's z."""
    say(f"gated forward {dt} M={M} K={K} N={N}")
    o, g, w = _gate_inputs(90 + M, M, K, dt)
    gain = synth.make_gain(91 + M, 0, 0, K, dt)
    W = synth.make_w(92 + M, 0, 0, N, K, zero_row_frac=0.05)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = check_pack(W)
    od, gd, wd, nd = o.to(DEV), g.to(DEV), w.to(DEV), gain.to(DEV)
    xdt = synth.DTYPES[dt]
    y = Guarded((M, N), xdt)
    ws = Guarded((max(16, tw.bitlinear_workspace_bytes(M, K, N)),), torch.uint8)
    tw.bitlinear_forward_gated(od, gd, wd, nd, d_packed, d_beta, N, y.t, ws.t, gate_eps=GATE_EPS)
    y.check("y")
    ws.check("workspace")
    # the same through the standalone gate and the plain forward
    z = torch.empty(M, K, dtype=xdt, device=DEV)
    tw.bitlinear_rmsnorm_swish_gate(od, gd, wd, z, eps=GATE_EPS)
    y2 = tw.forward(z, nd, d_packed, d_beta, N)
    torch.cuda.synchronize()
    assert torch.equal(y.t.view(torch.uint8), y2.view(torch.uint8))
    # z against the oracle's gate, y against the oracle's projection of the GPU's z
    zr = oracle.rmsnorm_swish_gate(synth.widen(o), synth.widen(g), synth.widen(w), eps=GATE_EPS)
    _check_z(y_to_np(z), zr, dt)
    ref = oracle.forward(synth.widen(z.cpu()), synth.widen(gain), o_Wq, o_beta)
    xq, s, _ = gpu_act_quant(z, nd)
    check_xq(xq, s, ref)
    check_y(y_to_np(y.t), ref, dt, Wq=o_Wq, beta=o_beta, xq_gpu=xq, s_gpu=s)


@pytest.mark.parametrize("M", [1, 8, 64, 512, 8192])
def test_gated_o_proj_2p7b_full_size(M):
    """The 2.7B o_proj (2560 -> 2560) with its gate at every token count of
    the stack's sweep; sampled rows against the oracle."""
    say(f"gated o_proj 2.7B M={M}")
    K = N = 2560
    o, g, w = _gate_inputs(7, M, K, "bf16")
    gain = synth.make_gain(8, 0, 0, K, "bf16")
    W = synth.make_w(9, 0, 0, N, K, zero_row_frac=0.05)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = check_pack(W)
    od, gd, wd, nd = o.to(DEV), g.to(DEV), w.to(DEV), gain.to(DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ws = tw.workspace(M, K, N, device=DEV)
    tw.bitlinear_forward_gated(od, gd, wd, nd, d_packed, d_beta, N, y, ws, gate_eps=GATE_EPS)
    z = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    tw.bitlinear_rmsnorm_swish_gate(od, gd, wd, z, eps=GATE_EPS)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, min(M, 4)).round().astype(int))
    zr = oracle.rmsnorm_swish_gate(synth.widen(o)[rows], synth.widen(g)[rows], synth.widen(w),
                                   eps=GATE_EPS)
    zg = z[torch.from_numpy(rows).to(DEV)]
    _check_z(y_to_np(zg), zr, "bf16")
    ref = oracle.forward(synth.widen(zg.cpu()), synth.widen(gain), o_Wq, o_beta)
    xq, s, _ = gpu_act_quant(zg.contiguous(), nd)
    check_xq(xq, s, ref)
    check_y(y_to_np(y[torch.from_numpy(rows).to(DEV)]), ref, "bf16", Wq=o_Wq, beta=o_beta,
            xq_gpu=xq, s_gpu=s)
