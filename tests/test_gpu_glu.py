"""GPU parity of the GLU MLP entry points (gate_proj packed in GLU order,
SiLU gate fused into the projection's epilogue) against the oracle.

Bar: packed bytes and beta bit-exact (as for any pack).  h is held to the
stated output tolerance itself, |h_gpu - h| <= 1e-3 + r |h| (r per output
dtype, as for y), h the oracle's fp64 silu(y_gate) * y_up: the kernels form
h in fp32 from the exact int32 accumulators, so only the fp32 rescale, the
SiLU evaluation (~1e-6 relative) and the output rounding separate the two.
Rows whose int8 codes differ under the .5-band rule are re-checked from the
GPU's own codes.  Outputs and workspaces carry guard bands.
"""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import ATOL, DEV, RTOL, Guarded, check_xq, gpu_act_quant, say, y_to_np

pytestmark = pytest.mark.gpu


def h_tolerance(h, dtype):
    return ATOL + RTOL[dtype] * np.abs(h)


def check_h(h_gpu, ref, F, dtype, Wq, beta, xq_gpu, s_gpu, rows=None):
    y = ref["y"] if rows is None else ref["y"][rows]
    h = oracle.glu(y)
    bad = np.abs(h_gpu - h) > h_tolerance(h, dtype)
    if not bad.any():
        return
    xo = ref["xq"] if rows is None else ref["xq"][rows]
    for r in np.unique(np.nonzero(bad)[0]):
        assert np.any(xq_gpu[r] != xo[r]), (
            f"row {r}: h mismatch with identical codes, max err "
            f"{float(np.max(np.abs(h_gpu[r] - h[r])))}")
        y_r = oracle.epilogue(oracle.contract(xq_gpu[r:r + 1], Wq), s_gpu[r:r + 1], beta)
        h_r = oracle.glu(y_r)
        assert np.all(np.abs(h_gpu[r] - h_r[0]) <= h_tolerance(h_r, dtype)[0])


def check_pack_glu(W_cpu):
    o_packed, o_beta, o_Wq = oracle.pack_glu_weights(W_cpu.numpy())
    d_packed, d_beta = tw.pack_glu(W_cpu.to(DEV))
    torch.cuda.synchronize()
    g_beta = np.float32(d_beta.cpu().item())
    assert g_beta == o_beta
    np.testing.assert_array_equal(d_packed.cpu().numpy(), o_packed)
    return o_Wq, o_beta, d_packed, d_beta


@pytest.mark.parametrize("F,K", [(16, 128), (48, 384), (80, 2560), (176, 1024)])
def test_pack_glu_bit_exact(F, K):
    say(f"pack_glu F={F} K={K}")
    W = synth.make_w(300 + F, 0, 0, 2 * F, K, zero_row_frac=0.05)
    check_pack_glu(W)


CASES = [
    # path, M, F, K, x dtype, h dtype
    (tw.BL_PATH_FUSED, 1, 80, 1024, "fp16", "fp16"),
    (tw.BL_PATH_FUSED, 3, 48, 2560, "bf16", "bf16"),
    (tw.BL_PATH_FUSED, 1, 16, 7040, "fp32", "fp32"),
    (tw.BL_PATH_AUTO, 4, 176, 1024, "bf16", "fp32"),
    (tw.BL_PATH_SKINNY, 1, 80, 1024, "bf16", "bf16"),
    (tw.BL_PATH_SKINNY, 8, 48, 2048, "fp16", "fp16"),
    (tw.BL_PATH_SKINNY, 45, 80, 1280, "bf16", "bf16"),
    (tw.BL_PATH_SKINNY, 64, 16, 640, "fp32", "fp32"),
    (tw.BL_PATH_SKINNY, 40, 48, 5632, "bf16", "bf16"),   # 8 waves, 8 tiles each
    (tw.BL_PATH_MFMA, 17, 80, 1280, "bf16", "bf16"),
    (tw.BL_PATH_MFMA, 130, 176, 1024, "fp16", "fp16"),
    (tw.BL_PATH_MFMA, 257, 48, 2048, "bf16", "fp32"),
    # K split over wave groups inside the workgroup: the 2.7B gate_proj at
    # 128 tokens (440 tiles of 32 rows, 2 groups of 10 k-blocks) and 4
    # groups over 17 k-blocks (5/5/5/2)
    (tw.BL_PATH_MFMA, 128, 7040, 2560, "bf16", "bf16"),
    (tw.BL_PATH_MFMA, 40, 2048, 2176, "fp16", "fp16"),
    (tw.BL_PATH_FUSED, 9, 80, 1024, "bf16", "bf16"),   # row mode, two rows per wave
    (tw.BL_PATH_FUSED, 16, 48, 2048, "fp32", "fp32"),
    (tw.BL_PATH_FUSED, 13, 80, 2560, "bf16", "fp16"),
    (tw.BL_PATH_FUSED, 6, 16, 7040, "bf16", "bf16"),   # past the decode kernel: skinny fused
    # the GLU gate in 128 x 256 tiles, ragged in M and in the packed rows
    # (2 F = 8224: the last tile column holds one packed tile), every h checked
    (tw.BL_PATH_MFMA, 3000, 4112, 128, "bf16", "bf16"),
]


@pytest.mark.parametrize("path,M,F,K,xdt,hdt", CASES)
def test_forward_glu_matches_oracle(path, M, F, K, xdt, hdt):
    say(f"forward_glu path={path} M={M} F={F} K={K} x={xdt} h={hdt}")
    seed = 700 + M * 7 + F + K
    x = synth.make_x(seed, 0, 0, M, K, xdt, outlier_p=0.01)
    g = synth.make_gain(seed, 0, 0, K, xdt)
    W = synth.make_w(seed, 0, 0, 2 * F, K, zero_row_frac=0.05)
    o_Wq, o_beta, d_packed, d_beta = check_pack_glu(W)
    xd, gd = x.to(DEV), g.to(DEV)
    h = Guarded((M, F), synth.DTYPES[hdt])
    ws = Guarded((max(16, tw.bitlinear_workspace_bytes(M, K, 2 * F)),), torch.uint8)
    tw.bitlinear_forward_glu(xd, gd, d_packed, d_beta, F, h.t, ws.t, path=path)
    h.check("h")
    ws.check("workspace")
    ref = oracle.forward_glu(synth.widen(x), synth.widen(g), o_Wq, o_beta)
    xq_gpu, s_gpu, _ = gpu_act_quant(xd, gd)
    check_xq(xq_gpu, s_gpu, ref)
    check_h(y_to_np(h.t), ref, F, hdt, o_Wq, o_beta, xq_gpu, s_gpu)


def test_glu_pairing_matches_unfused_projection():
    """Every path's fused gate equals the gate applied on the host to the
    same kernel's unfused fp32 output over the GLU-packed rows (the packed
    order puts gated row 16t + c at column 32t + c, its partner at 32t + 16 + c)."""
    say("glu pairing")
    F, K = 80, 1024
    W = synth.make_w(41, 0, 0, 2 * F, K)
    d_packed, d_beta = tw.pack_glu(W.to(DEV))
    for M, path in [(1, tw.BL_PATH_FUSED), (4, tw.BL_PATH_FUSED), (8, tw.BL_PATH_SKINNY),
                    (40, tw.BL_PATH_SKINNY), (300, tw.BL_PATH_MFMA)]:
        x = synth.make_x(42 + M, 0, 0, M, K, "bf16").to(DEV)
        g = synth.make_gain(42 + M, 0, 0, K, "bf16").to(DEV)
        y = tw.forward(x, g, d_packed, d_beta, 2 * F, out_dtype=torch.float32, path=path)
        h = tw.forward_glu(x, g, d_packed, d_beta, F, out_dtype=torch.float32, path=path)
        torch.cuda.synchronize()
        yp = y.cpu().numpy().astype(np.float32)
        src = oracle.glu_rows(F)
        gate_cols = np.array([r for r in range(2 * F) if src[r] < F])
        up_cols = np.array([r for r in range(2 * F) if src[r] >= F])
        order = np.argsort(src[gate_cols])
        yg, yu = yp[:, gate_cols[order]], yp[:, up_cols[order]]
        hh = (yg / (np.float32(1) + np.exp(-yg))) * yu
        np.testing.assert_allclose(h.cpu().numpy(), hh, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("M,F,K,path", [(4096, 5632, 2048, tw.BL_PATH_AUTO),
                                         (1, 7040, 2560, tw.BL_PATH_AUTO),
                                         (64, 7040, 2560, tw.BL_PATH_AUTO),
                                         (1100, 2048, 1024, tw.BL_PATH_AUTO)])
def test_forward_glu_full_size_sampled(M, F, K, path):
    """The MLP gate of the 1.3B layer at prefill and the 2.7B one at decode,
    full size, in the launch configuration the benchmark uses, and a gate
    whose GEMM takes 96-row tiles (1100 x 4096 packed rows: 384 of them);
    every packed byte is checked, h on sampled rows."""
    say(f"glu full size M={M} F={F} K={K}")
    x = synth.make_x(77, 0, 1, M, K, "bf16", outlier_p=0.01)
    g = synth.make_gain(77, 0, 1, K, "bf16")
    W = synth.make_w(77, 0, 1, 2 * F, K, zero_row_frac=0.05)
    o_Wq, o_beta, d_packed, d_beta = check_pack_glu(W)
    xd, gd = x.to(DEV), g.to(DEV)
    hg = Guarded((M, F), torch.bfloat16)
    ws = Guarded((max(16, tw.bitlinear_workspace_bytes(M, K, 2 * F)),), torch.uint8)
    tw.bitlinear_forward_glu(xd, gd, d_packed, d_beta, F, hg.t, ws.t, path=path)
    hg.check("h")
    ws.check("workspace")
    h = hg.t
    rows = np.unique(np.linspace(0, M - 1, min(M, 6)).round().astype(int))
    ref = oracle.forward_glu(synth.widen(x)[rows], synth.widen(g), o_Wq, o_beta)
    xq_gpu, s_gpu, _ = gpu_act_quant(xd, gd)
    check_xq(xq_gpu[rows], s_gpu[rows], ref)
    check_h(y_to_np(h)[rows], ref, F, "bf16", o_Wq, o_beta, xq_gpu[rows], s_gpu[rows])
