"""One whole HGRNBit block on the GPU (ternary_weight_lm_amd.block: i/f/g
grouped -> MLGRU scan -> swish-gated o_proj -> gate_proj + GLU -> down_proj),
each stage held to the oracle on the GPU's own input to that stage ("given
identical input", as the per-projection tests do): the three projections, the
o_proj behind the gate, gate_proj + GLU and down_proj on sampled rows within
the output tolerance; the scan's h on every element.  Prefill (one sequence)
and two decode steps of several sequences, the second continuing from the
state the first left.  2.7B shapes (D = 2560, F = 7040), bf16."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from ternary_weight_lm_amd.block import GATE_EPS, Block
from tests.parity import ATOL, DEV, RTOL, check_xq, check_y, gpu_act_quant, say, y_to_np

pytestmark = pytest.mark.gpu

D, F, DT = 2560, 7040, "bf16"
SEED = 21


@pytest.fixture(scope="module")
def block():
    say("block: packing the 2.7B block's six projections")
    names = Block.NAMES
    shapes = {"i_proj": (D, D), "f_proj": (D, D), "g_proj": (D, D), "o_proj": (D, D),
              "gate_proj": (2 * F, D), "down_proj": (D, F)}
    W = {n: synth.make_w(SEED, 0, k, *shapes[n], zero_row_frac=0.05) for k, n in enumerate(names)}
    gain = {n: synth.make_gain(SEED, 0, k, shapes[n][1], DT) for k, n in enumerate(names)}
    gate_w = synth.make_gain(SEED, 0, 9, D, DT)
    blk = Block(W, gain, gate_w, device=DEV)
    ref = {}
    for n in names:
        Wn = W[n].numpy()
        if n == "gate_proj":
            _, beta, Wq = oracle.pack_glu_weights(Wn)
        else:
            _, beta, Wq = oracle.pack_weights(Wn)
        assert float(blk.beta[n].item()) == float(beta), f"{n}: beta differs from the oracle's"
        ref[n] = (Wq, beta)
    return blk, ref, gain, gate_w


def _check_proj(name, x_dev, y_dev, ref, gain, rows, glu=False):
    Wq, beta = ref[name]
    x_rows = x_dev[rows].contiguous()
    g = synth.widen(gain[name])
    r = (oracle.forward_glu if glu else oracle.forward)(synth.widen(x_rows.cpu()), g, Wq, beta)
    xq, s, _ = gpu_act_quant(x_rows, gain[name].to(DEV))
    check_xq(xq, s, r)
    if glu:
        tol = ATOL + RTOL[DT] * np.abs(r["h"])
        err = np.abs(y_to_np(y_dev[rows]) - r["h"])
        assert np.all(err <= tol), f"{name}: max |dh| {err.max()}"
    else:
        check_y(y_to_np(y_dev[rows]), r, DT, Wq=Wq, beta=beta, xq_gpu=xq, s_gpu=s)


def _check_step(blk, ref, gain, gate_w, b, state_before):
    M, B, T = b["M"], b["B"], b["T"]
    rows = np.unique(np.linspace(0, M - 1, min(M, 4)).round().astype(int))
    for n in ("i_proj", "f_proj", "g_proj"):
        _check_proj(n, b["x"], b[n[0]], ref, gain, rows)
    # the scan on every element, from the GPU's i and f and the state it started from
    h_ref, hT_ref = oracle.mlgru_scan(synth.widen(b["i"].view(B, T, D).cpu()),
                                      synth.widen(b["f"].view(B, T, D).cpu()),
                                      state_before.astype(np.float64))
    tol = ATOL + RTOL[DT] * np.abs(h_ref)
    err = np.abs(y_to_np(b["h"].view(B, T, D)) - h_ref)
    assert np.all(err <= tol), f"scan: max |dh| {err.max()}"
    np.testing.assert_allclose(b["state"].cpu().numpy(), hT_ref, rtol=2e-3, atol=1e-3)
    # the gate on the GPU's h and g (the standalone gate kernel: the same bits
    # as the gated forward's prologue), then o_proj on the GPU's z
    h_rows, g_rows = b["h"][rows].contiguous(), b["g"][rows].contiguous()
    z_dev = torch.empty_like(h_rows)
    tw.bitlinear_rmsnorm_swish_gate(h_rows, g_rows, gate_w.to(DEV), z_dev, eps=GATE_EPS)
    z_ref = oracle.rmsnorm_swish_gate(synth.widen(h_rows.cpu()), synth.widen(g_rows.cpu()),
                                      synth.widen(gate_w), eps=GATE_EPS)
    tol = ATOL + RTOL[DT] * np.abs(z_ref)
    assert np.all(np.abs(y_to_np(z_dev) - z_ref) <= tol), "gate: z outside the tolerance"
    _check_proj("o_proj", z_dev, b["o"][rows], ref, gain, np.arange(len(rows)))
    _check_proj("gate_proj", b["o"], b["m"], ref, gain, rows, glu=True)
    _check_proj("down_proj", b["m"], b["y"], ref, gain, rows)


def test_block_prefill_one_sequence(block):
    blk, ref, gain, gate_w = block
    M = 512
    say(f"block prefill M={M}")
    b = blk.buffers(M, sequences=1, device=DEV)
    b["x"].copy_(synth.make_x(SEED, 1, 0, M, D, DT).to(DEV))
    blk.step(b)
    torch.cuda.synchronize()
    _check_step(blk, ref, gain, gate_w, b, np.zeros((1, D)))


def test_block_decode_two_steps(block):
    """Four sequences, one token each per step; the second step continues
    from the state the first left (the scan's h0 and hT are one buffer)."""
    blk, ref, gain, gate_w = block
    M = 4
    b = blk.buffers(M, sequences=M, device=DEV)
    for step in range(2):
        say(f"block decode M={M} step {step}")
        state = b["state"].cpu().numpy().astype(np.float64)
        b["x"].copy_(synth.make_x(SEED, 2 + step, 0, M, D, DT).to(DEV))
        blk.step(b)
        torch.cuda.synchronize()
        _check_step(blk, ref, gain, gate_w, b, state)
        assert step == 1 or np.any(b["state"].cpu().numpy() != 0)
