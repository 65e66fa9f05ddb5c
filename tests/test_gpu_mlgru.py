"""GPU parity of the MLGRU scan (the reading of the pages' description:
h_t = a h_{t-1} + (1 - a) i_t, a = sigmoid(f_t), per sequence and channel).

Bar: h (floating point, rounded to the activation dtype) within the output
tolerance 1e-3 + r |h| of the oracle's fp64 scan, every element; hT (fp32)
within 1e-3 + 2e-3 |hT| and equal to h's last step before rounding (bit for
bit once rounded to the dtype).  Saturated gates give exact results: f = +40
freezes the state (h = h0 rounded), f = -40 copies the input.  Outputs
guarded."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import ATOL, DEV, RTOL, Guarded, say, y_to_np

pytestmark = pytest.mark.gpu


def _inputs(seed, B, T, D, dt):
    """i like a projection output; f spread over the sigmoid's whole range,
    with a channel frozen (f = +40) and one copying (f = -40) in every
    sequence."""
    i = synth.make_x(seed, 0, 0, B * T, D, dt, outlier_p=0.01).reshape(B, T, D)
    f = (synth.make_x(seed, 0, 1, B * T, D, "fp32") * 3).reshape(B, T, D)
    f[:, :, 0] = 40.0
    if D > 1:
        f[:, :, 1] = -40.0
    h0 = synth.make_x(seed, 0, 2, B, D, "fp32")
    return i, f.to(synth.DTYPES[dt]), h0


def _check(h_gpu, h_ref, dt, what="h"):
    tol = ATOL + RTOL[dt] * np.abs(h_ref)
    err = np.abs(h_gpu - h_ref)
    k = int(np.argmax(err - tol))
    assert np.all(err <= tol), f"{what}: max |dh| {err.max()} (at {np.unravel_index(k, err.shape)}, tol {tol.flat[k]})"


def _run(i, f, h0, dt, with_h0=True, with_hT=True):
    B, T, D = i.shape
    xdt = synth.DTYPES[dt]
    h = Guarded((B, T, D), xdt)
    hT = Guarded((B, D), torch.float32) if with_hT else None
    need = tw.bitlinear_mlgru_workspace_bytes(B, T, D)
    ws = Guarded((max(16, need),), torch.uint8) if need else None
    tw.bitlinear_mlgru_scan(i.to(DEV), f.to(DEV), h.t, h0=h0.to(DEV) if with_h0 else None,
                            hT=hT.t if hT is not None else None, ws=ws.t if ws else None)
    h.check("h")
    if hT is not None:
        hT.check("hT")
    if ws is not None:
        ws.check("workspace")
    return h.t, hT.t if hT is not None else None


# one chunk (T <= 32) is one launch; past it three (chunks of 16 below 1024
# steps, of 32 from there, the last ragged), the carry in one batch up to 32 chunks, else
# in groups of 32 chunks over windows of 256 (20000 steps: two windows); D
# covers one and several 512-channel workgroups, ragged ones and the
# 8-channel minimum
CASES = [(1, 1, 8, "bf16", True), (2, 1, 2560, "fp16", True), (1, 32, 64, "fp16", False),
         (1, 33, 520, "bf16", True), (2, 300, 1032, "fp32", True), (3, 257, 24, "bf16", False),
         (4, 256, 2048, "fp16", True), (1, 1000, 2560, "bf16", True), (2, 400, 4104, "bf16", True),
         (1, 4100, 136, "fp16", True), (1, 2000, 40, "fp32", True), (2, 20000, 16, "bf16", True)]


@pytest.mark.parametrize("B,T,D,dt,with_h0", CASES)
def test_mlgru_scan_matches_oracle(B, T, D, dt, with_h0):
    say(f"mlgru scan {dt} B={B} T={T} D={D} h0={with_h0}")
    i, f, h0 = _inputs(300 + B + T + D, B, T, D, dt)
    h, hT = _run(i, f, h0, dt, with_h0=with_h0)
    ref, refT = oracle.mlgru_scan(synth.widen(i), synth.widen(f),
                                  synth.widen(h0).astype(np.float64) if with_h0 else None)
    hg = y_to_np(h)
    _check(hg, ref, dt)
    hTg = hT.cpu().numpy().astype(np.float64)
    _check(hTg, refT, "fp32", "hT")
    # hT is the last step's state, h that state rounded to the dtype
    assert torch.equal(hT.to(h.dtype).cpu(), h[:, -1, :].cpu())
    # channel 0 frozen (f = +40): the start state, exactly; channel 1 (f = -40)
    # copies the input (a = ~4e-18: within one rounding of it)
    start = synth.widen(h0)[:, 0] if with_h0 else np.zeros(B, np.float32)
    want = torch.from_numpy(start).to(h.dtype)
    assert torch.equal(h[:, :, 0].cpu(), want[:, None].expand(B, T))
    _check(hg[:, :, 1], synth.widen(i)[:, :, 1].astype(np.float64), dt, "copying channel")


@pytest.mark.parametrize("B,T", [(1, 8192), (8, 1024)])
def test_mlgru_scan_2p7b_full_size(B, T):
    """The 2.7B block's mixer width (D = 2560) at the prefill sizes the
    benchmark times (8192 tokens as one sequence, and as 8 of 1024), every
    element against the oracle."""
    D = 2560
    say(f"mlgru scan 2.7B B={B} T={T}")
    i, f, h0 = _inputs(11, B, T, D, "bf16")
    h, hT = _run(i, f, h0, "bf16")
    ref, refT = oracle.mlgru_scan(synth.widen(i), synth.widen(f), synth.widen(h0).astype(np.float64))
    _check(y_to_np(h), ref, "bf16")
    _check(hT.cpu().numpy().astype(np.float64), refT, "fp32", "hT")


def test_mlgru_scan_continues_from_its_final_state():
    """Two calls, the second from the first's hT, against one call over the
    whole sequence: the same function (both within the bar of the oracle),
    the way a decode step continues a prefill."""
    B, T, D = 2, 300, 264
    i, f, h0 = _inputs(5, B, T, D, "fp16")
    t0 = 173
    h_a, hT_a = _run(i[:, :t0].contiguous(), f[:, :t0].contiguous(), h0, "fp16")
    h_b, hT_b = _run(i[:, t0:].contiguous(), f[:, t0:].contiguous(), hT_a.cpu(), "fp16")
    ref, refT = oracle.mlgru_scan(synth.widen(i), synth.widen(f), synth.widen(h0).astype(np.float64))
    _check(np.concatenate([y_to_np(h_a), y_to_np(h_b)], axis=1), ref, "fp16")
    _check(hT_b.cpu().numpy().astype(np.float64), refT, "fp32", "hT")


def test_mlgru_scan_empty_is_a_no_op():
    h = torch.full((2, 0, 16), 7.0, dtype=torch.bfloat16, device=DEV)
    i = torch.empty(2, 0, 16, dtype=torch.bfloat16, device=DEV)
    tw.bitlinear_mlgru_scan(i, i, h)
    torch.cuda.synchronize()
