"""Shared helpers of the GPU parity tests: run the HIP path through the C
ABI, run the oracle on the same seeded inputs, compare.

Bars (decided before any kernel existed):
  packed bytes, beta, int32 accumulators, rowsum: bit-exact;
  xq: bit-exact except elements whose oracle pre-rounding value v lies within
      1e-4 of a .5 boundary, which may differ by one; any row holding such a
      difference is re-checked end to end from the GPU's own codes;
  y: |y_gpu - y_oracle| <= 1e-3 + 2e-3 |y_oracle| for fp32 / fp16 outputs,
      and <= 1e-3 + (2e-3 + 2^-8) |y_oracle| for bf16 outputs (bf16's own
      rounding alone reaches 2^-9 relative), against the oracle's fp64 y.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth

DEV = "cuda:0"
ATOL = 1e-3
RTOL = {"fp32": 2e-3, "fp16": 2e-3, "bf16": 2e-3 + 2.0 ** -8}
BAND = 1e-4


GUARD = 4096          # bytes of sentinel on each side of a guarded output
GUARD_BYTE = 0xA5


def say(*a):
    print(*a, flush=True)


class Guarded:
    """A device output with GUARD sentinel bytes on both sides: .t is the
    contiguous [shape] view the kernels write (16-byte aligned), .check()
    asserts that nothing was written outside it."""

    def __init__(self, shape, dtype, fill=None):
        self.shape = tuple(shape)
        esz = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(self.shape)) * esz
        self.n = n
        self.full = torch.full((GUARD + n + GUARD,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        self.t = self.full[GUARD:GUARD + n].view(dtype).view(self.shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what="output"):
        torch.cuda.synchronize()
        head = self.full[:GUARD]
        tail = self.full[GUARD + self.n:]
        assert bool(torch.all(head == GUARD_BYTE)), f"{what}: write before the buffer"
        assert bool(torch.all(tail == GUARD_BYTE)), f"{what}: write past the buffer"


def contract_rows(xq, Wq, workers=16):
    """oracle.contract over row blocks on a thread pool (rows are independent
    and the oracle releases the GIL); the blocks are the oracle's own calls."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    M = xq.shape[0]
    w = max(1, min(workers, len(os.sched_getaffinity(0)), M))
    bounds = np.linspace(0, M, w + 1).round().astype(int)
    with ThreadPoolExecutor(w) as ex:
        parts = list(ex.map(lambda i: oracle.contract(xq[bounds[i]:bounds[i + 1]], Wq), range(w)))
    return np.concatenate(parts, axis=0)


def band_mask(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    return np.abs(a - np.floor(a) - 0.5) < BAND


def gpu_pack(W_cpu: torch.Tensor):
    packed, beta = tw.pack(W_cpu.to(DEV))
    torch.cuda.synchronize()
    return packed.cpu().numpy(), np.float32(beta.cpu().item()), packed, beta


def check_pack(W_cpu: torch.Tensor):
    """GPU packer vs oracle packer on the same W: bytes and beta bit-exact.
    Returns the oracle (packed, beta, Wq) and the device (packed, beta)."""
    W = W_cpu.numpy()
    o_packed, o_beta, o_Wq = oracle.pack_weights(W)
    g_packed, g_beta, d_packed, d_beta = gpu_pack(W_cpu)
    if g_beta != o_beta:
        # Both sums are fp64; they may straddle an fp32 rounding boundary
        # only when the exact mean sits within ~1e-12 of it.
        exact = oracle.abs_sum(W) / W.size
        lo, hi = sorted([float(g_beta), float(o_beta)])
        assert np.nextafter(np.float32(lo), np.float32(np.inf)) == np.float32(hi)
        mid = (lo + hi) / 2
        assert abs(exact - mid) <= 1e-12 * exact, (g_beta, o_beta, exact)
        o_Wq = oracle.ternarize(W, g_beta)
        o_packed = oracle.pack(o_Wq)
        o_beta = g_beta
    np.testing.assert_array_equal(g_packed, o_packed)
    return (o_packed, o_beta, o_Wq), (d_packed, d_beta)


def gpu_act_quant(x_dev, g_dev, eps=1e-8):
    M, K = x_dev.shape
    xq = Guarded((M, K), torch.int8)
    s = Guarded((M,), torch.float32)
    rs = Guarded((M,), torch.int32)
    tw.bitlinear_act_quant(x_dev, g_dev, xq.t, s.t, rs.t, eps=eps)
    for b, name in ((xq, "xq"), (s, "s"), (rs, "rowsum")):
        b.check(name)
    return xq.t.cpu().numpy(), s.t.cpu().numpy(), rs.t.cpu().numpy()


def check_xq(xq_gpu, s_gpu, ref):
    """xq under the band rule; s bit-exact on rows whose xq agree."""
    diff = xq_gpu != ref["xq"]
    if diff.any():
        band = band_mask(ref["v"])
        assert np.all(band[diff]), "xq differs outside the .5 band"
        assert np.all(np.abs(xq_gpu[diff].astype(np.int32) - ref["xq"][diff]) == 1)
    same_rows = ~diff.any(axis=1)
    np.testing.assert_array_equal(s_gpu[same_rows], ref["s"][same_rows])
    return diff.any(axis=1)


def check_y(y_gpu: np.ndarray, ref, y_dtype: str, Wq=None, beta=None,
            xq_gpu=None, s_gpu=None, rows=None):
    """Compare y (fp64 view of the GPU output) with the oracle's fp64 y.
    rows: the oracle rows y_gpu corresponds to (all when None)."""
    yo = ref["y"]
    tol = ATOL + RTOL[y_dtype] * np.abs(yo)
    bad = np.abs(y_gpu - yo) > tol
    if not bad.any():
        return
    assert xq_gpu is not None, (
        f"y mismatch: {int(bad.sum())} elements, max err "
        f"{float(np.max(np.abs(y_gpu - yo)))}")
    for r in np.unique(np.nonzero(bad)[0]):
        diff = xq_gpu[r] != ref["xq"][r]
        assert diff.any(), f"row {r}: y mismatch with identical codes"
        acc = oracle.contract(xq_gpu[r:r + 1], Wq)
        y_r = oracle.epilogue(acc, s_gpu[r:r + 1], beta)[0]
        assert np.all(np.abs(y_gpu[r] - y_r) <= ATOL + RTOL[y_dtype] * np.abs(y_r))


def y_to_np(y: torch.Tensor) -> np.ndarray:
    return y.detach().float().cpu().numpy().astype(np.float64)


def run_forward(x_cpu, g_cpu, d_packed, d_beta, N, y_dtype, path=tw.BL_PATH_AUTO, eps=1e-8):
    """bitlinear_forward_path with the output and the workspace guarded."""
    x = x_cpu.to(DEV)
    g = g_cpu.to(DEV)
    M, K = x.shape
    y = Guarded((M, N), synth.DTYPES[y_dtype])
    ws = Guarded((max(16, tw.bitlinear_workspace_bytes(M, K, N)),), torch.uint8)
    tw.bitlinear_forward_path(x, g, d_packed, d_beta, N, y.t, ws.t, path, eps=eps)
    y.check("y")
    ws.check("workspace")
    return y_to_np(y.t), x, g
