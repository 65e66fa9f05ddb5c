"""MI355X (gfx950) FusedBitLinear: RMSNorm + per-token int8 activations +
absmean ternary weights packed at 2 bits + exact integer contraction +
rescale, in HIP kernels behind the C ABI of include/bitlinear.h.

The functions named bitlinear_* mirror the C entry points one to one.
pack() and forward() below only allocate outputs and workspaces with torch
and call them.
"""
from __future__ import annotations

import torch

from ._lib import (  # noqa: F401
    BL_BF16, BL_F16, BL_F32, BL_PATH_AUTO, BL_PATH_FUSED, BL_PATH_MFMA,
    BL_PATH_SKINNY, CODE_DTYPE, DTYPE_CODE, BitLinearError, lib,
    bitlinear_act_quant, bitlinear_contract, bitlinear_contract_glu, bitlinear_forward, bitlinear_forward_grouped,
    bitlinear_forward_grouped_ws, bitlinear_grouped_workspace_bytes,
    bitlinear_contract_grouped, make_contract_calls,
    bitlinear_forward_glu, bitlinear_forward_path, bitlinear_pack_glu_weights, make_calls,
    bitlinear_gemm_i32, bitlinear_pack_weights, bitlinear_pack_workspace_bytes,
    bitlinear_packed_bytes, bitlinear_select_path, bitlinear_status_string, bitlinear_unpack_weights,
    bitlinear_workspace_bytes, bitlinear_forward_noalloc, bitlinear_noalloc_max_scratch_bytes,
    BL_ERR_TIMEOUT, BlChain, make_chain_calls, bitlinear_chain_workspace_bytes,
    bitlinear_chain_plan, bitlinear_chain_run, bitlinear_chain_run_ex, bitlinear_chain_status,
    bitlinear_test_fail_launches, bitlinear_rmsnorm_swish_gate, bitlinear_forward_gated,
    bitlinear_mlgru_scan, bitlinear_mlgru_workspace_bytes,
    bitlinear_set_decode_contraction, bitlinear_get_decode_contraction,
    BL_DECODE_AUTO, BL_DECODE_MFMA, BL_DECODE_VALU,
)


def _bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def pack(W: torch.Tensor):
    """Pack latent fp32 weights [N, K] (on the GPU).  Returns
    (packed uint8 [N*K/4], beta fp32 [1])."""
    N, K = W.shape
    packed = torch.empty(bitlinear_packed_bytes(N, K), dtype=torch.uint8, device=W.device)
    beta = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = _bytes(bitlinear_pack_workspace_bytes(N, K), W.device)
    bitlinear_pack_weights(W, packed, beta, ws)
    return packed, beta


def forward(x: torch.Tensor, gain: torch.Tensor, packed: torch.Tensor,
            beta: torch.Tensor, N: int, eps: float = 1e-8, out_dtype=None,
            path: int = BL_PATH_AUTO, ws: torch.Tensor | None = None):
    """y [M, N] = FusedBitLinear(x [M, K]) with the packed weights."""
    M, K = x.shape
    y = torch.empty(M, N, dtype=out_dtype or x.dtype, device=x.device)
    if ws is None:
        ws = _bytes(bitlinear_workspace_bytes(M, K, N), x.device)
    bitlinear_forward_path(x, gain, packed, beta, N, y, ws, path, eps=eps)
    return y


def pack_glu(W: torch.Tensor):
    """Pack a gate_proj [2F, K] (fp32, on the GPU; rows 0..F-1 SiLU-gated,
    F..2F-1 multiplied) in the GLU row order.  Returns (packed, beta)."""
    N2, K = W.shape
    packed = torch.empty(bitlinear_packed_bytes(N2, K), dtype=torch.uint8, device=W.device)
    beta = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = _bytes(bitlinear_pack_workspace_bytes(N2, K), W.device)
    bitlinear_pack_glu_weights(W, packed, beta, ws)
    return packed, beta


def forward_glu(x: torch.Tensor, gain: torch.Tensor, packed: torch.Tensor,
                beta: torch.Tensor, F: int, eps: float = 1e-8, out_dtype=None,
                path: int = BL_PATH_AUTO, ws: torch.Tensor | None = None):
    """h [M, F] = silu(y[:, :F]) * y[:, F:] for y = gate_proj(x) (GLU-packed)."""
    M, K = x.shape
    h = torch.empty(M, F, dtype=out_dtype or x.dtype, device=x.device)
    if ws is None:
        ws = _bytes(bitlinear_workspace_bytes(M, K, 2 * F), x.device)
    bitlinear_forward_glu(x, gain, packed, beta, F, h, ws, path=path, eps=eps)
    return h


def workspace(M: int, K: int, N: int, device="cuda") -> torch.Tensor:
    return _bytes(bitlinear_workspace_bytes(M, K, N), device)
