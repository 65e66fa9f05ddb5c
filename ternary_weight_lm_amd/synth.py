"""Seeded synthetic inputs shaped like the HGRNBit projection layers.

This module only draws random numbers and rounds them to a storage dtype; it
holds none of the layer's arithmetic.  Tests, the benchmark and the oracle
all take their inputs from here, so both sides see the same bytes.

Every tensor comes from its own numpy PCG64 stream keyed by
(seed, layer, projection, tensor), so any one tensor can be regenerated
alone.  Distributions:
  x     ~ N(0, 1), optionally with a Bernoulli(p) subset of entries scaled
          by a factor (absmax stress), then rounded (RNE) to fp32/fp16/bf16;
  gain  = 1, or ~ U(0.5, 1.5) rounded to the activation dtype;
  W     ~ N(0, 0.02) in fp32, optionally with exactly round(frac * N) rows
          (chosen by a seeded permutation) set to zero.

Layer shapes follow the model zoo on the pages (370M: d=1024, 24 layers;
1.3B: d=2048, 24 layers; 2.7B: d=2560, 32 layers) and the printed MLP widths
of the 1.3B model (gate_proj 2048->11264, down_proj 5632->2048).  The 2.7B MLP
widths use the same expansion ratio (an assumption, the pages give none).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}

_TENSOR_KEYS = {"x": 1, "gain": 2, "W": 3, "outlier": 4, "zero_rows": 5}


def rng(seed: int, layer: int, proj: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed,
                                spawn_key=(layer, proj, _TENSOR_KEYS[tensor]))
    return np.random.Generator(np.random.PCG64(ss))


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DTYPES[dtype])


def make_x(seed, layer, proj, M, K, dtype, outlier_p=0.0, outlier_scale=20.0):
    r = rng(seed, layer, proj, "x")
    x = r.standard_normal((M, K), dtype=np.float32)
    if outlier_p > 0.0:
        ro = rng(seed, layer, proj, "outlier")
        mask = ro.random((M, K)) < outlier_p
        x = np.where(mask, x * np.float32(outlier_scale), x).astype(np.float32)
    return _to_dtype(x, dtype)


def make_gain(seed, layer, proj, K, dtype, kind="uniform"):
    if kind == "ones":
        return torch.ones(K, dtype=DTYPES[dtype])
    r = rng(seed, layer, proj, "gain")
    g = r.uniform(0.5, 1.5, size=K).astype(np.float32)
    return _to_dtype(g, dtype)


def make_w(seed, layer, proj, N, K, std=0.02, zero_row_frac=0.0):
    r = rng(seed, layer, proj, "W")
    W = r.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    if zero_row_frac > 0.0:
        nz = int(round(zero_row_frac * N))
        rz = rng(seed, layer, proj, "zero_rows")
        rows = rz.permutation(N)[:nz]
        W[rows, :] = 0.0
    return torch.from_numpy(W)


def widen(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a stored fp32/fp16/bf16 tensor to fp32 numpy."""
    return t.detach().cpu().to(torch.float32).numpy()


# ------------------------------------------------------------------ configs

@dataclass
class Proj:
    name: str
    K: int
    N: int


def _attn(d):
    return [Proj(n, d, d) for n in ("i_proj", "f_proj", "g_proj", "o_proj")]


def _mlp(d, inter):
    return [Proj("gate_proj", d, 2 * inter), Proj("down_proj", inter, d)]


@dataclass
class Config:
    name: str
    seed: int
    M_list: list
    projs: list
    layers: int
    dtype: str
    gain: str = "uniform"
    outlier_p: float = 0.0
    zero_row_frac: float = 0.0
    out_dtype: str | None = None
    extra: dict = field(default_factory=dict)

    @property
    def y_dtype(self):
        return self.out_dtype or self.dtype


# Seeds: the 16-token case names seed 0; the others are only "seeded", so
# they take seeds 1..4 in order.
CONFIGS = {
    "c1": Config("c1_single_M16_1024x1024_fp32", 0, [16],
                 [Proj("single", 1024, 1024)], 1, "fp32", gain="ones"),
    "c2": Config("c2_370M_attn_decode_M1_4x1024x1024_fp16", 1, [1],
                 _attn(1024), 1, "fp16"),
    "c3": Config("c3_1p3B_layer_decode_M32_fp16", 2, [32],
                 _attn(2048) + _mlp(2048, 5632), 1, "fp16"),
    "c4": Config("c4_1p3B_layer_prefill_M4096_bf16_outliers", 3, [4096],
                 _attn(2048) + _mlp(2048, 5632), 1, "bf16", outlier_p=0.01),
    "c5": Config("c5_2p7B_stack_32layers_Msweep_bf16", 4, [1, 8, 64, 512, 8192],
                 _attn(2560) + _mlp(2560, 7040), 32, "bf16", zero_row_frac=0.05),
}


# projections that read one block input (the first one names its seed)
SHARED_INPUT = ("i_proj", "f_proj", "g_proj")


def config_inputs(cfg: Config, M: int, layer: int, proj_index: int):
    """x, gain, W (torch CPU tensors) for one projection call of a config.

    i_proj, f_proj and g_proj read the same block input (HGRNBit's token
    mixer applies the three to one hidden state), so their x is drawn once,
    under i_proj's index; each keeps its own gain and weights.  In the 2.7B
    stack one activation tensor per (projection type, M) is reused across
    layers; weights differ per layer."""
    p = cfg.projs[proj_index]
    x_layer = 0 if cfg.layers > 1 else layer
    x_index = proj_index
    if p.name in SHARED_INPUT:
        x_index = next(i for i, q in enumerate(cfg.projs) if q.name == SHARED_INPUT[0])
    x = make_x(cfg.seed, x_layer, x_index, M, p.K, cfg.dtype,
               outlier_p=cfg.outlier_p)
    g = make_gain(cfg.seed, layer, proj_index, p.K, cfg.dtype, kind=cfg.gain)
    W = make_w(cfg.seed, layer, proj_index, p.N, p.K,
               zero_row_frac=cfg.zero_row_frac)
    return x, g, W
