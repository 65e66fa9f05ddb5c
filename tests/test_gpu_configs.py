"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times (bitlinear_forward, automatic path).  Every packed byte and
beta is compared with the oracle; outputs are compared on sampled token
rows (rows are independent given beta), always including the first and last
row.  The 2.7B stack is checked on its first and last layer."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, check_pack, check_xq, check_y, gpu_act_quant, say, y_to_np

pytestmark = pytest.mark.gpu


def sample_rows(M, n):
    return np.unique(np.linspace(0, M - 1, min(M, n)).round().astype(int))


def run_call(cfg, M, layer, pi, packs, rows_n=8):
    x, g, W = synth.config_inputs(cfg, M, layer, pi)
    key = (layer, pi)
    if key not in packs:
        packs[key] = check_pack(W)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = packs[key]
    N = cfg.projs[pi].N
    xd, gd = x.to(DEV), g.to(DEV)
    y = tw.forward(xd, gd, d_packed, d_beta, N, out_dtype=synth.DTYPES[cfg.y_dtype])
    torch.cuda.synchronize()
    rows = sample_rows(M, rows_n)
    yr = y_to_np(y[torch.from_numpy(rows).to(DEV)])
    xw = synth.widen(x)[rows]
    ref = oracle.forward(xw, synth.widen(g), o_Wq, o_beta)
    xq_all, s_all, _ = gpu_act_quant(xd, gd)
    xq, s = xq_all[rows], s_all[rows]
    check_xq(xq, s, ref)
    check_y(yr, ref, cfg.y_dtype, Wq=o_Wq, beta=o_beta, xq_gpu=xq, s_gpu=s)
    zero_rows = np.nonzero(~o_Wq.any(axis=1))[0]
    assert np.all(yr[:, zero_rows] == 0.0)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4"])
def test_config_full_size(key):
    cfg = synth.CONFIGS[key]
    M = cfg.M_list[0]
    packs = {}
    for pi, p in enumerate(cfg.projs):
        say(f"{key} {p.name} M={M} K={p.K} N={p.N}")
        run_call(cfg, M, 0, pi, packs)


@pytest.fixture(scope="module")
def c5_packs():
    return {}


@pytest.mark.parametrize("M", [1, 8, 64, 512, 8192])
def test_config_2p7b_stack(M, c5_packs):
    cfg = synth.CONFIGS["c5"]
    for layer in (0, cfg.layers - 1):
        for pi, p in enumerate(cfg.projs):
            say(f"c5 layer={layer} {p.name} M={M} K={p.K} N={p.N}")
            run_call(cfg, M, layer, pi, c5_packs, rows_n=4)
