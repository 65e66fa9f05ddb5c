"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times: its Workload / Weights / Buffers and launch_group build and
issue every launch group exactly as a benchmark step does (i/f/g grouped on
one input through bitlinear_forward_grouped or bitlinear_forward_grouped_ws;
in the 2.7B stack the layers chained, gate_proj through the fused GLU gate).
The 2.7B stack is also run at one token as the single chained launch of
bitlinear_chain_run (bench.py --launch chain), over per-call output buffers
so every output survives.

Every packed byte and beta of every projection (all 192 of the 2.7B stack)
is compared with the oracle's packer.  Every call's output is compared with
the oracle run on the GPU call's own input rows (rows are independent given
beta), on a fixed row sample that always includes the first and last row.
The groups run one layer at a time, so each layer's inputs and outputs are
read before the next layer reuses the buffers."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bench
import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, check_xq, check_y, gpu_act_quant, say, y_to_np
from tests.test_gpu_glu import check_h

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def sample_rows(M, n):
    return np.unique(np.linspace(0, M - 1, min(M, n)).round().astype(int))


def oracle_pack(c, cfg):
    _, _, W = synth.config_inputs(cfg, 1, c.layer, c.pi)
    W = W.numpy()
    return oracle.pack_glu_weights(W) if c.glu else oracle.pack_weights(W)


def check_call(c, cfg, d_packed, d_beta, samples):
    """Packed bytes and beta of call c against the oracle's packer, then each
    (M, x rows, y rows, rows' GPU codes and scales) sample against the
    oracle.  Runs on a worker thread (the oracle releases the GIL)."""
    o_packed, o_beta, o_Wq = oracle_pack(c, cfg)
    assert float(d_beta) == float(o_beta), (c.layer, c.name, d_beta, o_beta)
    np.testing.assert_array_equal(d_packed, o_packed, err_msg=f"{c.layer} {c.name}")
    g = synth.widen(synth.make_gain(cfg.seed, c.layer, c.pi, c.K, cfg.dtype, kind=cfg.gain))
    zero = np.nonzero(~o_Wq.any(axis=1))[0]
    for M, xr, yr, xq, s in samples:
        if c.glu:
            ref = oracle.forward(xr, g, o_Wq, o_beta)
            check_xq(xq, s, ref)
            check_h(yr, ref, c.n_out, cfg.y_dtype, o_Wq, o_beta, xq, s)
        else:
            ref = oracle.forward(xr, g, o_Wq, o_beta)
            check_xq(xq, s, ref)
            check_y(yr, ref, cfg.y_dtype, Wq=o_Wq, beta=o_beta, xq_gpu=xq, s_gpu=s)
            assert np.all(yr[:, zero] == 0.0), (c.layer, c.name, M)
    return c.idx


def run_config(key, Ms, rows_of, launch="per-call"):
    dev = torch.device(DEV)
    wls = {M: bench.Workload(key, M=M, launch=launch) for M in Ms}
    wl0 = wls[Ms[0]]
    cfg = wl0.cfg
    say(f"{key}: packing {len(wl0.calls)} projections")
    weights = bench.Weights(wl0, 0, dev, keep_host_layers=())
    bufs = {M: bench.Buffers(wls[M], weights, dev, distinct=wls[M].launch == "chain")
            for M in Ms}
    groups = {M: wls[M].groups() for M in Ms}
    pool = weights.pool[0]
    for M in Ms:
        if wls[M].launch == "chain":
            say(f"{key}: M={M} as one chained launch of {len(wls[M].calls)} calls")
            plan = bufs[M].chain_plans(wls[M], weights)[0][0]
            tw.bitlinear_chain_run(plan)
            assert tw.bitlinear_chain_status(plan) == 0
    done = set()
    futures = []
    with ThreadPoolExecutor(WORKERS) as ex:
        for layer in range(cfg.layers):
            calls = [c for c in wl0.calls if c.layer == layer]
            for M in Ms:
                if wls[M].launch == "chain":
                    continue
                for grp in groups[M]:
                    if grp[0].layer == layer:
                        bench.launch_group(wls[M], grp, weights, bufs[M], pool, [])
            torch.cuda.synchronize()
            for c in calls:
                samples = []
                for M in Ms:
                    rows = sample_rows(M, rows_of(M))
                    ridx = torch.from_numpy(rows).to(dev)
                    b = bufs[M]
                    x = b.inp[c.idx][ridx].contiguous()
                    xq, s, _ = gpu_act_quant(x, weights.gains[c.idx])
                    samples.append((M, synth.widen(x), y_to_np(b.out[c.idx][ridx]), xq, s))
                d_packed = weights.packed[c.idx].cpu().numpy()
                d_beta = np.float32(weights.betas[c.idx].cpu().item())
                futures.append(ex.submit(check_call, c, cfg, d_packed, d_beta, samples))
            say(f"{key}: layer {layer} launched, {len(futures)} calls queued for the oracle")
        for f in futures:
            done.add(f.result())
    assert done == {c.idx for c in wl0.calls}


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4"])
def test_config_full_size(key):
    cfg = synth.CONFIGS[key]
    run_config(key, [cfg.M_list[0]], lambda M: 8)


def test_config_2p7b_stack_chained():
    """All five token counts of the 2.7B stack, every one of its 192 calls,
    the launch groups of a benchmark step (i/f/g grouped; M = 8192 takes the
    grouped 4-tile-wave GEMM).  Rows: all of M = 1, first and last of M = 8,
    first, middle and last of M >= 64."""
    run_config("c5", list(bench.C5_SWEEP), lambda M: 1 if M == 1 else (2 if M <= 8 else 3))


def test_config_2p7b_stack_one_chained_launch():
    """The 2.7B stack at one token as one persistent chained launch
    (bitlinear_chain_run over all 192 calls), every call against the oracle."""
    run_config("c5", [1], lambda M: 1, launch="chain")
