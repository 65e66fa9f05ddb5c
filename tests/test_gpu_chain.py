"""GPU tests of the chained decode launch (bitlinear_chain_*): a chain of
dependent calls -- HGRN-shaped blocks: i/f/g on the block input, o_proj on
g_proj's output, gate_proj + GLU on o_proj's, down_proj on h, the next block
on down_proj's output -- in one persistent launch.

Bars: every call's output equals bitlinear_forward (bitlinear_forward_glu)
on the same input bit for bit (same arithmetic, same order), and stays
within the oracle's tolerance on the 2.7B shapes; a forced give-up of the
bounded wait ends every workgroup normally and is reported, and the next run
is correct again; graph replays redo the whole chain every time.  Every call
writes its own guarded output buffer."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, Guarded, check_xq, check_y, gpu_act_quant, say, y_to_np
from tests.test_gpu_glu import check_h

pytestmark = pytest.mark.gpu


class Chain:
    """layers x (i, f, g, o, gate+GLU, down) with model width d and GLU width
    F, random weights, one guarded output per call."""

    def __init__(self, layers, d, F, M, dtype, seed):
        self.M, self.dtype = M, dtype
        dt = synth.DTYPES[dtype]
        self.x0 = synth.make_x(seed, 0, 0, M, d, dtype, outlier_p=0.01).to(DEV)
        self.calls = []   # dicts: name, x (tensor), g, W (cpu), packed, beta, y (Guarded), glu
        prev = self.x0
        for l in range(layers):
            ys = {}
            for pi, (name, K, N, glu) in enumerate([("i", d, d, False), ("f", d, d, False),
                                                     ("g", d, d, False), ("o", d, d, False),
                                                     ("gate", d, 2 * F, True), ("down", F, d, False)]):
                x = {"i": prev, "f": prev, "g": prev, "o": ys.get("g"), "gate": ys.get("o"),
                     "down": ys.get("gate")}[name]
                g = synth.make_gain(seed, l, pi, K, dtype).to(DEV)
                W = synth.make_w(seed, l, pi, N, K, zero_row_frac=0.05)
                packed, beta = (tw.pack_glu if glu else tw.pack)(W.to(DEV))
                y = Guarded((M, N // 2 if glu else N), dt, fill=float("nan"))
                ys[name] = y.t
                self.calls.append(dict(name=f"{name}{l}", x=x, g=g, W=W, packed=packed, beta=beta,
                                       y=y, glu=glu, K=K, N=N))
            prev = ys["down"]
        self.arr = tw.make_chain_calls([(c["x"], c["g"], c["packed"], c["beta"], c["y"].t, c["glu"])
                                        for c in self.calls])
        nbytes = tw.bitlinear_chain_workspace_bytes(self.arr, M)
        assert nbytes > 0
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=DEV)
        off = (-self.ws.data_ptr()) % 256
        self.wsv = self.ws[off:off + nbytes]
        self.plan = tw.bitlinear_chain_plan(self.arr, M, dt, self.wsv)

    def clear(self):
        for c in self.calls:
            c["y"].t.fill_(float("nan"))

    def reference(self, c):
        """bitlinear_forward (or _glu) on the call's own input, as the chain fed it."""
        out = torch.empty_like(c["y"].t)
        ws = tw.workspace(self.M, c["K"], c["N"], device=DEV)
        if c["glu"]:
            tw.bitlinear_forward_glu(c["x"], c["g"], c["packed"], c["beta"], c["N"] // 2, out, ws)
        else:
            tw.bitlinear_forward(c["x"], c["g"], c["packed"], c["beta"], c["N"], out, ws)
        return out

    def check_bitwise(self):
        for c in self.calls:
            c["y"].check(c["name"])
            ref = self.reference(c)
            torch.cuda.synchronize()
            assert torch.equal(c["y"].t.view(torch.int16), ref.view(torch.int16)), c["name"]


@pytest.mark.parametrize("M,dtype", [(1, "bf16"), (2, "fp16"), (3, "bf16"), (4, "bf16")])
def test_chain_matches_per_call_forward(M, dtype):
    """Two blocks of width 1024 (GLU width 1536: K capacities 1 and 2 in one
    launch), every call bit-identical to the per-call forward."""
    say(f"chain small M={M} {dtype}")
    ch = Chain(2, 1024, 1536, M, dtype, seed=50 + M)
    tw.bitlinear_chain_run(ch.plan)
    assert tw.bitlinear_chain_status(ch.plan) == 0
    ch.check_bitwise()


@pytest.mark.parametrize("M", [1, 4])
def test_chain_2p7b_shapes_vs_oracle(M):
    """Two blocks at the 2.7B widths (K = 2560 and 7040: capacities 3 and
    8), bitwise against the per-call forward and every call against the
    oracle on the call's own input rows (codes under the band rule)."""
    say(f"chain 2.7B shapes M={M}")
    ch = Chain(2, 2560, 7040, M, "bf16", seed=70 + M)
    tw.bitlinear_chain_run(ch.plan)
    assert tw.bitlinear_chain_status(ch.plan) == 0
    ch.check_bitwise()
    for c in ch.calls:
        o_packed, o_beta, o_Wq = (oracle.pack_glu_weights if c["glu"] else oracle.pack_weights)(
            c["W"].numpy())
        assert np.array_equal(c["packed"].cpu().numpy(), o_packed)
        xw = synth.widen(c["x"])
        ref = oracle.forward(xw, synth.widen(c["g"]), o_Wq, o_beta)
        xq, s, _ = gpu_act_quant(c["x"], c["g"])
        check_xq(xq, s, ref)
        y = y_to_np(c["y"].t)
        if c["glu"]:
            check_h(y, ref, c["N"] // 2, "bf16", o_Wq, o_beta, xq, s)
        else:
            check_y(y, ref, "bf16", Wq=o_Wq, beta=o_beta, xq_gpu=xq, s_gpu=s)


def test_chain_wait_gives_up_and_recovers():
    """A run whose bounded wait is forced to give up at once (wait limit 0)
    ends normally and reports BL_ERR_TIMEOUT; the counters it leaves let the
    next normal run compute every call correctly."""
    say("chain forced give-up")
    ch = Chain(3, 1024, 1536, 1, "bf16", seed=90)
    tw.bitlinear_chain_run_ex(ch.plan, 0)
    assert tw.bitlinear_chain_status(ch.plan) == tw.BL_ERR_TIMEOUT
    assert tw.bitlinear_chain_status(ch.plan) == 0          # cleared
    ch.clear()
    tw.bitlinear_chain_run(ch.plan)
    assert tw.bitlinear_chain_status(ch.plan) == 0
    ch.check_bitwise()
    tw.bitlinear_chain_run_ex(ch.plan, 0)                    # again, then recover again
    assert tw.bitlinear_chain_status(ch.plan) == tw.BL_ERR_TIMEOUT
    ch.clear()
    for _ in range(3):
        tw.bitlinear_chain_run(ch.plan)
    assert tw.bitlinear_chain_status(ch.plan) == 0
    ch.check_bitwise()


def test_chain_graph_replays():
    """Three runs captured in a HIP graph; the graph is replayed three times
    with eager work (outputs cleared, a synchronization) in between, and
    every replay recomputes every call."""
    say("chain graph replays")
    ch = Chain(2, 1024, 1536, 1, "bf16", seed=95)
    tw.bitlinear_chain_run(ch.plan)                          # warm
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            tw.bitlinear_chain_run(ch.plan)
    for rep in range(3):
        ch.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert tw.bitlinear_chain_status(ch.plan) == 0, rep
        ch.check_bitwise()
