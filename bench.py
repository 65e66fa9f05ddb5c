#!/usr/bin/env python3
"""FusedBitLinear benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c5]

A step is one pass of the whole hot path -- RMSNorm, per-token int8
quantization, ternary contraction against pre-packed 2-bit weights and the
rescale -- over every projection of the workload, on seeded synthetic inputs
already resident in HBM.

Default workload (c5): the 2.7B-shaped stack, 32 layers of six projections
(i/f/g/o_proj 2560 -> 2560, gate_proj 2560 -> 2 x 7040 with its SiLU gate,
down_proj 7040 -> 2560), bf16 activations, swept over M in {1, 8, 64, 512,
8192} tokens, all in one JSON line: `value` and `roofline` are those of the
largest M (prefill), `sweep` holds every M.  The layers are chained as the
model chains them: i/f/g read the layer input, o_proj reads g_proj's output,
gate_proj (GLU-fused) reads o_proj's output, down_proj reads the gated h and
writes the next layer's input.  Other workloads: c5-M<M> (one M of the
stack), c1..c4 (the single-layer configurations, independent projections,
i/f/g on one shared input), and <c3|c4|c5-M<M>>-mlp (the MLP pair alone).

Method
  * Weights come from a rotating pool of distinct packed copies of at least
    --pool-mib MiB (default 1024 MiB, four times the 256 MiB Infinity Cache),
    so every step streams its weights from HBM.
  * Steps are captured into HIP graphs; W warm-up steps are replayed untimed,
    then exactly K steps are timed with events on the replay stream,
    bracketed by device synchronization.
  * Roofline of the dominant kernel (the path most of the step's calls take):
    a second graph holding only that kernel's launches, as the step issues
    them, is timed the same way, giving its average duration; when every
    launch of a step is that kernel, the timed steps themselves give it.
    Algorithmic bytes (packed weights + x + gain + y + beta) or ops (2 M N K)
    per launch over that duration give `achieved`.
  * cpu_baseline: the plain C oracle, single-threaded and pinned to one host
    core, on a fixed row sample of the largest M, timed for about
    --cpu-seconds and scaled to tokens/s.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FusedBitLinear tokens/s; decode HBM GB/s & prefill int8 TOPS as % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA
GRAPH_CHUNK = 512             # at most this many steps per captured graph
GRAPH_MAX_LAUNCHES = 8192     # and about this many kernel launches
C5_SWEEP = (1, 8, 64, 512, 8192)

# HBM bytes per launch of the dominant kernel, measured with rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (one run each) and scaled by what the same
# counters read for a plain 256 MiB device copy (2047.8 and 1024.0 bytes per
# unit); the commands and tables are under profiles/.  A figure holds only
# for the kernel sources it was taken on: they are hashed, and a changed
# kernel reports traffic null until it is measured again.
KERNEL_SOURCES = {"decode": ["decode.hip", "decode_kernels.h", "decode_f32.hip", "decode_f16.hip",
                             "decode_bf16.hip", "rowquant.h", "bl_common.h", "bl_launch.h"],
                  "gemm": ["gemm.hip", "bl_common.h", "bl_launch.h"],
                  "skinny": ["skinny.hip", "rowquant.h", "bl_common.h", "bl_launch.h"],
                  "mlgru": ["mlgru.hip", "bl_common.h", "bl_launch.h"]}
TRAFFIC = {  # workload: (kernel family, sources sha256[:16], bytes per launch; per call for -mlgru)
    "c5-M1": ("decode", "61df0d418fe5e71c", 5255087),
    "c5-M8": ("decode", "61df0d418fe5e71c", 5795857),
    "c5-M64": ("skinny", "7976ad7a222d303f", 8311517),
    "c5-M512": ("gemm", "a4312010841b3530", 24119056),
    "c5-M8192": ("gemm", "a4312010841b3530", 231211982),
    "c2": ("decode", "61df0d418fe5e71c", 648128),
    "c3": ("skinny", "7976ad7a222d303f", 4661509),
    "c4": ("gemm", "a4312010841b3530", 87154001),
    "c5-M8192-mlgru": ("mlgru", "9710b4206d609eee", 225843436),
    "c5-M512-mlgru": ("mlgru", "9710b4206d609eee", 15301697),
}


def sources_sha(family):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "ternary_weight_lm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(key):
    """Counter-measured HBM bytes per launch, or None if not measured for
    this workload or the kernel changed since."""
    if key not in TRAFFIC:
        return None
    family, sha, byt = TRAFFIC[key]
    return byt if sources_sha(family) == sha else None


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c5",
                    help="c5 (2.7B stack, M sweep) | c5-M<M> | c1 | c2 | c3 | c4, an MLP "
                         "workload c3-mlp | c4-mlp | c5-M<M>-mlp, the gated o_proj c5-M<M>-gate, "
                         "the MLGRU scan c5-M<M>-mlgru, or whole HGRNBit blocks c5-M<M>-block")
    ap.add_argument("--launch", choices=["per-call", "chain"], default="per-call",
                    help="per-call: one launch group per projection (default); chain: a "
                         "chained stack at 1..4 tokens runs as one persistent launch per step "
                         "(bitlinear_chain_run)")
    ap.add_argument("--pool-mib", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-reps", type=int, default=None,
                    help="passes of the dominant kernel's roofline graph; 0 skips it where "
                         "the steps do not give it (for kernel traces of the steps alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy three times "
                         "(reference for the HBM byte counters) and exit")
    return ap.parse_args(argv)


def calibrate_copy():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
    the scale between counter units and bytes."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": 3}), flush=True)


# ---------------------------------------------------------------- workload

class Call:
    """One FusedBitLinear call of a step.  x / y name the activation buffers
    it reads and writes; N is the packed row count (2F for a GLU gate_proj,
    whose output h is F wide)."""

    def __init__(self, idx, layer, pi, name, K, N, glu, x, y):
        self.idx, self.layer, self.pi, self.name = idx, layer, pi, name
        self.K, self.N, self.glu, self.x, self.y = K, N, glu, x, y

    @property
    def n_out(self):
        return self.N // 2 if self.glu else self.N


class Workload:
    """The calls of one step and how they are grouped into launches."""

    def __init__(self, key: str, M: int | None = None, launch: str = "per-call"):
        from ternary_weight_lm_amd import synth
        base = key.split("-M")[0]
        cfg = synth.CONFIGS[base]
        if M is None:
            M = int(key.split("-M")[1]) if "-M" in key else cfg.M_list[0]
        assert M in cfg.M_list, f"{base} runs at M in {cfg.M_list}"
        self.key, self.cfg, self.M, self.layers = base, cfg, M, cfg.layers
        self.chained = cfg.layers > 1
        names = [p.name for p in cfg.projs]
        self.calls = []
        for layer in range(cfg.layers):
            for pi, p in enumerate(cfg.projs):
                glu = self.chained and p.name == "gate_proj"
                if not self.chained:
                    # independent projections: i/f/g share the block input,
                    # every other projection reads an input of its own
                    src = names.index(synth.SHARED_INPUT[0]) if p.name in synth.SHARED_INPUT else pi
                    x, y = ("in", src), ("y", pi)
                elif p.name in synth.SHARED_INPUT:
                    x, y = ("x", layer), ("y", pi)
                elif p.name == "o_proj":
                    x, y = ("y", names.index("g_proj")), ("y", pi)
                elif p.name == "gate_proj":
                    x, y = ("y", names.index("o_proj")), ("h",)
                else:  # down_proj
                    x, y = ("h",), ("x", layer + 1)
                self.calls.append(Call(len(self.calls), layer, pi, p.name, p.K, p.N, glu, x, y))
        # launch == "chain": a chained stack at 1..4 tokens (16-bit
        # activations) runs as one persistent launch per step
        # (bitlinear_chain_run); otherwise (the default) one launch group per
        # projection, which measures faster on MI355X (see the design notes)
        chain_ok = self.chained and M <= 4 and cfg.dtype in ("fp16", "bf16") \
            and max(p.K for p in cfg.projs) <= 8192
        self.launch = "chain" if chain_ok and launch == "chain" else "per-call"

    def path(self, c):
        import ternary_weight_lm_amd as tw
        return tw.bitlinear_select_path(self.M, c.K)

    def groups(self):
        """Launch groups of a step: a layer's i/f/g (one input) go out as one
        grouped call -- one fused decode launch, or on the two-kernel paths
        one shared act-quant launch (and on the MFMA path one GEMM launch);
        every other projection is launched on its own."""
        from ternary_weight_lm_amd import synth
        out, cur = [], []
        for c in self.calls:
            if c.name in synth.SHARED_INPUT and cur and cur[0].layer == c.layer \
                    and self.path(cur[0]) == self.path(c):
                cur.append(c)
                continue
            if cur:
                out.append(cur)
                cur = []
            if c.name in synth.SHARED_INPUT:
                cur = [c]
            else:
                out.append([c])
        if cur:
            out.append(cur)
        return out

    def name(self):
        base = self.cfg.name
        if self.chained:
            base = base.replace("_Msweep", "") + "_chained"
            return f"{base}_M{self.M}"
        return base

    def describe(self):
        projs = [f"{p.name} {p.K}->{p.N}" + (" + SiLU gate (GLU, fused)" if self.chained and
                                              p.name == "gate_proj" else "")
                 for p in self.cfg.projs]
        d = {"workload": self.name(), "tokens_per_step": self.M, "layers": self.layers,
             "projections": projs, "x_dtype": self.cfg.dtype, "y_dtype": self.cfg.y_dtype}
        if self.chained:
            d["dataflow"] = ("per layer: i/f/g_proj(x_l); o_proj(g_proj output); gate_proj + GLU "
                             "(o_proj output) -> h; down_proj(h) -> x_(l+1)")
        return d


def algorithmic(wl, c):
    """Bytes (packed W + x + gain + y + beta) and ops (2 M N K) of one call."""
    xb = 4 if wl.cfg.dtype == "fp32" else 2
    yb = 4 if wl.cfg.y_dtype == "fp32" else 2
    M = wl.M
    byt = c.N * c.K // 4 + M * c.K * xb + c.K * xb + M * c.n_out * yb + 4
    return byt, 2 * M * c.N * c.K


class Weights:
    """Packed weights of every call of the stack (GLU order for a chained
    gate_proj), a pool of copies of at least pool_bytes, and the host copies
    the oracle needs (layer 0 and the last layer)."""

    def __init__(self, wl, pool_bytes, dev, keep_host_layers=None):
        import torch
        import ternary_weight_lm_amd as tw
        from concurrent.futures import ThreadPoolExecutor
        from ternary_weight_lm_amd import synth

        cfg = wl.cfg
        keep = set(keep_host_layers if keep_host_layers is not None else (0, wl.layers - 1))
        self.packed, self.betas, self.host = [], [], {}

        def gen(c):
            _, g, W = synth.config_inputs(cfg, 1, c.layer, c.pi)
            return g, W

        with ThreadPoolExecutor(8) as ex:
            for c, (g, W) in zip(wl.calls, ex.map(gen, wl.calls)):
                Wd = W.to(dev)
                pk, beta = tw.pack_glu(Wd) if c.glu else tw.pack(Wd)
                del Wd
                self.packed.append(pk)
                self.betas.append(beta)
                if c.layer in keep:
                    self.host[c.idx] = W
        self.gains = {}
        for c in wl.calls:
            self.gains[c.idx] = synth.make_gain(cfg.seed, c.layer, c.pi, c.K, cfg.dtype,
                                                kind=cfg.gain).to(dev)
        self.set_bytes = sum(p.numel() for p in self.packed)
        self.copies = max(1, math.ceil(pool_bytes / self.set_bytes))
        self.pool = [self.packed] + [[p.clone() for p in self.packed]
                                     for _ in range(self.copies - 1)]
        torch.cuda.synchronize()


class Buffers:
    """Activation buffers of one M: the synthetic inputs and every call's
    output, plus the workspaces.  inp[i] / out[i] are the tensors call i
    reads and writes.  distinct=False (the benchmark): outputs of one kind
    share a buffer across layers (each is consumed before the next layer
    writes it; x_l alternates between two buffers so the step input x_0 is
    never overwritten); distinct=True (tests): every call writes a buffer of
    its own, so every output survives the step."""

    def __init__(self, wl, weights, dev, distinct=False):
        import torch
        import ternary_weight_lm_amd as tw
        from ternary_weight_lm_amd import synth

        cfg, M = wl.cfg, wl.M
        xdt, ydt = synth.DTYPES[cfg.dtype], synth.DTYPES[cfg.y_dtype]
        self.t = {}
        for c in wl.calls:
            if c.x[0] == "in" and c.x not in self.t:
                x, _, _ = synth.config_inputs(cfg, M, c.layer, c.x[1])
                self.t[c.x] = x.to(dev)
            if c.x == ("x", 0) and c.x not in self.t:
                x, _, _ = synth.config_inputs(cfg, M, 0, 0)
                self.t[c.x] = x.to(dev)
        dt_of = {"x": xdt, "y": ydt, "h": xdt}
        self.inp, self.out = {}, {}
        writer = {}
        for c in wl.calls:
            self.inp[c.idx] = self.out[writer[c.x]] if c.x in writer else self.t[c.x]
            if distinct:
                self.out[c.idx] = torch.empty(M, c.n_out, dtype=dt_of[c.y[0]], device=dev)
            else:
                key = ("x", 1 + (c.y[1] - 1) % 2) if c.y[0] == "x" else c.y
                if key not in self.t:
                    self.t[key] = torch.empty(M, c.n_out, dtype=dt_of[c.y[0]], device=dev)
                self.out[c.idx] = self.t[key]
            writer[c.y] = c.idx
        self.ws = {}
        for c in wl.calls:
            key = (c.K, c.N)
            if key not in self.ws:
                self.ws[key] = tw.workspace(M, c.K, c.N, device=dev)
        gws = 256
        for grp in wl.groups():
            if len(grp) > 1:
                items = [self.item(c, weights, weights.pool[0]) for c in grp]
                gws = max(gws, tw.bitlinear_grouped_workspace_bytes(items, xdt))
        self.gws = torch.empty(gws, dtype=torch.uint8, device=dev)
        self.plans = None
        torch.cuda.synchronize()

    def item(self, c, weights, pool):
        return (self.inp[c.idx], weights.gains[c.idx], pool[c.idx], weights.betas[c.idx],
                self.out[c.idx])

    def chain_plans(self, wl, weights):
        """One planned chain per weight-pool copy (each in a workspace of its
        own): a step runs the chain of its copy in one launch."""
        import torch
        import ternary_weight_lm_amd as tw
        from ternary_weight_lm_amd import synth
        if self.plans is None:
            self.plans = []
            for pool in weights.pool:
                arr = tw.make_chain_calls([self.item(c, weights, pool) + (c.glu,)
                                           for c in wl.calls])
                nbytes = tw.bitlinear_chain_workspace_bytes(arr, wl.M)
                raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.gws.device)
                off = (-raw.data_ptr()) % 256
                ws = raw[off:off + nbytes]
                plan = tw.bitlinear_chain_plan(arr, wl.M, synth.DTYPES[wl.cfg.dtype], ws)
                self.plans.append((plan, raw, arr))
        return self.plans


def launch_group(wl, grp, weights, bufs, pool, keep):
    """Enqueue one launch group as the step issues it.  `keep` collects the
    ctypes descriptor arrays so they outlive graph capture."""
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    xdt, ydt = synth.DTYPES[wl.cfg.dtype], synth.DTYPES[wl.cfg.y_dtype]
    if len(grp) > 1:
        arr = tw.make_calls([bufs.item(c, weights, pool) for c in grp])
        keep.append(arr)
        if wl.path(grp[0]) == tw.BL_PATH_FUSED:
            tw.bitlinear_forward_grouped(arr, xdt, ydt)
        else:
            tw.bitlinear_forward_grouped_ws(arr, xdt, ydt, bufs.gws)
        return
    c = grp[0]
    x, g, pk, beta, y = bufs.item(c, weights, pool)
    ws = bufs.ws[(c.K, c.N)]
    if c.glu:
        tw.bitlinear_forward_glu(x, g, pk, beta, c.n_out, y, ws)
    else:
        tw.bitlinear_forward(x, g, pk, beta, c.N, y, ws)


def step_fn(wl, weights, bufs, s, keep):
    """Enqueue one step (weights from pool copy s)."""
    import ternary_weight_lm_amd as tw
    if wl.launch == "chain":
        tw.bitlinear_chain_run(bufs.chain_plans(wl, weights)[s % weights.copies][0])
        return
    pool = weights.pool[s % weights.copies]
    for grp in wl.groups():
        launch_group(wl, grp, weights, bufs, pool, keep)


def capture(fn, first, count, launches_per_step):
    import torch
    graphs = []
    s = first
    chunk = max(1, min(GRAPH_CHUNK, GRAPH_MAX_LAUNCHES // max(1, launches_per_step)))
    while count > 0:
        n = min(count, chunk)
        g = torch.cuda.CUDAGraph()
        keep = []
        with torch.cuda.graph(g):
            for k in range(n):
                fn(s + k, keep)
        graphs.append((g, keep))
        s += n
        count -= n
    return graphs


def timed_replay(graphs):
    import torch
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for g, _ in graphs:
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


# ---------------------------------------------------------------- roofline

KERNEL_NAME = {0: "bl::chain_kernel (the whole stack's calls in one persistent launch: "
                  "norm+quant+contract+rescale per tile column, inputs handed on in-kernel)",
               1: "bl::decode_kernel (norm+quant+contract+rescale in one launch)",
               2: "bl::skinny_kernel<pre-quantized> (contract+rescale)",
               3: "bl::gemm_mfma_kernel (contract+rescale)"}


def dominant_path(wl):
    """The path most of the step's calls take (ties: the one carrying more
    algorithmic bytes)."""
    paths = {}
    for c in wl.calls:
        p = wl.path(c)
        n, b = paths.get(p, (0, 0))
        paths[p] = (n + 1, b + algorithmic(wl, c)[0])
    return max(paths, key=lambda p: paths[p])


def roofline(wl, weights, bufs, reps, step_ms=None, steps=None):
    """Average duration of the dominant kernel's launches and the roofline
    fraction it reaches.  If every launch of a step is that kernel, the
    timed steps give it; otherwise a graph of only its launches (issued as
    in a step, reps passes, weights rotating through the pool) is timed.
    On the two-kernel paths the activations are quantized beforehand, so
    that graph holds nothing but contraction launches."""
    import torch
    import ternary_weight_lm_amd as tw

    path = 0 if wl.launch == "chain" else dominant_path(wl)
    sel = [c for c in wl.calls if path == 0 or wl.path(c) == path]
    bound = "hbm" if path in (0, tw.BL_PATH_FUSED, tw.BL_PATH_SKINNY) else "mfma"
    units = []
    for grp in wl.groups():
        mine = [c for c in grp if wl.path(c) == path]
        if not mine:
            continue
        if len(mine) > 1 and path in (tw.BL_PATH_MFMA, tw.BL_PATH_FUSED, tw.BL_PATH_SKINNY):
            units.append(mine)
        else:
            units.extend([c] for c in mine)
    if path == 0:
        units = [wl.calls]
    if len(sel) == len(wl.calls) and path in (0, tw.BL_PATH_FUSED) and step_ms is not None:
        passes, ms = steps, step_ms * steps
        timed_region = "the benchmark steps themselves (every launch is this kernel)"
    else:
        stage = {}
        if path != tw.BL_PATH_FUSED:
            for c in sel:
                x = bufs.inp[c.idx]
                xq = torch.empty(wl.M, c.K, dtype=torch.int8, device=x.device)
                sc = torch.empty(wl.M, dtype=torch.float32, device=x.device)
                rs = torch.empty(wl.M, dtype=torch.int32, device=x.device)
                tw.bitlinear_act_quant(x, weights.gains[c.idx], xq, sc, rs)
                stage[c.idx] = (xq, sc, rs)
        nunits = len(units)

        def launch(r, keep):
            s, u = divmod(r, nunits)
            unit = units[u]
            pool = weights.pool[(s + 7) % weights.copies]
            if path == tw.BL_PATH_FUSED:
                launch_group(wl, unit, weights, bufs, pool, keep)
                return
            if len(unit) > 1:
                items = []
                for c in unit:
                    xq, sc, rs = stage[c.idx]
                    items.append((xq, sc, rs, pool[c.idx], weights.betas[c.idx], bufs.out[c.idx]))
                arr = tw.make_contract_calls(items)
                keep.append(arr)
                tw.bitlinear_contract_grouped(arr, bufs.out[unit[0].idx].dtype, path=path)
                return
            c = unit[0]
            xq, sc, rs = stage[c.idx]
            if c.glu:
                tw.bitlinear_contract_glu(xq, sc, rs, pool[c.idx], weights.betas[c.idx], c.n_out,
                                          bufs.out[c.idx], path=path)
            else:
                tw.bitlinear_contract(xq, sc, rs, pool[c.idx], weights.betas[c.idx], c.N,
                                      bufs.out[c.idx], path=path)

        graphs = capture(launch, 0, reps * nunits, 1)
        graphs[0][0].replay()                      # warm the replay path
        torch.cuda.synchronize()
        passes, ms = reps, timed_replay(graphs)
        timed_region = "a graph of the dominant kernel's launches only"
    total = passes * len(units)
    byt = sum(algorithmic(wl, c)[0] for c in sel) * passes
    ops = sum(algorithmic(wl, c)[1] for c in sel) * passes
    sec = ms / 1e3
    if bound == "hbm":
        ach = byt / sec / 1e9
        out = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(ach / HBM_PEAK_GBS, 5)}
    else:
        ach = ops / sec / 1e12
        out = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
               "frac": round(ach / I8_PEAK_TOPS, 5)}
    out["traffic"] = None
    out["kernel"] = KERNEL_NAME[path] + (" (i/f/g grouped per launch; GLU gate variant for "
                                         "gate_proj)" if wl.chained and path != 0 else "")
    out["calls_timed"] = f"{len(sel)} of {len(wl.calls)} calls per step (those on this path)"
    out["launches"] = total
    out["avg_kernel_us"] = round(sec * 1e6 / total, 3)
    out["algorithmic_bytes_per_launch"] = round(byt / total, 1)
    out["ops_per_launch"] = round(ops / total, 1)
    out["timed_region"] = timed_region
    return out


# --------------------------------------------------------------- one M

def run_m(wl, weights, dev, args):
    """Time one workload at one M; returns (summary dict, bufs)."""
    import torch
    bufs = Buffers(wl, weights, dev)
    big = wl.M >= 512
    steps = args.steps if args.steps is not None else (20 if big else 100)
    warmup = args.warmup if args.warmup is not None else (3 if big else 10)
    reps = args.roofline_reps if args.roofline_reps is not None else (2 if big else 10)
    groups = wl.groups()
    # fused groups are one launch; the two-kernel paths an act-quant launch
    # and one contraction launch per group (grouped MFMA or grouped skinny)
    per_step = 1 if wl.launch == "chain" else \
        sum(1 if wl.path(g[0]) == 1 else 2 for g in groups)
    if wl.launch == "chain":
        bufs.chain_plans(wl, weights)

    def fn(s, keep):
        step_fn(wl, weights, bufs, s, keep)

    if warmup > 0:
        for g, _ in capture(fn, 0, warmup, per_step):
            g.replay()
    timed = capture(fn, warmup, steps, per_step)
    ms = timed_replay(timed)
    del timed
    if reps > 0 or wl.launch == "chain" or all(wl.path(c) == 1 for c in wl.calls):
        roof = roofline(wl, weights, bufs, max(reps, 1), step_ms=ms / steps, steps=steps)
        roof["traffic"] = traffic(wl.key if not wl.chained else f"c5-M{wl.M}")
        roof["traffic_unit"] = ("HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated)")
    else:
        roof = None    # --roofline-reps 0: only the steps run (kernel traces of a step)
    torch.cuda.synchronize()
    return {"M": wl.M, "tokens_per_s": round(wl.M * steps / (ms / 1e3), 2), "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms / steps, 6), "launch": wl.launch,
            "launches_per_step": 1 if wl.launch == "chain" else per_step,
            "launch_groups_per_step": len(groups), "roofline": roof}, bufs


# ------------------------------------------------ o_proj with its swish gate

GATE_EPS = 1e-6   # the gate's RMSNorm epsilon (a reading: the pages give none)


def run_gate(args):
    """o_proj with FusedRMSNormSwishGate as its prologue (bitlinear_forward_gated):
    per layer, the gate of the token mixer's output o and the gate input g
    (both synthetic, bf16) feeds the 2.7B o_proj (2560 -> 2560), the gate's z
    never leaving registers.  Workloads c5-M<M>-gate (32 layers)."""
    import numpy as np
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    import oracle

    base = args.workload[:-len("-gate")]
    cfg = synth.CONFIGS["c5"]
    M = int(base.split("-M")[1])
    layers = cfg.layers
    names = [p.name for p in cfg.projs]
    oi = names.index("o_proj")
    K, N = cfg.projs[oi].K, cfg.projs[oi].N
    dev = torch.device("cuda:0")
    xdt = synth.DTYPES[cfg.dtype]
    o = synth.make_x(cfg.seed, 0, oi, M, K, cfg.dtype).to(dev)
    g = (synth.make_x(cfg.seed, 1, oi, M, K, cfg.dtype) * 2).to(dev)
    gw = synth.make_gain(cfg.seed, 1, oi, K, cfg.dtype).to(dev)
    packed, betas, gains, host_W = [], [], [], None
    for layer in range(layers):
        _, gn, W = synth.config_inputs(cfg, M, layer, oi)
        if layer == 0:
            host_W = W
        pk, b = tw.pack(W.to(dev))
        packed.append(pk)
        betas.append(b)
        gains.append(gn.to(dev))
    set_bytes = sum(p.numel() for p in packed)
    copies = max(1, math.ceil((args.pool_mib << 20) / set_bytes))
    pool = [packed] + [[p.clone() for p in packed] for _ in range(copies - 1)]
    y = torch.empty(M, N, dtype=xdt, device=dev)
    ws = tw.workspace(M, K, N, device=dev)
    torch.cuda.synchronize()

    def step(s, keep):
        pl = pool[s % copies]
        for layer in range(layers):
            tw.bitlinear_forward_gated(o, g, gw, gains[layer], pl[layer], betas[layer], N, y, ws,
                                       gate_eps=GATE_EPS)

    big = M >= 512
    steps = args.steps if args.steps is not None else (20 if big else 100)
    warmup = args.warmup if args.warmup is not None else (3 if big else 10)
    for gr, _ in capture(step, 0, warmup, 2 * layers):
        gr.replay()
    ms = timed_replay(capture(step, warmup, steps, 2 * layers))
    launches = steps * layers
    sec = ms / 1e3
    ops = 2 * M * N * K
    byt = N * K // 4 + 2 * M * K * 2 + 2 * K * 2 + M * N * 2 + 4   # W + o, g + gate and o_proj gains + y
    path_mfma = M > 64
    if path_mfma:
        ach = ops * launches / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / I8_PEAK_TOPS, 5)}
    else:
        ach = byt * launches / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 5)}
    one_launch = M <= 8   # the decode kernel's gated row mode (16-bit activations)
    roof.update({"traffic": None,
                 "kernel": ("bl::decode_rows_gated_kernel (gate + norm + quant + contract + rescale "
                            "in one launch)" if one_launch else
                            "gated act-quant (gate + norm + quant) + "
                            + ("bl::gemm_mfma_kernel" if path_mfma else "bl::skinny_kernel<pre-quantized>")),
                 "launches": launches, "avg_call_us": round(sec * 1e6 / launches, 3),
                 "algorithmic_bytes_per_call": byt, "ops_per_call": ops,
                 "timed_region": "the benchmark steps (each call: " +
                                 ("one launch)" if one_launch else
                                  "the gated act-quant launch and the contraction launch)")})
    out = {
        "metric": METRIC, "value": round(M * steps / sec, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name.replace('_Msweep', '')}_M{M}_o_proj_swish_gate",
                   "tokens_per_step": M, "layers": layers,
                   "projections": [f"FusedRMSNormSwishGate({K}) -> o_proj {K}->{N} (fused prologue)"],
                   "x_dtype": cfg.dtype, "y_dtype": cfg.dtype, "gate_eps": GATE_EPS,
                   "weight_pool_MiB": round(set_bytes * copies / 2**20, 1),
                   "launch": "hipGraph; per layer bitlinear_forward_gated (one launch up to 8 tokens)",
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        facts = host_facts()
        rows = min(M, 8)
        sel = np.linspace(0, M - 1, rows).round().astype(int)
        ow, gw_, ww = synth.widen(o.cpu())[sel], synth.widen(g.cpu())[sel], synth.widen(gw.cpu())
        _, beta, Wq = oracle.pack_weights(host_W.numpy())
        gn0 = synth.widen(gains[0].cpu())
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {facts["pinned_core"]})
        try:
            t0, n = time.perf_counter(), 0
            while True:
                z = oracle.rmsnorm_swish_gate(ow, gw_, ww, eps=GATE_EPS).astype(np.float32)
                oracle.forward(z, gn0, Wq, beta)
                n += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        finally:
            os.sched_setaffinity(0, old)
        out["cpu_baseline"] = {
            "value": round(rows * n / el / layers, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} passes of {rows} of {M} token rows through one layer's gate + o_proj "
                      f"({el:.1f} s single-threaded; scaled to {layers} layers)",
            "host": {"nproc": facts["nproc"], "cpu_model": facts["model"],
                     "pinned": f"core {facts['pinned_core']}"}}
    print(json.dumps(out), flush=True)


def run_mlgru(args):
    """The MLGRU scan (bitlinear_mlgru_scan) at the 2.7B block's mixer width:
    per layer one scan over the i_proj and f_proj outputs (synthetic, bf16,
    a distinct pair per layer so each scan reads them from HBM).  M >= 512
    tokens are one sequence of M steps (prefill); fewer are M sequences of
    one step each, continuing from a start state (decode).  Workloads
    c5-M<M>-mlgru (32 layers)."""
    import numpy as np
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    import oracle

    base = args.workload[:-len("-mlgru")]
    cfg = synth.CONFIGS["c5"]
    M = int(base.split("-M")[1])
    layers = cfg.layers
    D = cfg.projs[[p.name for p in cfg.projs].index("i_proj")].N
    B, T = (1, M) if M >= 512 else (M, 1)
    dev = torch.device("cuda:0")
    xdt = synth.DTYPES[cfg.dtype]
    i_in, f_in = [], []
    for layer in range(layers):
        i_in.append(synth.make_x(cfg.seed, layer, 0, M, D, cfg.dtype).to(dev).view(B, T, D))
        f_in.append((synth.make_x(cfg.seed, layer, 1, M, D, "fp32") * 3).to(xdt).to(dev).view(B, T, D))
    h0 = [synth.make_x(cfg.seed, layer, 2, B, D, "fp32").to(dev) for layer in range(layers)]
    h = torch.empty(B, T, D, dtype=xdt, device=dev)
    hT = torch.empty(B, D, dtype=torch.float32, device=dev)
    need = tw.bitlinear_mlgru_workspace_bytes(B, T, D)
    ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(s, keep):
        for layer in range(layers):
            tw.bitlinear_mlgru_scan(i_in[layer], f_in[layer], h, h0=h0[layer], hT=hT, ws=ws)

    nlaunch = 1 if T <= 32 else 3
    big = M >= 512
    steps = args.steps if args.steps is not None else (20 if big else 100)
    warmup = args.warmup if args.warmup is not None else (3 if big else 10)
    for gr, _ in capture(step, 0, warmup, nlaunch * layers):
        gr.replay()
    ms = timed_replay(capture(step, warmup, steps, nlaunch * layers))
    calls = steps * layers
    sec = ms / 1e3
    byt = 6 * B * T * D + 8 * B * D          # i, f, h (bf16) + h0, hT (fp32)
    ach = byt * calls / sec / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 5), "traffic": traffic(args.workload),
            "kernel": ("bl::mlgru_apply_kernel (one chunk per sequence: one launch per scan)"
                       if nlaunch == 1 else
                       "bl::mlgru_chunk_kernel + mlgru_carry_kernel + mlgru_apply_kernel "
                       f"(chunks of {16 if 32 < T < 1024 else 32} steps joined through their "
                       "start states)"),
            "launches": calls * nlaunch, "avg_call_us": round(sec * 1e6 / calls, 3),
            "algorithmic_bytes_per_call": byt,
            "timed_region": f"the benchmark steps (each call: {nlaunch} launch"
                            f"{'es' if nlaunch > 1 else ''})",
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE over its "
                            "launches, copy-calibrated)"}
    out = {
        "metric": METRIC, "value": round(M * steps / sec, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name.replace('_Msweep', '')}_M{M}_mlgru_scan",
                   "tokens_per_step": M, "layers": layers, "sequences": B, "steps_per_sequence": T,
                   "channels": D, "x_dtype": cfg.dtype,
                   "launch": f"hipGraph; per layer one bitlinear_mlgru_scan ({nlaunch} launch"
                             f"{'es' if nlaunch > 1 else ''})",
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        facts = host_facts()
        iw = synth.widen(i_in[0].cpu())
        fw = synth.widen(f_in[0].cpu())
        hw = synth.widen(h0[0].cpu()).astype(np.float64)
        cols = min(D, 256)                   # a channel sample: the scan is per channel
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {facts["pinned_core"]})
        try:
            t0, n = time.perf_counter(), 0
            while True:
                oracle.mlgru_scan(iw[:, :, :cols], fw[:, :, :cols], hw[:, :cols])
                n += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        finally:
            os.sched_setaffinity(0, old)
        out["cpu_baseline"] = {
            "value": round(M * n * cols / D / el / layers, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} scans of {cols} of {D} channels over all {M} tokens of one layer "
                      f"({el:.1f} s single-threaded; scaled to {D} channels and {layers} layers)",
            "host": {"nproc": facts["nproc"], "cpu_model": facts["model"],
                     "pinned": f"core {facts['pinned_core']}"}}
    print(json.dumps(out), flush=True)


def run_block(args):
    """The 2.7B stack as whole HGRNBit blocks (ternary_weight_lm_amd.block):
    per layer i/f/g grouped on the block input, the MLGRU scan of i and f,
    o_proj behind the swish gate of (h, g), gate_proj + GLU and down_proj,
    whose output is the next layer's input.  M >= 512 tokens: one sequence
    of M steps; fewer: M sequences of one step each, the scan continuing from
    each sequence's state.  Workloads c5-M<M>-block (32 layers)."""
    import numpy as np
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    from ternary_weight_lm_amd.block import Block
    import oracle

    base = args.workload[:-len("-block")]
    cfg = synth.CONFIGS["c5"]
    M = int(base.split("-M")[1])
    layers = cfg.layers
    names = [p.name for p in cfg.projs]
    D = cfg.projs[names.index("i_proj")].N
    F = cfg.projs[names.index("down_proj")].K
    dev = torch.device("cuda:0")
    blocks, host = [], None
    for layer in range(layers):
        W, gain = {}, {}
        for n in Block.NAMES:
            _, gain[n], W[n] = synth.config_inputs(cfg, 1, layer, names.index(n))
        if layer == 0:
            host = (W, gain)
        gate_w = synth.make_gain(cfg.seed, layer, len(names), D, cfg.dtype)
        blocks.append(Block(W, gain, gate_w, device=dev))
    seqs = 1 if M >= 512 else M
    bufs = [blk.buffers(M, sequences=seqs, device=dev) for blk in blocks]
    bufs[0]["x"].copy_(synth.make_x(cfg.seed, 0, 0, M, D, cfg.dtype).to(dev))
    for layer in range(1, layers):          # layer l reads layer l - 1's output
        bufs[layer]["x"] = bufs[layer - 1]["y"]
        calls = [(bufs[layer]["x"], blocks[layer].gain[n], blocks[layer].packed[n],
                  blocks[layer].beta[n], bufs[layer][n[0]]) for n in ("i_proj", "f_proj", "g_proj")]
        bufs[layer]["calls"] = tw.make_calls(calls)
    torch.cuda.synchronize()

    def step(s, keep):
        for layer in range(layers):
            blocks[layer].step(bufs[layer])

    per_layer = 12   # launches per block at most
    big = M >= 512
    steps = args.steps if args.steps is not None else (10 if big else 50)
    warmup = args.warmup if args.warmup is not None else (2 if big else 5)
    for gr, _ in capture(step, 0, warmup, per_layer * layers):
        gr.replay()
    ms = timed_replay(capture(step, warmup, steps, per_layer * layers))
    sec = ms / 1e3
    proj_nk = 4 * D * D + 2 * F * D + F * D                      # weights per layer
    if big:
        ops = 2 * M * proj_nk * layers * steps
        ach = ops / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / I8_PEAK_TOPS, 5), "ops_per_step": ops // steps}
    else:
        byt = (proj_nk // 4 + M * 2 * (3 * D + D + D + D + F + F) + 16 * M * D) * layers * steps
        ach = byt / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 5), "algorithmic_bytes_per_step": byt // steps}
    roof.update({"traffic": None,
                 "kernel": "whole block step (every launch of the 32 blocks: i/f/g, scan, gated "
                           "o_proj, gate_proj + GLU, down_proj)",
                 "timed_region": "the benchmark steps; the roofline counts every projection's "
                                 + ("int8 ops" if big else "weight and activation bytes")
                                 + " against the whole step's time"})
    out = {
        "metric": METRIC, "value": round(M * steps / sec, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name.replace('_Msweep', '')}_M{M}_hgrn_blocks",
                   "tokens_per_step": M, "layers": layers, "sequences": seqs,
                   "steps_per_sequence": M // seqs, "x_dtype": cfg.dtype,
                   "block": "i/f/g grouped -> MLGRU scan -> FusedRMSNormSwishGate + o_proj -> "
                            "gate_proj + GLU -> down_proj",
                   "launch": "hipGraph; per layer ternary_weight_lm_amd.block.Block.step",
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        facts = host_facts()
        W0, g0 = host
        packs = {}
        for n in Block.NAMES:
            Wn = W0[n].numpy()
            packs[n] = (oracle.pack_glu_weights(Wn) if n == "gate_proj" else oracle.pack_weights(Wn))[1:]
        gw0 = synth.widen(synth.make_gain(cfg.seed, 0, len(names), D, cfg.dtype))
        rows = min(M, 8)
        x = synth.widen(synth.make_x(cfg.seed, 0, 0, rows, D, cfg.dtype))
        gn = {n: synth.widen(g0[n]) for n in Block.NAMES}
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {facts["pinned_core"]})
        try:
            t0, n = time.perf_counter(), 0
            while True:
                y = {k: oracle.forward(x, gn[k], *packs[k][::-1])["y"].astype(np.float32)
                     for k in ("i_proj", "f_proj", "g_proj")}
                # the rows as one sequence of `rows` steps: the scan needs every step
                h, _ = oracle.mlgru_scan(y["i_proj"][None], y["f_proj"][None])
                z = oracle.rmsnorm_swish_gate(h[0].astype(np.float32), y["g_proj"], gw0,
                                              eps=GATE_EPS).astype(np.float32)
                o = oracle.forward(z, gn["o_proj"], *packs["o_proj"][::-1])["y"].astype(np.float32)
                m = oracle.forward_glu(o, gn["gate_proj"], *packs["gate_proj"][::-1])["h"]
                oracle.forward(m.astype(np.float32), gn["down_proj"], *packs["down_proj"][::-1])
                n += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        finally:
            os.sched_setaffinity(0, old)
        out["cpu_baseline"] = {
            "value": round(rows * n / el / layers, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} passes of {rows} of {M} token rows through one block ({el:.1f} s "
                      f"single-threaded; scaled to {layers} blocks)",
            "host": {"nproc": facts["nproc"], "cpu_model": facts["model"],
                     "pinned": f"core {facts['pinned_core']}"}}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------ CPU baseline

def host_facts():
    """nproc, the CPU model and the core the oracle is pinned to."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = sorted(os.sched_getaffinity(0))
    return {"nproc": len(avail), "cpu_count": os.cpu_count(), "model": model,
            "pinned_core": avail[-1] if avail else None}


def cpu_baseline(wl, weights, seconds):
    """The oracle, as it stands, on one pinned host core: a fixed sample of
    token rows (all rows up to 8, else 8 spread over M) through one layer's
    calls (every call of a single-layer workload; layer 0 of the stack,
    chained through the oracle's own outputs), tokens/s scaled to every
    layer.  Every row and layer costs the same in the oracle."""
    import numpy as np
    import oracle
    from ternary_weight_lm_amd import synth

    facts = host_facts()
    cfg = wl.cfg
    rows = min(wl.M, 8)
    sel = np.linspace(0, wl.M - 1, rows).round().astype(int)
    layer_calls = [c for c in wl.calls if c.layer == 0]
    prep = {}
    for c in layer_calls:
        W = weights.host[c.idx].numpy()
        g = synth.widen(synth.make_gain(cfg.seed, c.layer, c.pi, c.K, cfg.dtype, kind=cfg.gain))
        if c.glu:
            _, beta, Wq = oracle.pack_glu_weights(W)
        else:
            _, beta, Wq = oracle.pack_weights(W)
        prep[c.idx] = (g, Wq, beta)
    inputs = {}
    for c in layer_calls:
        if c.x[0] in ("in", "x") and c.x not in inputs:
            x, _, _ = synth.config_inputs(cfg, wl.M, 0, c.x[1] if c.x[0] == "in" else 0)
            inputs[c.x] = synth.widen(x)[sel]

    def one_layer():
        vals = dict(inputs)
        for c in layer_calls:
            g, Wq, beta = prep[c.idx]
            if c.glu:
                out = oracle.forward_glu(vals[c.x], g, Wq, beta)["h"]
            else:
                out = oracle.forward(vals[c.x], g, Wq, beta)["y"]
            vals[c.y] = out.astype(np.float32)

    old = os.sched_getaffinity(0)
    if facts["pinned_core"] is not None:
        os.sched_setaffinity(0, {facts["pinned_core"]})
    try:
        t0, n = time.perf_counter(), 0
        while True:
            one_layer()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        os.sched_setaffinity(0, old)
    per_token = el / n / rows * wl.layers
    return {"value": round(1.0 / per_token, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"{n} passes of {rows} of {wl.M} token rows through the {len(layer_calls)} "
                       f"projections of one layer ({el:.1f} s single-threaded), scaled to "
                       f"{wl.layers} layer(s)"),
            "host": {"nproc": facts["nproc"], "os_cpu_count": facts["cpu_count"],
                     "cpu_model": facts["model"],
                     "pinned": f"core {facts['pinned_core']} (sched_setaffinity, 1 thread)"}}


# ------------------------------------------------------------- MLP (GLU)

def run_mlp(args):
    """The HGRNBit MLP alone: gate_proj with the SiLU gate fused into its
    epilogue (bitlinear_forward_glu, GLU-packed weights), then down_proj on
    the gated output.  Workloads <config>-mlp: c3-mlp (M = 32), c4-mlp
    (M = 4096), c5-M<M>-mlp (2.7B, 32 layers)."""
    import numpy as np
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    import oracle

    base = args.workload[:-len("-mlp")]
    cfg = synth.CONFIGS["c5" if base.startswith("c5") else base]
    M = int(base.split("-M")[1]) if "-M" in base else cfg.M_list[0]
    layers = cfg.layers
    names = [p.name for p in cfg.projs]
    gi, di = names.index("gate_proj"), names.index("down_proj")
    K, F2 = cfg.projs[gi].K, cfg.projs[gi].N
    F, N = F2 // 2, cfg.projs[di].N
    assert cfg.projs[di].K == F
    dev = torch.device("cuda:0")
    xdt, ydt = synth.DTYPES[cfg.dtype], synth.DTYPES[cfg.y_dtype]
    x, g_gate, W_gate = synth.config_inputs(cfg, M, 0, gi)
    _, g_down, W_down = synth.config_inputs(cfg, M, 0, di)
    pk_g, b_g = tw.pack_glu(W_gate.to(dev))
    pk_d, b_d = tw.pack(W_down.to(dev))
    set_bytes = pk_g.numel() + pk_d.numel()
    copies = max(layers, math.ceil((args.pool_mib << 20) / set_bytes))
    pool = [(pk_g, pk_d)] + [(pk_g.clone(), pk_d.clone()) for _ in range(copies - 1)]
    xd, ggd, gdd = x.to(dev), g_gate.to(dev), g_down.to(dev)
    h = torch.empty(M, F, dtype=xdt, device=dev)
    y = torch.empty(M, N, dtype=ydt, device=dev)
    ws_g = tw.workspace(M, K, F2)
    ws_d = tw.workspace(M, F, N)
    torch.cuda.synchronize()

    def step(s, keep):
        for l in range(layers):
            pg, pd = pool[(s * layers + l) % copies]
            tw.bitlinear_forward_glu(xd, ggd, pg, b_g, F, h, ws_g)
            tw.bitlinear_forward(h, gdd, pd, b_d, N, y, ws_d)

    big = M >= 512
    steps = args.steps if args.steps is not None else (20 if big else (100 if layers > 1 else 2000))
    warmup = args.warmup if args.warmup is not None else (3 if big else 10)
    for g, _ in capture(step, 0, warmup, 4 * layers):
        g.replay()
    ms = timed_replay(capture(step, warmup, steps, 4 * layers))

    reps = 2 if big else (10 if layers > 1 else 200)

    def glu_only(r, keep):
        pg, _ = pool[(r + 3) % copies]
        tw.bitlinear_forward_glu(xd, ggd, pg, b_g, F, h, ws_g)

    gms = timed_replay(capture(glu_only, 0, reps * layers, 2))
    launches = reps * layers
    sec = gms / 1e3
    ops = 2 * M * F2 * K
    xb = x.element_size()
    byt = F2 * K // 4 + M * K * xb + K * xb + M * F * xb + 4
    path = tw.bitlinear_select_path(M, K)
    kern = {tw.BL_PATH_FUSED: "bl::decode_kernel<GLU> (norm+quant+contract+SiLU gate)",
            tw.BL_PATH_SKINNY: "act_quant + bl::skinny_kernel<GLU> (contract+SiLU gate)",
            tw.BL_PATH_MFMA: "act_quant + bl::gemm_mfma_kernel<GLU> (contract+SiLU gate)"}[path]
    if path == tw.BL_PATH_MFMA:
        ach = ops * launches / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(ach / I8_PEAK_TOPS, 5)}
    else:
        ach = byt * launches / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 5)}
    roof.update({"traffic": None, "kernel": kern, "launches": launches,
                 "avg_kernel_us": round(sec * 1e6 / launches, 3),
                 "algorithmic_bytes_per_launch": byt, "ops_per_launch": ops,
                 "timed_region": "a graph of the gate_proj + GLU calls only"
                                 + (" (act-quant and contraction launches)" if path != tw.BL_PATH_FUSED else "")})
    out = {
        "metric": METRIC, "value": round(M * steps / (ms / 1e3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}{'_M%d' % M if base.startswith('c5') else ''}_mlp_glu",
                   "tokens_per_step": M, "layers": layers,
                   "projections": [f"gate_proj {K}->2x{F} + SiLU gate (fused)", f"down_proj {F}->{N}"],
                   "x_dtype": cfg.dtype, "y_dtype": cfg.y_dtype,
                   "weight_pool_MiB": round(set_bytes * copies / 2**20, 1),
                   "launch": "hipGraph; per layer bitlinear_forward_glu then bitlinear_forward",
                   "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        facts = host_facts()
        rows = min(M, 8)
        sel = np.linspace(0, M - 1, rows).round().astype(int)
        xw = synth.widen(x)[sel]
        _, beta_g, Wq_g = oracle.pack_glu_weights(W_gate.numpy())
        _, beta_d, Wq_d = oracle.pack_weights(W_down.numpy())
        gw, dw = synth.widen(g_gate), synth.widen(g_down)
        old = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {facts["pinned_core"]})
        try:
            t0, n = time.perf_counter(), 0
            while True:
                hh = oracle.forward_glu(xw, gw, Wq_g, beta_g)["h"].astype(np.float32)
                oracle.forward(hh, dw, Wq_d, beta_d)
                n += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        finally:
            os.sched_setaffinity(0, old)
        out["cpu_baseline"] = {
            "value": round(rows * n / el / layers, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} passes of {rows} of {M} token rows through one layer's MLP "
                      f"({el:.1f} s single-threaded; scaled to {layers} layer(s))",
            "host": {"nproc": facts["nproc"], "os_cpu_count": facts["cpu_count"],
                     "cpu_model": facts["model"],
                     "pinned": f"core {facts['pinned_core']} (sched_setaffinity, 1 thread)"}}
    print(json.dumps(out), flush=True)


# -------------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: --gpus {args.gpus} / WORLD_SIZE {world} "
              "is not supported (the FusedBitLinear hot path is measured per GPU; the "
              "multi-GPU sharding design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import ternary_weight_lm_amd as tw
    tw.lib()                                  # fail loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.calibrate_copy:
        calibrate_copy()
        return
    dev = torch.device("cuda:0")
    if args.workload.endswith("-mlp"):
        run_mlp(args)
        return
    if args.workload.endswith("-gate"):
        run_gate(args)
        return
    if args.workload.endswith("-mlgru"):
        run_mlgru(args)
        return
    if args.workload.endswith("-block"):
        run_block(args)
        return

    sweep = args.workload == "c5"
    Ms = list(C5_SWEEP) if sweep else [None]
    t_setup = time.perf_counter()
    wl0 = Workload(args.workload, M=Ms[0], launch=args.launch)
    weights = Weights(wl0, args.pool_mib << 20, dev)
    setup_s = time.perf_counter() - t_setup
    results, last = [], None
    for M in Ms:
        wl = Workload(args.workload, M=M, launch=args.launch)
        print(f"# timing {wl.name()} ({wl.launch})", file=sys.stderr, flush=True)
        res, bufs = run_m(wl, weights, dev, args)
        del bufs
        torch.cuda.empty_cache()
        results.append(res)
        last = wl
    head = results[-1]
    wl = last
    cfgd = dict(wl.describe(),
                weight_pool_MiB=round(weights.set_bytes * weights.copies / 2**20, 1),
                weight_copies=weights.copies,
                launch=(("hipGraph; the whole step as one persistent chained launch "
                         "(bitlinear_chain_run)" if wl.launch == "chain" else
                         "hipGraph; per layer i/f/g grouped on one input (one fused decode "
                         "launch, or one shared act-quant launch + one GEMM launch on the MFMA "
                         "path), every other projection one fused launch or act-quant + "
                         "contraction") if wl.chained else
                        f"hipGraph; {head['launch_groups_per_step']} launch groups per step (i/f/g "
                        "grouped on one input; every other projection one fused launch or "
                        "act-quant + contraction)"),
                parallelism="single GPU", setup_s=round(setup_s, 1))
    if sweep:
        cfgd["workload"] = wl.name().rsplit("_M", 1)[0] + "_Msweep"
        cfgd["value_at_M"] = wl.M
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": head["steps"], "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic", "config": cfgd,
        "roofline": head["roofline"],
    }
    if sweep:
        out["sweep"] = [dict({"M": r["M"], "tokens_per_s": r["tokens_per_s"],
                              "ms_per_step": r["ms_per_step"], "steps": r["steps"],
                              "launch": r["launch"], "launches_per_step": r["launches_per_step"]},
                             **({k: r["roofline"][k] for k in ("bound", "frac", "achieved", "unit",
                                                              "avg_kernel_us", "traffic", "kernel")}
                                if r["roofline"] else {})) for r in results]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, weights, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
