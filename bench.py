#!/usr/bin/env python3
"""FusedBitLinear benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2]

A step is one pass of the whole hot path -- RMSNorm, per-token int8
quantization, ternary contraction against pre-packed 2-bit weights and the
rescale -- over every projection of the workload, on seeded synthetic inputs
already resident in HBM.  Default workload: the 370M-shaped attention
projections at decode (M = 1 token, four 1024 -> 1024 FusedBitLinear layers,
fp16 activations).  Other workloads (--workload c1 | c3 | c4 | c5-M<M>) are
the parity configurations, measurable the same way; <config>-mlp runs the
block's MLP instead (gate_proj with the SiLU gate fused into its epilogue,
then down_proj on the gated output).

Method
  * Weights come from a rotating pool of distinct packed copies of at least
    --pool-mib MiB (default 1024 MiB, four times the 256 MiB Infinity Cache),
    so every step streams its weights from HBM.
  * Steps are captured into HIP graphs (chunks of at most 512 steps);
    W warm-up steps are replayed untimed, then exactly K steps are timed
    with events on the replay stream, bracketed by device synchronization.
  * Roofline of the dominant kernel: a second graph holding only that
    kernel's launches is timed the same way, giving its average duration
    (rocprofv3's per-dispatch average reads higher, by about 10 % on the
    long launches and up to a third on the 2-3 us decode launches: the
    tracer stamps and signals each dispatch on its own); algorithmic bytes (packed
    weights + x + gain + y + beta) or ops (2 M N K) per launch over it give
    `achieved`.
  * cpu_baseline: the plain C oracle, single-threaded, on the same inputs,
    timed for about --cpu-seconds on the host.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
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

# HBM bytes per launch of the dominant kernel, measured with rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (one run each) and scaled by what the same
# counters read for a plain 256 MiB device copy (2047.8 and 1024.0 bytes per
# unit); the commands and tables are under profiles/.  A figure holds only
# for the kernel sources it was taken on: they are hashed, and a changed
# kernel reports traffic null until it is measured again.
KERNEL_SOURCES = {"decode": ["decode.hip", "decode_kernels.h", "decode_f32.hip", "decode_f16.hip",
                             "decode_bf16.hip", "rowquant.h", "bl_common.h", "bl_launch.h"],
                  "gemm": ["gemm.hip", "bl_common.h", "bl_launch.h"],
                  "skinny": ["skinny.hip", "rowquant.h", "bl_common.h", "bl_launch.h"]}
TRAFFIC = {  # workload: (kernel family, sources sha256[:16], bytes per launch)
    "c2": ("decode", "a0400cf502a0437a", 647830),
    "c3": ("skinny", "f48b47180f28191b", 3130625),
    "c4": ("gemm", "f09c37220f1bdc87", 87518951),
    "c5-M1": ("decode", "a0400cf502a0437a", 5250590),
    "c5-M8192": ("gemm", "f09c37220f1bdc87", 260669374),
}


def launch_kinds(wl):
    """What one launch group of the workload runs, from the paths its calls take."""
    import ternary_weight_lm_amd as tw
    fused = {tw.bitlinear_select_path(wl.M, wl.shape(c)[0]) == tw.BL_PATH_FUSED for c in wl.calls}
    if fused == {True}:
        return "one fused decode launch per group"
    if fused == {False}:
        return "two-kernel paths: act-quant + contraction per group"
    return "one fused decode launch per group where the row length allows, else act-quant + contraction"


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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c2",
                    help="c1 | c2 | c3 | c4 | c5-M1 | c5-M8 | c5-M64 | c5-M512 | c5-M8192, "
                         "or an MLP workload c3-mlp | c4-mlp | c5-M<M>-mlp (gate_proj with the fused "
                         "GLU gate, then down_proj)")
    ap.add_argument("--pool-mib", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-reps", type=int, default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy three times "
                         "(reference for the HBM byte counters) and exit")
    return ap.parse_args()


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

class Workload:
    def __init__(self, key: str):
        from ternary_weight_lm_amd import synth
        if key.startswith("c5"):
            cfg = synth.CONFIGS["c5"]
            M = int(key.split("-M")[1]) if "-M" in key else 1
            assert M in cfg.M_list, f"c5 runs at M in {cfg.M_list}"
            layers = cfg.layers
        else:
            cfg = synth.CONFIGS[key]
            M = cfg.M_list[0]
            layers = cfg.layers
        self.key, self.cfg, self.M, self.layers = key, cfg, M, layers
        # (layer, projection index) for every call of a step
        self.calls = [(l, i) for l in range(layers) for i in range(len(cfg.projs))]

    def groups(self):
        """Launch groups of a step.  HGRNBit's i/f/g projections of one layer
        read the same block input, so when they take the fused decode path
        they go out as one grouped decode launch; on the two-kernel paths they
        share one act-quant launch (and on the MFMA path one GEMM launch:
        bitlinear_forward_grouped_ws); every other projection (o_proj after
        the recurrence, the MLP pair) is launched on its own."""
        import ternary_weight_lm_amd as tw
        out, cur, cur_path = [], [], None
        for j, (layer, pi) in enumerate(self.calls):
            name = self.cfg.projs[pi].name
            path = tw.bitlinear_select_path(self.M, self.cfg.projs[pi].K)
            groupable = name in ("i_proj", "f_proj", "g_proj")
            if groupable and cur and self.calls[cur[0]][0] == layer and path == cur_path:
                cur.append(j)
                continue
            if cur:
                out.append(cur)
                cur = []
            if groupable:
                cur, cur_path = [j], path
            else:
                out.append([j])
        if cur:
            out.append(cur)
        return out

    def shape(self, call):
        p = self.cfg.projs[call[1]]
        return p.K, p.N

    def xkey(self, call):
        """The activation tensor a call reads: one per (layer, input), where
        i/f/g share their block input (synth.SHARED_INPUT) and the 2.7B
        stack reuses one per projection type across layers."""
        from ternary_weight_lm_amd import synth
        layer, pi = call
        names = [q.name for q in self.cfg.projs]
        if names[pi] in synth.SHARED_INPUT:
            pi = names.index(synth.SHARED_INPUT[0])
        return (0 if self.layers > 1 else layer, pi)

    def describe(self):
        projs = [f"{p.name} {p.K}->{p.N}" for p in self.cfg.projs]
        return {"workload": self.cfg.name + ("" if not self.key.startswith("c5") else f"_M{self.M}"),
                "tokens_per_step": self.M, "layers": self.layers, "projections": projs,
                "x_dtype": self.cfg.dtype, "y_dtype": self.cfg.y_dtype}


def build_inputs(wl: Workload, pool_bytes: int, dev):
    """Device inputs: x and gain per (layer-shared) projection, a pool of
    packed weight copies, per-call beta, outputs and workspaces."""
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth

    cfg, M = wl.cfg, wl.M
    xs, gs, host = {}, {}, {}
    packed, betas = [], []
    for call in wl.calls:
        layer, pi = call
        x, g, W = synth.config_inputs(cfg, M, layer, pi)
        key = wl.xkey(call)
        if key not in xs:
            xs[key] = x.to(dev)
        gs[call] = g.to(dev)
        pk, beta = tw.pack(W.to(dev))
        packed.append(pk)
        betas.append(beta)
        if wl.layers == 1 or layer in (0, wl.layers - 1):
            host[("W",) + call] = (x, g, W)       # oracle sample
        del W
    set_bytes = sum(p.numel() for p in packed)
    copies = max(1, math.ceil(pool_bytes / set_bytes))
    pool = []
    for c in range(copies):
        pool.append([p if c == 0 else p.clone() for p in packed])
    # outputs and workspaces are shared by the layers of a projection type:
    # each layer's output is consumed before the next layer runs
    ydt = synth.DTYPES[cfg.y_dtype]
    per_type_y = {pi: torch.empty(M, p.N, dtype=ydt, device=dev) for pi, p in enumerate(cfg.projs)}
    per_type_ws = {pi: tw.workspace(M, p.K, p.N, device=dev) for pi, p in enumerate(cfg.projs)}
    ys = [per_type_y[c[1]] for c in wl.calls]
    wss = [per_type_ws[c[1]] for c in wl.calls]
    groups = wl.groups()
    # one workspace for the grouped two-kernel launches (they run one after
    # another on the stream)
    gws_bytes = 0
    for grp in groups:
        if len(grp) > 1:
            items = [(xs[wl.xkey(wl.calls[j])],
                      gs[wl.calls[j]], pool[0][j], betas[j], ys[j]) for j in grp]
            gws_bytes = max(gws_bytes, tw.bitlinear_grouped_workspace_bytes(
                items, synth.DTYPES[cfg.dtype]))
    gws = torch.empty(max(gws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return {"xs": xs, "gs": gs, "pool": pool, "betas": betas, "ys": ys, "wss": wss, "gws": gws,
            "set_bytes": set_bytes, "copies": copies, "host": host, "groups": groups}


def step_fn(wl, inp, s, keep):
    """Enqueue one step (weights from pool copy s).  `keep` collects the
    ctypes descriptor arrays so they outlive graph capture."""
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    pool = inp["pool"][s % inp["copies"]]
    for grp in inp["groups"]:
        if len(grp) > 1:
            items = []
            for j in grp:
                call = wl.calls[j]
                x = inp["xs"][wl.xkey(call)]
                items.append((x, inp["gs"][call], pool[j], inp["betas"][j], inp["ys"][j]))
            arr = tw.make_calls(items)
            keep.append(arr)
            call = wl.calls[grp[0]]
            if tw.bitlinear_select_path(wl.M, wl.shape(call)[0]) == tw.BL_PATH_FUSED:
                tw.bitlinear_forward_grouped(arr, synth.DTYPES[wl.cfg.dtype],
                                             synth.DTYPES[wl.cfg.y_dtype])
            else:
                tw.bitlinear_forward_grouped_ws(arr, synth.DTYPES[wl.cfg.dtype],
                                                synth.DTYPES[wl.cfg.y_dtype], inp["gws"])
            continue
        j = grp[0]
        call = wl.calls[j]
        K, N = wl.shape(call)
        x = inp["xs"][wl.xkey(call)]
        tw.bitlinear_forward(x, inp["gs"][call], pool[j], inp["betas"][j], N, inp["ys"][j],
                             inp["wss"][j])


def capture(wl, inp, first, count):
    import torch
    graphs = []
    s = first
    per_step = sum(1 if len(grp) > 1 else 2 for grp in inp["groups"])  # upper bound
    chunk = max(1, min(GRAPH_CHUNK, GRAPH_MAX_LAUNCHES // per_step))
    while count > 0:
        n = min(count, chunk)
        g = torch.cuda.CUDAGraph()
        keep = []
        with torch.cuda.graph(g):
            for k in range(n):
                step_fn(wl, inp, s + k, keep)
        graphs.append((g, n))
        s += n
        count -= n
    return graphs


# ---------------------------------------------------------------- roofline

def algorithmic(wl, call):
    """Bytes (packed W + x + gain + y + beta) and ops (2 M N K) of one call."""
    from ternary_weight_lm_amd import synth
    import torch
    K, N = wl.shape(call)
    xb = torch.tensor([], dtype=synth.DTYPES[wl.cfg.dtype]).element_size()
    yb = torch.tensor([], dtype=synth.DTYPES[wl.cfg.y_dtype]).element_size()
    M = wl.M
    byt = N * K // 4 + M * K * xb + K * xb + M * N * yb + 4
    return byt, 2 * M * N * K


def roofline_from_steps(wl, inp, steps, ms):
    """Fused decode path: every launch of a step is the dominant kernel, so
    the timed steps themselves give its average duration."""
    import ternary_weight_lm_amd as tw
    launches = steps * len(inp["groups"])
    sec = ms / 1e3
    byt = sum(algorithmic(wl, c)[0] for c in wl.calls) * steps
    ops = sum(algorithmic(wl, c)[1] for c in wl.calls) * steps
    ach = byt / sec / 1e9
    grouped = any(len(g) > 1 for g in inp["groups"])
    return {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 5), "traffic": None,
            "kernel": "bl::decode_kernel (norm+quant+contract+rescale in one launch)"
                      + (", i/f/g grouped per launch" if grouped else ""),
            "launches": launches, "avg_kernel_us": round(sec * 1e6 / launches, 3),
            "algorithmic_bytes_per_launch": round(byt / launches, 1),
            "ops_per_launch": round(ops / launches, 1),
            "timed_region": "the benchmark steps themselves (one kernel per launch)"}


def roofline(wl, inp, reps):
    """Average duration of the dominant kernel: a HIP graph holding only its
    launches (reps passes over every call, weights rotating through the
    pool) is timed with events on the replay stream.  For the two-kernel
    paths the activations are quantized once beforehand, so the graph holds
    nothing but contraction launches."""
    import torch
    import ternary_weight_lm_amd as tw
    from ternary_weight_lm_amd import synth
    # the dominant kernel: the path most of the step's calls take
    paths = [tw.bitlinear_select_path(wl.M, wl.shape(c)[0]) for c in wl.calls]
    path = max(set(paths), key=paths.count)
    sel = [j for j, p in enumerate(paths) if p == path]
    bound = "hbm" if path in (tw.BL_PATH_FUSED, tw.BL_PATH_SKINNY) else "mfma"
    ncalls = len(sel)
    stage = {}
    if path != tw.BL_PATH_FUSED:
        for j in sel:
            call = wl.calls[j]
            K, N = wl.shape(call)
            # per call: calls that share x still quantize it with their own gain
            if j not in stage:
                xq = torch.empty(wl.M, K, dtype=torch.int8, device="cuda")
                sc = torch.empty(wl.M, dtype=torch.float32, device="cuda")
                rs = torch.empty(wl.M, dtype=torch.int32, device="cuda")
                tw.bitlinear_act_quant(inp["xs"][wl.xkey(call)], inp["gs"][call], xq, sc, rs)
                stage[j] = (xq, sc, rs)

    # the step's launch groups restricted to the dominant path: grouped i/f/g
    # calls are one grouped launch (decode kernel, resp. contraction), as in
    # a step
    units = []
    for grp in inp["groups"]:
        mine = [j for j in grp if j in sel]
        if not mine:
            continue
        if len(mine) > 1 and path in (tw.BL_PATH_MFMA, tw.BL_PATH_FUSED):
            units.append(mine)
        else:
            units.extend([j] for j in mine)
    nunits = len(units)
    keep = []

    def launch(r):
        s, uu = divmod(r, nunits)
        unit = units[uu]
        items = []
        for j in unit:
            call = wl.calls[j]
            K, N = wl.shape(call)
            pk = inp["pool"][(s + 7) % inp["copies"]][j]
            xkey = wl.xkey(call)
            if path == tw.BL_PATH_FUSED and len(unit) == 1:
                tw.bitlinear_forward_path(inp["xs"][xkey], inp["gs"][call], pk, inp["betas"][j],
                                          N, inp["ys"][j], inp["wss"][j], path)
            elif path == tw.BL_PATH_FUSED:
                items.append((inp["xs"][xkey], inp["gs"][call], pk, inp["betas"][j], inp["ys"][j]))
            elif len(unit) == 1:
                xq, sc, rs = stage[j]
                tw.bitlinear_contract(xq, sc, rs, pk, inp["betas"][j], N, inp["ys"][j], path=path)
            else:
                xq, sc, rs = stage[j]
                items.append((xq, sc, rs, pk, inp["betas"][j], inp["ys"][j]))
        if items and path == tw.BL_PATH_FUSED:
            arr = tw.make_calls(items)
            keep.append(arr)
            tw.bitlinear_forward_grouped(arr, synth.DTYPES[wl.cfg.dtype],
                                         synth.DTYPES[wl.cfg.y_dtype])
        elif items:
            arr = tw.make_contract_calls(items)
            keep.append(arr)
            tw.bitlinear_contract_grouped(arr, synth.DTYPES[wl.cfg.y_dtype])

    total = reps * nunits
    graphs = []
    r = 0
    while r < total:
        n = min(total - r, GRAPH_MAX_LAUNCHES)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for q in range(r, r + n):
                launch(q)
        graphs.append(g)
        r += n
    graphs[0].replay()                      # warm the replay path
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for g in graphs:
        g.replay()
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / 1e3
    byt = ops = 0
    for j in sel:
        cb, co = algorithmic(wl, wl.calls[j])
        byt += cb * reps
        ops += co * reps
    kernel = {tw.BL_PATH_FUSED: "bl::decode_kernel (norm+quant+contract+rescale)",
              tw.BL_PATH_SKINNY: "bl::skinny_kernel<fused=false> (contract+rescale)",
              tw.BL_PATH_MFMA: "bl::gemm_mfma_kernel (contract+rescale)"}[path]
    if bound == "hbm":
        ach = byt / sec / 1e9
        out = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(ach / HBM_PEAK_GBS, 5)}
    else:
        ach = ops / sec / 1e12
        out = {"bound": "mfma", "achieved": round(ach, 2), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
               "frac": round(ach / I8_PEAK_TOPS, 5)}
    out["traffic"] = None
    out["kernel"] = kernel
    out["calls_timed"] = (f"{len(sel)} of {len(wl.calls)} calls per step (those on this path) in "
                          f"{nunits} launches")
    out["launches"] = total
    out["avg_kernel_us"] = round(sec * 1e6 / total, 3)
    out["algorithmic_bytes_per_launch"] = round(byt / total, 1)
    out["ops_per_launch"] = round(ops / total, 1)
    return out


# ------------------------------------------------------------- MLP (GLU)

def run_mlp(args):
    """The HGRNBit MLP: gate_proj with the SiLU gate fused into its
    epilogue (bitlinear_forward_glu, GLU-packed weights), then down_proj on
    the gated output -- the real dependency chain.  Workloads <config>-mlp:
    c3-mlp (M = 32), c4-mlp (M = 4096), c5-M<M>-mlp (2.7B, 32 layers)."""
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

    def step(s):
        for l in range(layers):
            pg, pd = pool[(s * layers + l) % copies]
            tw.bitlinear_forward_glu(xd, ggd, pg, b_g, F, h, ws_g)
            tw.bitlinear_forward(h, gdd, pd, b_d, N, y, ws_d)

    big = M >= 512
    steps = args.steps if args.steps is not None else (20 if big else (100 if layers > 1 else 2000))
    warmup = args.warmup if args.warmup is not None else (3 if big else 10)
    per_graph = max(1, min(GRAPH_CHUNK, GRAPH_MAX_LAUNCHES // (4 * layers)))

    def capture(first, count, fn, per):
        graphs, s0 = [], first
        while count > 0:
            n = min(count, per)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(n):
                    fn(s0 + k)
            graphs.append(g)
            s0 += n
            count -= n
        return graphs

    def timed(graphs):
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for g in graphs:
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    for g in capture(0, warmup, step, per_graph):
        g.replay()
    ms = timed(capture(warmup, steps, step, per_graph))

    # roofline of the fused gate_proj + GLU launches alone
    reps = 2 if big else (10 if layers > 1 else 200)

    def glu_only(r):
        pg, _ = pool[(r + 3) % copies]
        tw.bitlinear_forward_glu(xd, ggd, pg, b_g, F, h, ws_g)

    gms = timed(capture(0, reps * layers, glu_only, GRAPH_MAX_LAUNCHES // 2))
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
        rows = M if M <= 32 else 8
        sel = np.linspace(0, M - 1, rows).round().astype(int)
        xw = synth.widen(x)[sel]
        _, beta_g, Wq_g = oracle.pack_glu_weights(W_gate.numpy())
        _, beta_d, Wq_d = oracle.pack_weights(W_down.numpy())
        gw, dw = synth.widen(g_gate), synth.widen(g_down)
        t0, n = time.perf_counter(), 0
        while True:
            hh = oracle.forward_glu(xw, gw, Wq_g, beta_g)["h"].astype(np.float32)
            oracle.forward(hh, dw, Wq_d, beta_d)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {
            "value": round(rows * n / el / layers, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} passes of {rows} of {M} token rows through one layer's MLP "
                      f"({el:.1f} s single-threaded; scaled to {layers} layer(s))"}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, inp, seconds):
    """The oracle, as it stands, on one host core: full steps for the small
    workloads, a fixed row sample for the large ones (tokens/s scaled by the
    sampled row count; every row costs the same in the oracle)."""
    import numpy as np
    import oracle
    from ternary_weight_lm_amd import synth

    host = inp["host"]
    rows = wl.M if wl.M <= 32 else 8
    sample_calls = [c for c in wl.calls if ("W",) + c in host]
    prepared = []
    for call in sample_calls:
        x, g, W = host[("W",) + call]
        W = W.numpy()
        _, beta, Wq = oracle.pack_weights(W)
        xw = synth.widen(x)
        sel = np.linspace(0, wl.M - 1, rows).round().astype(int)
        prepared.append((xw[sel], synth.widen(g), Wq, beta))
    t0 = time.perf_counter()
    n = 0
    while True:
        for xw, gw, Wq, beta in prepared:
            oracle.forward(xw, gw, Wq, beta)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_pass = el / n                               # seconds for `rows` rows of sample_calls
    per_token_all_calls = per_pass / rows * (len(wl.calls) / len(sample_calls))
    return {"value": round(1.0 / per_token_all_calls, 4), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{n} passes of {rows} of {wl.M} token rows through "
                       f"{len(sample_calls)} of {len(wl.calls)} projections "
                       f"({el:.1f} s single-threaded on {platform.processor() or 'host'}; "
                       f"scaled to every projection of a step)")}


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

    wl = Workload(args.workload)
    big = wl.M >= 512 or wl.key == "c5-M64"
    stack = wl.layers > 1
    steps = args.steps if args.steps is not None else (20 if big else (100 if stack else 2000))
    warmup = args.warmup if args.warmup is not None else (3 if big else (10 if stack else 100))
    reps = args.roofline_reps if args.roofline_reps is not None else (
        2 if big else (10 if stack else 200))

    inp = build_inputs(wl, args.pool_mib << 20, dev)

    warm_graphs = capture(wl, inp, 0, warmup) if warmup > 0 else []
    timed_graphs = capture(wl, inp, warmup, steps)
    for g, _ in warm_graphs:
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for g, _ in timed_graphs:
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / steps
    tokens_per_s = wl.M * steps / (ms / 1e3)

    import ternary_weight_lm_amd as tw
    paths = {tw.bitlinear_select_path(wl.M, wl.shape(c)[0]) for c in wl.calls}
    if paths == {tw.BL_PATH_FUSED}:
        roof = roofline_from_steps(wl, inp, steps, ms)
    else:
        roof = roofline(wl, inp, reps)
        roof["timed_region"] = "a graph of the dominant kernel's launches only"

    roof["traffic"] = traffic(wl.key)
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": dict(wl.describe(), weight_pool_MiB=round(inp["set_bytes"] * inp["copies"] / 2**20, 1),
                       weight_copies=inp["copies"],
                       launch=f"hipGraph; {len(inp['groups'])} launch groups per step "
                              f"({'i/f/g grouped' if any(len(g) > 1 for g in inp['groups']) else 'one per projection'}; "
                              f"{launch_kinds(wl)})",
                       parallelism="single GPU"),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
