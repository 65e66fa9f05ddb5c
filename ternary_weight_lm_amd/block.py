"""One HGRNBit block through the C ABI, in the order the pages give its
parts (hysenlabs ja review, section "HGRNBit という層構成を読む"; datacamp
"MatMul-freie LLMs", section "Kernkomponenten: MLGRU und GLU"):

    i, f, g = i_proj(x), f_proj(x), g_proj(x)      one grouped launch group
    h       = MLGRU scan of (i, f)                  bitlinear_mlgru_scan
    o       = o_proj(FusedRMSNormSwishGate(h, g))   bitlinear_forward_gated
    m       = GLU(gate_proj(o))                     bitlinear_forward_glu
    y       = down_proj(m)                          bitlinear_forward_path

Every projection is a FusedBitLinear with its own RMSNorm; the scan and the
gate are this library's readings of the parts the pages name without a
formula.  The block's input rows are either one sequence of M steps
(prefill) or M sequences of one step each, continuing from a per-sequence
state (decode).  Buffers are allocated once, so a step can be captured in a
HIP graph.  Argument marshalling only: every step runs in the HIP kernels."""
import torch

from . import _lib
from ._lib import DTYPE_CODE  # noqa: F401  (re-exported for callers)

GATE_EPS = 1e-6


class Block:
    """Packed weights of one block.  W: dict name -> fp32 [N, K] weights
    (i_proj, f_proj, g_proj, o_proj: [D, D]; gate_proj: [2F, D], rows 0..F-1
    the SiLU-gated half; down_proj: [D, F]); gain: dict name -> [K] gains in
    the activation dtype; gate_w: [D] gain of the swish gate."""

    NAMES = ("i_proj", "f_proj", "g_proj", "o_proj", "gate_proj", "down_proj")

    def __init__(self, W, gain, gate_w, device="cuda"):
        from . import pack, pack_glu
        self.D = W["i_proj"].shape[0]
        self.F = W["down_proj"].shape[1]
        self.packed, self.beta = {}, {}
        for n in self.NAMES:
            w = W[n].to(device=device, dtype=torch.float32)
            self.packed[n], self.beta[n] = (pack_glu(w) if n == "gate_proj" else pack(w))
        self.gain = {n: gain[n].to(device) for n in self.NAMES}
        self.gate_w = gate_w.to(device)
        self.dtype = self.gate_w.dtype

    def buffers(self, M, sequences=1, device="cuda"):
        """Outputs and workspaces of one step of M token rows: one sequence of
        M steps (sequences=1) or M sequences of one step (sequences=M)."""
        assert sequences in (1, M)
        D, F, dt = self.D, self.F, self.dtype
        e = lambda *s: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
        B, T = (1, M) if sequences == 1 else (M, 1)
        b = {"M": M, "B": B, "T": T, "x": e(M, D), "i": e(M, D), "f": e(M, D), "g": e(M, D),
             "h": e(M, D), "o": e(M, D), "m": e(M, F), "y": e(M, D),
             "state": torch.zeros(B, D, dtype=torch.float32, device=device)}
        calls = [(b["x"], self.gain[n], self.packed[n], self.beta[n], b[n[0]])
                 for n in ("i_proj", "f_proj", "g_proj")]
        b["calls"] = _lib.make_calls(calls)
        b["ws_grouped"] = torch.empty(max(16, _lib.bitlinear_grouped_workspace_bytes(b["calls"], dt)),
                                      dtype=torch.uint8, device=device)
        b["ws_scan"] = torch.zeros(max(16, _lib.bitlinear_mlgru_workspace_bytes(B, T, D)),
                                   dtype=torch.uint8, device=device)
        ws = max(_lib.bitlinear_workspace_bytes(M, D, D), _lib.bitlinear_workspace_bytes(M, D, 2 * F),
                 _lib.bitlinear_workspace_bytes(M, F, D))
        b["ws"] = torch.empty(max(16, ws), dtype=torch.uint8, device=device)
        return b

    def step(self, b, eps=1e-8, stream=None):
        """One block over b["x"] into b["y"]; the scan continues from and
        updates b["state"] (the last step's state of each sequence)."""
        D, F, dt, M, B, T = self.D, self.F, self.dtype, b["M"], b["B"], b["T"]
        _lib.bitlinear_forward_grouped_ws(b["calls"], dt, dt, b["ws_grouped"], eps=eps, stream=stream)
        _lib.bitlinear_mlgru_scan(b["i"].view(B, T, D), b["f"].view(B, T, D), b["h"].view(B, T, D),
                                  h0=b["state"], hT=b["state"], ws=b["ws_scan"], stream=stream)
        _lib.bitlinear_forward_gated(b["h"], b["g"], self.gate_w, self.gain["o_proj"],
                                     self.packed["o_proj"], self.beta["o_proj"], D, b["o"], b["ws"],
                                     gate_eps=GATE_EPS, eps=eps, stream=stream)
        _lib.bitlinear_forward_glu(b["o"], self.gain["gate_proj"], self.packed["gate_proj"],
                                   self.beta["gate_proj"], F, b["m"], b["ws"], eps=eps, stream=stream)
        _lib.bitlinear_forward_path(b["m"], self.gain["down_proj"], self.packed["down_proj"],
                                    self.beta["down_proj"], D, b["y"], b["ws"], _lib.BL_PATH_AUTO,
                                    eps=eps, stream=stream)
