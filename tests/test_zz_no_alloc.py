"""bitlinear_forward_noalloc (the static-scratch forward for callers that
cannot allocate) against bitlinear_forward with its own workspace: same
kernels, so the outputs must be identical bit for bit.  Two calls in a row
on the shared scratch, the second smaller, on the two-kernel paths that use
it (MFMA, then skinny) and on the one-launch path that does not; outputs
guarded.  Runs alone in a fresh process or after the other GPU tests."""
import numpy as np
import pytest
import torch

import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, Guarded, say

pytestmark = pytest.mark.gpu


def _case(seed, M, K, N, xdt):
    x = synth.make_x(seed, 0, 0, M, K, xdt, outlier_p=0.01).to(DEV)
    g = synth.make_gain(seed, 0, 0, K, xdt).to(DEV)
    packed, beta = tw.pack(synth.make_w(seed, 0, 0, N, K, zero_row_frac=0.05).to(DEV))
    return x, g, packed, beta


@pytest.mark.parametrize("shapes", [
    [(900, 2048, 1024), (130, 1024, 512)],     # MFMA path, then a smaller MFMA call
    [(3000, 2560, 2560), (40, 5632, 256)],     # large MFMA call, then skinny
    [(48, 7040, 512), (2, 1024, 1024)],        # skinny, then the one-launch decode
])
def test_noalloc_matches_forward(shapes):
    for j, (M, K, N) in enumerate(shapes):
        say(f"noalloc call {j}: M={M} K={K} N={N}")
        x, g, packed, beta = _case(900 + 31 * j + M, M, K, N, "bf16")
        ref = tw.forward(x, g, packed, beta, N)
        y = Guarded((M, N), torch.bfloat16, fill=float("nan"))
        tw.bitlinear_forward_noalloc(x, g, packed, beta, N, y.t)
        y.check("y")
        assert torch.equal(y.t.view(torch.int16), ref.view(torch.int16)), f"call {j}"


def test_noalloc_rejects_beyond_scratch():
    say("noalloc limit")
    cap = tw.bitlinear_noalloc_max_scratch_bytes()
    K = 8192
    M = cap // K + 1                       # M * K alone exceeds the scratch
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(K, dtype=torch.bfloat16, device=DEV)
    packed = torch.empty(32 * K // 4, dtype=torch.uint8, device=DEV)
    beta = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.empty(M, 32, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tw.BitLinearError) as e:
        tw.bitlinear_forward_noalloc(x, g, packed, beta, 32, y)
    assert e.value.status == -10
    assert np.isfinite(cap) and cap == 32 << 20
