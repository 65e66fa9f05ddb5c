"""Failure paths on the GPU, forced from the host so every kernel that does
run exits normally: a launch the library is told to fail (test hook) comes
back as BitLinearError(BL_ERR_HIP) with the outputs untouched, and the next
call computes as usual."""
import numpy as np
import pytest
import torch

import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import DEV, Guarded, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 1024, 1024), (40, 2048, 512), (600, 2048, 1024)])
def test_forced_launch_failure_is_reported_and_harmless(M, K, N):
    say(f"forced launch failure M={M} K={K} N={N}")
    x = synth.make_x(5, 0, 0, M, K, "bf16").to(DEV)
    g = synth.make_gain(5, 0, 0, K, "bf16").to(DEV)
    packed, beta = tw.pack(synth.make_w(5, 0, 0, N, K).to(DEV))
    ref = tw.forward(x, g, packed, beta, N)
    y = Guarded((M, N), torch.bfloat16, fill=7.0)
    ws = torch.empty(tw.bitlinear_workspace_bytes(M, K, N), dtype=torch.uint8, device=DEV)
    try:
        tw.bitlinear_test_fail_launches(1)
        with pytest.raises(tw.BitLinearError) as e:
            tw.bitlinear_forward(x, g, packed, beta, N, y.t, ws)
        assert e.value.status == -7
    finally:
        tw.bitlinear_test_fail_launches(0)
    torch.cuda.synchronize()
    y.check("y")
    assert bool(torch.all(y.t == 7.0))          # nothing ran
    tw.bitlinear_forward(x, g, packed, beta, N, y.t, ws)
    y.check("y")
    assert torch.equal(y.t.view(torch.int16), ref.view(torch.int16))
