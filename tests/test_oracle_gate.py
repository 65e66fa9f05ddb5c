"""Pins of the oracle's FusedRMSNormSwishGate (the reading of the module's
name: z = RMSNorm(o) * w * swish(g), swish = the GLU's SiLU).  CPU only.
Each pin is a closed form, an exact invariant or a property that a plausible
slip breaks: the wrong input normalized, a sigmoid where the swish belongs,
eps outside the root, a dropped gain or 1/K."""
import math

import numpy as np
import pytest


def _inputs(seed, M, K):
    r = np.random.default_rng(seed)
    o = r.standard_normal((M, K)).astype(np.float32)
    g = (r.standard_normal((M, K)) * 2).astype(np.float32)
    w = r.uniform(0.5, 1.5, K).astype(np.float32)
    return o, g, w


def test_gate_zero_gate_input_gives_zero(orc):
    o, g, w = _inputs(1, 3, 64)
    z = orc.rmsnorm_swish_gate(o, np.zeros_like(g), w)
    assert np.all(z == 0.0)


def test_gate_constant_row_with_saturated_gate(orc):
    """o = c on the whole row and g = 40 (sigmoid(40) rounds to 1 in fp64, so
    swish(40) = 40 exactly): z = 40 w c / sqrt(c^2 + eps), the RMSNorm closed
    form; pins eps inside the root, the 1/K, the swish factor and the gain."""
    K = 96
    w = np.random.default_rng(2).uniform(0.5, 1.5, K).astype(np.float32)
    for c, eps in [(0.75, 1e-6), (3.0, 1e-6), (1e-3, 1e-6), (2.0, 0.5)]:
        o = np.full((1, K), c, np.float32)
        g = np.full((1, K), 40.0, np.float32)
        z = orc.rmsnorm_swish_gate(o, g, w, eps=eps)[0]
        cf = np.float64(np.float32(c))          # the value the row holds
        want = 40.0 * w.astype(np.float64) * (cf / math.sqrt(cf * cf + eps))
        np.testing.assert_allclose(z, want, rtol=1e-14, atol=0)


def test_gate_swish_odd_part_is_the_identity(orc):
    """swish(a) - swish(-a) = a (sigmoid(a) + sigmoid(-a) = 1): rows with g
    and -g and the same o; a sigmoid in place of the swish gives 1 instead."""
    o, g, w = _inputs(3, 1, 128)
    z1 = orc.rmsnorm_swish_gate(o, g, w)
    z2 = orc.rmsnorm_swish_gate(o, -g, w)
    n = orc.rmsnorm_swish_gate(o, np.full_like(g, 40.0), w) / 40.0     # = norm(o) * w
    np.testing.assert_allclose(z1 - z2, n * g.astype(np.float64), rtol=1e-12, atol=1e-14)


def test_gate_normalizes_o_not_g(orc):
    """Scaling o by 4 with eps = 0 leaves z bit-identical (power-of-two
    scaling commutes with every fp64 rounding of the norm); scaling g by 4
    changes it."""
    o, g, w = _inputs(4, 3, 160)
    z = orc.rmsnorm_swish_gate(o, g, w, eps=0.0)
    assert np.array_equal(orc.rmsnorm_swish_gate(o * 4, g, w, eps=0.0), z)
    assert not np.allclose(orc.rmsnorm_swish_gate(o, g * 4, w, eps=0.0), z)


def test_gate_unit_mean_square_of_the_normalized_part(orc):
    """With w = 1 and g = 40, z / 40 is o * r, whose mean square is
    ms / (ms + eps) for the row's ms = mean(o^2)."""
    o, _, _ = _inputs(5, 4, 256)
    eps = 1e-2
    z = orc.rmsnorm_swish_gate(o, np.full_like(o, 40.0), np.ones(256, np.float32), eps=eps) / 40.0
    ms = np.mean(o.astype(np.float64) ** 2, axis=1)
    np.testing.assert_allclose(np.mean(z * z, axis=1), ms / (ms + eps), rtol=1e-13)


def test_gate_linear_in_the_gain_and_rows_independent(orc):
    o, g, w = _inputs(6, 5, 64)
    z = orc.rmsnorm_swish_gate(o, g, w)
    assert np.array_equal(orc.rmsnorm_swish_gate(o, g, w * 2), 2 * z)
    perm = np.array([3, 0, 4, 1, 2])
    assert np.array_equal(orc.rmsnorm_swish_gate(o[perm], g[perm], w), z[perm])


@pytest.mark.parametrize("a", [-30.0, -3.0, -0.5, 0.25, 1.0, 7.0])
def test_gate_swish_values(orc, a):
    """The gate factor on a single element with o normalized to 1 (K = 1,
    o = 1, eps = 0, w = 1): z = swish(a) = a e^a / (1 + e^a), evaluated here
    through the odd form -- swish(a) - a = swish(-a) -- so the check is not
    the oracle's own expression."""
    z = orc.rmsnorm_swish_gate(np.ones((1, 1), np.float32), np.full((1, 1), a, np.float32),
                               np.ones(1, np.float32), eps=0.0)[0, 0]
    zm = orc.rmsnorm_swish_gate(np.ones((1, 1), np.float32), np.full((1, 1), -a, np.float32),
                                np.ones(1, np.float32), eps=0.0)[0, 0]
    assert z - zm == pytest.approx(a, rel=1e-14, abs=1e-15)
    t = math.exp(a) if a < 0 else 1.0 / math.exp(-a) if a < 700 else 0.0
    assert z == pytest.approx(a * t / (1.0 + t) if a < 0 else a / (1.0 + math.exp(-a)), rel=1e-13)
