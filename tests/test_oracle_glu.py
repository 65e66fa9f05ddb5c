"""Pins of the oracle's GLU MLP pieces (SiLU, the gating, the GLU row order)
against mathematics and the structure the pages describe (datacamp
"MatMul-freie LLMs: Zentrale Konzepte erklärt", section "Kernkomponenten:
MLGRU und GLU": one BitLinear output passes SiLU and multiplies the other
elementwise).  Each pin compares with something other than the oracle's own
formula: identities of the logistic function, its tanh form, limits, and
reductions of the gate to already pinned pieces.  CPU only.
"""
import math

import numpy as np


def test_silu_odd_part_identity(orc):
    """silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)."""
    for x in [1e-9, 0.25, 1.0, 2.5, 7.0, 19.0, 33.0]:
        d = orc.silu(x) - orc.silu(-x)
        assert abs(d - x) <= 4e-16 * max(1.0, x), x


def test_silu_tanh_form(orc):
    """silu(x) = (x / 2) * (1 + tanh(x / 2))."""
    for x in [-30.0, -6.0, -1.5, -0.3, 0.0, 0.3, 1.5, 6.0, 30.0]:
        ref = 0.5 * x * (1.0 + math.tanh(0.5 * x))
        assert abs(orc.silu(x) - ref) <= 1e-15 * max(1.0, abs(x)), x


def test_silu_limits_and_minimum(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(60.0) == 60.0                 # sigmoid(60) rounds to 1
    assert -1e-20 < orc.silu(-60.0) < 0.0         # ~ -60 e^-60
    assert orc.silu(-800.0) == 0.0                # exp overflows: the limit
    # the global minimum of silu is at x* with x* = -1 - W(e^-1)... checked
    # numerically: it lies in (-1.28, -1.27) and its value is about -0.2785
    xs = np.linspace(-1.4, -1.15, 2501)
    v = np.array([orc.silu(float(x)) for x in xs])
    i = int(np.argmin(v))
    assert -1.28 < xs[i] < -1.27
    assert abs(v[i] + 0.27846) < 1e-4


def test_silu_slope_at_zero(orc):
    """derivative 1/2 at 0 (central difference of the odd part)."""
    e = 1e-6
    assert abs((orc.silu(e) - orc.silu(-e)) / (2 * e) - 0.5) < 1e-9


def test_glu_reduces_to_silu_and_product(orc):
    r = np.random.default_rng(5)
    M, F = 3, 48
    g = r.normal(size=(M, F)) * 3
    # multiplied half = 1: the gate is silu of the gated half
    h = orc.glu(np.concatenate([g, np.ones((M, F))], axis=1))
    for m in range(M):
        for j in range(0, F, 7):
            assert h[m, j] == orc.silu(float(g[m, j]))
    # multiplied half = 0, or gated half = 0: zero output
    assert np.all(orc.glu(np.concatenate([g, np.zeros((M, F))], axis=1)) == 0.0)
    assert np.all(orc.glu(np.concatenate([np.zeros((M, F)), g], axis=1)) == 0.0)
    # linear in the multiplied half, and not in the gated half
    u = r.normal(size=(M, F))
    h1 = orc.glu(np.concatenate([g, u], axis=1))
    h3 = orc.glu(np.concatenate([g, 3 * u], axis=1))
    np.testing.assert_allclose(h3, 3 * h1, rtol=1e-15, atol=0)
    hg = orc.glu(np.concatenate([3 * g, u], axis=1))
    assert not np.allclose(hg, 3 * h1)
    # a large positive gate passes the product through, a large negative one blocks it
    big = orc.glu(np.concatenate([np.full((M, F), 50.0), u], axis=1))
    np.testing.assert_allclose(big, 50.0 * u, rtol=1e-15)
    small = orc.glu(np.concatenate([np.full((M, F), -50.0), u], axis=1))
    assert np.all(np.abs(small) < 1e-19)


def test_glu_rows_pair_each_tile(orc):
    """The GLU packed order is a permutation whose 32-row tiles hold 16
    gated rows and exactly the 16 rows they multiply: a consumer that pairs
    rows c and 16 + c of tile t into output 16 t + c reproduces glu()."""
    F = 80
    src = orc.glu_rows(F)
    assert sorted(src.tolist()) == list(range(2 * F))
    for t in range(2 * F // 32):
        gate = src[32 * t:32 * t + 16]
        up = src[32 * t + 16:32 * t + 32]
        assert np.all(gate < F) and np.all(up >= F)
        assert np.all(up - F == gate)
        assert np.all(gate == np.arange(16 * t, 16 * t + 16))
    r = np.random.default_rng(9)
    y = r.normal(size=(2, 2 * F))
    y_packed = y[:, src]                       # what a kernel sees, tile by tile
    h = np.empty((2, F))
    for t in range(2 * F // 32):
        for c in range(16):
            a, b = y_packed[:, 32 * t + c], y_packed[:, 32 * t + 16 + c]
            h[:, 16 * t + c] = [orc.silu(float(v)) * w for v, w in zip(a, b)]
    np.testing.assert_array_equal(h, orc.glu(y))


def test_glu_rows_rejects_bad_width(orc):
    for F in (0, 8, 24, 100):
        try:
            orc.glu_rows(F)
        except ValueError:
            continue
        raise AssertionError(F)


def test_glu_pack_keeps_scale_and_codes(orc):
    """Packing gate_proj in GLU order is a row permutation: one per-tensor
    scale over all 2F rows (unchanged by the order), the same codes per
    original row, and the packed tiles decode to the permuted matrix."""
    r = np.random.default_rng(11)
    F, K = 48, 256
    W = (r.normal(size=(2 * F, K)) * 0.02).astype(np.float32)
    packed, beta, Wq = orc.pack_glu_weights(W)
    p2, beta2, Wq2 = orc.pack_weights(W)
    assert beta == beta2
    np.testing.assert_array_equal(Wq, Wq2)
    np.testing.assert_array_equal(orc.unpack(packed, 2 * F, K), Wq2[orc.glu_rows(F)])


def test_glu_forward_identity_weights(orc):
    """gate and up rows both one-hot on input k: y_g = y_u = xq[:, k] / s * beta,
    so h = silu(d) * d with d the dequantized activation (closed form from
    the FusedBitLinear pins)."""
    r = np.random.default_rng(13)
    M, F, K = 4, 16, 128
    x = r.normal(size=(M, K)).astype(np.float32)
    g = np.ones(K, np.float32)
    Wq = np.zeros((2 * F, K), np.int8)
    for j in range(F):
        Wq[j, 3 * j] = 1
        Wq[F + j, 3 * j] = 1
    beta = np.float32(0.5)
    out = orc.forward_glu(x, g, Wq, beta)
    d = out["xq"][:, 0:3 * F:3].astype(np.float64) / out["s"][:, None].astype(np.float64) * 0.5
    expect = np.array([[orc.silu(float(v)) * v for v in row] for row in d])
    np.testing.assert_allclose(out["h"], expect, rtol=1e-15, atol=0)
