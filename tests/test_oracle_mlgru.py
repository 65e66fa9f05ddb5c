"""Pins of the oracle's MLGRU scan (the reading of the pages' word-only
description: h_t = a h_{t-1} + (1 - a) i_t with the gate a = sigmoid(f_t)).
CPU only.  Each pin is a closed form, an exact invariant or a property that a
plausible slip breaks: i and f swapped, the gate on the wrong term, f used
without the sigmoid (or with e^+f), h stored before the update, h0 ignored or
not reset per sequence, a transposed [B, T, D] layout."""
import math

import numpy as np


def _inputs(seed, B, T, D):
    r = np.random.default_rng(seed)
    i = r.standard_normal((B, T, D)).astype(np.float32)
    f = (r.standard_normal((B, T, D)) * 3).astype(np.float32)
    return i, f


def test_scan_saturated_open_gate_freezes_the_state(orc):
    """f = 40: sigmoid(40) rounds to 1 in fp64 and 1 - a to 0, so every step
    keeps h0 exactly, whatever i holds (a gate on the wrong term would copy i)."""
    B, T, D = 2, 9, 5
    i, _ = _inputs(1, B, T, D)
    f = np.full((B, T, D), 40.0, np.float32)
    h0 = np.random.default_rng(2).standard_normal((B, D))
    h, hT = orc.mlgru_scan(i, f, h0)
    assert np.array_equal(h, np.broadcast_to(h0[:, None, :], (B, T, D)))
    assert np.array_equal(hT, h0)


def test_scan_saturated_closed_gate_copies_the_input(orc):
    """f = -40: a = e^-40 / (1 + e^-40) ~ 4.2e-18, so h_t = i_t to within
    1e-16 relative at the same step t (an off-by-one store or a missing
    sigmoid shows here)."""
    B, T, D = 2, 7, 6
    i, _ = _inputs(3, B, T, D)
    f = np.full((B, T, D), -40.0, np.float32)
    h0 = np.full((B, D), 1e3)
    h, hT = orc.mlgru_scan(i, f, h0)
    np.testing.assert_allclose(h, i.astype(np.float64), rtol=1e-15, atol=1e-13)
    np.testing.assert_allclose(hT, i[:, -1, :].astype(np.float64), rtol=1e-15, atol=1e-13)


def test_scan_zero_gate_input_halves_towards_the_input(orc):
    """f = 0: a = 1/2 exactly, so with a constant input c the state is the
    binary closed form h_t = c + (h0 - c) 2^-(t+1), exact in fp64 for small
    dyadic c and h0 (f used without the sigmoid gives a = 0: h_t = c)."""
    T, D = 12, 3
    c = np.array([0.75, -2.5, 8.0])
    h0 = np.array([[4.0, 1.0, -8.0]])
    i = np.broadcast_to(c.astype(np.float32), (1, T, D)).copy()
    f = np.zeros((1, T, D), np.float32)
    h, hT = orc.mlgru_scan(i, f, h0)
    t = np.arange(T)[:, None]
    want = c + (h0[0] - c) * np.ldexp(1.0, -(t + 1))
    assert np.array_equal(h[0], want)
    assert np.array_equal(hT[0], want[-1])


def test_scan_constant_gate_geometric_closed_form(orc):
    """Constant f and i: h_t = c + (h0 - c) a^(t+1), a = 1/(1 + e^-f); pins
    the sign inside the exponential and which term the gate weighs."""
    T = 40
    for fv, c, h0v in [(1.5, 0.3, -2.0), (-0.7, -1.25, 5.0), (3.0, 2.0, 0.0)]:
        a = 1.0 / (1.0 + math.exp(-float(np.float32(fv))))
        cf = float(np.float32(c))
        i = np.full((1, T, 1), c, np.float32)
        f = np.full((1, T, 1), fv, np.float32)
        h, _ = orc.mlgru_scan(i, f, np.array([[h0v]]))
        want = np.array([cf + (h0v - cf) * a ** (t + 1) for t in range(T)])
        np.testing.assert_allclose(h[0, :, 0], want, rtol=1e-12, atol=1e-14)


def test_scan_is_causal_and_splits_at_any_step(orc):
    """Changing inputs after step t0 leaves h[:, :t0+1] bit-identical, and
    running the first t0+1 steps, then the rest from their final state,
    gives the whole scan bit for bit (the same sequential operations)."""
    B, T, D = 3, 20, 4
    i, f = _inputs(5, B, T, D)
    h0 = np.random.default_rng(6).standard_normal((B, D))
    h, hT = orc.mlgru_scan(i, f, h0)
    t0 = 8
    i2, f2 = i.copy(), f.copy()
    i2[:, t0 + 1:] += 1.0
    f2[:, t0 + 1:] -= 2.0
    h2, _ = orc.mlgru_scan(i2, f2, h0)
    assert np.array_equal(h2[:, :t0 + 1], h[:, :t0 + 1])
    ha, hTa = orc.mlgru_scan(i[:, :t0 + 1], f[:, :t0 + 1], h0)
    hb, hTb = orc.mlgru_scan(i[:, t0 + 1:], f[:, t0 + 1:], hTa)
    assert np.array_equal(np.concatenate([ha, hb], axis=1), h)
    assert np.array_equal(hTb, hT)


def test_scan_sequences_and_channels_are_independent(orc):
    """Each sequence starts from its own h0 (its outputs ignore the other
    sequences' inputs), and permuting channels permutes the outputs exactly
    (a transposed layout mixes them)."""
    B, T, D = 3, 11, 7
    i, f = _inputs(7, B, T, D)
    h0 = np.random.default_rng(8).standard_normal((B, D))
    h, _ = orc.mlgru_scan(i, f, h0)
    for b in range(B):
        hb, _ = orc.mlgru_scan(i[b:b + 1], f[b:b + 1], h0[b:b + 1])
        assert np.array_equal(hb[0], h[b])
    perm = np.random.default_rng(9).permutation(D)
    hp, _ = orc.mlgru_scan(i[:, :, perm], f[:, :, perm], h0[:, perm])
    assert np.array_equal(hp, h[:, :, perm])


def test_scan_is_linear_in_input_and_state(orc):
    """For a fixed gate the map (i, h0) -> h is linear: scaling both by 4
    scales h by 4 bit for bit, and the scan of i1 + i2 from h0 = 0 is the sum
    of the two scans to rounding."""
    B, T, D = 2, 30, 5
    i1, f = _inputs(10, B, T, D)
    i2, _ = _inputs(11, B, T, D)
    # multiples of 2^-10 below 8: i1 + i2 is exact in fp32
    i1 = (np.round(i1 * 1024) / 1024).astype(np.float32)
    i2 = (np.round(i2 * 1024) / 1024).astype(np.float32)
    h0 = np.random.default_rng(12).standard_normal((B, D))
    h, _ = orc.mlgru_scan(i1, f, h0)
    h4, _ = orc.mlgru_scan(i1 * 4, f, h0 * 4)
    assert np.array_equal(h4, 4 * h)
    s12, _ = orc.mlgru_scan(i1 + i2, f)
    s1, _ = orc.mlgru_scan(i1, f)
    s2, _ = orc.mlgru_scan(i2, f)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-12, atol=1e-12)


def test_scan_state_is_a_convex_mix(orc):
    """Every state lies between the smallest and the largest of h0 and the
    inputs seen so far (gates in (0, 1)); without the sigmoid (or with 1 + a
    in place of 1 - a) large |f| leaves that hull."""
    B, T, D = 2, 50, 8
    i, f = _inputs(13, B, T, D)
    h0 = np.random.default_rng(14).standard_normal((B, D))
    h, _ = orc.mlgru_scan(i, f, h0)
    lo = np.minimum.accumulate(np.concatenate([h0[:, None], i.astype(np.float64)], 1), axis=1)[:, 1:]
    hi = np.maximum.accumulate(np.concatenate([h0[:, None], i.astype(np.float64)], 1), axis=1)[:, 1:]
    assert np.all(h >= lo - 1e-12) and np.all(h <= hi + 1e-12)
