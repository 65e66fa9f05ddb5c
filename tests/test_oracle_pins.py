"""Pins of the C oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: the
worked example printed on the pages, brute force on tiny inputs, closed
forms, exact invariants and error bounds.  They are chosen so that a
plausible slip (a dropped term, a sign, an index, a transposed operand, a
wrong rounding or scale direction) fails at least one of them;
test_oracle_mutants.py plants such slips and checks that they are caught.
"""
import itertools
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_matrices(path):
    mats, name, rows, want = {}, None, [], 0
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0].isalpha():
                name, want, rows = parts[0], int(parts[1]), []
                mats[name] = rows
                continue
            rows.append([int(p) for p in parts])
    return {k: np.array(v, dtype=np.int64) for k, v in mats.items()}


# ------------------------------------------------------------ contraction

def test_matmul_worked_example(orc):
    """C_ij = sum_p A_ip B_pj, the 2x3 by 3x2 example printed on the page."""
    m = _read_matrices(os.path.join(GOLDEN, "matmul_worked_example.txt"))
    np.testing.assert_array_equal(orc.matmul_i64(m["A"], m["B"]), m["C"])
    # The contraction uses the same product with the weight operand stored
    # as [out, in]: acc[m, n] = sum_k xq[m, k] * Wq[n, k].
    acc = orc.contract(m["A"].astype(np.int8), m["B"].T.astype(np.int8))
    np.testing.assert_array_equal(acc, m["C"])


def test_contract_brute_force_every_ternary_row(orc):
    """All 3^6 ternary rows against random int8 activations, pure-Python sums."""
    K = 6
    Wq = np.array(list(itertools.product((-1, 0, 1), repeat=K)), np.int8)
    r = np.random.default_rng(11)
    xq = r.integers(-128, 128, size=(5, K), dtype=np.int64)
    xq[0] = 127
    xq[1] = -128
    xq = xq.astype(np.int8)
    acc = orc.contract(xq, Wq)
    for m in range(xq.shape[0]):
        for n in range(Wq.shape[0]):
            want = 0
            for k in range(K):
                w = int(Wq[n, k])
                x = int(xq[m, k])
                want += x if w == 1 else (-x if w == -1 else 0)
            assert acc[m, n] == want


def test_contract_invariants(orc):
    r = np.random.default_rng(3)
    M, K = 7, 300
    xq = r.integers(-128, 128, size=(M, K)).astype(np.int8)
    zero = np.zeros((1, K), np.int8)
    ones = np.ones((1, K), np.int8)
    assert np.all(orc.contract(xq, zero) == 0)
    np.testing.assert_array_equal(orc.contract(xq, ones)[:, 0],
                                  xq.astype(np.int64).sum(1))
    np.testing.assert_array_equal(orc.contract(xq, -ones)[:, 0],
                                  -xq.astype(np.int64).sum(1))
    eye = np.eye(K, dtype=np.int8)
    np.testing.assert_array_equal(orc.contract(xq, eye), xq.astype(np.int32))
    # linearity in the activations (exact integers)
    a = r.integers(-60, 60, size=(M, K)).astype(np.int8)
    b = r.integers(-60, 60, size=(M, K)).astype(np.int8)
    Wq = r.integers(-1, 2, size=(9, K)).astype(np.int8)
    np.testing.assert_array_equal(orc.contract(a + b, Wq),
                                  orc.contract(a, Wq) + orc.contract(b, Wq))
    # extreme sums stay exact
    big = np.full((1, 4096), 127, np.int8)
    assert orc.contract(big, np.ones((1, 4096), np.int8))[0, 0] == 127 * 4096
    assert orc.contract(np.full((1, 4096), -128, np.int8),
                        np.ones((1, 4096), np.int8))[0, 0] == -128 * 4096


# --------------------------------------------------------- weight quantizer

def test_weight_scale_is_correctly_rounded_mean(orc):
    """beta equals fp32(exact sum|W| / count); math.fsum is exactly rounded."""
    r = np.random.default_rng(5)
    for N, K in [(32, 128), (64, 384), (96, 1024)]:
        W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
        exact = math.fsum(abs(float(w)) for w in W.ravel()) / (N * K)
        assert orc.weight_scale(W) == np.float32(exact)
        assert abs(orc.abs_sum(W) - exact * N * K) <= 1e-12 * exact * N * K


def test_weight_scale_floor_and_constant_magnitude(orc):
    r = np.random.default_rng(6)
    for c in (np.float32(0.015625), np.float32(0.02), np.float32(3.0)):
        signs = np.where(r.random((64, 256)) < 0.5, -1.0, 1.0).astype(np.float32)
        W = signs * c
        beta = orc.weight_scale(W)
        assert beta == c            # mean |W| of a constant-magnitude matrix
        # dividing by the scale maps every entry to its sign; multiplying by
        # it instead would round them all to zero
        np.testing.assert_array_equal(orc.ternarize(W, beta), signs.astype(np.int8))
    assert orc.weight_scale(np.zeros((32, 128), np.float32)) == np.float32(1e-5)


def test_ternarize_ties_round_half_to_even(orc):
    beta = np.float32(2.0 ** -6)
    half = np.float32(beta / 2)
    W = np.array([half, -half,
                  np.nextafter(half, np.float32(1)), np.nextafter(-half, np.float32(-1)),
                  np.nextafter(half, np.float32(0)),
                  np.float32(1.5) * beta, np.float32(-1.5) * beta,
                  np.float32(2.5) * beta, np.float32(1e9), np.float32(-1e9),
                  np.float32(0.0), np.float32(-0.0)], np.float32)
    want = [0, 0, 1, -1, 0, 1, -1, 1, 1, -1, 0, 0]
    np.testing.assert_array_equal(orc.ternarize(W, beta), np.array(want, np.int8))


def test_ternary_codes_in_set_and_gaussian_fractions(orc):
    """For Gaussian W the scale is sigma*sqrt(2/pi) and a weight is zero when
    |Z| <= 0.5*sqrt(2/pi): P = erf(0.5/sqrt(pi)) = 0.31006, +-1 each 0.34497."""
    r = np.random.default_rng(7)
    N, K = 512, 1024
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    packed, beta, Wq = orc.pack_weights(W)
    assert set(np.unique(Wq).tolist()) <= {-1, 0, 1}
    n = W.size
    assert abs(beta / 0.015957691216057307 - 1.0) < 5e-3
    p0 = 0.3100642654488372
    pp = 0.3449678672755814
    tol = 4.5 * math.sqrt(p0 * (1 - p0) / n)
    assert abs((Wq == 0).mean() - p0) < tol + 2e-3
    assert abs((Wq == 1).mean() - pp) < tol + 2e-3
    assert abs((Wq == -1).mean() - pp) < tol + 2e-3
    # codes never leave the set, even for extreme magnitudes
    Wx = W.copy()
    Wx[0, :8] = [1e30, -1e30, 1e-30, -1e-30, 5.0, -5.0, 0.0, 1e-40]
    _, _, Wq2 = orc.pack_weights(Wx)
    assert set(np.unique(Wq2).tolist()) <= {-1, 0, 1}


def test_weight_scale_linear_in_power_of_two(orc):
    r = np.random.default_rng(8)
    W = (r.standard_normal((64, 256)) * 0.02).astype(np.float32)
    p0, b0, q0 = orc.pack_weights(W)
    for j in (-3, 4):
        p1, b1, q1 = orc.pack_weights(W * np.float32(2.0 ** j))
        assert b1 == b0 * np.float32(2.0 ** j)
        np.testing.assert_array_equal(q1, q0)
        np.testing.assert_array_equal(p1, p0)


# ------------------------------------------------------------------ packing

def test_pack_roundtrip_and_uniform_bytes(orc):
    r = np.random.default_rng(9)
    for N, K in [(32, 128), (64, 256), (96, 640)]:
        Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
        p = orc.pack(Wq)
        assert p.size == N * K // 4
        np.testing.assert_array_equal(orc.unpack(p, N, K), Wq)
    # code = Wq + 1 in every 2-bit field
    assert np.all(orc.pack(np.zeros((32, 128), np.int8)) == 0x55)
    assert np.all(orc.pack(np.ones((32, 128), np.int8)) == 0xAA)
    assert np.all(orc.pack(-np.ones((32, 128), np.int8)) == 0x00)
    with pytest.raises(ValueError):
        orc.pack(np.full((32, 128), 2, np.int8))
    with pytest.raises(ValueError):
        orc.pack(np.zeros((16, 128), np.int8))
    with pytest.raises(ValueError):
        orc.unpack(np.full(32 * 128 // 4, 0xFF, np.uint8), 32, 128)


def test_pack_feeds_mfma_lanes(orc):
    """The tile layout exists so that one 16-byte load per lane of a 64-lane
    wave yields, after (word >> 2q) & 0x03030303, the 16x16x64 MFMA operand
    bytes: lane L holds output row 16h + L%16 and k-group 2*(L/16) + s in
    word 2h + s, element 4q + b in byte b of step q.  Simulate that consumer."""
    r = np.random.default_rng(10)
    N, K = 64, 384
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    p = orc.pack(Wq)
    words = p.view("<u4")
    for nt in range(N // 32):
        for kb in range(K // 128):
            tile = words[(nt * (K // 128) + kb) * 256:][:256]
            for L in range(64):
                for i in range(4):
                    h, s = divmod(i, 2)
                    w = int(tile[4 * L + i])
                    row = 32 * nt + 16 * h + L % 16
                    k0 = 128 * kb + 16 * (2 * (L // 16) + s)
                    for q in range(4):
                        v = (w >> (2 * q)) & 0x03030303
                        for b in range(4):
                            code = (v >> (8 * b)) & 0xFF
                            assert code - 1 == Wq[row, k0 + 4 * q + b]


# -------------------------------------------------------------- activations

def test_rmsnorm_constant_row_closed_form(orc):
    """x = c * ones -> xn = g * c / sqrt(c^2 + eps); at c = 1e-4 the eps term
    is as large as the mean square, which pins where eps enters."""
    r = np.random.default_rng(12)
    K = 512
    g = r.uniform(0.5, 1.5, K).astype(np.float32)
    for c in (1e-4, -3e-4, 0.75, 3.0, -40.0):
        x = np.full((1, K), np.float32(c), np.float32)
        xn, _ = orc.rmsnorm(x, g, 1e-8)
        cc = float(np.float32(c))
        want = g.astype(np.float64) * cc / math.sqrt(cc * cc + 1e-8)
        np.testing.assert_allclose(xn[0], want, rtol=5 * 2.0 ** -24, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance(orc):
    r = np.random.default_rng(13)
    M, K = 6, 1024
    x = r.standard_normal((M, K)).astype(np.float32)
    ones = np.ones(K, np.float32)
    xn, _ = orc.rmsnorm(x, ones, 1e-8)
    # with g = 1 the normalized row has mean square ms / (ms + eps) ~ 1
    msq = (xn.astype(np.float64) ** 2).mean(1)
    np.testing.assert_allclose(msq, 1.0, rtol=2e-6)
    # the direction of every row is kept
    assert np.all(np.sign(xn) == np.sign(x))
    # power-of-four scaling (mean square >= 0.25, so eps is below half an ulp)
    g = r.uniform(0.5, 1.5, K).astype(np.float32)
    xn0, _ = orc.rmsnorm(x, g, 1e-8)
    for j in (1, 2, 5):
        xn1, _ = orc.rmsnorm(x * np.float32(4.0 ** j), g, 1e-8)
        np.testing.assert_array_equal(xn1, xn0)
    # below a mean square of ~0.17 eps is no longer absorbed: x/4 differs
    xn_small, _ = orc.rmsnorm(x * np.float32(0.25), g, 1e-8)
    assert np.any(xn_small != xn0)
    # zero row -> zero output, zero codes
    z = np.zeros((1, K), np.float32)
    xz, _ = orc.rmsnorm(z, g, 1e-8)
    assert np.all(xz == 0)
    xq, s, _ = orc.act_quant(xz)
    assert np.all(xq == 0) and s[0] == np.float32(127.0) / np.float32(1e-5)


def test_act_quant_nearest_integer_and_qmax(orc):
    r = np.random.default_rng(14)
    M, K = 16, 256
    xn = r.standard_normal((M, K)).astype(np.float32)
    xn[3] *= 1e-3
    xn[4, 17] = 40.0                      # one outlier dominates the scale
    xq, s, v = orc.act_quant(xn)
    gamma = np.abs(xn).max(1)
    for m in range(M):
        # per-token absmax: the largest entry maps to +-127 exactly
        assert np.abs(xq[m]).max() == 127
        # the scale is 127 over the row absmax, to fp32 rounding
        assert abs(float(s[m]) * float(gamma[m]) - 127.0) <= 127.0 * 2 ** -23
    # every code is the integer nearest to v (ties to even), by search
    cand = np.arange(-128, 128, dtype=np.float64)
    for m in range(M):
        for k in range(K):
            d = np.abs(float(v[m, k]) - cand)
            best = cand[d == d.min()]
            if best.size == 2:
                best = best[best % 2 == 0]
            assert xq[m, k] == int(best[0])
    # dequantization error is at most half a step
    err = np.abs(xq / s[:, None].astype(np.float64) - xn.astype(np.float64))
    assert np.all(err <= (0.5 + 1e-5) / s[:, None])
    assert np.all((np.sign(xq) == np.sign(xn)) | (xq == 0))


def test_act_quant_ties_go_to_even(orc):
    # row absmax 127 -> s = 1 exactly, so v = xn and ties are visible
    xn = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.4999998]], np.float32)
    xq, s, v = orc.act_quant(xn)
    assert s[0] == 1.0
    np.testing.assert_array_equal(xq[0], [127, 0, 2, 2, 0, -2, -2, 3])


# ------------------------------------------------------------ whole forward

def test_identity_weights_reproduce_dequantized_activations(orc):
    """W = c*I -> beta = c/K, Wq = I, so y = dequant(xq) * beta and, within
    the quantization step, y = RMSNorm(x) * beta."""
    r = np.random.default_rng(15)
    M, K = 5, 128
    c = np.float32(0.125)
    W = np.eye(K, dtype=np.float32) * c
    packed, beta, Wq = orc.pack_weights(W)
    assert beta == np.float32(c / K)
    np.testing.assert_array_equal(Wq, np.eye(K, dtype=np.int8))
    x = r.standard_normal((M, K)).astype(np.float32)
    g = r.uniform(0.5, 1.5, K).astype(np.float32)
    out = orc.forward(x, g, Wq, beta)
    np.testing.assert_array_equal(out["acc"], out["xq"].astype(np.int32))
    s = out["s"].astype(np.float64)[:, None]
    np.testing.assert_allclose(out["y"] * s / float(beta), out["xq"], rtol=1e-14, atol=1e-12)
    xn, _ = orc.rmsnorm(x, g, 1e-8)
    assert np.all(np.abs(out["y"] - xn * float(beta)) <= (0.5 + 1e-5) / s * float(beta))


def test_forward_zero_rows_scale_linearity_and_error_bound(orc):
    r = np.random.default_rng(16)
    M, N, K = 4, 64, 256
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[[3, 40]] = 0.0
    x = r.standard_normal((M, K)).astype(np.float32)
    g = r.uniform(0.5, 1.5, K).astype(np.float32)
    _, beta, Wq = orc.pack_weights(W)
    out = orc.forward(x, g, Wq, beta)
    y = out["y"]
    assert np.all(y[:, [3, 40]] == 0.0) and not np.any(np.signbit(y[:, [3, 40]]))
    # y is linear in the per-tensor scale
    _, beta2, Wq2 = orc.pack_weights(W * np.float32(8.0))
    out2 = orc.forward(x, g, Wq2, beta2)
    np.testing.assert_array_equal(out2["y"], y * 8.0)
    # activation quantization error bound: |y - (xn . Wq) beta| <= sum|Wq| beta / (2 s)
    xn, _ = orc.rmsnorm(x, g, 1e-8)
    exact = xn.astype(np.float64) @ Wq.T.astype(np.float64) * float(beta)
    bound = (np.abs(Wq).sum(1)[None, :] * float(beta)
             / (2.0 * out["s"].astype(np.float64)[:, None]))
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-12)
