"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, on
seeded inputs at sizes the oracle finishes in seconds, spanning several
tiles, ragged token counts, partial 128-wide output tiles and K-block counts
that do not divide evenly among the waves."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_lm_amd as tw
from ternary_weight_lm_amd import synth
from tests.parity import (DEV, Guarded, check_pack, check_xq, check_y, contract_rows,
                          gpu_act_quant, run_forward, say, y_to_np)

pytestmark = pytest.mark.gpu

PACK_SHAPES = [(32, 128), (64, 384), (96, 1024), (1024, 1024), (160, 1280), (2048, 5632)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_bit_exact(N, K):
    say(f"pack N={N} K={K}")
    W = synth.make_w(101, 0, N, N, K, zero_row_frac=0.05 if N >= 64 else 0.0)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = check_pack(W)
    # decoding the device bytes gives the oracle's ternary matrix
    Wq = torch.empty(N, K, dtype=torch.int8, device=DEV)
    tw.bitlinear_unpack_weights(d_packed, N, K, Wq)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Wq.cpu().numpy(), o_Wq)


def test_pack_exact_ties_and_extremes():
    """A matrix whose mean |W| is exactly 2^-6 and that holds entries at
    exactly beta/2 (round half to even -> 0) and one ulp above (-> +-1)."""
    say("pack ties")
    N, K = 64, 256
    r = np.random.default_rng(5)
    c = np.float32(2.0 ** -6)
    W = (np.where(r.random((N, K)) < 0.5, -1.0, 1.0) * c).astype(np.float32)
    half = np.float32(2.0 ** -7)
    up = np.nextafter(half, np.float32(1))
    W[0, :6] = [half, -half, up, -up, np.float32(2.0 ** -5),
                np.nextafter(np.float32(2.0 ** -5), np.float32(0))]
    assert np.abs(W.astype(np.float64)).sum() == 256.0      # mean exactly 2^-6
    (o_packed, o_beta, o_Wq), _ = check_pack(torch.from_numpy(W))
    assert o_beta == c
    np.testing.assert_array_equal(o_Wq[0, :6], [0, 0, 1, -1, 1, 1])
    # all-zero matrix: the scale floor, every code zero
    (_, zb, zq), _ = check_pack(torch.zeros(N, K))
    assert zb == np.float32(1e-5) and not zq.any()
    # huge magnitudes: the scale follows them, the largest saturate at +-1
    Wx = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wx[5, :4] = [1e30, -1e30, 3e38, -3e38]
    (_, _, xq_), _ = check_pack(torch.from_numpy(Wx))
    np.testing.assert_array_equal(xq_[5, :4], [0, 0, 1, -1])


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
# M <= 1024 or 4096 < K <= 8192: the split kernel, every chunk-round capacity (1..4 rounds per
# wave); M > 1024 with K <= 4096: one wave per row, every register-cache instance (2, 4, 6, 8
# chunks per lane); K > 8192: one wave per row re-reading the row per pass
@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (33, 1280), (64, 2048), (6, 3072), (9, 4096),
                                 (7, 4224), (12, 5632), (5, 6144), (7, 7040), (1030, 8192),
                                 (3, 9216), (1100, 1024), (1027, 2048), (1025, 2944), (1029, 4096)])
def test_act_quant(dtype, M, K):
    say(f"act_quant {dtype} M={M} K={K}")
    x = synth.make_x(7, 0, 0, M, K, dtype, outlier_p=0.01)
    g = synth.make_gain(7, 0, 0, K, dtype)
    if M >= 5:
        x[3] = 0        # all-zero row
        x[4] = x[4] * 1e-4
    xq, s, rs = gpu_act_quant(x.to(DEV), g.to(DEV))
    xn, _ = oracle.rmsnorm(synth.widen(x), synth.widen(g))
    oq, os_, ov = oracle.act_quant(xn)
    ref = {"xq": oq, "s": os_, "v": ov}
    check_xq(xq, s, ref)
    np.testing.assert_array_equal(rs, xq.astype(np.int64).sum(1))


@pytest.mark.parametrize("K", [1024, 2048, 3072, 4096])
def test_act_quant_kernels_agree(K):
    """The same rows through both act-quant kernels -- 1100 rows take one wave
    per row, their first 1000 one workgroup per row split over four waves --
    give the same codes, scales and row sums, bit for bit (both keep the
    fixed association of the sum of squares)."""
    say(f"act_quant one-wave vs split K={K}")
    x = synth.make_x(21, 0, 0, 1100, K, "bf16", outlier_p=0.01).to(DEV)
    g = synth.make_gain(21, 0, 0, K, "bf16").to(DEV)
    xq1, s1, rs1 = gpu_act_quant(x, g)
    xq2, s2, rs2 = gpu_act_quant(x[:1000].contiguous(), g)
    np.testing.assert_array_equal(xq1[:1000], xq2)
    np.testing.assert_array_equal(s1[:1000].view(np.uint32), s2.view(np.uint32))
    np.testing.assert_array_equal(rs1[:1000], rs2)


def _random_codes(M, K, seed):
    r = np.random.default_rng(seed)
    xq = r.integers(-128, 128, size=(M, K)).astype(np.int8)
    xq[0, :] = 127
    if M > 1:
        xq[1, :] = -128
    return xq


@pytest.mark.parametrize("path", [tw.BL_PATH_SKINNY, tw.BL_PATH_MFMA])
@pytest.mark.parametrize("M,N,K", [(1, 32, 128), (3, 96, 384), (16, 160, 1280),
                                   (17, 160, 1280), (33, 1024, 1024), (130, 96, 640),
                                   (16, 64, 7040), (200, 256, 2048), (32, 96, 2560),
                                   (48, 64, 7040), (64, 160, 1280), (40, 64, 9216),
                                   (5, 8192, 4224), (20, 8224, 1024), (64, 8224, 2560),
                                   (1100, 4096, 384)])   # 96-row tiles
def test_gemm_i32_bit_exact(path, M, N, K):
    if path == tw.BL_PATH_SKINNY and M > 64:
        pytest.skip("skinny path is for M <= 64")
    say(f"gemm_i32 path={path} M={M} N={N} K={K}")
    xq = _random_codes(M, K, M * 7 + K)
    r = np.random.default_rng(N + K)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    Wq[N // 3] = 0
    Wq[N // 2] = 1
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = Guarded((M, N), torch.int32, fill=-7)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc.t, path=path)
    acc.check("acc")
    np.testing.assert_array_equal(acc.t.cpu().numpy(), contract_rows(xq, Wq))


@pytest.mark.parametrize("M,N,K", [(3072, 8192, 128), (3000, 8224, 128), (4096, 2560, 256)])
def test_gemm_i32_wide_tile_launches_full(M, N, K):
    """Launches of at least 768 tiles of 128 x 256, the ones whose waves each
    hold four packed tiles (3072 x 8192: exactly 768; 3000 x 8224: 792 with a
    ragged last tile row and tile column; 4096 x 2560: 320 tiles, below the
    threshold, for contrast), every element of the int32 result against the
    oracle's contraction, with guard bands around the output."""
    say(f"gemm_i32 wide tiles M={M} N={N} K={K}")
    xq = _random_codes(M, K, M + N + K)
    r = np.random.default_rng(M * 3 + N)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    Wq[N - 1] = 1
    Wq[N - 2] = -1
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = Guarded((M, N), torch.int32, fill=-7)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc.t, path=tw.BL_PATH_MFMA)
    acc.check("acc")
    np.testing.assert_array_equal(acc.t.cpu().numpy(), contract_rows(xq, Wq))


@pytest.mark.parametrize("K", [128, 256, 384, 512, 640])
def test_gemm_i32_stage_ring_tails(K):
    """128-row tiles (2000 x 2048: 256 tiles, the last tile row ragged) whose
    k-blocks run in steps of three with one or two left over: 1 to 5
    k-blocks cover no full step, one step, and each remainder, every element
    against the oracle's contraction."""
    M, N = 2000, 2048
    say(f"gemm_i32 stage ring M={M} N={N} K={K}")
    xq = _random_codes(M, K, K + 5)
    r = np.random.default_rng(K)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = Guarded((M, N), torch.int32, fill=-7)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc.t, path=tw.BL_PATH_MFMA)
    acc.check("acc")
    np.testing.assert_array_equal(acc.t.cpu().numpy(), contract_rows(xq, Wq))


# (M, N, K) -> (tile height, K groups) under the launch rule in gemm.hip:
# (20, 992, 2176) 32 rows, 4 groups over 17 k-blocks (5/5/5/2);
# (100, 2560, 7040) 32, 4 over 55 (14/14/14/13); (512, 2560, 2560) 32, 2;
# (400, 2560, 7040) 32, 2 over 55 (28/27); (40, 3072, 1280) 32, 2 over 10;
# (300, 1024, 1024) 32, 2 over 8; (700, 2976, 1152) 64, 2 over 9 (5/4);
# (1000, 2560, 7040) 64, 2; (1000, 2048, 2560) 64, 4; (64, 512, 512) 32, 1
# (too few k-blocks to split); (2048, 2560, 7040) 96 rows, not split.
K_GROUP_SHAPES = [(20, 992, 2176), (100, 2560, 7040), (512, 2560, 2560), (400, 2560, 7040),
                  (40, 3072, 1280), (300, 1024, 1024), (700, 2976, 1152), (1000, 2560, 7040),
                  (1000, 2048, 2560), (64, 512, 512), (2048, 2560, 7040)]


@pytest.mark.parametrize("M,N,K", K_GROUP_SHAPES)
def test_gemm_i32_k_groups_full(M, N, K):
    """Launches with few tiles split K over 2 or 4 wave groups of one
    workgroup and add the groups' int32 accumulators in LDS: every element
    against the oracle's contraction (ragged M, N and uneven k-block shares
    included), guard bands around the output."""
    say(f"gemm_i32 k-groups M={M} N={N} K={K}")
    xq = _random_codes(M, K, 5 * M + N + K)
    r = np.random.default_rng(M + 11 * N + K)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    Wq[0] = 1
    Wq[N - 1] = -1
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = Guarded((M, N), torch.int32, fill=-7)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc.t, path=tw.BL_PATH_MFMA)
    acc.check("acc")
    np.testing.assert_array_equal(acc.t.cpu().numpy(), contract_rows(xq, Wq))


@pytest.mark.parametrize("ydt,M,N,K", [("bf16", 3072, 4096, 128), ("fp16", 3072, 4096, 128),
                                         ("bf16", 256, 2560, 2560), ("fp16", 100, 1024, 2176)])
def test_contract_grouped_full(ydt, M, N, K):
    """A grouped launch of three same-shape contractions, every output
    element against the oracle's int32 contraction rescaled as the epilogue
    does it (fp32 acc times the correctly rounded fp32 beta / s, rounded once
    to the output dtype), each output guarded.  3072 x 4096 x 128: 1152 tiles
    of 128 x 256 across the calls (the grouped kernel's 4-tile waves, as
    i/f/g at prefill); 256 x 2560 x 2560: 480 tiles of 32 rows, K split over
    2 wave groups (i/f/g of the 2.7B layer at 256 tokens); 100 x 1024 x
    2176: 96 tiles, K split over 4 groups with uneven shares."""
    say(f"contract_grouped M={M} N={N} K={K} y={ydt}")
    items, refs, outs = [], [], []
    for j in range(3):
        xq = _random_codes(M, K, 500 + j)
        r = np.random.default_rng(600 + j)
        Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
        s = r.uniform(0.5, 40.0, size=M).astype(np.float32)
        beta = np.float32(0.0155 + 0.001 * j)
        d_xq = torch.from_numpy(xq).to(DEV)
        d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
        y = Guarded((M, N), synth.DTYPES[ydt])
        items.append((d_xq, torch.from_numpy(s).to(DEV), d_rs,
                      torch.from_numpy(oracle.pack(Wq)).to(DEV),
                      torch.tensor([beta], dtype=torch.float32, device=DEV), y.t))
        outs.append(y)
        refs.append((contract_rows(xq, Wq), s, beta))
    tw.bitlinear_contract_grouped(items, synth.DTYPES[ydt])
    for j, (y, (acc, s, beta)) in enumerate(zip(outs, refs)):
        y.check(f"y[{j}]")
        scale = (torch.tensor(beta) / torch.from_numpy(s)).to(torch.float32)
        want = (torch.from_numpy(acc).to(torch.float32) * scale[:, None]).to(y.t.dtype)
        assert torch.equal(y.t.cpu().view(torch.int16), want.view(torch.int16)), f"call {j}"


FWD_CASES = [
    # path, M, N, K, x dtype, y dtype
    (tw.BL_PATH_FUSED, 1, 1024, 1024, "fp16", "fp16"),
    (tw.BL_PATH_FUSED, 3, 160, 1280, "bf16", "bf16"),
    (tw.BL_PATH_FUSED, 16, 96, 384, "fp32", "fp32"),
    (tw.BL_PATH_FUSED, 2, 64, 7040, "bf16", "fp32"),
    (tw.BL_PATH_SKINNY, 1, 160, 1280, "fp16", "fp16"),
    (tw.BL_PATH_SKINNY, 11, 1024, 1024, "bf16", "bf16"),
    (tw.BL_PATH_SKINNY, 16, 64, 2048, "fp32", "fp16"),
    (tw.BL_PATH_SKINNY, 32, 160, 2048, "fp16", "fp16"),
    (tw.BL_PATH_SKINNY, 45, 96, 5632, "bf16", "bf16"),
    (tw.BL_PATH_SKINNY, 64, 64, 1024, "fp32", "fp32"),
    (tw.BL_PATH_MFMA, 1, 96, 384, "fp16", "fp16"),
    (tw.BL_PATH_MFMA, 17, 160, 1280, "bf16", "bf16"),
    (tw.BL_PATH_MFMA, 33, 1024, 1024, "fp32", "fp32"),
    (tw.BL_PATH_MFMA, 130, 256, 640, "fp16", "bf16"),
    (tw.BL_PATH_MFMA, 257, 128, 2048, "bf16", "bf16"),
    (tw.BL_PATH_AUTO, 1, 1024, 1024, "fp16", "fp16"),
    (tw.BL_PATH_AUTO, 8, 256, 2560, "bf16", "bf16"),
    (tw.BL_PATH_AUTO, 64, 256, 2560, "bf16", "bf16"),
    (tw.BL_PATH_AUTO, 3, 96, 7040, "fp16", "fp32"),
    (tw.BL_PATH_AUTO, 2, 64, 1024, "fp32", "fp32"),
    # decode row mode with two rows per wave (9..16 rows)
    (tw.BL_PATH_FUSED, 12, 160, 2048, "bf16", "bf16"),
    (tw.BL_PATH_FUSED, 10, 96, 4096, "fp16", "fp16"),
    (tw.BL_PATH_AUTO, 16, 256, 1024, "fp32", "fp32"),
    (tw.BL_PATH_FUSED, 16, 64, 2560, "fp32", "fp32"),   # fp32 past K = 2048: skinny fused
    # 128 x 256 tiles (waves side by side, two packed tiles each), ragged in
    # both M and N: 24 x 33 = 792 such tiles, the last tile column one packed
    # tile wide, so one wave of it holds a tile and three hold none
    (tw.BL_PATH_MFMA, 3000, 8224, 128, "bf16", "bf16"),
    (tw.BL_PATH_MFMA, 3001, 8224, 256, "fp16", "fp16"),
    (tw.BL_PATH_MFMA, 3072, 8224, 128, "fp32", "fp32"),
]


@pytest.mark.parametrize("path,M,N,K,xdt,ydt", FWD_CASES)
def test_forward_matches_oracle(path, M, N, K, xdt, ydt):
    say(f"forward path={path} M={M} N={N} K={K} x={xdt} y={ydt}")
    seed = 1000 + M * 13 + N + K
    x = synth.make_x(seed, 0, 0, M, K, xdt, outlier_p=0.01)
    g = synth.make_gain(seed, 0, 0, K, xdt)
    if M >= 3:
        x[2] = 0
    W = synth.make_w(seed, 0, 0, N, K, zero_row_frac=0.05)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = check_pack(W)
    y, x_dev, g_dev = run_forward(x, g, d_packed, d_beta, N, ydt, path=path)
    ref = oracle.forward(synth.widen(x), synth.widen(g), o_Wq, o_beta)
    xq_gpu, s_gpu, _ = gpu_act_quant(x_dev, g_dev)
    check_xq(xq_gpu, s_gpu, ref)
    check_y(y, ref, ydt, Wq=o_Wq, beta=o_beta, xq_gpu=xq_gpu, s_gpu=s_gpu)
    # zeroed weight rows give exact zeros
    zero_rows = np.nonzero(~o_Wq.any(axis=1))[0]
    assert np.all(y[:, zero_rows] == 0.0)
    if M >= 3:
        assert np.all(y[2] == 0.0)


def test_paths_agree_and_repeat_bitwise():
    say("paths agree")
    M, N, K = 4, 512, 2048
    x = synth.make_x(77, 0, 0, M, K, "fp16")
    g = synth.make_gain(77, 0, 0, K, "fp16")
    W = synth.make_w(77, 0, 0, N, K)
    packed, beta = tw.pack(W.to(DEV))
    xd, gd = x.to(DEV), g.to(DEV)
    outs = [tw.forward(xd, gd, packed, beta, N, path=p)
            for p in (tw.BL_PATH_FUSED, tw.BL_PATH_SKINNY, tw.BL_PATH_MFMA, tw.BL_PATH_FUSED)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_grouped_matches_single_calls():
    say("grouped")
    # (M, N, K); consecutive same-shape runs share launches: split mode for
    # M = 1, the row mode (4 and 8 waves) for 2 <= M <= 8 up to K = 4096
    shapes = [(1, 1024, 1024), (1, 2048, 1024), (3, 96, 384), (2, 64, 7040), (4, 160, 1280),
              (0, 64, 256)] + [(6, 256, 2048)] * 3 + [(3, 96, 1024)] * 3 + [(8, 64, 4096)] * 2 \
        + [(12, 96, 1024)] * 3 + [(14, 64, 2048)] * 3
    items, singles = [], []
    for i, (M, N, K) in enumerate(shapes):
        x = synth.make_x(900 + i, 0, 0, M, K, "bf16").to(DEV)
        g = synth.make_gain(900 + i, 0, 0, K, "bf16").to(DEV)
        packed, beta = tw.pack(synth.make_w(900 + i, 0, 0, N, K).to(DEV))
        y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
        items.append((x, g, packed, beta, y))
        singles.append(tw.forward(x, g, packed, beta, N, path=tw.BL_PATH_FUSED))
    tw.bitlinear_forward_grouped(items, torch.bfloat16, torch.bfloat16)
    torch.cuda.synchronize()
    for (x, g, packed, beta, y), ref in zip(items, singles):
        assert torch.equal(y, ref)
    # more calls than one launch carries (16): split into several launches
    many = [(items[0][0], items[0][1], items[0][2], items[0][3],
             torch.empty(1, 1024, dtype=torch.bfloat16, device=DEV)) for _ in range(37)]
    tw.bitlinear_forward_grouped(many, torch.bfloat16, torch.bfloat16)
    torch.cuda.synchronize()
    for it in many:
        assert torch.equal(it[4], singles[0])


@pytest.mark.parametrize("xdt", ["fp16", "bf16", "fp32"])
def test_grouped_shared_input(xdt):
    """Grouped calls that read one activation tensor (HGRN's i/f/g, as the
    benchmark runs them) and calls whose third x is a copy: every output
    equals its single call bit for bit, for split-mode triples (M = 1, 4 and
    8 waves), a split-mode pair, and row-mode triples (8 and 16 waves)."""
    say(f"grouped shared x {xdt}")
    runs = [(1, 96, 1024, 3), (1, 64, 2560, 3), (1, 160, 1024, 2), (2, 64, 2048, 3),
            (3, 96, 1024, 3), (6, 64, 2048, 3), (14, 64, 1024, 3)]
    if xdt == "fp32":  # fp32 rows: split mode one row at a time, row mode to 8 rows
        runs = [r for r in runs if r[0] <= 8]
    ydt = "fp32" if xdt == "fp32" else xdt
    for r, (M, N, K, n) in enumerate(runs):
        x = synth.make_x(700 + r, 0, 0, M, K, xdt).to(DEV)
        for shared in (True, False):
            items, singles = [], []
            for i in range(n):
                xi = x if shared or i < n - 1 else x.clone()
                g = synth.make_gain(700 + r, 0, i, K, xdt).to(DEV)
                packed, beta = tw.pack(synth.make_w(700 + r, 0, i, N, K).to(DEV))
                y = torch.full((M, N), 7.0, dtype=synth.DTYPES[ydt], device=DEV)
                items.append((xi, g, packed, beta, y))
                singles.append(tw.forward(xi, g, packed, beta, N, path=tw.BL_PATH_FUSED,
                                          out_dtype=synth.DTYPES[ydt]))
            tw.bitlinear_forward_grouped(items, synth.DTYPES[xdt], synth.DTYPES[ydt])
            torch.cuda.synchronize()
            for (_, _, _, _, y), ref in zip(items, singles):
                assert torch.equal(y, ref), (M, N, K, n, shared)


@pytest.mark.parametrize("case", ["mixed", "prefill_1p3b", "prefill_shared_x", "skinny_runs"])
def test_grouped_ws_matches_single_calls(case):
    """bitlinear_forward_grouped_ws gives bitlinear_forward's result on every
    call, bit for bit: runs of three same-shape MFMA-path calls sharing an
    act-quant and a GEMM launch (ragged M, partial output tiles, a run of
    four split 3 + 1), an MFMA call of another shape, a skinny-path call,
    calls the fused kernels take and a triple whose grouped GEMM takes 96-row
    tiles (single calls of that shape take 32-row ones) -- and, full size,
    the 1.3B i/f/g triple at prefill, also with one x shared by the triple
    (one act-quant pass per row for all three calls, which must still give
    each call's own bits).  skinny_runs: triples that go out as one skinny
    launch (the 2.7B i/f/g at 64 tokens, 12 sub-calls of 16 rows; 20 tokens
    over 288 tile columns, not split; 33 tokens at K = 7040)."""
    shared = case == "prefill_shared_x"
    if case == "mixed":
        shapes = [(300, 384, 640)] * 4 + [(100, 96, 256), (20, 160, 512), (1, 64, 1024),
                                          (3, 96, 384), (0, 64, 256), (65, 160, 1280),
                                          (65, 160, 1280)] + [(40, 96, 512)] * 3 \
            + [(1100, 1408, 1024)] * 3   # grouped GEMM in 96-row tiles
    elif case == "prefill_1p3b":
        shapes = [(4096, 2048, 2048)] * 3
    elif case == "skinny_runs":
        shapes = [(64, 2560, 2560)] * 3 + [(20, 3072, 1024)] * 3 + [(33, 2560, 7040)] * 3
    else:
        shapes = [(4096, 2048, 2048)] * 3 + [(3101, 384, 2944)] * 3
    say(f"grouped_ws {case}")
    items, singles = [], []
    for i, (M, N, K) in enumerate(shapes):
        x = synth.make_x(950 + i, 0, 0, M, K, "bf16").to(DEV)
        if shared and i % 3:
            x = items[i - 1][0]   # the same tensor as the run's first call
        g = synth.make_gain(950 + i, 0, 0, K, "bf16").to(DEV)
        packed, beta = tw.pack(synth.make_w(950 + i, 0, 0, N, K).to(DEV))
        y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
        items.append((x, g, packed, beta, y))
        singles.append(tw.forward(x, g, packed, beta, N))
    calls = tw.make_calls(items)
    nbytes = tw.bitlinear_grouped_workspace_bytes(calls, torch.bfloat16)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    tw.bitlinear_forward_grouped_ws(calls, torch.bfloat16, torch.bfloat16, ws)
    torch.cuda.synchronize()
    for (x, g, packed, beta, y), ref in zip(items, singles):
        assert torch.equal(y, ref)


@pytest.mark.parametrize("path", [tw.BL_PATH_MFMA, tw.BL_PATH_SKINNY, tw.BL_PATH_AUTO])
def test_contract_grouped_matches_single_calls(path):
    """bitlinear_contract_grouped (runs of up to three same-shape calls per
    launch) gives bitlinear_contract(..., same path) bit for bit: on the MFMA
    kernel, and on the skinny kernel (the 2.7B i/f/g at 64 tokens as 12
    sub-calls of 16 rows, a run of four split 3 + 1, a run over 288 tile
    columns that is not split), and with the path chosen per run."""
    say(f"contract_grouped path={path}")
    if path == tw.BL_PATH_MFMA:
        shapes = [(300, 384, 640)] * 4 + [(40, 96, 256), (300, 384, 640), (0, 64, 256)]
    else:
        shapes = [(64, 2560, 2560)] * 3 + [(40, 96, 256)] * 4 + [(20, 3072, 1024)] * 3 \
            + [(0, 64, 256), (7, 160, 1280)]
        if path == tw.BL_PATH_AUTO:
            shapes += [(300, 384, 640)] * 3
    items, singles = [], []
    for i, (M, N, K) in enumerate(shapes):
        xq = (torch.from_numpy(_random_codes(M, K, 70 + i)) if M else
              torch.empty((0, K), dtype=torch.int8)).to(DEV)
        rs = xq.to(torch.int32).sum(1, dtype=torch.int32)
        sc = (torch.rand(M, device=DEV) * 30 + 0.5).to(torch.float32)
        packed, beta = tw.pack(synth.make_w(970 + i, 0, 0, N, K).to(DEV))
        y = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
        ref = torch.empty_like(y)
        tw.bitlinear_contract(xq, sc, rs, packed, beta, N, ref, path=path)
        items.append((xq, sc, rs, packed, beta, y))
        singles.append(ref)
    tw.bitlinear_contract_grouped(items, torch.float16, path=path)
    torch.cuda.synchronize()
    for it, ref in zip(items, singles):
        assert torch.equal(it[5], ref)


def test_paths_agree_bitwise_mid_m():
    say("paths agree mid M")
    for M in (24, 40, 64):
        N, K = 160, 2560
        x = synth.make_x(78 + M, 0, 0, M, K, "bf16", outlier_p=0.01)
        g = synth.make_gain(78 + M, 0, 0, K, "bf16")
        packed, beta = tw.pack(synth.make_w(78 + M, 0, 0, N, K).to(DEV))
        xd, gd = x.to(DEV), g.to(DEV)
        a = tw.forward(xd, gd, packed, beta, N, path=tw.BL_PATH_SKINNY)
        b = tw.forward(xd, gd, packed, beta, N, path=tw.BL_PATH_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_grouped_mixed_kernels():
    """Calls the decode kernel does not take (M of 5..16, fp32 rows with
    M > 1) share launches of the skinny kernel; results equal single calls."""
    say("grouped mixed")
    for dt, shapes in (("bf16", [(8, 96, 1024), (1, 96, 1024), (16, 64, 2560), (1, 96, 1024),
                                 (1, 96, 1024), (1, 96, 1024), (12, 32, 384)]),
                       ("fp32", [(2, 64, 1024), (1, 64, 1024), (3, 32, 512)])):
        tdt = synth.DTYPES[dt]
        items, singles = [], []
        for i, (M, N, K) in enumerate(shapes):
            x = synth.make_x(950 + i, 0, 0, M, K, dt).to(DEV)
            g = synth.make_gain(950 + i, 0, 0, K, dt).to(DEV)
            packed, beta = tw.pack(synth.make_w(950 + i, 0, 0, N, K).to(DEV))
            y = torch.full((M, N), 7.0, dtype=tdt, device=DEV)
            items.append((x, g, packed, beta, y))
            singles.append(tw.forward(x, g, packed, beta, N, path=tw.BL_PATH_FUSED))
        tw.bitlinear_forward_grouped(items, tdt, tdt)
        torch.cuda.synchronize()
        for (x, g, packed, beta, y), ref in zip(items, singles):
            assert torch.equal(y, ref)


def test_empty_batch_is_noop():
    say("empty batch")
    N, K = 64, 256
    packed, beta = tw.pack(synth.make_w(3, 0, 0, N, K).to(DEV))
    x = torch.empty(0, K, dtype=torch.float16, device=DEV)
    g = torch.ones(K, dtype=torch.float16, device=DEV)
    y = tw.forward(x, g, packed, beta, N)
    torch.cuda.synchronize()
    assert y.shape == (0, N)


@pytest.mark.parametrize("path,M,N,K,xdt", [
    (tw.BL_PATH_FUSED, 1, 64, 8192, "bf16"),      # largest K of the one-launch kernel
    (tw.BL_PATH_FUSED, 4, 96, 8192, "fp16"),
    (tw.BL_PATH_AUTO, 1, 64, 8320, "bf16"),       # just past it: two kernels
    (tw.BL_PATH_AUTO, 2, 32, 65536, "bf16"),      # largest K: act-quant re-reads the row
    (tw.BL_PATH_MFMA, 3, 160, 65536, "fp16"),
])
def test_forward_size_limits(path, M, N, K, xdt):
    say(f"size limits path={path} M={M} N={N} K={K}")
    seed = 4000 + M + K
    x = synth.make_x(seed, 0, 0, M, K, xdt)
    g = synth.make_gain(seed, 0, 0, K, xdt)
    W = synth.make_w(seed, 0, 0, N, K)
    (o_packed, o_beta, o_Wq), (d_packed, d_beta) = check_pack(W)
    y, x_dev, g_dev = run_forward(x, g, d_packed, d_beta, N, xdt, path=path)
    ref = oracle.forward(synth.widen(x), synth.widen(g), o_Wq, o_beta)
    xq_gpu, s_gpu, _ = gpu_act_quant(x_dev, g_dev)
    check_xq(xq_gpu, s_gpu, ref)
    check_y(y, ref, xdt, Wq=o_Wq, beta=o_beta, xq_gpu=xq_gpu, s_gpu=s_gpu)


@pytest.mark.parametrize("path", [tw.BL_PATH_SKINNY, tw.BL_PATH_MFMA])
def test_gemm_i32_largest_k(path):
    """K = 65536: |acc| up to 128 * 65536, and the skinny kernel's weight
    registers are refilled 8 times per wave."""
    say(f"gemm_i32 K=65536 path={path}")
    M, N, K = 5, 64, 65536
    xq = _random_codes(M, K, 99)
    r = np.random.default_rng(100)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    Wq[0] = 1
    Wq[1] = -1
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc, path=path)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), oracle.contract(xq, Wq))


@pytest.mark.parametrize("ydt,M,N,K", [("bf16", 2000, 11264, 2048), ("fp16", 2000, 11264, 2048),
                                        ("bf16", 4000, 11264, 2048), ("fp16", 4000, 11264, 2048),
                                        ("bf16", 3000, 2048, 5632), ("fp16", 3000, 2048, 2048)])
def test_long_launch_epilogue_bitwise(ydt, M, N, K):
    """Long launches of the MFMA kernel: 2000 x 11264 x 2048 (1408 tiles of
    128 x 128, 16 k-blocks each: output tiles staged through LDS), 4000 x
    11264 x 2048 (1408 tiles of 128 x 256, waves of 4 packed tiles, stored
    directly) and 3000 x 2048 (512 tiles of 96 x 128; at K = 5632 staged,
    at K = 2048 stored directly), each with a ragged last tile row.  Every
    output element must equal the exact int32 contraction rescaled by
    fl32(beta / s) in fp32 and rounded to the output dtype -- the epilogue's
    arithmetic, done on the host from the int32 result -- and sampled rows
    must match the oracle."""
    say(f"long-launch epilogue M={M} N={N} K={K} y={ydt}")
    xq = _random_codes(M, K, 11)
    r = np.random.default_rng(12)
    Wq = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed = torch.from_numpy(oracle.pack(Wq)).to(DEV)
    beta = torch.tensor([0.0173], dtype=torch.float32, device=DEV)
    s = torch.from_numpy(r.uniform(0.5, 40.0, size=M).astype(np.float32)).to(DEV)
    d_xq = torch.from_numpy(xq).to(DEV)
    d_rs = torch.from_numpy(xq.astype(np.int64).sum(1).astype(np.int32)).to(DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitlinear_gemm_i32(d_xq, d_rs, packed, N, acc, path=tw.BL_PATH_MFMA)
    y = torch.empty((M, N), dtype=synth.DTYPES[ydt], device=DEV)
    tw.bitlinear_contract(d_xq, s, d_rs, packed, beta, N, y, path=tw.BL_PATH_MFMA)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, 9).round().astype(int))
    np.testing.assert_array_equal(acc.cpu().numpy()[rows], oracle.contract(xq[rows], Wq))
    scale = (beta.cpu() / s.cpu()).to(torch.float32)          # fp32, correctly rounded
    want = (acc.cpu().to(torch.float32) * scale[:, None]).to(y.dtype)
    assert torch.equal(y.cpu().view(torch.int16), want.view(torch.int16))
