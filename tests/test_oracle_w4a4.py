"""Pins of the oracle's W4A4 NVFP4 variant (kernel_check.rs page, the NVFP4 MMQ W4A4 arms: E2M1
activations with a per-token row scale and a UE4M3 micro-scale per 16-element sub-block; the
sub-block-only quantizer it replaced; the DYNAMIC-RANGE and RESIDUAL-CHANNEL arms).

Independent checks: a brute-force nearest-grid-point search for the E2M1 encoder, exact round trips
of representable rows, the per-element error bound of the quantizer, numpy's f64 matmul for the
GEMM, and the pages' own two hard comparisons (the row scale beats sub-block-only scaling on
decade-spread tokens; keeping the 8 injected outlier channels beats keeping none) plus their
informational band (max-normalized relative error below 0.2 on 0.1-scale activations)."""
import numpy as np
import pytest

import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_e2m1(v):
    a = min(abs(float(v)), 6.0)
    d = np.abs(GRID - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return code | (8 if np.signbit(np.float32(v)) else 0)


def test_e2m1_encode_is_the_nearest_grid_point(orc):
    mids = (GRID[:-1] + GRID[1:]) / 2
    vals = np.concatenate([GRID, mids, mids + 1e-6, mids - 1e-6, np.linspace(-8, 8, 4001), [6.5, 100.0, -0.0]])
    vals = vals.astype(np.float32)
    got = orc.e2m1_encode(vals)
    assert [int(c) for c in got] == [brute_e2m1(v) for v in vals]


def test_representable_rows_round_trip(orc):
    # sub-block g < 7 holds E2M1 values times 2^(g-3) with amax 6 * 2^(g-3) (micro 2^(g-3)); the last
    # holds E2M1 values times 448 with amax 2688, so rs = 2688 / 2688 = 1 and its micro is 448
    rng = np.random.default_rng(1)
    k = 128
    x = np.zeros((3, k), dtype=np.float32)
    for g in range(k // 16):
        vals = GRID[rng.integers(0, 8, 16)] * np.where(rng.random(16) < 0.5, -1, 1)
        vals[0] = 6.0
        x[:, 16 * g:16 * g + 16] = vals * (448.0 if g == k // 16 - 1 else 2.0 ** (g - 3))
    x[1] *= 2.0 ** 20                      # any power-of-two row scale: rs = 2^20, same codes
    x[2] *= 2.0 ** -30
    codes, micro, rs = orc.act_quant_fp4(x)
    assert rs.tolist() == [1.0, 2.0 ** 20, 2.0 ** -30]
    assert np.array_equal(codes[0], codes[1]) and np.array_equal(codes[0], codes[2])
    assert micro[0, -1] == 0x7E and micro[0, 3] == 0x38     # 448 and 2^0
    np.testing.assert_array_equal(orc.dequant_acts_fp4(codes, micro, rs), x.astype(np.float64))


@pytest.mark.parametrize("two_level", [True, False])
def test_quantizer_error_bound(orc, two_level):
    # per element: |deq - x| <= amax_sub * (1/6 + 1/12): half the widest E2M1 gap (1 of a scale of
    # amax_sub/6) plus the micro-scale's E4M3 rounding (at most 1/16 relative) at the cap of 6
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-3, 3, (40, 1)))).astype(np.float32)
    codes, micro, rs = orc.act_quant_fp4(x, two_level)
    d = orc.dequant_acts_fp4(codes, micro, rs)
    asub = np.abs(x.astype(np.float64)).reshape(40, 16, 16).max(axis=2).repeat(16, axis=1)
    assert np.all(np.abs(d - x) <= asub * (1 / 6 + 1 / 12))
    if two_level:
        assert np.all(micro.max(axis=1) == 0x7E)    # the loudest sub-block of each row gets 448


def test_subblock_only_clamps_where_the_row_scale_does_not(orc):
    x = np.full((2, 32), 1e-5, dtype=np.float32)
    x[1] *= 1e8                                      # 1e3: amax/6 = 167, inside UE4M3
    _, micro1, _ = orc.act_quant_fp4(x, two_level=False)
    _, micro2, rs2 = orc.act_quant_fp4(x, two_level=True)
    assert micro1[0, 0] == 0x01                      # wants 1.7e-6 < 2^-9: clamped to the smallest
    assert micro2[0, 0] == 0x7E and micro2[1, 0] == 0x7E
    assert rs2[0] == pytest.approx(1e-5 / 2688, rel=1e-6)


def test_w4a4_gemm_matches_numpy(orc):
    x, ex = workloads.w4a4_case(3, 9, 40, 256, "res")
    codes, micro, rs = orc.act_quant_fp4(x)
    out, absout = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2)
    A = orc.dequant_acts_fp4(codes, micro, rs)
    W = orc.dequant_weights(ex.w, ex.s, ex.scale2, workloads.NVFP4)
    np.testing.assert_allclose(out, A @ W.T, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(absout, np.abs(A) @ np.abs(W).T, rtol=1e-12)
    idx = np.array(workloads.w4a4_hot_channels(256), dtype=np.int32)
    out2, _ = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2, x, idx)
    np.testing.assert_allclose(out2 - out, x[:, idx].astype(np.float64) @ W[:, idx].T, rtol=1e-9, atol=1e-300)


def rel_max(y, ref):
    return np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-3)


def per_token_rel(y, ref):
    s = np.abs(ref).max(axis=1)
    return float(np.max(np.where(s > 0, np.abs(y - ref).max(axis=1) / np.where(s > 0, s, 1), 0.0)))


def exact_product(orc, x, ex):
    """The unquantized product on the dequantized weights (what the pages' rel is measured against)."""
    return x.astype(np.float64) @ orc.dequant_weights(ex.w, ex.s, ex.scale2, workloads.NVFP4).T


@pytest.mark.parametrize("T", [16, 64])
def test_informational_band(orc, T):
    x, ex = workloads.w4a4_case(4, T, 256, 1024, "uniform")
    ref = exact_product(orc, x, ex)
    codes, micro, rs = orc.act_quant_fp4(x)
    y, _ = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2)
    assert rel_max(y, ref) < 0.2


@pytest.mark.parametrize("T", [16, 128])
def test_dynamic_range_gate(orc, T):
    x, ex = workloads.w4a4_case(5, T, 256, 1024, "dyn")
    ref = exact_product(orc, x, ex)
    rels = []
    for two_level in (True, False):
        codes, micro, rs = orc.act_quant_fp4(x, two_level)
        y, _ = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2)
        rels.append(per_token_rel(y, ref))
    assert rels[0] < rels[1], rels


def test_residual_channel_gate(orc):
    k = 1024
    x, ex = workloads.w4a4_case(6, 128, 256, k, "res")
    ref = exact_product(orc, x, ex)
    hot = sorted(workloads.w4a4_hot_channels(k))
    rels = {}
    for k_res in (0, 4, 8, 16):
        idx = orc.loud_channels(x, k_res)
        if k_res == 8:
            assert sorted(idx.tolist()) == hot
        xq = x.copy()
        xq[:, idx] = 0.0
        codes, micro, rs = orc.act_quant_fp4(xq)
        y, _ = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2, x, idx)
        rels[k_res] = per_token_rel(y, ref)
    assert rels[8] < rels[0] and rels[16] < rels[0], rels
