"""Pins of the oracle's bf16-dequant rung (dsv4_native_gemm_gate.rs page, comparison 3: activations
converted to bf16, weights dequantized to bf16, a bf16 GEMM; the class shift of the native path
against it, predicted as (u_q / sqrt 3) ||x (.) w||_2 per output).

Independent references: torch's own f32 -> bf16 conversion, the f64 dequantization of the weights
(pinned elsewhere), numpy's f64 matmul, and the closed form of the prediction; the prediction's
meaning (the RMS shift caused by act-quant rounding) is checked against the measured shift of the
oracle's own quantized GEMM against the unquantized product."""
import math

import numpy as np
import pytest
import torch

import workloads

NV, MX = workloads.NVFP4, workloads.MXFP4


def torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_cvt_bf16_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(50000) * 1e-39).astype(np.float32),                 # subnormals
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.01171875, -1.00390625, 3.389e38, 3.4e38,
                  -3.4e38, np.inf, -np.inf, 1.1754944e-38, 9.2e-41], dtype=np.float32),
    ])
    # every bf16 tie: the midpoint between two neighbouring bf16 values
    hi = rng.integers(0, 0x7F7F, 5000).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    assert np.array_equal(orc.cvt_bf16(x), torch_bf16_bits(x))
    nan = orc.cvt_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.isnan(orc.bf16_value(nan)).all()


def test_cvt_bf16_is_exact_on_bf16_values_and_within_half_ulp(orc):
    rng = np.random.default_rng(2)
    b = rng.integers(0, 0x7F80, 10000).astype(np.uint16)          # finite positive bf16 patterns
    v = orc.bf16_value(b).astype(np.float32)
    assert np.array_equal(orc.cvt_bf16(v), b)
    x = (rng.standard_normal(10000) * 100).astype(np.float32)
    err = np.abs(orc.bf16_value(orc.cvt_bf16(x)) - x.astype(np.float64))
    assert np.all(err <= 2.0 ** -8 * np.abs(x.astype(np.float64)))     # half of 2^-7 relative


@pytest.mark.parametrize("kind,scale2", [(NV, 2.0 ** -6), (NV, 1.0), (MX, 0.0)])
def test_dequant_bf16_is_exact_for_pow2_scales(orc, kind, scale2):
    # E2M1 x E4M3 x 2^j (or x E8M0) has at most 5 significant bits: exact in bf16
    rng = np.random.default_rng(3)
    n, k = 48, 256
    w = workloads.random_nibbles(rng, n, k)
    s = workloads.random_scale_codes(rng, kind, n, k)
    got = orc.bf16_value(orc.dequant_bf16(w, s, scale2, kind))
    assert np.array_equal(got, orc.dequant_weights(w, s, scale2, kind))


def test_dequant_bf16_rounds_the_f32_product(orc):
    # non-power-of-two scale2: the f32 product E2M1 x f32(E4M3 x scale2), rounded by torch
    rng = np.random.default_rng(4)
    n, k = 32, 256
    w = workloads.random_nibbles(rng, n, k)
    s = workloads.random_scale_codes(rng, NV, n, k)
    scale2 = np.float32(0.37)
    wd = orc.dequant_weights(w, s, scale2, NV)             # f64 of E2M1 x f32(ws): exact products
    f32_product = wd.astype(np.float32)                     # the f32 multiply: one rounding of it
    assert np.array_equal(orc.dequant_bf16(w, s, scale2, NV), torch_bf16_bits(f32_product))


def test_gemm_bf16_matches_numpy(orc):
    rng = np.random.default_rng(5)
    a = orc.cvt_bf16((rng.standard_normal((7, 96)) * 2).astype(np.float32))
    w = orc.cvt_bf16((rng.standard_normal((11, 96)) * 0.5).astype(np.float32))
    out, absout = orc.gemm_bf16(a, w)
    A, W = orc.bf16_value(a), orc.bf16_value(w)
    np.testing.assert_allclose(out, A @ W.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(absout, np.abs(A) @ np.abs(W).T, rtol=1e-13)


def test_prediction_closed_form(orc):
    x = np.array([[1.0, 2.0]], dtype=np.float32)
    wd = np.array([[3.0, 4.0], [0.0, -1.0]])
    pred = orc.class_shift_prediction(x, wd)
    assert pred[0, 0] == pytest.approx(2.0 ** -4 / math.sqrt(3.0) * math.sqrt(73.0), rel=1e-15)
    assert pred[0, 1] == pytest.approx(2.0 ** -4 / math.sqrt(3.0) * 2.0, rel=1e-15)


@pytest.mark.parametrize("name", ["config0", "config1", "config2"])
def test_prediction_measures_the_act_quant_shift(orc, name):
    # the quantized GEMM (f64) against the unquantized product on the same dequantized weights: the
    # shift comes from act-quant rounding alone; relative E4M3 rounding errors are at most U_FP8 and
    # smaller on average than the uniform model, so |shift| / prediction has a median near 0.5
    wl = {"config0": workloads.config0, "config1": lambda: workloads.config1(8), "config2": workloads.config2}[name]()
    e = wl.expert
    codes, scales = orc.act_quant(wl.x)
    native = orc.expert_gemm(codes, scales, e.w, e.s, e.scale2, e.kind)[0]
    wd = orc.dequant_weights(e.w, e.s, e.scale2, e.kind)
    shift = np.abs(native - wl.x.astype(np.float64) @ wd.T)
    ratio = shift / orc.class_shift_prediction(wl.x, wd)
    assert 0.4 < np.median(ratio) < 0.6
    assert np.quantile(ratio, 0.99) < 3.0
