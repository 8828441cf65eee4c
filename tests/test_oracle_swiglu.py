"""Pins of the oracle's expert activation (swiglu with limit), the step between the gate/up and the
down projection: memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, the swiglu_limit saturation
cell (clamp math: the up projection clamped on both sides, the gate from above only, both before
silu; silu(t) = t / (1 + exp(-t))).  The checks use closed forms of the logistic function, the
clamp boundaries and the algebraic structure (linearity in the up value and the row weight), not a
second copy of the formula."""
import math

import numpy as np
import pytest

LIMIT = 7.0


def one(orc, g, u, limit=LIMIT, w=None):
    gu = np.array([[g, u]], dtype=np.float32)
    weights = None if w is None else np.array([w], dtype=np.float32)
    return float(orc.swiglu(gu, 1, limit, weights)[0, 0])


def test_logistic_closed_forms(orc):
    # sigma(0) = 1/2, so silu(0) = 0 for any up value
    assert one(orc, 0.0, 5.0) == 0.0
    # sigma(1) = 1 / (1 + 1/e) = 0.7310585786300049 (textbook value)
    assert one(orc, 1.0, 1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    # sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4; the gate is the f32 value of ln 3
    g = float(np.float32(math.log(3.0)))
    assert one(orc, g, 2.0) == pytest.approx(2.0 * 0.75 * g, rel=1e-7)
    assert one(orc, -g, 2.0) == pytest.approx(2.0 * 0.25 * -g, rel=1e-7)
    # large positive gate: silu(t) = t (1 - e^-t + ...)
    e = math.exp(-6.5)
    assert one(orc, 6.5, 1.0) == pytest.approx(6.5 * (1.0 - e + e * e - e ** 3), rel=1e-10)


def test_gate_clamped_from_above_only(orc):
    # above the limit the gate is the limit: h = limit * sigma(limit) * u
    sig7 = 1.0 / (1.0 + math.exp(-7.0))
    assert one(orc, 100.0, 1.0) == pytest.approx(7.0 * sig7, rel=1e-15)
    assert one(orc, 7.0, 1.0) == one(orc, 1e30, 1.0)
    # a very negative gate is not clamped to -limit: silu(-100) ~ -100 e^-100, not -7 sigma(-7)
    h = one(orc, -100.0, 1.0)
    assert h < 0 and abs(h) < 1e-40
    assert one(orc, -7.5, 1.0) == pytest.approx(-7.5 / (1.0 + math.exp(7.5)), rel=1e-12)


def test_up_clamped_on_both_sides(orc):
    base = one(orc, 1.0, 1.0)
    assert one(orc, 1.0, 50.0) == pytest.approx(7.0 * base, rel=1e-15)
    assert one(orc, 1.0, -50.0) == pytest.approx(-7.0 * base, rel=1e-15)
    assert one(orc, 1.0, 7.0) == one(orc, 1.0, 7.5)
    # inside the limits the result is linear in the up value and odd in it
    assert one(orc, 1.0, 3.0) == pytest.approx(3.0 * base, rel=1e-15)
    assert one(orc, 1.0, -3.0) == -one(orc, 1.0, 3.0)


def test_limit_changes_both_clamps(orc):
    # with limit 2, gate 3 -> 2 and up -5 -> -2
    sig2 = 1.0 / (1.0 + math.exp(-2.0))
    assert one(orc, 3.0, -5.0, limit=2.0) == pytest.approx(2.0 * sig2 * -2.0, rel=1e-15)


def test_row_weight_is_a_row_scalar(orc):
    rng = np.random.default_rng(11)
    gu = (rng.standard_normal((5, 2 * 256)) * 4).astype(np.float32)
    w = np.array([0.5, 2.0, 0.0, -1.0, 0.125], dtype=np.float32)
    h1 = orc.swiglu(gu, 256, LIMIT)
    hw = orc.swiglu(gu, 256, LIMIT, w)
    np.testing.assert_allclose(hw, h1 * w[:, None].astype(np.float64), rtol=1e-15, atol=0)


def test_gate_and_up_column_halves(orc):
    # row layout [gate_0 .. gate_{I-1}, up_0 .. up_{I-1}]: each output pairs gate i with up i
    inter = 128
    gu = np.zeros((2, 2 * inter), dtype=np.float32)
    gu[0, :inter] = 1.0                       # gate 1 everywhere
    gu[0, inter:] = np.arange(inter) / 64.0   # up = i/64
    gu[1, :inter] = np.arange(inter) / 16.0   # gate = i/16 (crosses the limit at i = 112)
    gu[1, inter:] = 1.0
    h = orc.swiglu(gu, inter, LIMIT)
    base = one(orc, 1.0, 1.0)
    np.testing.assert_allclose(h[0], base * np.arange(inter) / 64.0, rtol=1e-15, atol=0)
    g = np.minimum(np.arange(inter) / 16.0, LIMIT)
    assert h[1, 0] == 0.0
    assert np.all(np.diff(h[1]) >= 0)         # silu is increasing for t >= 0
    assert np.all(h[1, 112:] == h[1, 112])    # saturated from the limit on
    assert h[1, 64] == pytest.approx(one(orc, float(g[64]), 1.0), rel=1e-15)


def test_saturation_cell_engages_both_clamps(orc):
    # the pages' cell: a row scaled x50 drives gate/up outputs past the limit on both sides
    rng = np.random.default_rng(5)
    gu = (rng.standard_normal((1, 2 * 512)) * 50).astype(np.float32)
    h = orc.swiglu(gu, 512, LIMIT)
    gate, up = gu[0, :512], gu[0, 512:]
    assert np.sum(gate > LIMIT) > 0 and np.sum(np.abs(up) > LIMIT) > 0
    sig7 = 1.0 / (1.0 + math.exp(-7.0))
    both = (gate > LIMIT) & (np.abs(up) > LIMIT)
    assert np.any(both)
    expect = 7.0 * sig7 * 7.0 * np.sign(up[both]).astype(np.float64)
    np.testing.assert_allclose(h[0, both], expect, rtol=1e-15)
    assert np.max(np.abs(h)) <= 7.0 * sig7 * 7.0 * (1 + 1e-15)
