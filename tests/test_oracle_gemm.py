"""Pins of the oracle's quantized GEMM (f64 route): exact rational brute force with independent
decoders, a textbook special case, the dequantize-then-dense route, the grouped form, and the
exact-by-construction inputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from conftest import read_golden

NV, MX = workloads.NVFP4, workloads.MXFP4
E4M3_TORCH = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E8M0_TORCH = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
E2M1_GOLD = np.array([float(v) for _, v in read_golden("e2m1_grid.txt")])


def brute_force(a_codes, a_scales, w, s, scale2, kind):
    """Exact rational sum with torch/golden decoders and numpy unpacking (shares nothing with the
    oracle's C code)."""
    g, k = a_codes.shape
    n = w.shape[0]
    gs = 16 if kind == NV else 32
    lo, hi = w & 0x0F, w >> 4
    nib = np.stack([lo, hi], axis=2).reshape(n, k)                 # even k low nibble
    wv = E2M1_GOLD[nib]
    if kind == NV:
        ws = (E4M3_TORCH[s].astype(np.float32) * np.float32(scale2)).astype(np.float32)
    else:
        ws = E8M0_TORCH[s].astype(np.float32)
    ws_full = np.repeat(ws, gs, axis=1)                               # [n, k]
    as_full = np.repeat(a_scales, 128, axis=1)                        # [g, k]
    av = E4M3_TORCH[a_codes]
    out = np.empty((g, n), dtype=object)
    absp = np.empty((g, n), dtype=object)
    for r in range(g):
        for c in range(n):
            acc = Fraction(0)
            aab = Fraction(0)
            for kk in range(k):
                p = (Fraction(float(av[r, kk])) * Fraction(float(wv[c, kk]))
                     * Fraction(float(ws_full[c, kk])) * Fraction(float(as_full[r, kk])))
                acc += p
                aab += abs(p)
            out[r, c] = acc
            absp[r, c] = aab
    return out, absp


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_exact_rational(orc, kind, seed):
    rng = np.random.default_rng(seed)
    g, n, k = 2, 3, 256
    x = (rng.standard_normal((g, k)) * np.array([[1.0], [300.0]])).astype(np.float32)
    x[:, 128:] *= np.float32(0.01)                                   # distinct act scale per block
    a_codes, a_scales = orc.act_quant(x)
    ex = workloads.single_random(seed, 1, n, k, kind).expert
    scale2 = 0.37 if kind == NV else 0.0                             # non-power-of-two scale2
    ref, absp = orc.expert_gemm(a_codes, a_scales, ex.w, ex.s, scale2, kind, threads=1)
    exact, eabs = brute_force(a_codes, a_scales, ex.w, ex.s, scale2, kind)
    for r in range(g):
        for c in range(n):
            assert abs(Fraction(ref[r, c]) - exact[r, c]) <= Fraction((k - 1) * 2.0 ** -53) * eabs[r, c]
            assert abs(Fraction(absp[r, c]) - eabs[r, c]) <= Fraction((k - 1) * 2.0 ** -53) * eabs[r, c]


@pytest.mark.parametrize("kind", [NV, MX])
def test_textbook_special_case(orc, kind):
    # every weight scale 1, activation scales 1, exactly one nonzero weight (value 1.0, nibble 2)
    # per column at a position p[c]: out[r, c] is the decoded activation at p[c].
    rng = np.random.default_rng(5)
    g, n, k = 3, 5, 384
    a_codes = rng.integers(0, 256, size=(g, k), dtype=np.uint8)
    a_codes[(a_codes & 0x7F) == 0x7F] = 0x38
    a_scales = np.ones((g, k // 128), dtype=np.float32)
    pos = rng.choice(k, size=n, replace=False)
    nib = np.zeros((n, k), dtype=np.uint8)
    nib[np.arange(n), pos] = 2
    w = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    gs = 16 if kind == NV else 32
    s = np.full((n, k // gs), 0x38 if kind == NV else 127, dtype=np.uint8)
    ref, _ = orc.expert_gemm(a_codes, a_scales, w, s, 1.0, kind)
    assert np.array_equal(ref, E4M3_TORCH[a_codes[:, pos]])


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("g,n,k", [(4, 256, 512), (5, 200, 640), (1, 64, 2048)])
def test_dequant_dense_route_equivalence(orc, kind, g, n, k):
    wl = workloads.single_random(11 + g, g, n, k, kind, x_scale=3.0)
    a_codes, a_scales = orc.act_quant(wl.x)
    ex = wl.expert
    ref, absp = orc.expert_gemm(a_codes, a_scales, ex.w, ex.s, ex.scale2, kind)
    dense = orc.dense_route(a_codes, a_scales, ex.w, ex.s, ex.scale2, kind)
    assert np.all(np.abs(dense - ref) <= 2 * k * 2.0 ** -53 * absp)
    # a misplaced scale is an O(1) change: shifting the weight-scale plane by one group must break it
    s_bad = np.roll(ex.s, 1, axis=1)
    bad = orc.dense_route(a_codes, a_scales, ex.w, s_bad, ex.scale2, kind)
    assert np.max(np.abs(bad - ref) / (absp + 1e-300)) > 1e-3


def test_points_match_full(orc):
    wl = workloads.single_random(3, 6, 96, 384, NV)
    a_codes, a_scales = orc.act_quant(wl.x)
    ex = wl.expert
    ref, absp = orc.expert_gemm(a_codes, a_scales, ex.w, ex.s, ex.scale2, NV)
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, 6, 50), rng.integers(0, 96, 50)
    pr, pa = orc.expert_gemm_points(a_codes, a_scales, ex.w, ex.s, ex.scale2, NV, rows, cols)
    assert np.array_equal(pr, ref[rows, cols]) and np.array_equal(pa, absp[rows, cols])


def test_grouped_equals_per_expert(orc):
    kinds = [NV, MX, NV, NV, MX, NV]
    wl = workloads.grouped_random(1, T=24, E=6, top=2, n=80, k=256, kinds=kinds, empty_experts=(3,))
    assert wl.offsets[4] == wl.offsets[3]                          # expert 3 has no rows
    codes, scales = orc.act_quant(wl.x)
    pc, ps = codes[wl.row_ids], scales[wl.row_ids]
    ws = [wl.w_of(e) for e in range(wl.E)]
    ss = [wl.s_of(e) for e in range(wl.E)]
    ref, absp = orc.grouped_gemm(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n)
    for e in range(wl.E):
        lo, hi = wl.offsets[e], wl.offsets[e + 1]
        if hi == lo:
            continue
        r1, a1 = orc.expert_gemm(pc[lo:hi], ps[lo:hi], ws[e], ss[e], wl.scale2[e], wl.kinds[e])
        assert np.array_equal(ref[lo:hi], r1) and np.array_equal(absp[lo:hi], a1)
    rows = np.arange(wl.R)
    cols = (rows * 7) % wl.n
    pr, _ = orc.grouped_gemm_points(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n, rows, cols)
    assert np.array_equal(pr, ref[rows, cols])
    sub, _ = orc.grouped_gemm(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n, row0=5, row1=17)
    assert np.array_equal(sub, ref[5:17])


@pytest.mark.parametrize("kind", [NV, MX])
def test_exact_arm_is_exact_in_f32(orc, kind):
    a_codes, a_scales, ex = workloads.exact_arm(0, 3, 48, 7168, kind)
    ref, absp = orc.expert_gemm(a_codes, a_scales, ex.w, ex.s, ex.scale2, kind)
    assert np.all(absp < 2.0 ** 22)
    assert np.all(ref * 4 == np.round(ref * 4))                     # multiples of 1/4
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)


def test_bound_helpers(orc):
    assert orc.gemm_bound(np.array([1.0]), 7168)[0] == 7168 * 2.0 ** -24
    assert orc.pages_op_count(NV, 7168) == 15 + 4 + 7
    assert orc.pages_op_count(MX, 7168) == 31 + 2 + 7
