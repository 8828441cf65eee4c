"""Pins of the oracle's routing steps: top-k with softmax weights, packing per expert, the combine of
expert outputs and the row gather (qwen4exp_gpu_gate.rs page, the device-router arm; kernel_check.rs
page, f16g grouped GEMM section).

The checks do not retype the oracle: hand-worked examples (tests/golden/route_*_example.txt), the
closed forms of the softmax (equal logits, two experts = the logistic function, ln-integer logits =
fractions, shift invariance, sums), Python's own sort as an independent ranking, invariants that fix
a stable packing uniquely, the combine as a sparse matrix product done by numpy, and the input
generator's independent table builder."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from conftest import GOLDEN

import workloads


def _logit(tok):
    if tok.startswith("ln"):
        return np.float32(math.log(int(tok[2:])))
    return np.float32(float(tok))


def _frac(tok):
    return float("nan") if tok == "nan" else float(Fraction(tok))


def read_golden_pipe(name):
    """Rows of '|'-separated field groups from tests/golden/<name>, comments stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([part.split() for part in line.split("|")])
    return rows


@pytest.mark.parametrize("normalize", [False, True])
def test_worked_example(orc, normalize):
    rows = read_golden_pipe("route_topk_example.txt")
    logits = np.array([[_logit(t) for t in r[0]] for r in rows], dtype=np.float32)
    ids, w = orc.route_topk(logits, 3, normalize=normalize)
    for i, r in enumerate(rows):
        assert ids[i].tolist() == [int(v) for v in r[1]], f"row {i}"
        want = np.array([_frac(v) for v in r[3 if normalize else 2]])
        # the ln<c> logits carry an f32 rounding of at most 2^-24 |ln c|, so exp(logit) = c (1 + d)
        # with |d| < 2^-24 * ln(5) + tiny; the fractions hold to a relative 4e-7
        np.testing.assert_allclose(w[i], want, rtol=4e-7, atol=0, equal_nan=True, err_msg=f"row {i}")


def _python_rank(l):
    """Expert order by an independent route: Python's sort on (NaN last, larger first, lower id)."""
    return sorted(range(len(l)), key=lambda e: (math.isnan(l[e]), 0.0 if math.isnan(l[e]) else -float(l[e]), e))


@pytest.mark.parametrize("E,k,levels", [(8, 3, None), (16, 16, 3), (64, 8, 4), (256, 8, None), (33, 5, 2)])
def test_selection_matches_a_sort(orc, E, k, levels):
    rng = np.random.default_rng(E * 100 + k)
    T = 60
    if levels is None:
        l = rng.standard_normal((T, E)).astype(np.float32)
    else:                                    # few distinct values: ties everywhere, also at the cut
        l = rng.integers(0, levels, size=(T, E)).astype(np.float32) - 1.0
    l[0, :] = 0.0
    l[1, ::2] = -0.0                         # +0 and -0 are equal
    l[2, : E // 2] = np.nan
    ids, _ = orc.route_topk(l, k)
    for t in range(T):
        assert ids[t].tolist() == _python_rank(l[t].tolist())[:k], f"token {t}"


def test_softmax_closed_forms(orc):
    # equal logits: every expert 1/E, renormalized 1/k
    l = np.full((1, 10), 0.3, dtype=np.float32)
    _, w = orc.route_topk(l, 4)
    np.testing.assert_allclose(w, 0.1, rtol=1e-15)
    _, wn = orc.route_topk(l, 4, normalize=True)
    np.testing.assert_allclose(wn, 0.25, rtol=1e-15)
    # two experts: the logistic function of the difference
    for a, b in [(1.0, 0.0), (0.25, -3.5), (10.0, 9.0)]:
        _, w = orc.route_topk(np.array([[a, b]], dtype=np.float32), 2)
        assert w[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-15)
        assert w[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(a - b)), rel=1e-15)
    # huge logits do not overflow: the maximum is taken out first
    _, w = orc.route_topk(np.array([[1000.0, 999.0]], dtype=np.float32), 1)
    assert w[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def test_softmax_sums_and_shift(orc):
    rng = np.random.default_rng(7)
    # logits on a 2^-10 grid inside (-16, 16): adding 4 to them is exact in f32
    l = (np.round(np.clip(rng.standard_normal((20, 32)) * 3, -15, 15) * 1024) / 1024).astype(np.float32)
    ids, w = orc.route_topk(l, 32)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)   # best first means non-increasing weights
    # a shift of every logit leaves the softmax unchanged
    _, w2 = orc.route_topk(l + np.float32(4.0), 32)
    np.testing.assert_allclose(w2, w, rtol=1e-13)
    # the renormalized weights of a top-k are the softmax weights over the selection
    ids8, w8 = orc.route_topk(l, 8)
    _, wn8 = orc.route_topk(l, 8, normalize=True)
    np.testing.assert_allclose(wn8, w8 / w8.sum(axis=1, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(wn8.sum(axis=1), 1.0, rtol=1e-14)
    assert np.array_equal(ids8, ids[:, :8])


def test_underflow_battery(orc):
    # probabilities far below f32's range still order by logit and keep their f64 values
    l = np.array([[-400.0, 0.0, -200.0, -800.0, -0.5]], dtype=np.float32)
    ids, w = orc.route_topk(l, 5)
    assert ids[0].tolist() == [1, 4, 2, 0, 3]
    s = 1.0 + math.exp(-0.5) + math.exp(-200.0) + math.exp(-400.0)
    assert w[0, 2] == pytest.approx(math.exp(-200.0) / s, rel=1e-13)
    assert w[0, 3] == pytest.approx(math.exp(-400.0) / s, rel=1e-13)
    assert w[0, 3] > 0 and w[0, 4] == 0.0    # exp(-800) underflows f64 as well


def test_nan_and_infinite_rows(orc):
    l = np.array([[1.0, np.nan, 2.0, 0.0],
                  [-np.inf] * 4,
                  [np.inf, 1.0, 2.0, 3.0]], dtype=np.float32)
    ids, w = orc.route_topk(l, 2)
    assert ids.tolist() == [[2, 0], [0, 1], [0, 3]]
    assert np.isnan(w).all()                 # NaN input, and inf - inf in the softmax


def _pack_rows():
    out = []
    for r in read_golden_pipe("route_pack_example.txt"):
        out.append([[int(v) for v in part] for part in r])
    return out


def test_pack_worked_example(orc):
    for ids, offsets, row_ids, pair_rows in _pack_rows():
        ids = np.array(ids, dtype=np.int32).reshape(4, 2)
        w = np.arange(8, dtype=np.float32).reshape(4, 2) + 0.5
        off, rid, pr, rw = orc.route_pack(ids, 4, w)
        assert off.tolist() == offsets
        assert rid.tolist() == row_ids
        assert pr.reshape(-1).tolist() == pair_rows
        for p in range(8):
            if pair_rows[p] >= 0:
                assert rw[pair_rows[p]] == w.reshape(-1)[p]


def check_pack_invariants(ids, E, off, rid, pr, w=None, rw=None):
    """The properties that fix a stable per-expert packing uniquely."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=E))]))
    prf = pr.reshape(-1)
    assert np.all(prf[~valid] == -1)
    assert np.array_equal(np.sort(prf[valid]), np.arange(int(off[-1])))     # a bijection onto rows
    pairs = np.flatnonzero(valid)
    assert np.array_equal(rid[prf[pairs]], pairs // k)                      # the row's token
    e_of_row = np.repeat(np.arange(E), np.diff(off))
    assert np.array_equal(e_of_row[prf[pairs]], flat[pairs])                # the row's expert
    for e in range(E):                                                      # ascending (t, j)
        seg = np.sort(pairs[flat[pairs] == e])
        assert np.array_equal(prf[seg], np.arange(off[e], off[e + 1]))
    if rw is not None:
        assert np.array_equal(rw[prf[pairs]], w.reshape(-1)[pairs])


@pytest.mark.parametrize("T,k,E,bad", [(50, 8, 16, False), (7, 3, 64, True), (300, 2, 5, True),
                                       (1, 1, 1, False)])
def test_pack_invariants(orc, T, k, E, bad):
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(-2 if bad else 0, E + (2 if bad else 0), size=(T, k)).astype(np.int32)
    w = rng.uniform(0, 1, size=(T, k)).astype(np.float32)
    off, rid, pr, rw = orc.route_pack(ids, E, w)
    check_pack_invariants(ids, E, off, rid, pr, w, rw)


def test_pack_of_topk_matches_the_input_generator(orc):
    # the generator's own tables (a separate numpy implementation) for the decode-sized router and
    # a tie-heavy one
    rng = np.random.default_rng(3)
    for logits in (rng.standard_normal((512, 256)).astype(np.float32),
                   rng.integers(0, 3, size=(200, 40)).astype(np.float32)):
        row_ids, offsets = workloads.route_topk(logits, 8)
        ids, _ = orc.route_topk(logits, 8)
        off, rid, _, _ = orc.route_pack(ids, logits.shape[1])
        assert np.array_equal(off, offsets) and np.array_equal(rid, row_ids)


def test_combine_is_a_sparse_product(orc):
    rng = np.random.default_rng(9)
    T, k, R, n = 12, 3, 30, 17
    pr = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    w = rng.standard_normal((T, k)).astype(np.float32)
    y = rng.standard_normal((R, n)).astype(np.float32)
    S = np.zeros((T, R))
    A = np.zeros((T, R))
    for t in range(T):
        for j in range(k):
            if pr[t, j] >= 0:
                S[t, pr[t, j]] += float(w[t, j])
                A[t, pr[t, j]] += abs(float(w[t, j]))
    out, absout = orc.combine(y, pr, w)
    np.testing.assert_allclose(out, S @ y.astype(np.float64), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(absout, A @ np.abs(y.astype(np.float64)), rtol=1e-12, atol=1e-12)
    C = np.zeros((T, R))                               # no weights: plain sums
    for t in range(T):
        for j in range(k):
            if pr[t, j] >= 0:
                C[t, pr[t, j]] += 1.0
    out1, _ = orc.combine(y, pr)
    np.testing.assert_allclose(out1, C @ y.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_combine_bad_row_is_nan(orc):
    y = np.ones((4, 3), dtype=np.float32)
    pr = np.array([[0, 1], [4, 0], [-1, -1]], dtype=np.int32)
    out, _ = orc.combine(y, pr)
    assert out[0].tolist() == [2.0, 2.0, 2.0]
    assert np.isnan(out[1]).all()
    assert out[2].tolist() == [0.0, 0.0, 0.0]


def test_gather_rows(orc):
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(9, 256), dtype=np.uint8)
    scales = rng.uniform(0.1, 1, size=(9, 2)).astype(np.float32)
    row_ids = np.array([3, 3, 0, 8, -1, 9, 5], dtype=np.int32)
    oc, osc = orc.gather_rows(codes, scales, row_ids)
    ok = (row_ids >= 0) & (row_ids < 9)
    assert np.array_equal(oc[ok], codes[row_ids[ok]])
    assert np.array_equal(osc[ok], scales[row_ids[ok]])
    assert (oc[~ok] == 0).all() and np.isnan(osc[~ok]).all()
