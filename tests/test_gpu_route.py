"""GPU parity of the routing steps: route_softmax_topk, route_pack, gather_quant_rows, moe_combine, and
the whole expert layer from router logits to the combined output (qwen4exp_gpu_gate.rs page, the
device-router arm; kernel_check.rs page, f16g grouped GEMM section).

Bars:
  * ids and their order, offsets, row_ids, pair_rows, moved weights and gathered rows: exact.
  * softmax weights: the GPU evaluates exp(x - m) in f32 (x - m rounded once, relative error of the
    argument <= 2^-24, so exp carries |x - m| 2^-24 more; the device expf adds about 2 ulp), sums the
    terms in a tree of depth D (D = ceil(E/64) + 7 over all experts, k + 1 over the selection) and
    divides once.  Hence, per weight w_i of expert i, with g_e = |l_e - m| and S the e-weighted
    mean of g over the summed experts:
        |w_gpu - w_f64| <= 2^-24 (g_i + S + D + 5) |w_f64| + 2^-126
    (the absolute floor covers results in f32's subnormal range).  NaN where the oracle has NaN.
  * combine: each output is a sum of top_k terms with one f32 rounding per fused multiply-add, so
        |out_gpu - out_f64| <= top_k 2^-24 sum_j |w_j y_j|."""
import functools
import math

import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import U32, check_bound, dev, first_byte_diff, require_gpu

pytestmark = pytest.mark.gpu
NV, MX = workloads.NVFP4, workloads.MXFP4


def weight_bound(logits, ids, ref, normalize):
    T, E = logits.shape
    k = ids.shape[1]
    l = logits.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.nanmax(np.where(np.isnan(l), -np.inf, l), axis=1, keepdims=True)
        g = np.abs(l - m)
        e = np.exp(l - m)
    with np.errstate(invalid="ignore"):
        eg = np.where(e > 0, e * g, 0.0)           # experts with e = 0 add nothing (g may be inf)
    if normalize:
        es, egs = np.take_along_axis(e, ids, axis=1), np.take_along_axis(eg, ids, axis=1)
        D = k + 1
    else:
        es, egs = e, eg
        D = math.ceil(E / 64) + 7
    with np.errstate(invalid="ignore", divide="ignore"):
        S = np.nansum(egs, axis=1, keepdims=True) / np.nansum(es, axis=1, keepdims=True)
        gi = np.take_along_axis(g, ids, axis=1)
        rel = np.where(ref != 0, U32 * (gi + S + D + 5) * np.abs(ref), 0.0)
    return rel + 2.0 ** -126


def check_topk(orc, logits, k, normalize, what):
    d = require_gpu()
    ids, w = fp4.route_softmax_topk(dev(logits, d), k, normalize=normalize)
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    rid, rw = orc.route_topk(logits, k, normalize=normalize)
    if not np.array_equal(ids, rid):
        t = int(np.flatnonzero((ids != rid).any(axis=1))[0])
        raise AssertionError(f"{what}: ids differ at token {t}: gpu {ids[t].tolist()} ref {rid[t].tolist()} "
                             f"logits {logits[t][np.union1d(ids[t], rid[t])].tolist()}")
    nan_ref = np.isnan(rw)
    assert np.array_equal(np.isnan(w), nan_ref), f"{what}: NaN pattern differs"
    bound = weight_bound(logits, rid, rw, normalize)
    err = np.abs(w - rw)
    bad = ~nan_ref & ~(err <= bound)
    if bad.any():
        t, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} weights outside the bound; first token {t} slot {j}: "
                             f"gpu {w[t, j]!r} ref {rw[t, j]!r} err {err[t, j]:.3e} bound {bound[t, j]:.3e}")
    return ids, w


@functools.lru_cache(maxsize=None)
def workload_logits(name):
    return {"config3": workloads.config3_logits, "config4": workloads.config4_logits}[name]()


@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("name", ["config3", "config4"])
def test_topk_workload_routers(orc, name, normalize):
    logits = workload_logits(name)
    ids, _ = check_topk(orc, logits, 8, normalize, name)
    # the same tables as the generator's: packing the device ids reproduces the GEMM inputs
    off, rid, _, _ = orc.route_pack(ids, logits.shape[1])
    row_ids, offsets = workloads.route_topk(logits, 8)
    assert np.array_equal(off, offsets) and np.array_equal(rid, row_ids)


@pytest.mark.parametrize("E", [1, 7, 63, 64, 65, 129, 256, 512, 1000, 1024])
@pytest.mark.parametrize("normalize", [False, True])
def test_topk_shapes(orc, E, normalize):
    rng = np.random.default_rng(E)
    logits = (rng.standard_normal((37, E)) * 3).astype(np.float32)
    for k in sorted({1, min(E, 8), min(E, 64)}):
        check_topk(orc, logits, k, normalize, f"E={E} k={k}")


def tie_battery(E, rng):
    rows = [
        np.zeros(E),                                            # all equal
        np.where(np.arange(E) % 2 == 0, 0.0, -0.0),             # +0 and -0 are equal
        rng.integers(0, 2, E).astype(np.float64),               # two levels: duplicates across the cut
        rng.integers(0, 4, E).astype(np.float64) - 2.0,         # four levels
        np.full(E, 1.5),
        -np.arange(E) * 200.0,                                  # underflowing probabilities
        -np.arange(E) * 0.01 - 100.0,                           # close values far from zero
        np.where(np.arange(E) == E // 2, 3e38, -3e38),          # the extremes of f32
        np.full(E, -np.inf),                                    # every logit -inf
        np.where(np.arange(E) < 3, 1.0, -np.inf),               # masked experts
        np.where(np.arange(E) == E - 1, np.inf, 0.0),           # +inf
        np.where(np.arange(E) % 5 == 1, np.nan, rng.standard_normal(E)),   # NaN
        np.full(E, np.nan),
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("E,k", [(8, 3), (64, 8), (256, 8), (300, 20), (1024, 64)])
@pytest.mark.parametrize("normalize", [False, True])
def test_topk_tie_battery(orc, E, k, normalize):
    logits = tie_battery(E, np.random.default_rng(E + k))
    check_topk(orc, logits, k, normalize, f"ties E={E} k={k}")


def test_topk_empty():
    d = require_gpu()
    ids, w = fp4.route_softmax_topk(torch.empty((0, 16), dtype=torch.float32, device=d), 4)
    assert ids.shape == (0, 4) and w.shape == (0, 4)


# ------------------------------------------------------------------------------------- packing

def check_pack(orc, ids, E, w=None, what=""):
    d = require_gpu()
    T, k = ids.shape
    off, rid, pr, rw = fp4.route_pack(dev(ids, d), E, None if w is None else dev(w, d))
    torch.cuda.synchronize()
    ro, rr, rp, rrw = orc.route_pack(ids, E, w)
    off = off.cpu().numpy()
    assert np.array_equal(off, ro), f"{what}: offsets differ"
    R = int(ro[-1])
    assert np.array_equal(rid.cpu().numpy()[:R], rr), f"{what}: row_ids differ"
    assert np.array_equal(pr.cpu().numpy(), rp), f"{what}: pair_rows differ"
    if w is not None:
        assert np.array_equal(rw.cpu().numpy()[:R], rrw), f"{what}: row weights differ"
    return off, rid, pr, rw


@pytest.mark.parametrize("name", ["config3", "config4"])
def test_pack_workload_routers(orc, name):
    logits = workload_logits(name)
    ids, w = orc.route_topk(logits, 8)
    check_pack(orc, ids, logits.shape[1], w.astype(np.float32), name)


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (63, 3, 5), (64, 8, 256), (65, 9, 256), (1000, 17, 64),
                                   (130, 33, 1024), (77, 64, 100), (4096, 8, 256)])
def test_pack_random(orc, T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)     # repeats and dropped ids
    w = rng.uniform(0, 1, size=(T, k)).astype(np.float32)
    check_pack(orc, ids, E, w, f"T={T} k={k} E={E}")
    check_pack(orc, ids, E, None, f"T={T} k={k} E={E} no weights")


def test_pack_empty_and_all_dropped(orc):
    d = require_gpu()
    off, _, _, _ = fp4.route_pack(torch.empty((0, 8), dtype=torch.int32, device=d), 16)
    assert off.cpu().numpy().tolist() == [0] * 17
    ids = np.full((70, 4), 99, dtype=np.int32)
    off, _, pr, _ = check_pack(orc, ids, 16, None, "all dropped")
    assert (pr.cpu().numpy() == -1).all()


# -------------------------------------------------------------------------------------- gather

def test_gather_rows(orc):
    d = require_gpu()
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 384)).astype(np.float32)
    codes, scales = fp4.act_quant_fp8(dev(x, d))
    row_ids = np.concatenate([rng.integers(0, 50, 200), [-1, 50, 49, 0]]).astype(np.int32)
    oc, osc = fp4.gather_quant_rows(codes, scales, dev(row_ids, d))
    rc, rs = orc.gather_rows(codes.cpu().numpy(), scales.cpu().numpy(), row_ids)
    assert np.array_equal(oc.cpu().numpy(), rc), first_byte_diff(oc.cpu().numpy(), rc)
    assert np.array_equal(osc.cpu().numpy(), rs, equal_nan=True)


# ------------------------------------------------------------------------------------- combine

def check_combine(orc, y, pr, w, what, y_dev=None, out=None):
    d = require_gpu()
    got = fp4.moe_combine(dev(y, d) if y_dev is None else y_dev, dev(pr, d), None if w is None else dev(w, d),
                          out=out).cpu().numpy()
    ref, absr = orc.combine(y, pr, w)
    bad_rows = np.isnan(ref).all(axis=1)
    assert np.isnan(got[bad_rows]).all(), f"{what}: rows with an out-of-range pair must be NaN"
    check_bound(got[~bad_rows], ref[~bad_rows], absr[~bad_rows], pr.shape[1], what)


@pytest.mark.parametrize("T,k,n", [(40, 8, 7168), (33, 3, 4096), (9, 2, 5), (17, 64, 1027), (1, 1, 1)])
@pytest.mark.parametrize("weighted", [False, True])
def test_combine(orc, T, k, n, weighted):
    rng = np.random.default_rng(T + k + n)
    ids = rng.integers(-1, 12, size=(T, k)).astype(np.int32)
    _, _, pr, _ = orc.route_pack(ids, 10)
    R = T * k
    y = (rng.standard_normal((R, n)) * 4).astype(np.float32)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32) if weighted else None
    check_combine(orc, y, pr, w, f"T={T} k={k} n={n} weighted={weighted}")


def test_combine_unaligned_and_bad_rows(orc):
    d = require_gpu()
    rng = np.random.default_rng(5)
    T, k, n, R = 20, 4, 256, 60
    y = rng.standard_normal((R, n)).astype(np.float32)
    pr = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    pr[3, 1] = R                       # past the rows: the token's output is NaN
    w = rng.uniform(0, 1, size=(T, k)).astype(np.float32)
    flat = torch.empty(R * n + 1, dtype=torch.float32, device=d)
    y_view = flat[1:].view(R, n)       # rows start 4 bytes off a 16-byte boundary
    y_view.copy_(dev(y, d))
    check_combine(orc, y, pr, w, "unaligned y", y_dev=y_view)
    check_combine(orc, y, pr, None, "bad row")


# ------------------------------------------------------- the expert layer from logits to output

def _upload_bank(gw, d):
    w_bank = dev(gw.w_bank, d)
    s_bank = dev(gw.s_bank, d)
    w_ptrs = dev((w_bank.data_ptr() + gw.w_off).astype(np.int64), d)
    s_ptrs = dev((s_bank.data_ptr() + gw.s_off).astype(np.int64), d)
    return w_bank, s_bank, w_ptrs, s_ptrs, dev(gw.scale2.astype(np.float32), d)


@pytest.mark.parametrize("seed,T,E,top,hidden,inter,normalize", [(11, 48, 8, 2, 512, 256, False),
                                                                 (12, 200, 16, 4, 384, 128, True)])
def test_expert_layer_from_logits(orc, schedule, seed, T, E, top, hidden, inter, normalize):
    """router logits -> top-k -> pack -> act-quant -> gate/up GEMM -> swiglu x routing weight ->
    down GEMM -> combine; every leg against the oracle on the same inputs as the GPU leg."""
    from test_gpu_swiglu import check_h
    d = require_gpu()
    kinds = [NV if e % 3 else MX for e in range(E)]
    ch = workloads.expert_chain(seed, T, E, top, hidden, inter, kinds=kinds)
    up, dn = _upload_bank(ch.up, d), _upload_bank(ch.down, d)
    kinds_d = dev(ch.kinds, d)
    ids, w = fp4.route_softmax_topk(dev(ch.logits, d), top, normalize=normalize)
    offsets, row_ids, pair_rows, row_w = fp4.route_pack(ids, E, w)
    codes_x, scales_x = fp4.act_quant_fp8(dev(ch.x, d))
    R = T * top
    gu = fp4.fp4_grouped_gemm_gather(codes_x, scales_x, row_ids, offsets, up[2], up[3], kinds_d, up[4], 2 * inter)
    h = torch.empty((R, inter), dtype=torch.float32, device=d)
    codes_h, scales_h = fp4.swiglu_quant_fp8(gu, ch.limit, row_weights=row_w, h_out=h)
    y = fp4.fp4_grouped_gemm_gather(codes_h, scales_h, None, offsets, dn[2], dn[3], kinds_d, dn[4], hidden,
                             out=torch.empty((R, hidden), dtype=torch.float32, device=d))
    out = fp4.moe_combine(y, pair_rows)
    torch.cuda.synchronize()

    rid, rw = orc.route_topk(ch.logits, top, normalize=normalize)
    assert np.array_equal(ids.cpu().numpy(), rid)
    ro, rr, rp, rrw = orc.route_pack(rid, E, w.cpu().numpy())
    assert np.array_equal(offsets.cpu().numpy(), ro) and np.array_equal(row_ids.cpu().numpy(), rr)
    assert np.array_equal(offsets.cpu().numpy(), ch.offsets) and np.array_equal(rr, ch.row_ids)
    rc, rs = orc.act_quant(ch.x)
    gu_np = gu.cpu().numpy()
    ref, absp = orc.grouped_gemm(rc[rr], rs[rr], ro, [ch.up.w_of(e) for e in range(E)],
                                 [ch.up.s_of(e) for e in range(E)], ch.kinds, ch.up.scale2, 2 * inter)
    check_bound(gu_np, ref, absp, hidden, "gate/up")
    h_np = h.cpu().numpy()
    check_h(h_np, orc.swiglu(gu_np, inter, ch.limit, rrw), "h")
    hc, hs = orc.act_quant(h_np)
    assert np.array_equal(codes_h.cpu().numpy(), hc) and np.array_equal(scales_h.cpu().numpy(), hs)
    y_np = y.cpu().numpy()
    ref2, absp2 = orc.grouped_gemm(hc, hs, ro, [ch.down.w_of(e) for e in range(E)],
                                   [ch.down.s_of(e) for e in range(E)], ch.kinds, ch.down.scale2, hidden)
    check_bound(y_np, ref2, absp2, inter, "down")
    ref3, absr3 = orc.combine(y_np, rp)
    check_bound(out.cpu().numpy(), ref3, absr3, top, "combine")
