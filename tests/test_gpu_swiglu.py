"""GPU parity of swiglu_quant_fp8 and of the expert chain gate/up -> activation -> down.

The activation h is compared with the oracle's f64 evaluation (memra-engine 0.98.0
dsv4_native_gemm_gate.rs page, the swiglu_limit saturation cell).  The GPU evaluates it in f32 with
the device expf, so h must agree to a few f32 ulps:

    |h_gpu - h_f64| <= 2^-20 * |h_f64| + 1e-35

(2^-20 = 16 ulp; the f32 chain min/clamp, expf, 1 + e, one division and three multiplies is
within about 5 ulp.  Below a gate of about -88.7, exp(-g) overflows f32 and the f32 result is 0
where the exact h is |g| e^g |u w| < 3e-37 |u w|; 1e-35 covers that for |u w| up to 30.  Values
that small quantize to code 0 against the act-quant scale floor of 1e-4 / 448 either way).  The codes and scales are an integer decision taken from h, so they are
compared bit for bit with the oracle's act-quant of the GPU's own h, and the GEMM legs with the
oracle's f64 GEMM on the same codes within |gpu - f64| <= k * 2^-24 * sum|p|, as the pages' cell does
for its down projection."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import check_bound, dev, first_byte_diff, require_gpu

pytestmark = pytest.mark.gpu
NV, MX = workloads.NVFP4, workloads.MXFP4
H_REL = 2.0 ** -20
H_ABS = 1e-35


def check_h(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = H_REL * np.abs(ref) + H_ABS
    bad = ~(err <= bound)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} h values outside the bound; first "
                             f"flat {i}: gpu {got.ravel()[i]!r} ref {ref.ravel()[i]!r}")


def run_swiglu(gu, limit, w=None):
    d = require_gpu()
    gu_d = dev(gu, d)
    w_d = None if w is None else dev(w, d)
    rows, inter = gu.shape[0], gu.shape[1] // 2
    h = torch.empty((rows, inter), dtype=torch.float32, device=d)
    codes, scales = fp4.swiglu_quant_fp8(gu_d, limit, row_weights=w_d, h_out=h)
    codes2, scales2 = fp4.swiglu_quant_fp8(gu_d, limit, row_weights=w_d)      # without h_out
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    return h.cpu().numpy(), codes.cpu().numpy(), scales.cpu().numpy()


def check_swiglu(orc, gu, limit, w=None, what=""):
    inter = gu.shape[1] // 2
    h, codes, scales = run_swiglu(gu, limit, w)
    check_h(h, orc.swiglu(gu, inter, limit, w), what)
    rc, rs = orc.act_quant(h)
    assert np.array_equal(scales, rs), f"{what}: scales differ"
    assert np.array_equal(codes, rc), f"{what}: " + first_byte_diff(codes, rc, h)
    return h


@pytest.mark.parametrize("rows,inter,scale", [(1, 128, 1.0), (37, 384, 3.0), (64, 2048, 10.0),
                                              (5, 256, 50.0)])
@pytest.mark.parametrize("weighted", [False, True])
def test_swiglu_quant_random(orc, rows, inter, scale, weighted):
    rng = np.random.default_rng(rows * 1000 + inter)
    gu = (rng.standard_normal((rows, 2 * inter)) * scale).astype(np.float32)
    w = rng.uniform(0.05, 1.0, rows).astype(np.float32) if weighted else None
    check_swiglu(orc, gu, 7.0, w, f"rows={rows} inter={inter} scale={scale} weighted={weighted}")


def test_swiglu_quant_edges(orc):
    inter = 256
    gu = np.zeros((6, 2 * inter), dtype=np.float32)
    t = np.linspace(-120, 120, inter).astype(np.float32)
    gu[0, :inter] = t                       # gates across the whole range (exp over/underflow)
    gu[0, inter:] = 1.0
    gu[1, :inter] = 1.0
    gu[1, inter:] = t                       # up values across both clamps
    gu[2, :] = 0.0                          # all-zero row: h = 0, scale floored at 1e-4
    gu[3, :inter] = 1e-3                    # tiny h: the act-quant scale floor decides
    gu[3, inter:] = 1e-3
    gu[4, :inter] = 7.0                     # exactly at the limit
    gu[4, inter:] = -7.0
    gu[5, :inter] = np.float32(6.9999995)   # one ulp below the limit
    gu[5, inter:] = np.float32(-7.0000005)  # one ulp beyond
    check_swiglu(orc, gu, 7.0, None, "edges")
    check_swiglu(orc, gu, 2.5, np.full(6, 0.5, np.float32), "edges, limit 2.5")
    h, _, _ = run_swiglu(gu, float("inf"))  # no clamping at all
    check_h(h, orc.swiglu(gu, inter, float("inf")), "limit inf")


def test_swiglu_saturation_row(orc):
    # the pages' cell: one row scaled x50 saturates both clamps; every saturated output is +-limit
    # * silu(limit)
    rng = np.random.default_rng(50)
    gu = (rng.standard_normal((1, 2 * 1024)) * 50).astype(np.float32)
    h = check_swiglu(orc, gu, 7.0, None, "x50 row")
    gate, up = gu[0, :1024], gu[0, 1024:]
    sat = (gate > 7.0) & (np.abs(up) > 7.0)
    assert sat.sum() > 0
    assert len(set(np.abs(h[0, sat]).tolist())) == 1


def _upload_bank(gw, d):
    w_bank = dev(gw.w_bank, d)
    s_bank = dev(gw.s_bank, d)
    w_ptrs = dev((w_bank.data_ptr() + gw.w_off).astype(np.int64), d)
    s_ptrs = dev((s_bank.data_ptr() + gw.s_off).astype(np.int64), d)
    return w_bank, s_bank, w_ptrs, s_ptrs, dev(gw.scale2.astype(np.float32), d)


def run_chain(ch, orc, what):
    """GPU: act-quant -> grouped gate/up GEMM -> swiglu_quant -> grouped down GEMM; every leg is
    checked against the oracle on the same inputs as the GPU leg (as the pages' cell does)."""
    d = require_gpu()
    x = dev(ch.x, d)
    row_ids, offsets, kinds = dev(ch.row_ids, d), dev(ch.offsets, d), dev(ch.kinds, d)
    rw = dev(ch.route_w, d)
    up = _upload_bank(ch.up, d)
    dn = _upload_bank(ch.down, d)
    R, I, Hd = ch.R, ch.inter, ch.hidden
    codes_x, scales_x = fp4.act_quant_fp8(x)
    gu = fp4.fp4_grouped_gemm_gather(codes_x, scales_x, row_ids, offsets, up[2], up[3], kinds, up[4], 2 * I)
    h = torch.empty((R, I), dtype=torch.float32, device=d)
    codes_h, scales_h = fp4.swiglu_quant_fp8(gu, ch.limit, row_weights=rw, h_out=h)
    y = fp4.fp4_grouped_gemm_gather(codes_h, scales_h, None, offsets, dn[2], dn[3], kinds, dn[4], Hd,
                             out=torch.empty((R, Hd), dtype=torch.float32, device=d))
    torch.cuda.synchronize()

    kinds_np = ch.kinds
    # leg 1: act-quant bit-exact, gate/up GEMM within the bound
    rc, rs = orc.act_quant(ch.x)
    assert np.array_equal(codes_x.cpu().numpy(), rc) and np.array_equal(scales_x.cpu().numpy(), rs)
    gu_np = gu.cpu().numpy()
    ref, absp = orc.grouped_gemm(rc[ch.row_ids], rs[ch.row_ids], ch.offsets,
                                 [ch.up.w_of(e) for e in range(len(kinds_np))],
                                 [ch.up.s_of(e) for e in range(len(kinds_np))], kinds_np, ch.up.scale2, 2 * I)
    check_bound(gu_np, ref, absp, Hd, what + " gate/up")
    # leg 2: the activation on the GPU's gate/up output, and its codes
    h_np = h.cpu().numpy()
    check_h(h_np, orc.swiglu(gu_np, I, ch.limit, ch.route_w), what + " h")
    hc, hs = orc.act_quant(h_np)
    assert np.array_equal(scales_h.cpu().numpy(), hs), what + ": h scales differ"
    assert np.array_equal(codes_h.cpu().numpy(), hc), what + ": " + first_byte_diff(codes_h.cpu().numpy(), hc, h_np)
    # leg 3: the down projection on the same codes
    ref2, absp2 = orc.grouped_gemm(hc, hs, ch.offsets, [ch.down.w_of(e) for e in range(len(kinds_np))],
                                   [ch.down.s_of(e) for e in range(len(kinds_np))], kinds_np,
                                   ch.down.scale2, Hd)
    check_bound(y.cpu().numpy(), ref2, absp2, I, what + " down")
    return gu_np, h_np


@pytest.mark.parametrize("seed,T,E,top,hidden,inter,x_scale", [(1, 40, 8, 2, 512, 256, 1.0),
                                                               (2, 96, 6, 3, 384, 384, 2.0),
                                                               (3, 600, 4, 2, 256, 128, 1.0)])
def test_expert_chain(orc, schedule, seed, T, E, top, hidden, inter, x_scale):
    kinds = [NV if e % 3 else MX for e in range(E)]
    ch = workloads.expert_chain(seed, T, E, top, hidden, inter, kinds=kinds, x_scale=x_scale)
    run_chain(ch, orc, ch.name)


@pytest.mark.parametrize("kind", [NV, MX])
def test_expert_chain_saturation_cell(orc, kind):
    # x50 activations drive the gate/up outputs past the limit on both sides; the whole chain
    # (quant -> GEMM -> clamp -> quant -> GEMM) stays within the oracle's bounds on every leg
    ch = workloads.expert_chain(50 + kind, 8, 2, 1, 1024, 512, kinds=[kind, kind], x_scale=50.0)
    gu, h = run_chain(ch, orc, f"saturation kind={kind}")
    I = ch.inter
    gate, up = gu[:, :I], gu[:, I:]
    assert np.sum(gate > ch.limit) > 0, "the gate clamp never engaged"
    assert np.sum(np.abs(up) > ch.limit) > 0, "the up clamp never engaged"


# --------------------------------------------------------------------------- fused gate/up + activation

def run_fused_vs_unfused(ch, limit=None, row_ids=None, kinds=None, weighted=True, x=None):
    """fp4_grouped_gemm_swiglu_quant against the unfused route it replaces (the tiled grouped GEMM,
    then swiglu_quant_fp8) on the same inputs: codes, scales and h must agree bit for bit, and every
    output element must be written (the outputs start poisoned, with two different poisons)."""
    d = require_gpu()
    limit = ch.limit if limit is None else limit
    xd = dev(ch.x if x is None else x, d)
    rid = dev(ch.row_ids if row_ids is None else row_ids, d)
    offsets = dev(ch.offsets, d)
    kd = dev(ch.kinds if kinds is None else np.asarray(kinds, dtype=np.int32), d)
    rw = dev(ch.route_w, d) if weighted else None
    up = _upload_bank(ch.up, d)
    R, I = ch.R, ch.inter
    codes_x, scales_x = fp4.act_quant_fp8(xd)
    fp4.set_gemm_schedule(fp4.SCHEDULE_TILED)
    try:
        gu = fp4.fp4_grouped_gemm_gather(codes_x, scales_x, rid, offsets, up[2], up[3], kd, up[4], 2 * I)
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    h_ref = torch.empty((R, I), dtype=torch.float32, device=d)
    c_ref, s_ref = fp4.swiglu_quant_fp8(gu, limit, row_weights=rw, h_out=h_ref)
    outs = []
    for poison, with_h in ((0xA5, True), (0x5A, False)):
        hc = torch.full((R, I), poison, dtype=torch.uint8, device=d)
        hs = torch.full((R, I // 128), float(poison), dtype=torch.float32, device=d)
        h = torch.full((R, I), float(poison), dtype=torch.float32, device=d) if with_h else None
        fp4.fp4_grouped_gemm_swiglu_quant(codes_x, scales_x, rid, offsets, up[2], up[3], kd, up[4], I, limit,
                                          row_weights=rw, h_codes=hc, h_scales=hs, h_out=h)
        outs.append((hc, hs, h))
    torch.cuda.synchronize()
    i32 = torch.int32
    for hc, hs, h in outs:
        assert torch.equal(hc, c_ref), first_byte_diff(hc.cpu().numpy(), c_ref.cpu().numpy(), h_ref.cpu().numpy())
        assert torch.equal(hs.view(i32), s_ref.view(i32)), "scales differ from the unfused route"
        if h is not None:
            assert torch.equal(h.view(i32), h_ref.view(i32)), "h differs from the unfused route"
    return gu, outs[0][2], c_ref, s_ref


@pytest.mark.parametrize("seed,T,E,top,hidden,inter,x_scale", [(1, 40, 8, 2, 512, 256, 1.0),
                                                               (2, 96, 6, 3, 384, 384, 2.0),
                                                               (3, 600, 4, 2, 256, 128, 1.0),
                                                               (4, 700, 8, 2, 1024, 512, 1.0),
                                                               (5, 9, 3, 1, 128, 1024, 0.5)])
def test_fused_gate_up_matches_the_unfused_route(orc, seed, T, E, top, hidden, inter, x_scale):
    kinds = [NV if e % 3 else MX for e in range(E)]
    ch = workloads.expert_chain(seed, T, E, top, hidden, inter, kinds=kinds, x_scale=x_scale)
    gu, h, codes, scales = (t.cpu().numpy() for t in run_fused_vs_unfused(ch, weighted=seed % 2 == 1))
    if seed == 1:
        # anchored to the oracle as well: h within the f32 bound of the exact activation of the same gate/up
        # values, and the codes its act-quant
        check_h(h, orc.swiglu(gu, inter, ch.limit, ch.route_w), "fused h")
        rc, rs = orc.act_quant(h)
        assert np.array_equal(codes, rc) and np.array_equal(scales, rs)


@pytest.mark.parametrize("seed", range(10))
def test_fused_gate_up_random_sweep(seed):
    # seeded random chains: 1..600 tokens, 1..12 experts of both formats, 1..3 per token, uniform or
    # Zipf(1.1) routing, hidden (k) 128..1024, inter 128..1024, activation scales from 0.1 to 20,
    # with and without row weights; the fused launch must give the unfused route's bits
    rng = np.random.default_rng([6502, seed])
    E = int(rng.integers(1, 13))
    top = int(rng.integers(1, min(3, E) + 1))
    T = int(rng.integers(1, 601))
    hidden = 128 * int(rng.integers(1, 9))
    inter = 128 * int(rng.integers(1, 9))
    kinds = [int(v) for v in rng.integers(0, 2, size=E)]
    x_scale = float(10.0 ** rng.uniform(-1.0, 1.3))
    ch = workloads.expert_chain(7100 + seed, T, E, top, hidden, inter, kinds=kinds, x_scale=x_scale,
                                zipf=1.1 if seed % 2 else None)
    run_fused_vs_unfused(ch, weighted=seed % 3 != 0)


@pytest.mark.parametrize("limit", [7.0, float("inf")])
def test_fused_gate_up_saturation(limit):
    ch = workloads.expert_chain(58, 70, 3, 2, 512, 256, kinds=[NV, MX, NV], x_scale=50.0)
    gu = run_fused_vs_unfused(ch, limit=limit)[0].cpu().numpy()
    if limit == 7.0:
        assert np.sum(gu[:, :256] > 7.0) > 0 and np.sum(np.abs(gu[:, 256:]) > 7.0) > 0


@pytest.mark.parametrize("factor", [1e-5, 3e5])
def test_fused_gate_up_outside_the_f16_range(factor):
    # rows scaled so that some NVFP4 tiles take the bf16 operand route, the others the f16 one
    ch = workloads.expert_chain(59, 300, 4, 2, 512, 256, kinds=[NV] * 4)
    x = ch.x.copy()
    x[::29] *= np.float32(factor)
    run_fused_vs_unfused(ch, x=x)


def test_fused_gate_up_invalid_rows_and_kinds():
    # packed rows whose activation row is out of range, and an expert of an unknown format, enter the
    # activation as NaN gate/up values in both routes
    ch = workloads.expert_chain(60, 120, 5, 2, 256, 256, kinds=[NV, MX, NV, NV, MX])
    rid = ch.row_ids.copy()
    rid[::17] = -1
    rid[5::23] = len(ch.x) + 3
    run_fused_vs_unfused(ch, row_ids=rid, kinds=[NV, MX, 7, NV, MX])


def test_config4_fused_gate_up_full_size():
    # the prefill layer's gate/up projection at full size (8192 tokens, top-8, 256 experts, n = 4096,
    # k = 7168, limit 7, routing-weighted rows), in the launch the chain benchmark times: bit-identical
    # to the unfused route over all 65536 x 2048 outputs
    ch = workloads.config4_chain()
    gu, h, codes, _ = run_fused_vs_unfused(ch)
    assert gu.shape == (ch.R, 2 * ch.inter) and codes.shape == (ch.R, ch.inter)
    assert torch.isfinite(h).all()
