"""The grouped GEMM's two C-ABI forms and the boundary's device-side checks, on the GPU:

- fp4_grouped_gemm (activation rows packed per expert, explicit workspace) gives the same bits as
  fp4_grouped_gemm_gather over the same packed rows, and meets the oracle's bound;
- fp4moe_set_debug_checks: valid tables run unchanged; each kind of invalid table makes the call
  return FP4MOE_EDEVICE without launching the GEMM;
- activation scales outside the contract (not positive powers of two) never give silently wrong
  outputs: the tiled kernel writes NaN rows, the other kernels apply the value exactly;
- the binding rejects a mis-shaped a_scales before any launch.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import GroupedDevice, check_bound, dev

pytestmark = pytest.mark.gpu
NV, MX = workloads.NVFP4, workloads.MXFP4


def _packed(gd):
    codes, scales = fp4.act_quant_fp8(gd.x)
    ids = gd.row_ids.long()
    return codes, scales, codes[ids].contiguous(), scales[ids].contiguous()


def _oracle(gd, orc, pc=None, ps=None):
    wl = gd.wl
    if pc is None:
        codes, scales = orc.act_quant(wl.x)
        pc, ps = codes[wl.row_ids], scales[wl.row_ids]
    return orc.grouped_gemm(pc, ps, wl.offsets, [wl.w_of(e) for e in range(wl.E)],
                            [wl.s_of(e) for e in range(wl.E)], wl.kinds, wl.scale2, wl.n)


@pytest.mark.parametrize("seed,T,E,top,n,k", [(41, 60, 8, 2, 200, 512), (42, 300, 6, 3, 320, 1024)])
def test_packed_form_matches_gather_form(orc, schedule, seed, T, E, top, n, k):
    wl = workloads.grouped_random(seed, T, E, top, n, k, kinds=[NV if e % 3 else MX for e in range(E)],
                                  empty_experts=(2,))
    gd = GroupedDevice(wl)
    codes, scales, pc, ps = _packed(gd)
    assert fp4.grouped_gemm_workspace_size(E, wl.R, n, k) == 0
    ref_out = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                          gd.scale2, n)
    o1 = fp4.fp4_grouped_gemm(pc, ps, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds, gd.scale2, n)
    ws = torch.empty(256, dtype=torch.uint8, device=pc.device)      # an (unused) caller workspace
    o2 = fp4.fp4_grouped_gemm(pc, ps, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds, gd.scale2, n, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, ref_out) and torch.equal(o2, ref_out)
    ref, absp = _oracle(gd, orc)
    check_bound(o1.cpu().numpy(), ref, absp, k, wl.name)


def test_packed_form_through_ctypes(orc):
    """The C entry point called directly (device pointers, sizes, a NULL workspace of 0 bytes)."""
    import ctypes
    wl = workloads.grouped_random(43, 40, 4, 2, 96, 256, kinds=[NV, MX, NV, NV])
    gd = GroupedDevice(wl)
    _, _, pc, ps = _packed(gd)
    out = torch.full((wl.R, wl.n), 7.0, device=pc.device)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = fp4.lib().fp4_grouped_gemm(p(pc), p(ps), p(gd.offsets), wl.E, wl.R, p(gd.w_ptrs), p(gd.s_ptrs), p(gd.kinds),
                                    p(gd.scale2), p(out), wl.n, wl.k, None, 0,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, fp4.lib().fp4moe_last_error()
    torch.cuda.synchronize()
    ref, absp = _oracle(gd, orc)
    check_bound(out.cpu().numpy(), ref, absp, wl.k, "ctypes packed form")


@pytest.fixture
def debug_checks():
    fp4.set_debug_checks(True)
    yield
    fp4.set_debug_checks(False)


def test_debug_checks_pass_valid_tables(debug_checks, schedule):
    wl = workloads.grouped_random(44, 50, 6, 2, 128, 256, kinds=[NV, MX] * 3, empty_experts=(4,))
    gd = GroupedDevice(wl)
    codes, scales, pc, ps = _packed(gd)
    fp4.set_debug_checks(False)
    want = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                       gd.scale2, wl.n)
    fp4.set_debug_checks(True)
    got = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                      gd.scale2, wl.n)
    got2 = fp4.fp4_grouped_gemm(pc, ps, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds, gd.scale2, wl.n)
    torch.cuda.synchronize()
    assert torch.equal(got, want) and torch.equal(got2, want)


def _bad_tables(gd, case):
    offs, rid, kinds = gd.offsets.clone(), gd.row_ids.clone(), gd.kinds.clone()
    if case == "first":
        offs[0] = 1
        return offs, rid, kinds, "offsets[0]"
    if case == "decreasing":
        offs[3] = offs[4] + 1
        return offs, rid, kinds, "offsets decrease at expert 3"
    if case == "total":
        offs[-1] = offs[-1] + 1
        return offs, rid, kinds, "total_rows"
    if case == "row_id":
        rid[5] = gd.x.shape[0]
        return offs, rid, kinds, "row_ids[5]"
    kinds[2] = 5
    return offs, rid, kinds, "kinds[2]"


@pytest.mark.parametrize("case", ["first", "decreasing", "total", "row_id", "kind"])
def test_debug_checks_report_invalid_tables(debug_checks, case):
    wl = workloads.grouped_random(45, 50, 6, 2, 256, 256)       # n = 2 x 128: the fused call takes it too
    gd = GroupedDevice(wl)
    codes, scales, pc, ps = _packed(gd)
    offs, rid, kinds, what = _bad_tables(gd, case)
    out = torch.full((wl.R, wl.n), 3.0, device=codes.device)
    with pytest.raises(fp4.Fp4MoeCallError) as ei:
        fp4.fp4_grouped_gemm_gather(codes, scales, rid, offs, gd.w_ptrs, gd.s_ptrs, kinds, gd.scale2, wl.n, out=out)
    assert ei.value.rc == fp4.EDEVICE and what in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())                     # the GEMM was not launched
    if case != "row_id":                                # the packed form has no row_ids
        with pytest.raises(fp4.Fp4MoeCallError) as ei:
            fp4.fp4_grouped_gemm(pc, ps, offs, gd.w_ptrs, gd.s_ptrs, kinds, gd.scale2, wl.n, out=out)
        assert ei.value.rc == fp4.EDEVICE and what in str(ei.value), str(ei.value)
        with pytest.raises(fp4.Fp4MoeCallError) as ei:
            fp4.fp4_grouped_gemm_swiglu_quant(codes, scales, rid, offs, gd.w_ptrs, gd.s_ptrs, kinds, gd.scale2,
                                              wl.n // 2, 10.0)
        assert ei.value.rc == fp4.EDEVICE and what in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def _non_pow2(scales, rows_groups):
    s = scales.clone()
    for r, q, f in rows_groups:
        s[r, q] = s[r, q] * f
    return s


@pytest.mark.parametrize("sched", [fp4.SCHEDULE_ROWSTREAM, fp4.SCHEDULE_TILED, fp4.SCHEDULE_SPLITK],
                         ids=["rowstream", "tiled", "splitk"])
@pytest.mark.parametrize("kind", [NV, MX])
def test_non_pow2_act_scales_single_expert(orc, sched, kind):
    """Rows 3 and 9 get an activation scale with mantissa bits (x1.5, x0.75) in one group each: the
    row-streaming and split-k kernels apply it exactly (within the bound of the oracle, which
    applies any f32 scale); the tiled kernel, which folds only a scale's exponent into its operand,
    writes those two rows as NaN and every other row within the bound."""
    g, n, k = 16, 96, 512
    wl = workloads.single_random(46 + kind, g, n, k, kind)
    codes, scales = fp4.act_quant_fp8(dev(wl.x))
    bad = [(3, 1, 1.5), (9, 3, 0.75)]
    s2 = _non_pow2(scales, bad)
    fp4.set_gemm_schedule(sched)
    try:
        out = fp4.fp4_expert_gemm(codes, s2, dev(wl.expert.w), dev(wl.expert.s), wl.expert.scale2, kind)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    got = out.cpu().numpy()
    ref, absp = orc.expert_gemm(codes.cpu().numpy(), s2.cpu().numpy(), wl.expert.w, wl.expert.s, wl.expert.scale2,
                                kind)
    bad_rows = sorted({r for r, _, _ in bad})
    if sched == fp4.SCHEDULE_TILED:
        assert np.isnan(got[bad_rows]).all()
        keep = [r for r in range(g) if r not in bad_rows]
        check_bound(got[keep], ref[keep], absp[keep], k, "tiled, valid rows")
    else:
        check_bound(got, ref, absp, k, f"schedule {sched}")


def test_non_pow2_act_scales_grouped_tiled(orc):
    """The same contract on a grouped launch of the tiled kernel, fused activation epilogue included:
    a packed row that reads a bad scale is NaN (its h codes are those of NaN gate/up values), all
    others keep the bits of the unmodified launch."""
    wl = workloads.grouped_random(47, 200, 4, 2, 256, 512, kinds=[NV, MX, NV, NV])
    gd = GroupedDevice(wl)
    codes, scales = fp4.act_quant_fp8(gd.x)
    s2 = _non_pow2(scales, [(7, 2, 1.25)])
    fp4.set_gemm_schedule(fp4.SCHEDULE_TILED)
    try:
        good = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                           gd.scale2, wl.n)
        out = fp4.fp4_grouped_gemm_gather(codes, s2, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                          gd.scale2, wl.n)
        hc_good, hs_good = fp4.fp4_grouped_gemm_swiglu_quant(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs,
                                                             gd.s_ptrs, gd.kinds, gd.scale2, wl.n // 2, 7.0)
        hc, hs = fp4.fp4_grouped_gemm_swiglu_quant(codes, s2, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs,
                                                   gd.kinds, gd.scale2, wl.n // 2, 7.0)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    hit = (gd.row_ids == 7).cpu().numpy()
    assert hit.any()
    o, gdd = out.cpu().numpy(), good.cpu().numpy()
    assert np.isnan(o[hit]).all()
    assert np.array_equal(o[~hit], gdd[~hit])
    hc, hs, hc_good, hs_good = (t.cpu().numpy() for t in (hc, hs, hc_good, hs_good))
    assert np.array_equal(hc[~hit], hc_good[~hit]) and np.array_equal(hs[~hit], hs_good[~hit])
    # the bad rows carry the activation of NaN gate/up values: one code byte and scale in every row
    for r in np.flatnonzero(hit):
        assert len(set(hc[r].tolist())) == 1 and len(set(hs[r].tolist())) == 1


def test_binding_rejects_misshaped_act_scales():
    wl = workloads.grouped_random(48, 20, 2, 1, 32, 256)
    gd = GroupedDevice(wl)
    codes, scales = fp4.act_quant_fp8(gd.x)
    short = scales[:, :1].contiguous()
    for call in (lambda: fp4.fp4_grouped_gemm_gather(codes, short, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs,
                                                     gd.kinds, gd.scale2, wl.n),
                 lambda: fp4.fp4_grouped_gemm(codes, short, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                                              gd.scale2, wl.n),
                 lambda: fp4.fp4_grouped_gemm_swiglu_quant(codes, short, gd.row_ids, gd.offsets, gd.w_ptrs,
                                                           gd.s_ptrs, gd.kinds, gd.scale2, 128, 7.0),
                 lambda: fp4.fp4_grouped_gemm_gather(codes, scales[:-1].contiguous(), gd.row_ids, gd.offsets,
                                                     gd.w_ptrs, gd.s_ptrs, gd.kinds, gd.scale2, wl.n)):
        with pytest.raises(ValueError):
            call()
