"""The swizzled weight layout on the GPU: fp4_weight_swizzle byte for byte against the numpy
statement of the layout, and the GEMMs on swizzled planes (kinds 2 and 3) bit-identical to the
same GEMMs on the plain planes and within the oracle's bound, single and grouped, in both
schedules."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import swizzle_ref
import workloads
from gpu_util import GroupedDevice, check_bound, dev

pytestmark = pytest.mark.gpu
NV, MX, SWZ = workloads.NVFP4, workloads.MXFP4, fp4.SWIZZLED


@pytest.mark.parametrize("kind,n,k", [(NV, 16, 128), (MX, 20, 384), (NV, 130, 640), (MX, 256, 7168),
                                      (NV, 2048, 7168), (NV, 7, 2048)])
def test_swizzle_bytes(kind, n, k):
    rng = np.random.default_rng(n + k + kind)
    gs = workloads.GROUP_SIZE[kind]
    w = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (n, k // gs), dtype=np.uint8)
    w_swz, s_swz = fp4.fp4_weight_swizzle(dev(w), dev(s), kind)
    torch.cuda.synchronize()
    rw, rs = swizzle_ref.swizzle(w, s, kind)
    assert np.array_equal(w_swz.cpu().numpy(), rw)
    assert np.array_equal(s_swz.cpu().numpy(), rs)


def _swz(ex):
    return fp4.fp4_weight_swizzle(dev(ex.w), dev(ex.s), ex.kind)


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("g,n,k", [(1, 16, 128), (4, 256, 512), (5, 200, 384), (17, 72, 640), (33, 96, 256),
                                   (100, 48, 1152), (129, 300, 256), (8, 2048, 7168)])
def test_single_expert_bits_equal_plain(orc, schedule, kind, g, n, k):
    wl = workloads.single_random(31 * g + n + k, g, n, k, kind, scale2=2.0 ** -6, x_scale=2.0)
    ex = wl.expert
    codes, scales = fp4.act_quant_fp8(dev(wl.x))
    plain = fp4.fp4_expert_gemm(codes, scales, dev(ex.w), dev(ex.s), ex.scale2, kind)
    w_swz, s_swz = _swz(ex)
    got = fp4.fp4_expert_gemm(codes, scales, w_swz, s_swz, ex.scale2, kind | SWZ, n=n)
    torch.cuda.synchronize()
    assert torch.equal(got, plain), f"{int((got != plain).sum())} outputs differ from the plain layout"
    rc, rs = orc.act_quant(wl.x)
    ref, absp = orc.expert_gemm(rc, rs, ex.w, ex.s, ex.scale2, kind)
    check_bound(got.cpu().numpy(), ref, absp, k, f"swizzled g={g} n={n} k={k} kind={kind}")


def _swizzled_tables(gd: GroupedDevice, which):
    """Swizzle the planes of experts e with which(e) true; returns (w_ptrs, s_ptrs, kinds, keep)."""
    wl = gd.wl
    w_ptrs = gd.w_ptrs.clone()
    s_ptrs = gd.s_ptrs.clone()
    kinds = gd.kinds.clone()
    keep = []
    for e in range(wl.E):
        if not which(e):
            continue
        k_e = int(wl.kinds[e])
        w_swz, s_swz = fp4.fp4_weight_swizzle(dev(wl.w_of(e)), dev(wl.s_of(e)), k_e)
        keep += [w_swz, s_swz]
        w_ptrs[e] = w_swz.data_ptr()
        s_ptrs[e] = s_swz.data_ptr()
        kinds[e] = k_e | SWZ
    return w_ptrs, s_ptrs, kinds, keep


@pytest.mark.parametrize("seed,T,E,top,n,k", [(1, 40, 8, 2, 96, 512), (2, 64, 16, 4, 200, 384),
                                              (3, 300, 12, 3, 64, 1024), (8, 700, 6, 2, 272, 384)])
def test_grouped_mixed_layouts_bits_equal_plain(orc, schedule, seed, T, E, top, n, k):
    kinds = [NV if e % 3 else MX for e in range(E)]
    wl = workloads.grouped_random(seed, T, E, top, n, k, kinds=kinds, empty_experts=(1, E - 2))
    gd = GroupedDevice(wl)
    codes, scales, plain = gd.step()
    w_ptrs, s_ptrs, kinds_t, keep = _swizzled_tables(gd, lambda e: e % 2 == 0)
    got = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, w_ptrs, s_ptrs, kinds_t, gd.scale2, wl.n)
    torch.cuda.synchronize()
    assert torch.equal(got, plain)
    del keep


def test_grouped_kind_outside_range_gives_nan(orc, schedule):
    wl = workloads.grouped_random(6, 24, 4, 2, 64, 256)
    gd = GroupedDevice(wl)
    codes, scales, good = gd.step()
    bad_kinds = gd.kinds.clone()
    bad_kinds[2] = 4                           # not 0..3
    out = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, bad_kinds,
                               gd.scale2, wl.n)
    torch.cuda.synchronize()
    lo, hi = int(wl.offsets[2]), int(wl.offsets[3])
    assert bool(torch.isnan(out[lo:hi]).all())
    assert torch.equal(out[:lo], good[:lo]) and torch.equal(out[hi:], good[hi:])


def test_config3_swizzled_bits_equal_plain():
    """The decode step at its full size (512 tokens, 256 NVFP4 experts, k=7168, n=2048), as the
    bench times it with swizzled planes: bit-identical to the plain layout's result."""
    gd = GroupedDevice(workloads.config3())
    codes, scales, plain = gd.step()
    w_ptrs, s_ptrs, kinds_t, keep = _swizzled_tables(gd, lambda e: True)
    got = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, w_ptrs, s_ptrs, kinds_t, gd.scale2, gd.n)
    torch.cuda.synchronize()
    assert torch.equal(got, plain)
    del keep


def test_config4_swizzled_bits_equal_plain():
    """The prefill step at its full size (8192 tokens, Zipf top-8, 255 NVFP4 + 1 MXFP4 experts,
    k=7168, n=4096) on swizzled planes: bit-identical to the plain layout's result, which the
    sampled oracle check covers."""
    gd = GroupedDevice(workloads.config4())
    codes, scales, plain = gd.step()
    w_ptrs, s_ptrs, kinds_t, keep = _swizzled_tables(gd, lambda e: True)
    got = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, w_ptrs, s_ptrs, kinds_t, gd.scale2, gd.n)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(got).any())
    assert torch.equal(got, plain)
    del keep


def test_swiglu_fused_swizzled_bits_equal_plain(orc):
    inter, k = 256, 512
    wl = workloads.grouped_random(12, 200, 6, 2, 2 * inter, k, kinds=[NV, MX, NV, NV, MX, NV])
    gd = GroupedDevice(wl)
    codes, scales = fp4.act_quant_fp8(gd.x)
    rw = torch.rand(wl.R, device=codes.device, dtype=torch.float32)
    plain = fp4.fp4_grouped_gemm_swiglu_quant(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs,
                                              gd.kinds, gd.scale2, inter, 7.0, row_weights=rw)
    w_ptrs, s_ptrs, kinds_t, keep = _swizzled_tables(gd, lambda e: e != 3)
    got = fp4.fp4_grouped_gemm_swiglu_quant(codes, scales, gd.row_ids, gd.offsets, w_ptrs, s_ptrs,
                                            kinds_t, gd.scale2, inter, 7.0, row_weights=rw)
    torch.cuda.synchronize()
    for a, b in zip(plain, got):
        assert torch.equal(a, b)
    del keep
