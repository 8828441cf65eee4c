"""GPU FP4 expert GEMM (single and grouped) vs the oracle: every output within
k * 2^-24 * sum|p|, bit identity on exact-by-construction inputs, determinism, batch invariance,
and the degenerate cases (empty experts, invalid table entries, ragged shapes)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import GroupedDevice, check_bound, dev, require_gpu

pytestmark = pytest.mark.gpu
NV, MX = workloads.NVFP4, workloads.MXFP4


def run_single(wl, orc, check_codes=True):
    """act_quant + fp4_expert_gemm on the GPU; full oracle comparison."""
    x = dev(wl.x)
    codes, scales = fp4.act_quant_fp8(x)
    ex = wl.expert
    out = fp4.fp4_expert_gemm(codes, scales, dev(ex.w), dev(ex.s), ex.scale2, ex.kind)
    torch.cuda.synchronize()
    rc, rs = orc.act_quant(wl.x)
    if check_codes:
        assert np.array_equal(codes.cpu().numpy(), rc)
    ref, absp = orc.expert_gemm(rc, rs, ex.w, ex.s, ex.scale2, ex.kind)
    return out.cpu().numpy(), ref, absp


def test_config0(orc):
    wl = workloads.config0()
    got, ref, absp = run_single(wl, orc)
    worst = check_bound(got, ref, absp, wl.k, "config0")
    print(f"config0 worst err / (2^-24 sum|p|) = {worst:.2f}; pages' op count "
          f"{orc.pages_op_count(NV, wl.k):.0f}")


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_config1(orc, g):
    wl = workloads.config1(g)
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, wl.k, f"config1 g={g}")


def test_config2(orc):
    wl = workloads.config2()
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, wl.k, "config2")


SHAPES = [(1, 16, 128), (5, 200, 256), (16, 64, 640), (17, 72, 384), (31, 130, 512),
          (32, 256, 1024), (33, 96, 256), (50, 64, 2048), (100, 48, 384), (129, 300, 256),
          (300, 520, 640)]


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("g,n,k", SHAPES)
def test_random_shapes(orc, schedule, kind, g, n, k):
    wl = workloads.single_random(1000 + g * 7 + n + k, g, n, k, kind, scale2=2.0 ** -5, x_scale=2.0)
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, k, f"g={g} n={n} k={k} kind={kind}")


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_tiled_output_any_float_alignment(orc, shift):
    # the tiled kernel writes whole 16-byte row pieces only when n % 4 == 0 and the output base is
    # 16-byte aligned; any other float-aligned base takes per-element stores of the same values, and
    # nothing outside the output is written
    g, n, k = 150, 256, 1024
    wl = workloads.single_random(600 + shift, g, n, k, NV)
    ex = wl.expert
    fp4.set_gemm_schedule(fp4.SCHEDULE_TILED)
    try:
        codes, scales = fp4.act_quant_fp8(dev(wl.x))
        aligned = fp4.fp4_expert_gemm(codes, scales, dev(ex.w), dev(ex.s), ex.scale2, ex.kind)
        buf = torch.full((g * n + 8,), 7.0, dtype=torch.float32, device="cuda")
        out = buf[shift:shift + g * n].view(g, n)
        fp4.fp4_expert_gemm(codes, scales, dev(ex.w), dev(ex.s), ex.scale2, ex.kind, out=out)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    assert torch.equal(out, aligned)
    assert bool((buf[:shift] == 7.0).all()) and bool((buf[shift + g * n:] == 7.0).all())
    rc, rs = orc.act_quant(wl.x)
    ref, absp = orc.expert_gemm(rc, rs, ex.w, ex.s, ex.scale2, ex.kind)
    check_bound(out.cpu().numpy(), ref, absp, k, f"output base + {4 * shift} bytes")


@pytest.mark.parametrize("seed", range(12))
def test_single_random_sweep(orc, schedule, seed):
    # seeded random single-expert shapes: g 1..300 (split-k sizes g <= 16 in a third of the seeds),
    # any n 1..600, k up to 2048, both formats, power-of-two and other scale2 values
    rng = np.random.default_rng([4096, seed])
    g = int(rng.integers(1, 17)) if seed % 3 == 0 else int(rng.integers(1, 301))
    n = int(rng.integers(1, 601))
    k = 128 * int(rng.integers(1, 17))
    kind = NV if seed % 2 == 0 else MX
    scale2 = float(2.0 ** -int(rng.integers(4, 9))) if seed % 4 else 0.3
    wl = workloads.single_random(7000 + seed, g, n, k, kind, scale2=scale2, x_scale=float(rng.uniform(0.1, 4.0)))
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, k, f"sweep seed={seed} g={g} n={n} k={k} kind={kind}")


@pytest.mark.parametrize("kind", [NV, MX])
def test_wide_dynamic_range_within_blocks(orc, schedule, kind):
    # activation magnitudes log-uniform over 6 decades: inside one 128-wide block the products span
    # about 20 binades, so any summation that aligns products to the largest one and drops low bits
    # (as the block-scaled FP8 x FP4 MFMA does) fails the f32 bound here
    rng = np.random.default_rng(99 + kind)
    g, n, k = 24, 160, 1024
    wl = workloads.single_random(4242 + kind, g, n, k, kind, scale2=2.0 ** -6)
    mags = 10.0 ** rng.uniform(-5.0, 1.0, size=(g, k))
    wl.x[:] = (np.where(rng.random((g, k)) < 0.5, -1.0, 1.0) * mags).astype(np.float32)
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, k, f"wide range kind={kind}")


def test_non_pow2_scale2(orc, schedule):
    wl = workloads.single_random(77, 9, 80, 512, NV, scale2=0.37)
    got, ref, absp = run_single(wl, orc)
    check_bound(got, ref, absp, 512, "scale2=0.37")


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("g,n,k", [(3, 48, 512), (16, 64, 7168), (29, 130, 2048), (200, 260, 1024)])
def test_exact_arm_bit_identity(orc, schedule, kind, g, n, k):
    a_codes, a_scales, ex = workloads.exact_arm(g + n, g, n, k, kind)
    out = fp4.fp4_expert_gemm(dev(a_codes), dev(a_scales), dev(ex.w), dev(ex.s), ex.scale2, kind)
    ref, _ = orc.expert_gemm(a_codes, a_scales, ex.w, ex.s, ex.scale2, kind)
    got = out.cpu().numpy()
    assert np.array_equal(got.astype(np.float64), ref), \
        f"{int(np.sum(got != ref))} outputs differ; max diff {np.max(np.abs(got - ref))}"


def test_determinism_and_row_invariance(orc, schedule):
    # 24 rows, or 16 under the split-k schedule (the largest batch that kernel takes: the batch and
    # its single rows must run on the same kernel)
    g = 16 if schedule == fp4.SCHEDULE_SPLITK else 24
    wl = workloads.single_random(5, g, 256, 1024, NV)
    codes, scales = fp4.act_quant_fp8(dev(wl.x))
    w, s = dev(wl.expert.w), dev(wl.expert.s)
    o1 = fp4.fp4_expert_gemm(codes, scales, w, s, wl.expert.scale2, NV)
    o2 = fp4.fp4_expert_gemm(codes, scales, w, s, wl.expert.scale2, NV)
    assert torch.equal(o1, o2)
    # each row alone gives the same bits as in the batched launch
    for r in (0, 7, g - 8, g - 1):
        o_r = fp4.fp4_expert_gemm(codes[r:r + 1].contiguous(), scales[r:r + 1].contiguous(), w, s,
                                  wl.expert.scale2, NV)
        assert torch.equal(o_r[0], o1[r])


def grouped_check(gd: GroupedDevice, orc, out, rows=None):
    wl = gd.wl
    codes, scales = orc.act_quant(wl.x)
    pc, ps = codes[wl.row_ids], scales[wl.row_ids]
    ws = [wl.w_of(e) for e in range(wl.E)]
    ss = [wl.s_of(e) for e in range(wl.E)]
    got = out.cpu().numpy()
    if rows is None:
        ref, absp = orc.grouped_gemm(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n)
        return check_bound(got, ref, absp, wl.k, wl.name)
    r, c = rows
    ref, absp = orc.grouped_gemm_points(pc, ps, wl.offsets, ws, ss, wl.kinds, wl.scale2, wl.n, r, c)
    return check_bound(got[r, c], ref, absp, wl.k, wl.name + " (sampled)")


@pytest.mark.parametrize("seed,T,E,top,n,k", [(1, 40, 8, 2, 96, 512), (2, 64, 16, 4, 200, 384),
                                              (3, 300, 12, 3, 64, 1024), (8, 700, 6, 2, 272, 384)])
def test_grouped_small_mixed(orc, schedule, seed, T, E, top, n, k):
    kinds = [NV if e % 3 else MX for e in range(E)]
    wl = workloads.grouped_random(seed, T, E, top, n, k, kinds=kinds, empty_experts=(1, E - 2))
    gd = GroupedDevice(wl)
    _, _, out = gd.step()
    grouped_check(gd, orc, out)


@pytest.mark.parametrize("seed", range(16))
def test_grouped_random_sweep(orc, schedule, seed):
    # seeded random grouped problems: any n (1..600, so ragged column tiles and n % 4 != 0), k up to
    # 1024, experts of both formats with some left empty, 1..4 experts per token, normal or
    # Student-t(3) activations, uniform or Zipf(1.1) routing; every fourth seed has 1..4 experts and
    # up to 600 tokens, so that experts span several 128-row slices, the others 1..20 experts and up
    # to 200 tokens (the short tail slices of every 32-row class)
    rng = np.random.default_rng([8128, seed])
    few = seed % 4 == 0
    E = int(rng.integers(1, 5)) if few else int(rng.integers(1, 21))
    n_empty = int(rng.integers(0, E // 3 + 1))
    empties = tuple(int(e) for e in rng.choice(E, n_empty, replace=False)) if n_empty else ()
    top = int(rng.integers(1, min(4, E - n_empty) + 1))
    T = int(rng.integers(100, 601)) if few else int(rng.integers(1, 201))
    n = int(rng.integers(1, 601))
    k = 128 * int(rng.integers(1, 5 if few else 9))
    kinds = [int(v) for v in rng.integers(0, 2, size=E)]
    x_dist = "t3" if seed % 2 else "normal"
    zipf = 1.1 if seed % 3 == 0 else None
    wl = workloads.grouped_random(9000 + seed, T, E, top, n, k, kinds=kinds, empty_experts=empties, zipf=zipf,
                                  x_dist=x_dist)
    gd = GroupedDevice(wl)
    _, _, out = gd.step()
    grouped_check(gd, orc, out)


@pytest.mark.parametrize("sched", [fp4.SCHEDULE_ROWSTREAM, fp4.SCHEDULE_TILED], ids=["rowstream", "tiled"])
@pytest.mark.parametrize("E,T,top", [(9, 90, 2), (37, 200, 4), (505, 700, 8), (512, 700, 8), (520, 700, 8)])
def test_many_experts_every_output(orc, E, T, top, sched):
    """Every expert computed exactly once into a NaN-filled output.  The row-streaming kernel hands
    each XCD its experts with more than 16 rows first (up to 512 experts; more keep the plain order):
    expert counts whose per-XCD lists differ in length (E % 8 != 0), that fill all 64 lanes of the
    ballot (512) or exceed it (520).  The tiled kernel scans the offsets of several 64-expert chunks
    per tile, and with n = 72 and rows that leave most 32-row tiles partial, its loads of columns past
    n and rows outside the slice run on every tile (they may read any bytes of the planes but must
    never reach the output).  Empty, short, long and multi-pass experts."""
    kinds = [NV if e % 5 else MX for e in range(E)]
    wl = workloads.grouped_random(7100 + E, T, E, top, 72, 256, kinds=kinds, zipf=1.1)
    rows = np.diff(wl.offsets)
    assert (rows > 16).any() and ((rows > 0) & (rows <= 16)).any()
    gd = GroupedDevice(wl)
    out = torch.full((wl.R, wl.n), float("nan"), dtype=torch.float32, device=gd.x.device)
    fp4.set_gemm_schedule(sched)
    try:
        _, _, out = gd.step(out=out)
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    grouped_check(gd, orc, out)


def test_grouped_matches_single_expert_bits(orc, schedule):
    if schedule == fp4.SCHEDULE_SPLITK:
        pytest.skip("split-k runs single-expert calls only: its additions are ordered differently "
                    "from the grouped kernels' (both within the bound, tested elsewhere)")
    wl = workloads.grouped_random(4, 96, 8, 3, 128, 512, kinds=[NV, MX] * 4)
    gd = GroupedDevice(wl)
    codes, scales, out = gd.step()
    for e in range(wl.E):
        lo, hi = int(wl.offsets[e]), int(wl.offsets[e + 1])
        if hi == lo:
            continue
        ids = gd.row_ids[lo:hi].long()
        o = fp4.fp4_expert_gemm(codes[ids].contiguous(), scales[ids].contiguous(),
                                dev(wl.w_of(e)), dev(wl.s_of(e)), float(wl.scale2[e]), int(wl.kinds[e]))
        assert torch.equal(o, out[lo:hi]), f"expert {e}"


def test_grouped_without_row_ids(orc, schedule):
    wl = workloads.grouped_random(5, 32, 4, 2, 64, 256, kinds=[NV, MX, NV, MX])
    gd = GroupedDevice(wl)
    codes, scales = fp4.act_quant_fp8(gd.x)
    pc, ps = codes[gd.row_ids.long()].contiguous(), scales[gd.row_ids.long()].contiguous()
    out = fp4.fp4_grouped_gemm_gather(pc, ps, None, gd.offsets, gd.w_ptrs, gd.s_ptrs, gd.kinds,
                               gd.scale2, wl.n, out=torch.empty((wl.R, wl.n), device=pc.device))
    _, _, ref_out = gd.step()
    assert torch.equal(out, ref_out)


def test_grouped_invalid_entries_give_nan(orc, schedule):
    wl = workloads.grouped_random(6, 24, 4, 2, 64, 256)
    gd = GroupedDevice(wl)
    codes, scales, good = gd.step()
    bad_ids = gd.row_ids.clone()
    bad_ids[3] = 10 ** 6                       # outside [0, a_rows)
    bad_ids[5] = -1
    bad_kinds = gd.kinds.clone()
    bad_kinds[2] = 7
    out = fp4.fp4_grouped_gemm_gather(codes, scales, bad_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, bad_kinds,
                               gd.scale2, wl.n)
    torch.cuda.synchronize()
    nan_rows = {3, 5} | set(range(int(wl.offsets[2]), int(wl.offsets[3])))
    for r in range(wl.R):
        if r in nan_rows:
            assert bool(torch.isnan(out[r]).all()), r
        else:
            assert torch.equal(out[r], good[r]), r


def test_grouped_offsets_are_clamped(orc, schedule):
    # offsets past total_rows are clamped: rows beyond R are never touched and every row is written
    wl = workloads.grouped_random(7, 16, 4, 2, 32, 128)
    gd = GroupedDevice(wl)
    codes, scales, good = gd.step()
    offs = gd.offsets.clone()
    offs[2] = offs[2] + 10 ** 6                # expert 1 now claims rows past the end
    sentinel = torch.full((wl.R + 8, wl.n), 123.0, device=codes.device)
    out = sentinel[:wl.R]
    fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, offs, gd.w_ptrs, gd.s_ptrs, gd.kinds, gd.scale2,
                         wl.n, out=out)
    torch.cuda.synchronize()
    assert bool((sentinel[wl.R:] == 123.0).all())
    lo = int(wl.offsets[1])
    assert torch.equal(out[:lo], good[:lo])


def _sample(R, n, count, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([rng.integers(0, R, count - 2 * n // 16), np.zeros(n // 16, np.int64),
                           np.full(n // 16, R - 1)])
    cols = np.concatenate([rng.integers(0, n, count - 2 * n // 16), np.arange(0, n, 16),
                           np.arange(0, n, 16)])
    return rows.astype(np.int64), cols.astype(np.int64)


@pytest.fixture(scope="module")
def config3_dev():
    return GroupedDevice(workloads.config3())


@pytest.fixture(scope="module")
def config4_dev():
    return GroupedDevice(workloads.config4())


def test_config3_sampled(orc, config3_dev):
    gd = config3_dev
    _, _, out = gd.step()
    _, _, out2 = gd.step()
    assert torch.equal(out, out2)                              # run-to-run bit identity
    assert not bool(torch.isnan(out).any())
    rows, cols = _sample(gd.R, gd.n, 16384, 3)
    worst = grouped_check(gd, orc, out, (rows, cols))
    print(f"config3 worst err / (2^-24 sum|p|) over {rows.size} samples = {worst:.2f}")


@pytest.fixture(scope="module")
def config3_full(orc, config3_dev):
    """The decode step as the benchmark runs it (swizzled planes, the automatic schedule), and the
    oracle's act-quant of its tokens."""
    gd = config3_dev
    w_ptrs, s_ptrs, kinds, _ = _swizzled_planes(gd)
    codes, scales = fp4.act_quant_fp8(gd.x)
    out = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, w_ptrs, s_ptrs, kinds, gd.scale2, gd.n)
    rc, rs = orc.act_quant(gd.wl.x)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)
    return out.cpu().numpy(), rc[gd.wl.row_ids], rs[gd.wl.row_ids]


@pytest.mark.parametrize("quarter", [0, 1, 2, 3])
def test_config3_every_output(orc, config3_dev, config3_full, quarter):
    """Every one of the 4096 x 2048 outputs of the decode step against the oracle, a quarter of the
    256 experts per case (each case streams its experts' packed rows through the f64 oracle)."""
    gd, (got, pc, ps) = config3_dev, config3_full
    wl = gd.wl
    e0, e1 = 64 * quarter, 64 * quarter + 64
    r0, r1 = int(wl.offsets[e0]), int(wl.offsets[e1])
    ref, absp = orc.grouped_gemm(pc, ps, wl.offsets, [wl.w_of(e) for e in range(wl.E)],
                                 [wl.s_of(e) for e in range(wl.E)], wl.kinds, wl.scale2, wl.n, row0=r0, row1=r1)
    worst = check_bound(got[r0:r1], ref, absp, wl.k, f"config3 experts {e0}..{e1 - 1}")   # ref: rows r0..r1
    print(f"config3 experts {e0}..{e1 - 1}: {r1 - r0} rows x {wl.n}, worst err / (2^-24 sum|p|) = {worst:.2f}")


def test_schedules_agree_within_bound(orc):
    """The two kernels on the same large-row grouped input: both within the bound of the oracle,
    each bit-reproducible run to run."""
    wl = workloads.grouped_random(9, 600, 8, 2, 512, 1024, kinds=[NV] * 7 + [MX], zipf=1.1, x_dist="t3")
    gd = GroupedDevice(wl)
    outs = []
    for sch in (fp4.SCHEDULE_ROWSTREAM, fp4.SCHEDULE_TILED):
        fp4.set_gemm_schedule(sch)
        try:
            _, _, o1 = gd.step()
            _, _, o2 = gd.step()
        finally:
            fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
        assert torch.equal(o1, o2)
        grouped_check(gd, orc, o1)
        outs.append(o1)


def _config4_tile_points(wl, seed):
    """Output coordinates that touch every (expert, 128-row slice, 256-column slice) tile of the tiled
    kernel once, plus every row of each expert's last, partial row slice (one column each)."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for e in range(wl.E):
        lo, hi = int(wl.offsets[e]), int(wl.offsets[e + 1])
        for m0 in range(lo, hi, 128):
            m1 = min(m0 + 128, hi)
            for c0 in range(0, wl.n, 256):
                rows.append(int(rng.integers(m0, m1)))
                cols.append(int(rng.integers(c0, min(c0 + 256, wl.n))))
            if m1 - m0 < 128:
                rows.extend(range(m0, m1))
                cols.extend(rng.integers(0, wl.n, m1 - m0).tolist())
    return np.array(rows, np.int64), np.array(cols, np.int64)


def test_config4_sampled(orc, config4_dev):
    """The prefill step at full size: every tile of every expert (the MXFP4 expert included) and every
    row of each expert's last partial row slice, against the oracle point by point; plus random
    outputs."""
    gd = config4_dev
    _, _, out = gd.step()
    assert not bool(torch.isnan(out).any())
    tr, tc = _config4_tile_points(gd.wl, 40)
    rr, rcol = _sample(gd.R, gd.n, 4096, 4)
    rows, cols = np.concatenate([tr, rr]), np.concatenate([tc, rcol])
    lo, hi = int(gd.wl.offsets[-2]), int(gd.wl.offsets[-1])
    assert hi > lo and np.any((rows >= lo) & (rows < hi))        # the MXFP4 expert is covered
    worst = grouped_check(gd, orc, out, (rows, cols))
    print(f"config4 worst err / (2^-24 sum|p|) over {rows.size} points "
          f"({tr.size} covering every tile and partial-slice row) = {worst:.2f}")


@pytest.mark.parametrize("factor", [1.0, 1e-5, 3e5])
def test_tiles_outside_the_f16_range(orc, schedule, factor):
    # The tiled kernel feeds NVFP4 tiles to f16 MFMAs only when every activation block scale of the
    # tile lies in [2^-15, 2^7]; a few rows scaled by 1e-5 (scales near 2^-18) or 3e5 (near 2^10)
    # send their tiles to the bf16 route while the other tiles stay on f16.  Every tile must meet
    # the same bound.
    wl = workloads.grouped_random(77, 400, 4, 2, 96, 512, kinds=[NV] * 4)
    wl.x[::37] *= np.float32(factor)
    gd = GroupedDevice(wl)
    _, scales, out = gd.step()
    s = scales.cpu().numpy()
    if factor != 1.0:
        assert ((s < 2.0 ** -15) | (s > 2.0 ** 7)).any()
    grouped_check(gd, orc, out)


@pytest.mark.parametrize("kind", [NV, MX])
@pytest.mark.parametrize("swz", [False, True])
@pytest.mark.parametrize("g,n,k", [(16, 2048, 8192), (1, 100, 128), (7, 2000, 1152), (16, 7168, 2048),
                                   (2, 33, 640)])
def test_splitk_single_expert(orc, kind, swz, g, n, k):
    """The split-k kernel at its limits (g = 16, k = 8192), ragged n and k, both layouts: within the
    bound, run-to-run identical, and each row alone gives the batch's bits."""
    fp4.set_gemm_schedule(fp4.SCHEDULE_SPLITK)
    try:
        wl = workloads.single_random(900 + g + n + k + kind, g, n, k, kind, scale2=2.0 ** -7, x_scale=3.0)
        ex = wl.expert
        codes, scales = fp4.act_quant_fp8(dev(wl.x))
        if swz:
            w, s = fp4.fp4_weight_swizzle(dev(ex.w), dev(ex.s), kind)
            kd = kind | fp4.SWIZZLED
        else:
            w, s, kd = dev(ex.w), dev(ex.s), kind
        o1 = fp4.fp4_expert_gemm(codes, scales, w, s, ex.scale2, kd, n=n)
        o2 = fp4.fp4_expert_gemm(codes, scales, w, s, ex.scale2, kd, n=n)
        last = fp4.fp4_expert_gemm(codes[g - 1:].contiguous(), scales[g - 1:].contiguous(), w, s, ex.scale2, kd, n=n)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    assert torch.equal(o1, o2)
    assert torch.equal(last[0], o1[g - 1])
    rc, rs = orc.act_quant(wl.x)
    ref, absp = orc.expert_gemm(rc, rs, ex.w, ex.s, ex.scale2, kind)
    check_bound(o1.cpu().numpy(), ref, absp, k, f"split-k g={g} n={n} k={k} kind={kind} swz={swz}")


def test_splitk_limits_fall_back(orc):
    """g = 17 or k = 8320 do not fit the split-k kernel: the call runs the row-streaming kernel and
    still meets the bound."""
    for g, k in ((17, 1024), (4, 8320)):
        fp4.set_gemm_schedule(fp4.SCHEDULE_SPLITK)
        try:
            wl = workloads.single_random(31 + g + k, g, 96, k, NV)
            got, ref, absp = run_single(wl, orc)
        finally:
            fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
        check_bound(got, ref, absp, k, f"fallback g={g} k={k}")


@pytest.mark.parametrize("sched", [fp4.SCHEDULE_AUTO, fp4.SCHEDULE_SPLITK], ids=["auto", "splitk"])
@pytest.mark.parametrize("T", [1, 2, 4, 16])
@pytest.mark.parametrize("swz", [False, True])
def test_grouped_few_tokens_splitk(orc, config3_dev, T, swz, sched):
    """A decode step of a few tokens over the 256 NVFP4 experts of the decode workload (k = 7168,
    n = 2048, top-8: 8 to 128 packed rows), under the automatic schedule (split-k for 8 rows,
    row-streaming above 16) and with split-k forced.  Every output within the bound, run-to-run
    identical."""
    gd = config3_dev
    fp4.set_gemm_schedule(sched)
    try:
        _few_tokens_case(orc, gd, T, swz)
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)


@pytest.mark.parametrize("seed,T,E,n,ks", [(21, 2, 16, 1592, 4), (22, 16, 128, 200, 2), (23, 16, 128, 1000, 1)],
                         ids=["ks4", "ks2", "ks1"])
def test_grouped_splitk_tile_groups(orc, seed, T, E, n, ks):
    """Grouped split-k launches whose size gives a 16-column tile 4, 2 or 1 wavefronts (the workgroup
    then owns 2, 4 or 8 tiles): min(E, rows) x ceil(tiles * ks / 8) first reaches 512 items at that
    ks.  n is not a multiple of the group width, so the last tile group holds a ragged tile and tiles
    past n.  Mixed NVFP4/MXFP4 experts, top-8, k = 256; every output within the bound, run-to-run
    identical."""
    tiles = (n + 15) // 16
    est = min(E, 8 * T)
    pick = next((c for c in (1, 2, 4) if est * -(-tiles * c // 8) >= 512), 8)
    assert pick == ks and (n % (16 * 8 // ks)) != 0
    kinds = [NV if e % 3 else MX for e in range(E)]
    wl = workloads.grouped_random(seed, T, E, 8, n, 256, kinds=kinds)
    gd = GroupedDevice(wl)
    fp4.set_gemm_schedule(fp4.SCHEDULE_SPLITK)
    try:
        _, _, o1 = gd.step()
        _, _, o2 = gd.step()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    assert torch.equal(o1, o2)
    assert not bool(torch.isnan(o1).any())
    grouped_check(gd, orc, o1)


@pytest.mark.parametrize("seed,T,E,n", [(24, 2, 16, 1592), (25, 16, 128, 200), (26, 16, 128, 1000)],
                         ids=["ks4", "ks2", "ks1"])
def test_grouped_splitk_tile_groups_unknown_kind(seed, T, E, n):
    """The same tile-group launches with one expert of a kind the kernels do not take: all of that
    expert's outputs (every tile of its groups, ragged tile included) are NaN, the other experts'
    outputs keep their bits."""
    wl = workloads.grouped_random(seed, T, E, 8, n, 256, kinds=[NV if e % 3 else MX for e in range(E)])
    gd = GroupedDevice(wl)
    counts = np.diff(wl.offsets)
    bad = int(np.argmax(counts))
    fp4.set_gemm_schedule(fp4.SCHEDULE_SPLITK)
    try:
        codes, scales, good = gd.step()
        bad_kinds = gd.kinds.clone()
        bad_kinds[bad] = 6
        out = fp4.fp4_grouped_gemm_gather(codes, scales, gd.row_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, bad_kinds,
                                   gd.scale2, wl.n)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    lo, hi = int(wl.offsets[bad]), int(wl.offsets[bad + 1])
    assert hi > lo
    assert bool(torch.isnan(out[lo:hi]).all())
    assert torch.equal(out[:lo], good[:lo]) and torch.equal(out[hi:], good[hi:])


def _few_tokens_case(orc, gd, T, swz):
    wl = gd.wl
    row_ids, offsets = workloads.route_topk(wl.logits[:T], 8)
    x = wl.x[:T]
    codes, scales = fp4.act_quant_fp8(dev(x))
    rid, offs = dev(row_ids), dev(offsets)
    if swz:
        w_ptrs, s_ptrs, kinds, keep = _swizzled_planes(gd)
    else:
        w_ptrs, s_ptrs, kinds, keep = gd.w_ptrs, gd.s_ptrs, gd.kinds, None
    o1 = fp4.fp4_grouped_gemm_gather(codes, scales, rid, offs, w_ptrs, s_ptrs, kinds, gd.scale2, wl.n)
    o2 = fp4.fp4_grouped_gemm_gather(codes, scales, rid, offs, w_ptrs, s_ptrs, kinds, gd.scale2, wl.n)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    rc, rs = orc.act_quant(x)
    ref, absp = orc.grouped_gemm(rc[row_ids], rs[row_ids], offsets, [wl.w_of(e) for e in range(wl.E)],
                                 [wl.s_of(e) for e in range(wl.E)], wl.kinds, wl.scale2, wl.n)
    check_bound(o1.cpu().numpy(), ref, absp, wl.k, f"{T} tokens swz={swz}")
    del keep


_SWZ_CACHE = {}


def _swizzled_planes(gd):
    """Swizzled copies of every expert of a GroupedDevice (kept for the module)."""
    key = id(gd)
    if key not in _SWZ_CACHE:
        wl = gd.wl
        w_ptrs, s_ptrs, kinds = gd.w_ptrs.clone(), gd.s_ptrs.clone(), gd.kinds.clone()
        keep = []
        for e in range(wl.E):
            kd = int(wl.kinds[e])
            w_swz, s_swz = fp4.fp4_weight_swizzle(gd.w_bank[int(wl.w_off[e]):int(wl.w_off[e]) + wl.n * wl.k // 2]
                                                  .view(wl.n, wl.k // 2),
                                                  gd.s_bank[int(wl.s_off[e]):int(wl.s_off[e]) + wl.n * wl.k // 16]
                                                  .view(wl.n, wl.k // 16) if kd == NV else
                                                  gd.s_bank[int(wl.s_off[e]):int(wl.s_off[e]) + wl.n * wl.k // 32]
                                                  .view(wl.n, wl.k // 32), kd)
            keep += [w_swz, s_swz]
            w_ptrs[e], s_ptrs[e], kinds[e] = w_swz.data_ptr(), s_swz.data_ptr(), kd | fp4.SWIZZLED
        _SWZ_CACHE[key] = (w_ptrs, s_ptrs, kinds, keep)
    return _SWZ_CACHE[key]


@pytest.mark.parametrize("schedule_id", [fp4.SCHEDULE_SPLITK, fp4.SCHEDULE_ROWSTREAM], ids=["splitk", "rowstream"])
def test_grouped_multipass_few_experts(orc, schedule_id):
    """40 tokens over 2 experts at top-1 (about 20 rows per expert, over the split-k kernel's
    16-row pass, so forced split-k runs two passes per expert; the automatic schedule would pick the
    row-streaming kernel for 40 packed rows) and ragged n, k: within the bound under forced split-k
    and under the row-streaming schedule; invalid row ids and kinds give NaN rows."""
    wl = workloads.grouped_random(24, 40, 2, 1, 200, 640, kinds=[NV, MX])
    gd = GroupedDevice(wl)
    fp4.set_gemm_schedule(schedule_id)
    try:
        codes, scales, out = gd.step()
        bad_ids = gd.row_ids.clone()
        bad_ids[3] = -5
        bad_kinds = gd.kinds.clone()
        bad_kinds[1] = 9
        bad = fp4.fp4_grouped_gemm_gather(codes, scales, bad_ids, gd.offsets, gd.w_ptrs, gd.s_ptrs, bad_kinds,
                                   gd.scale2, wl.n)
        torch.cuda.synchronize()
    finally:
        fp4.set_gemm_schedule(fp4.SCHEDULE_AUTO)
    grouped_check(gd, orc, out)
    lo1 = int(wl.offsets[1])
    for r in range(wl.R):
        if r == 3 or r >= lo1:
            assert bool(torch.isnan(bad[r]).all()), r
        else:
            assert torch.equal(bad[r], out[r]), r
