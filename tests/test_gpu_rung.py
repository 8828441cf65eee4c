"""GPU parity of the bf16-dequant rung and the class-shift characterization (dsv4_native_gemm_gate.rs
page, comparison 3).

cvt_bf16 and fp4_dequant_bf16 are bit-exact against the oracle (both follow the same f32 evaluation
and the same rounding).  gemm_bf16 sums exact products in f32, so |gpu - f64| <= k 2^-24 sum|p|.
The class shift of the native path (act_quant_fp8 + the FP4 GEMM) against the rung is informational
on the pages; here it is printed and held to a loose band around the oracle's own measurement
(median |shift| / prediction about 0.5, see the oracle's pins)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import check_bound, dev, require_gpu

pytestmark = pytest.mark.gpu
NV, MX = workloads.NVFP4, workloads.MXFP4


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def is_nan_bf16(b):
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def same_bf16(got, ref):
    """bf16 bit patterns equal wherever the oracle's value is a number, and NaN exactly where the
    oracle's is: IEEE fixes neither the sign nor the payload of a NaN an operation produces, so only
    its position is compared."""
    gn, rn = is_nan_bf16(got), is_nan_bf16(ref)
    bad = (gn != rn) | (~rn & (got != ref))
    return not bad.any(), int(bad.sum())


def test_cvt_bf16(orc):
    d = require_gpu()
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 0xFFFF, 20000).astype(np.uint32)
    x = np.concatenate([(rng.standard_normal(100003) * 5).astype(np.float32),
                        ((hi << 16) | 0x8000).view(np.float32),                      # ties (and NaN)
                        ((hi << 16) | rng.integers(0, 0x10000, 20000).astype(np.uint32)).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, 1e-40], np.float32)])
    got = bits(fp4.cvt_bf16(dev(x, d)))
    ref = orc.cvt_bf16(x)
    ok, nbad = same_bf16(got, ref)
    assert ok, f"{nbad} differ"


@pytest.mark.parametrize("kind,scale2,lo,hi", [(NV, 2.0 ** -6, None, None), (NV, 0.37, None, None),
                                               (NV, 1.0, 0, 255), (MX, 0.0, None, None), (MX, 0.0, 1, 254)])
def test_dequant_bf16(orc, kind, scale2, lo, hi):
    d = require_gpu()
    rng = np.random.default_rng(kind * 10 + (lo or 0))
    n, k = 96, 512
    w = workloads.random_nibbles(rng, n, k)
    if lo is None:
        s = workloads.random_scale_codes(rng, kind, n, k)
    else:                                    # every scale byte the format allows, NaN codes included
        s = rng.integers(lo, hi + 1, size=(n, k // workloads.GROUP_SIZE[kind]), dtype=np.uint8)
    got = bits(fp4.fp4_dequant_bf16(dev(w, d), dev(s, d), scale2, kind))
    ref = orc.dequant_bf16(w, s, scale2, kind)
    ok, nbad = same_bf16(got, ref)
    assert ok, f"{nbad} of {ref.size} differ"
    if lo is not None and kind == NV:
        assert is_nan_bf16(ref).any()        # the E4M3 NaN scale codes are exercised


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (37, 70, 96), (64, 64, 512), (100, 33, 7168)])
def test_gemm_bf16(orc, m, n, k):
    d = require_gpu()
    rng = np.random.default_rng(m + n + k)
    a = orc.cvt_bf16((rng.standard_normal((m, k)) * 3).astype(np.float32))
    w = orc.cvt_bf16(rng.standard_normal((n, k)).astype(np.float32))
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(d)
    tw = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(d)
    got = fp4.gemm_bf16(ta, tw).cpu().numpy()
    ref, absp = orc.gemm_bf16(a, w)
    check_bound(got, ref, absp, k, f"gemm_bf16 {m}x{n}x{k}")


def class_shift(orc, wl):
    """native (act_quant + FP4 GEMM) vs the rung (bf16 x, bf16 weights, bf16 GEMM), both on the GPU."""
    d = require_gpu()
    e = wl.expert
    x = dev(wl.x, d)
    w, s = dev(e.w, d), dev(e.s, d)
    codes, scales = fp4.act_quant_fp8(x)
    native = fp4.fp4_expert_gemm(codes, scales, w, s, e.scale2, e.kind).cpu().numpy().astype(np.float64)
    rung = fp4.gemm_bf16(fp4.cvt_bf16(x), fp4.fp4_dequant_bf16(w, s, e.scale2, e.kind)).cpu().numpy()
    wd = orc.dequant_weights(e.w, e.s, e.scale2, e.kind)
    pred = orc.class_shift_prediction(wl.x, wd)
    return np.abs(native - rung) / pred


@pytest.mark.parametrize("name", ["config0", "config1", "config2"])
def test_class_shift(orc, name):
    wl = {"config0": workloads.config0, "config1": lambda: workloads.config1(8), "config2": workloads.config2}[name]()
    ratio = class_shift(orc, wl)
    q = np.quantile(ratio, [0.1, 0.5, 0.9, 0.99])
    print(f"\n{name}: |native - rung| / ((2^-4/sqrt 3) ||x.w||_2): p10 {q[0]:.3f} median {q[1]:.3f} "
          f"p90 {q[2]:.3f} p99 {q[3]:.3f} max {ratio.max():.3f} over {ratio.size} outputs")
    assert 0.35 < q[1] < 0.65
    assert np.isfinite(ratio).all()
