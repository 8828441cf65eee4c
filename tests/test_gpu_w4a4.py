"""GPU parity of the W4A4 NVFP4 variant (kernel_check.rs page, the NVFP4 MMQ W4A4 arms).

The quantizer and the channel selection are integer decisions taken in f32 on both sides: bit-exact
against the oracle.  The GEMM sums exact bf16 products in f32 and applies the row scale, scale2 and
the kept channels after, so |gpu - f64| <= (k + k_res + 2) 2^-24 sum|p| on the same quantized
operands.  The pages' accuracy contract on top: informational max-normalized rel below 0.2 on
0.1-scale activations, and two hard comparisons (row scale beats sub-block-only scaling on
decade-spread tokens; keeping the 8 outlier channels beats keeping none)."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import check_bound, dev, require_gpu
from test_oracle_w4a4 import exact_product, per_token_rel, rel_max

pytestmark = pytest.mark.gpu


def gpu_w4a4(x, ex, two_level=True, k_res=0):
    d = require_gpu()
    xd = dev(x, d)
    idx = fp4.loud_channels(xd, k_res) if k_res else None
    codes, micro, rs = fp4.act_quant_fp4(xd, two_level, skip_channels=idx)
    y = fp4.w4a4_gemm(codes, micro, rs, dev(ex.w, d), dev(ex.s, d), ex.scale2, x=xd if k_res else None, res_idx=idx)
    return (codes.cpu().numpy(), micro.cpu().numpy(), rs.cpu().numpy(), y.cpu().numpy(),
            None if idx is None else idx.cpu().numpy())


@pytest.mark.parametrize("arm,T,k", [("uniform", 16, 1024), ("dyn", 33, 512), ("res", 128, 1024),
                                     ("uniform", 1, 128), ("dyn", 7, 7168), ("res", 9, 2048),
                                     ("dyn", 3, 8320)])           # k > 8192: the two-pass kernel
@pytest.mark.parametrize("two_level", [True, False])
def test_quantizer_bit_exact(orc, arm, T, k, two_level):
    x, ex = workloads.w4a4_case(10 + T, T, 64, k, arm)
    codes, micro, rs, _, _ = gpu_w4a4(x, ex, two_level)
    rc, rm, rr = orc.act_quant_fp4(x, two_level)
    assert np.array_equal(rs, rr)
    assert np.array_equal(micro, rm), f"{int((micro != rm).sum())} micro-scales differ"
    assert np.array_equal(codes, rc), f"{int((codes != rc).sum())} code bytes differ"


def test_quantizer_edges(orc):
    k = 256
    x = np.zeros((6, k), dtype=np.float32)
    x[1, :] = -0.0
    x[2, 7] = 1e-30                                       # a lone tiny value
    x[3, :] = np.linspace(-6.5, 6.5, k)                   # crosses every E2M1 midpoint
    x[4, :16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0]
    x[5, :] = 3e38 * np.sin(np.arange(k))
    for tl in (True, False):
        codes, micro, rs, _, _ = gpu_w4a4(x, workloads.w4a4_case(1, 1, 32, k)[1], tl)
        rc, rm, rr = orc.act_quant_fp4(x, tl)
        assert np.array_equal(rs, rr) and np.array_equal(micro, rm) and np.array_equal(codes, rc)


def test_loud_channels(orc):
    d = require_gpu()
    for arm, T, k in (("res", 128, 1024), ("uniform", 9, 8192), ("dyn", 50, 300 * 16)):
        x, _ = workloads.w4a4_case(3, T, 32, k, arm)
        x[:, 5] = x[:, 900 % k]                           # an exact tie between two channels
        for k_res in (1, 8, 64):
            got = fp4.loud_channels(dev(x, d), k_res).cpu().numpy()
            assert np.array_equal(got, orc.loud_channels(x, k_res)), (arm, k_res)


@pytest.mark.parametrize("arm,T,n,k,k_res", [("uniform", 16, 256, 1024, 0), ("dyn", 37, 70, 512, 0),
                                             ("res", 128, 96, 1024, 8), ("res", 5, 33, 2048, 64)])
def test_gemm_parity(orc, arm, T, n, k, k_res):
    x, ex = workloads.w4a4_case(20 + T, T, n, k, arm)
    codes, micro, rs, y, idx = gpu_w4a4(x, ex, True, k_res)
    ref, absp = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2, x if k_res else None, idx)
    check_bound(y, ref, absp, k + k_res + 2, f"w4a4 {arm} T={T} n={n} k={k} k_res={k_res}")


@pytest.mark.parametrize("seed", range(8))
def test_gemm_random_sweep(orc, seed):
    # seeded random shapes on the tiled kernel's W4A4 path: 1..300 tokens (every 32-row tail class),
    # any n 1..400, k up to 2048, 0, 8 or 64 kept channels, all three activation arms
    rng = np.random.default_rng([1729, seed])
    T = int(rng.integers(1, 301))
    n = int(rng.integers(1, 401))
    k = 128 * int(rng.integers(1, 17))
    k_res = (0, 8, 64)[seed % 3]
    arm = ("uniform", "dyn", "res")[seed % 3]
    x, ex = workloads.w4a4_case(300 + seed, T, n, k, arm)
    codes, micro, rs, y, idx = gpu_w4a4(x, ex, seed % 4 != 3, k_res)
    xq = x.copy()
    if idx is not None:
        xq[:, idx] = 0.0                                  # kept channels enter the quantizer as zeros
    rc, rm, rr = orc.act_quant_fp4(xq, seed % 4 != 3)
    assert np.array_equal(codes, rc) and np.array_equal(micro, rm) and np.array_equal(rs, rr)
    ref, absp = orc.w4a4_gemm(codes, micro, rs, ex.w, ex.s, ex.scale2, x if k_res else None, idx)
    check_bound(y, ref, absp, k + k_res + 2, f"w4a4 sweep seed={seed} T={T} n={n} k={k} k_res={k_res}")


@pytest.mark.parametrize("T", [16, 64, 128, 512])
def test_informational_band(orc, T):
    x, ex = workloads.w4a4_case(4, T, 256, 1024, "uniform")
    rel = rel_max(gpu_w4a4(x, ex)[3], exact_product(orc, x, ex))
    print(f"\nW4A4 T={T}: rel = {rel:.3e}")
    assert rel < 0.2


@pytest.mark.parametrize("T", [16, 128])
def test_dynamic_range_gate(orc, T):
    x, ex = workloads.w4a4_case(5, T, 256, 1024, "dyn")
    ref = exact_product(orc, x, ex)
    two = per_token_rel(gpu_w4a4(x, ex, True)[3], ref)
    one = per_token_rel(gpu_w4a4(x, ex, False)[3], ref)
    print(f"\nW4A4 DYN T={T}: two-level rel {two:.3e}, sub-block-only {one:.3e}")
    assert two < one


def test_residual_channel_gate(orc):
    x, ex = workloads.w4a4_case(6, 128, 256, 1024, "res")
    ref = exact_product(orc, x, ex)
    rels = {k_res: per_token_rel(gpu_w4a4(x, ex, True, k_res)[3], ref) for k_res in (0, 4, 8, 16, 32, 64)}
    print("\nW4A4 RES: " + ", ".join(f"k={k}: {r:.3e}" for k, r in rels.items()))
    for k_res in (8, 16, 32, 64):
        assert rels[k_res] < rels[0], rels
