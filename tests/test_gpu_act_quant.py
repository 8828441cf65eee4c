"""GPU act_quant_fp8 vs the oracle: codes and scales bit-exact on every workload, an exhaustive
sweep of the encoder over every f32 in [-448, 448], and edge rows."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads
from gpu_util import dev, first_byte_diff, require_gpu

pytestmark = pytest.mark.gpu


def _check(x_np, orc):
    codes, scales = fp4.act_quant_fp8(dev(x_np))
    torch.cuda.synchronize()
    rc, rs = orc.act_quant(x_np)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(gc, rc), first_byte_diff(gc, rc, x_np)
    bad = np.flatnonzero(gs.view(np.uint32) != rs.view(np.uint32))
    assert bad.size == 0, f"{bad.size} scale diffs, first group {bad[0]}: gpu {gs.ravel()[bad[0]]} ref {rs.ravel()[bad[0]]}"


@pytest.mark.parametrize("name", ["config0", "config1_g8", "config2"])
def test_single_expert_configs(orc, name):
    wl = {"config0": workloads.config0, "config1_g8": lambda: workloads.config1(8),
          "config2": workloads.config2}[name]()
    _check(wl.x, orc)


def test_config3_tokens(orc):
    rng = workloads.rng_for(3)
    x = rng.standard_normal((512, 7168), dtype=np.float32)     # the token rows of config3
    _check(x, orc)


def test_config4_tokens(orc):
    rng = workloads.rng_for(4)
    x = rng.standard_t(3, size=(8192, 7168)).astype(np.float32)  # the token rows of config4
    _check(x, orc)


def test_edge_rows(orc):
    rng = np.random.default_rng(9)
    k = 640
    x = np.zeros((9, k), dtype=np.float32)
    x[1] = -0.0
    x[2] = 3e-5                                               # under the 1e-4 floor
    x[3] = rng.standard_normal(k) * 1e30                      # huge: s = 2^90-ish
    x[4] = rng.standard_normal(k) * 1e-30                     # tiny: all codes round to zero
    x[5] = (rng.integers(1, 1 << 23, size=k).astype(np.uint32)).view(np.float32)  # denormals
    x[5, ::2] *= -1
    x[6] = 448.0 * np.float32(2.0) ** rng.integers(-20, 20, size=k)   # amax exactly 448 * 2^j
    x[7] = rng.standard_t(1, size=k)                          # Cauchy tails
    x[8] = np.float32(3.4e38) * rng.uniform(-1, 1, size=k)    # near f32 max
    _check(x.astype(np.float32), orc)


@pytest.mark.parametrize("rows,k", [(1, 128), (3, 384), (37, 1152), (129, 7168)])
def test_ragged_group_counts(orc, rows, k):
    rng = np.random.default_rng(rows)
    _check((rng.standard_normal((rows, k)) * 3).astype(np.float32), orc)


def test_zero_rows_is_noop():
    d = require_gpu()
    x = torch.empty((0, 256), dtype=torch.float32, device=d)
    codes, scales = fp4.act_quant_fp8(x)
    assert codes.shape == (0, 256) and scales.shape == (0, 2)


@pytest.mark.slow
def test_exhaustive_encoder_sweep(orc):
    """Every f32 with |x| <= 448 (both signs) goes through the kernel with scale 1: each 128-column
    group holds 448.0 in column 0 (so s = 1) and 127 sweep values; codes are compared with the
    oracle's encoder."""
    d = require_gpu()
    top = int(np.frombuffer(np.float32(448.0).tobytes(), dtype=np.uint32)[0])
    per_row = 127
    chunk = per_row * (1 << 19)                               # 66.6M values per chunk
    threads = min(16, len(os.sched_getaffinity(0)))
    pool = ThreadPoolExecutor(threads)
    total = 0
    for sign in (0, 0x80000000):
        for start in range(0, top + 1, chunk):
            stop = min(start + chunk, top + 1)
            cnt = stop - start
            rows = (cnt + per_row - 1) // per_row
            bits = torch.arange(start, start + rows * per_row, dtype=torch.int64, device=d)
            bits = torch.clamp(bits, max=top)
            if sign:                                   # bit 31 set, as a signed 32-bit value
                bits = bits - (1 << 31)
            vals = bits.to(torch.int32).view(torch.float32).view(rows, per_row)
            x = torch.empty((rows, 128), dtype=torch.float32, device=d)
            x[:, 0] = 448.0
            x[:, 1:] = vals
            codes, scales = fp4.act_quant_fp8(x)
            assert bool((scales == 1.0).all())
            got = codes[:, 1:].reshape(-1)[:cnt].cpu().numpy()
            xin = vals.reshape(-1)[:cnt].cpu().numpy()
            parts = np.array_split(np.arange(cnt), threads)
            refs = list(pool.map(lambda ix: orc.e4m3_encode(xin[ix[0]:ix[-1] + 1]) if ix.size else
                                 np.empty(0, np.uint8), parts))
            ref = np.concatenate(refs)
            assert np.array_equal(got, ref), first_byte_diff(got, ref, xin)
            total += cnt
            print(f"  sweep sign={sign >> 31} values {start}..{stop - 1}: ok", flush=True)
    pool.shutdown()
    assert total == 2 * (top + 1)
