"""Pins of the oracle's act-quant: worked scales, torch's independent E4M3 cast of x/s, the
closed-form quantization error bound, and the invariants the definition implies."""
import numpy as np
import torch

import workloads
from conftest import read_golden


def _group_with_amax(amax, rng):
    x = (rng.uniform(-1, 1, size=128) * np.float32(amax) * np.float32(0.5)).astype(np.float32)
    x[rng.integers(0, 128)] = np.float32(amax) * (1 if rng.integers(0, 2) else -1)
    return x


def test_worked_scales(orc):
    rng = np.random.default_rng(1)
    for amax, s in read_golden("act_quant_scales.txt"):
        x = _group_with_amax(float(amax), rng)[None, :]
        codes, scales = orc.act_quant(x)
        assert scales.shape == (1, 1)
        assert float(scales[0, 0]) == float(s), (amax, scales[0, 0], s)


def test_codes_equal_torch_cast_of_scaled_input(orc):
    w = workloads.config2()          # outliers drive some group amaxes
    codes, scales = orc.act_quant(w.x)
    s_full = np.repeat(scales, 128, axis=1)
    assert np.all(np.log2(scales) == np.round(np.log2(scales)))          # powers of two
    v = (w.x / s_full).astype(np.float32)                                 # exact: s is 2^e
    assert np.all(np.abs(v) <= 448.0)                                     # clamp never engages
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_scale_invariants(orc):
    x = workloads.config0().x
    codes, scales = orc.act_quant(x)
    g = x.reshape(x.shape[0], -1, 128)
    amax = np.maximum(np.abs(g).max(axis=2), np.float32(1e-4))
    assert np.all(scales >= amax / 448.0)                      # s >= amax/448 ...
    assert np.all(scales < 2 * amax / 448.0 * (1 + 2.0 ** -23))  # ... and the smallest such 2^e
    dec = orc.e4m3_value(codes).reshape(g.shape)
    top = np.abs(dec).max(axis=2)
    assert np.all((top > 224.0) & (top <= 448.0))              # largest code lands in (224, 448]


def test_quantization_error_bound(orc):
    # |dec(code) * s - x| <= half an E4M3 ulp of x/s, times s: 2^-4 relative in the normal range,
    # 2^-10 * s absolute in the subnormal range.
    rng = np.random.default_rng(7)
    x = (rng.standard_t(3, size=(8, 1024)) * 10.0 ** rng.integers(-6, 6, size=(8, 1))).astype(np.float32)
    codes, scales = orc.act_quant(x)
    s_full = np.repeat(scales, 128, axis=1).astype(np.float64)
    err = np.abs(orc.e4m3_value(codes) * s_full - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s_full)
    assert np.all(err <= bound)


def test_zero_and_floor_groups(orc):
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = 3e-5                                   # below the 1e-4 floor
    codes, scales = orc.act_quant(x)
    assert np.all(scales == np.float32(2.0 ** -22))
    assert np.all(codes[0] == 0x00) and np.all(codes[1, :128] == 0x80)
    # 3e-5 / 2^-22 = 125.8 lies between the E4M3 neighbours 120 and 128, above their midpoint 124
    assert orc.e4m3_value(codes[1, 128:129])[0] == 128.0


def test_group_independence_and_permutation(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    codes, scales = orc.act_quant(x)
    # each group depends on its own 128 values only; a permutation inside a group permutes codes
    perm = rng.permutation(128)
    xp = x.copy()
    xp[:, 128:256] = x[:, 128:256][:, perm]
    cp, sp = orc.act_quant(xp)
    assert np.array_equal(sp, scales)
    assert np.array_equal(cp[:, 128:256], codes[:, 128:256][:, perm])
    assert np.array_equal(np.delete(cp, np.s_[128:256], 1), np.delete(codes, np.s_[128:256], 1))
    # rows are independent: quantizing one row alone gives the same bytes
    c1, s1 = orc.act_quant(x[1:2])
    assert np.array_equal(c1, codes[1:2]) and np.array_equal(s1, scales[1:2])
