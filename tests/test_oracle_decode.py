"""Pins of the oracle's element decoders (E2M1, E4M3, E8M0) against the pages and against torch's
independent float8 implementations."""
import math

import numpy as np
import torch

import workloads
from conftest import read_golden


def test_e2m1_matches_golden_grid(orc):
    rows = read_golden("e2m1_grid.txt")
    assert len(rows) == 16
    for code, val in rows:
        v = orc.e2m1_value([int(code)])[0]
        assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val)), code


def test_e2m1_grid_properties(orc):
    vals = orc.e2m1_value(np.arange(16))
    mags = sorted(set(abs(v) for v in vals))
    assert len(mags) == 8 and max(mags) == 6.0          # 8 grid points, largest magnitude 6
    assert np.all(vals[8:] == -vals[:8])                 # bit 3 is the sign
    assert np.all(np.diff(vals[:8]) > 0)                 # magnitudes increase with the code


def test_e4m3_exhaustive_vs_torch(orc):
    codes = np.arange(256)
    ours = orc.e4m3_value(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert set(np.flatnonzero(nan_ours)) == {0x7F, 0xFF}
    ok = ~nan_ours
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_golden_points(orc):
    for byte, val in read_golden("e4m3_points.txt"):
        v = orc.e4m3_value([int(byte, 16)])[0]
        if val == "nan":
            assert math.isnan(v)
        else:
            assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val)), byte


def test_e4m3_monotone_and_ranges(orc):
    pos = orc.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9
    # the generator's NVFP4 scale range is exactly the 41 E4M3 values in [2^-3, 2^2]
    lo, hi = workloads.NVFP4_SCALE_CODE_RANGE
    inside = [c for c in range(0x7F) if 2.0 ** -3 <= pos[c] <= 2.0 ** 2]
    assert inside == list(range(lo, hi + 1)) and len(inside) == 41
    # qwen4exp page: bytes 0x28..0x40 are positive, non-NaN and end at 2.0
    assert pos[0x28] == 0.25 and pos[0x40] == 2.0


def test_e8m0_exhaustive_vs_torch(orc):
    ours = orc.e8m0_value(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert math.isnan(ours[255]) and math.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127
    lo, hi = workloads.MXFP4_SCALE_CODE_RANGE
    assert ours[lo] == 2.0 ** -10 and ours[hi] == 2.0 ** -3


def test_exact_arm_code_lists(orc):
    vals = orc.e4m3_value(np.array(workloads.EXACT_INT_E4M3_CODES))
    assert list(vals) == list(range(17))
    assert list(orc.e4m3_value(np.array(workloads.EXACT_NVFP4_SCALE_CODES))) == [1.0, 2.0, 4.0]
    assert list(orc.e8m0_value(np.array(workloads.EXACT_MXFP4_SCALE_CODES))) == [0.5, 1.0, 2.0]
