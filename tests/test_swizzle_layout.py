"""The numpy statement of the swizzled weight layout (tests/swizzle_ref.py) against the header's
index formulas evaluated one byte at a time, and its inverse.  The GPU tests compare the library's
fp4_weight_swizzle with this statement."""
import numpy as np
import pytest

import swizzle_ref


@pytest.mark.parametrize("kind,n,k", [(0, 16, 128), (0, 20, 384), (1, 33, 640), (1, 16, 512), (0, 7, 1024)])
def test_formula_by_loops(kind, n, k):
    rng = np.random.default_rng(n * 1000 + k + kind)
    gs = 16 if kind == 0 else 32
    w = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (n, k // gs), dtype=np.uint8)
    w_swz, s_swz = swizzle_ref.swizzle(w, s, kind)
    n16, nblk, nq = swizzle_ref.dims(n, k)
    assert w_swz.size == n16 * 16 * k // 2
    assert s_swz.size == n16 * nq * 64 * (8 if kind == 0 else 4)
    for t in range(n16):
        for j in range(16):
            c = 16 * t + j
            for b in range(nblk):
                for p in range(4):
                    for i in range(16):
                        want = w[c, 64 * b + 16 * p + i] if c < n else 0
                        assert w_swz[((t * nblk + b) * 64 + 16 * p + j) * 16 + i] == want
            for q in range(nq):
                for p in range(4):
                    for m in range(4):
                        blk = 4 * q + m
                        if kind == 0:
                            for e in range(2):
                                want = s[c, 8 * blk + 2 * p + e] if (c < n and blk < nblk) else 0
                                assert s_swz[((t * nq + q) * 64 + 16 * p + j) * 8 + 2 * m + e] == want
                        else:
                            want = s[c, 4 * blk + p] if (c < n and blk < nblk) else 0
                            assert s_swz[((t * nq + q) * 64 + 16 * p + j) * 4 + m] == want


@pytest.mark.parametrize("kind,n,k", [(0, 2048, 7168), (1, 2048, 7168), (0, 130, 384), (1, 7, 128)])
def test_inverse(kind, n, k):
    rng = np.random.default_rng(5)
    gs = 16 if kind == 0 else 32
    w = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (n, k // gs), dtype=np.uint8)
    w2, s2 = swizzle_ref.unswizzle(*swizzle_ref.swizzle(w, s, kind), kind, n, k)
    assert np.array_equal(w, w2) and np.array_equal(s, s2)
