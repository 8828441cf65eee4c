"""The swizzled weight layout of fp4_weight_swizzle, written with numpy from the index formulas
the header states (a test helper: no part of the library or the oracle).

Column c = 16t + j, 128-wide k block b, k piece p (k = 128b + 32p .. +32), chunk q of 4 blocks:
  w_swz[((t*nblk + b)*64 + 16p + j)*16 + i]     = w[c, 64b + 16p + i]
  NVFP4: s_swz[((t*nq + q)*64 + 16p + j)*8 + 2m + e] = s[c, 8(4q+m) + 2p + e]
  MXFP4: s_swz[((t*nq + q)*64 + 16p + j)*4 + m]      = s[c, 4(4q+m) + p]
with zeros for columns >= n and blocks >= nblk.
"""
from __future__ import annotations

import numpy as np


def dims(n: int, k: int):
    n16 = -(-n // 16)
    nblk = k // 128
    nq = -(-nblk // 4)
    return n16, nblk, nq


def swizzle(w: np.ndarray, s: np.ndarray, kind: int):
    """Plain planes w u8 [n, k/2], s u8 [n, k/gs] -> (w_swz, s_swz) u8 1-D."""
    n, k = w.shape[0], 2 * w.shape[1]
    n16, nblk, nq = dims(n, k)
    wp = np.zeros((n16 * 16, k // 2), np.uint8)
    wp[:n] = w
    # [t, j, b, p, i] -> [t, b, p, j, i]
    w_swz = wp.reshape(n16, 16, nblk, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    per_blk = 8 if kind == 0 else 4
    sp = np.zeros((n16 * 16, nq * 4 * per_blk), np.uint8)
    sp[:n, :nblk * per_blk] = s
    if kind == 0:
        # [t, j, q, m, p, e] -> [t, q, p, j, m, e]
        s_swz = sp.reshape(n16, 16, nq, 4, 4, 2).transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    else:
        # [t, j, q, m, p] -> [t, q, p, j, m]
        s_swz = sp.reshape(n16, 16, nq, 4, 4).transpose(0, 2, 4, 1, 3).reshape(-1)
    return np.ascontiguousarray(w_swz), np.ascontiguousarray(s_swz)


def unswizzle(w_swz: np.ndarray, s_swz: np.ndarray, kind: int, n: int, k: int):
    """Inverse of swizzle (drops the padding)."""
    n16, nblk, nq = dims(n, k)
    w = w_swz.reshape(n16, nblk, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(n16 * 16, k // 2)[:n]
    per_blk = 8 if kind == 0 else 4
    if kind == 0:
        s = s_swz.reshape(n16, nq, 4, 16, 4, 2).transpose(0, 3, 1, 4, 2, 5)
    else:
        s = s_swz.reshape(n16, nq, 4, 16, 4).transpose(0, 3, 1, 4, 2)
    s = s.reshape(n16 * 16, nq * 4 * per_blk)[:n, :nblk * per_blk]
    return np.ascontiguousarray(w), np.ascontiguousarray(s)
