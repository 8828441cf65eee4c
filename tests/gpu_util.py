"""Helpers for the GPU parity tests: device upload of workloads and the acceptance checks."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_fp4_quant_amd as fp4
import workloads

U32 = 2.0 ** -24


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (run them with -m gpu on an MI355X)")
    return torch.device("cuda", 0)


def dev(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device or require_gpu())


class GroupedDevice:
    """A GroupedWorkload resident on the device, with the per-expert address tables."""

    def __init__(self, wl: workloads.GroupedWorkload, device=None):
        d = device or require_gpu()
        self.wl = wl
        self.x = dev(wl.x, d)
        self.row_ids = dev(wl.row_ids, d)
        self.offsets = dev(wl.offsets, d)
        self.kinds = dev(wl.kinds, d)
        self.scale2 = dev(wl.scale2.astype(np.float32), d)
        self.w_bank = dev(wl.w_bank, d)
        self.s_bank = dev(wl.s_bank, d)
        self.w_ptrs = dev((self.w_bank.data_ptr() + wl.w_off).astype(np.int64), d)
        self.s_ptrs = dev((self.s_bank.data_ptr() + wl.s_off).astype(np.int64), d)
        self.R = wl.R
        self.n, self.k = wl.n, wl.k

    def step(self, out=None, codes=None, scales=None):
        """act_quant of the token rows, then the grouped GEMM over the packed rows."""
        codes, scales = fp4.act_quant_fp8(self.x, codes, scales)
        out = fp4.fp4_grouped_gemm_gather(codes, scales, self.row_ids, self.offsets, self.w_ptrs,
                                   self.s_ptrs, self.kinds, self.scale2, self.n, out=out)
        return codes, scales, out


def check_bound(got, ref, absp, k, what=""):
    """|got - ref| <= k * 2^-24 * absp elementwise; returns the worst err / (2^-24 absp)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bound = k * U32 * absp
    bad = ~(err <= bound)                       # NaN counts as a failure
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside the bound; first flat {i}: "
            f"gpu {got.ravel()[i]!r} ref {ref.ravel()[i]!r} err {err.ravel()[i]:.3e} "
            f"bound {bound.ravel()[i]:.3e}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(absp > 0, err / (U32 * absp), 0.0)
    return float(np.max(ratio)) if ratio.size else 0.0


def first_byte_diff(got: np.ndarray, ref: np.ndarray, x: np.ndarray | None = None):
    diff = np.flatnonzero(got.ravel() != ref.ravel())
    if diff.size == 0:
        return ""
    i = diff[0]
    msg = f"{diff.size} differing bytes; first at flat {i}: gpu {got.ravel()[i]:#04x} ref {ref.ravel()[i]:#04x}"
    if x is not None:
        v = np.float32(x.ravel()[i])
        msg += f" input {v!r} (bits {v.view(np.uint32):08x})"
    return msg
