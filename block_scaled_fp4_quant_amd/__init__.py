"""block_scaled_fp4_quant_amd -- FP8 E4M3 activation quantization and the block-scaled FP4
(NVFP4 / MXFP4) expert GEMM on AMD Instinct MI355X.

Thin ctypes binding over libfp4moe.so (C ABI in include/fp4moe.h).  The functions here only
marshal arguments: torch provides device memory and the current stream, every arithmetic step runs
in the library's HIP kernels.  There is no fallback: if the library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

NVFP4 = 0
MXFP4 = 1
GROUP_SIZE = {NVFP4: 16, MXFP4: 32}

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp4moe.so")
_lib = None


class Fp4MoeError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded libfp4moe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp4MoeError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_scaled_fp4_quant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        L.act_quant_fp8.argtypes = [P, P, P, I32, I32, P]
        L.act_quant_fp8.restype = ctypes.c_int
        L.swiglu_quant_fp8.argtypes = [P, P, F32, P, P, P, I32, I32, P]
        L.swiglu_quant_fp8.restype = ctypes.c_int
        L.fp4_expert_gemm.argtypes = [P, P, P, P, F32, I32, P, I32, I32, I32, P]
        L.fp4_expert_gemm.restype = ctypes.c_int
        L.fp4_grouped_gemm.argtypes = [P, P, I32, P, P, I32, I32, P, P, P, P, P, I32, I32, P]
        L.fp4_grouped_gemm.restype = ctypes.c_int
        L.fp4moe_last_error.argtypes = []
        L.fp4moe_last_error.restype = ctypes.c_char_p
        L.fp4moe_version.argtypes = []
        L.fp4moe_version.restype = ctypes.c_char_p
        L.fp4moe_set_gemm_schedule.argtypes = [I32]
        L.fp4moe_set_gemm_schedule.restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> str:
    return lib().fp4moe_version().decode()


SCHEDULE_AUTO, SCHEDULE_ROWSTREAM, SCHEDULE_TILED = 0, 1, 2


def set_gemm_schedule(schedule: int) -> None:
    """Force the GEMM kernel choice (0 automatic, 1 row-streaming, 2 tiled); a test hook."""
    _check(lib().fp4moe_set_gemm_schedule(int(schedule)), "fp4moe_set_gemm_schedule")


def _check(rc: int, what: str):
    if rc != 0:
        raise Fp4MoeError(f"{what} failed (rc={rc}): {lib().fp4moe_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def act_quant_fp8(x: torch.Tensor, codes=None, scales=None, stream=None):
    """x f32 [rows, k] -> (codes u8 [rows, k], scales f32 [rows, k/128])."""
    _dev(x, torch.float32, "x", 2)
    rows, k = x.shape
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // 128), dtype=torch.float32, device=x.device)
    _dev(codes, torch.uint8, "codes", 2)
    _dev(scales, torch.float32, "scales", 2)
    if codes.shape != (rows, k) or scales.shape != (rows, k // 128):
        raise ValueError("codes/scales shapes do not match x")
    _check(lib().act_quant_fp8(_ptr(x), _ptr(codes), _ptr(scales), rows, k, _stream(stream)),
           "act_quant_fp8")
    return codes, scales


def swiglu_quant_fp8(gu: torch.Tensor, limit: float, row_weights=None, codes=None, scales=None,
                     h_out=None, stream=None):
    """gu f32 [rows, 2*inter] (gate columns first, then up) -> (codes u8 [rows, inter],
    scales f32 [rows, inter/128]) of h = silu(min(gate, limit)) * clamp(up, +-limit) * row weight.
    h_out (f32 [rows, inter]) receives h itself when given."""
    _dev(gu, torch.float32, "gu", 2)
    rows, two_inter = gu.shape
    if two_inter % 2:
        raise ValueError("gu must have 2*inter columns")
    inter = two_inter // 2
    if row_weights is not None:
        _dev(row_weights, torch.float32, "row_weights", 1)
        if row_weights.shape != (rows,):
            raise ValueError("row_weights must be [rows]")
    if codes is None:
        codes = torch.empty((rows, inter), dtype=torch.uint8, device=gu.device)
    if scales is None:
        scales = torch.empty((rows, inter // 128), dtype=torch.float32, device=gu.device)
    _dev(codes, torch.uint8, "codes", 2)
    _dev(scales, torch.float32, "scales", 2)
    if codes.shape != (rows, inter) or scales.shape != (rows, inter // 128):
        raise ValueError("codes/scales shapes do not match gu")
    if h_out is not None:
        _dev(h_out, torch.float32, "h_out", 2)
        if h_out.shape != (rows, inter):
            raise ValueError("h_out must be [rows, inter]")
    _check(lib().swiglu_quant_fp8(_ptr(gu), _ptr(row_weights), float(limit), _ptr(codes), _ptr(scales),
                                  _ptr(h_out), rows, inter, _stream(stream)), "swiglu_quant_fp8")
    return codes, scales


def fp4_expert_gemm(a_codes, a_scales, w_packed, w_scales, scale2: float, kind: int, out=None,
                    stream=None):
    """One expert: a_codes u8 [g, k], a_scales f32 [g, k/128], w_packed u8 [n, k/2],
    w_scales u8 [n, k/gs] -> out f32 [g, n]."""
    _dev(a_codes, torch.uint8, "a_codes", 2)
    _dev(a_scales, torch.float32, "a_scales", 2)
    _dev(w_packed, torch.uint8, "w_packed", 2)
    _dev(w_scales, torch.uint8, "w_scales", 2)
    g, k = a_codes.shape
    n = w_packed.shape[0]
    if kind not in GROUP_SIZE:
        raise ValueError(f"kind must be 0 (NVFP4) or 1 (MXFP4), got {kind}")
    if a_scales.shape != (g, k // 128) or w_packed.shape != (n, k // 2) \
            or w_scales.shape != (n, k // GROUP_SIZE[kind]):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((g, n), dtype=torch.float32, device=a_codes.device)
    _dev(out, torch.float32, "out", 2)
    if out.shape != (g, n):
        raise ValueError("out shape must be [g, n]")
    _check(lib().fp4_expert_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_packed), _ptr(w_scales),
                                 float(scale2), int(kind), _ptr(out), g, n, k, _stream(stream)),
           "fp4_expert_gemm")
    return out


def fp4_grouped_gemm(a_codes, a_scales, row_ids, offsets, w_ptrs, s_ptrs, kinds, scale2, n: int,
                     out=None, stream=None):
    """Routed rows packed per expert.  a_codes u8 [a_rows, k], a_scales f32 [a_rows, k/128],
    row_ids int32 [R] or None, offsets int32 [E+1], w_ptrs/s_ptrs int64 [E] (device addresses),
    kinds int32 [E], scale2 f32 [E] -> out f32 [R, n] with R = offsets[-1] (read on the host
    only from `out`'s shape when out is given; otherwise from row_ids' length)."""
    _dev(a_codes, torch.uint8, "a_codes", 2)
    _dev(a_scales, torch.float32, "a_scales", 2)
    _dev(offsets, torch.int32, "offsets", 1)
    _dev(w_ptrs, torch.int64, "w_ptrs", 1)
    _dev(s_ptrs, torch.int64, "s_ptrs", 1)
    _dev(kinds, torch.int32, "kinds", 1)
    _dev(scale2, torch.float32, "scale2", 1)
    a_rows, k = a_codes.shape
    E = offsets.shape[0] - 1
    if not (w_ptrs.shape[0] == s_ptrs.shape[0] == kinds.shape[0] == scale2.shape[0] == E):
        raise ValueError("per-expert tables must all have num_experts entries")
    if row_ids is not None:
        _dev(row_ids, torch.int32, "row_ids", 1)
        R = row_ids.shape[0]
    elif out is not None:
        R = out.shape[0]
    else:
        raise ValueError("give row_ids or out so that the number of packed rows is known")
    if out is None:
        out = torch.empty((R, n), dtype=torch.float32, device=a_codes.device)
    _dev(out, torch.float32, "out", 2)
    if out.shape != (R, n):
        raise ValueError("out shape must be [total_rows, n]")
    _check(lib().fp4_grouped_gemm(_ptr(a_codes), _ptr(a_scales), a_rows, _ptr(row_ids),
                                  _ptr(offsets), E, R, _ptr(w_ptrs), _ptr(s_ptrs), _ptr(kinds),
                                  _ptr(scale2), _ptr(out), int(n), k, _stream(stream)),
           "fp4_grouped_gemm")
    return out
