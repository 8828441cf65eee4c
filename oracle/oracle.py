"""numpy driver for the plain C oracle (fp4moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.  It shares no code with the HIP library and never imports it.

Every arithmetic step lives in fp4moe_oracle.c (see that file's header for the passages of the
pages each function follows).  This module builds the C file with gcc, marshals numpy arrays, and
adds one independent route: the dequantize-then-dense product, whose dense step is numpy's f64
matmul (a library primitive standing in for the pages' bf16-dequant rung, computed in f64 here).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

NVFP4 = 0
MXFP4 = 1
GROUP_SIZE = {NVFP4: 16, MXFP4: 32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4moe_oracle.c")
_LIB = os.path.join(_HERE, "libfp4moe_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle (host-only C, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
               "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.or_e2m1_value.restype = ctypes.c_double
            lib.or_e2m1_value.argtypes = [ctypes.c_uint]
            lib.or_e4m3_value.restype = ctypes.c_double
            lib.or_e4m3_value.argtypes = [ctypes.c_uint]
            lib.or_e8m0_value.restype = ctypes.c_double
            lib.or_e8m0_value.argtypes = [ctypes.c_uint]
            lib.or_e4m3_encode.restype = ctypes.c_uint
            lib.or_e4m3_encode.argtypes = [ctypes.c_float]
            lib.or_e4m3_encode_many.restype = None
            lib.or_e4m3_encode_many.argtypes = [P, I64, P]
            lib.or_pow2_ceil.restype = ctypes.c_float
            lib.or_pow2_ceil.argtypes = [ctypes.c_float]
            lib.or_act_quant.restype = None
            lib.or_act_quant.argtypes = [P, I64, I64, P, P]
            lib.or_expert_gemm.restype = None
            lib.or_expert_gemm.argtypes = [P, P, P, P, ctypes.c_float, ctypes.c_int, I64, I64, I64,
                                           P, P, ctypes.c_int]
            lib.or_expert_gemm_points.restype = None
            lib.or_expert_gemm_points.argtypes = [P, P, P, P, ctypes.c_float, ctypes.c_int, I64,
                                                  P, P, I64, P, P]
            lib.or_grouped_gemm.restype = None
            lib.or_grouped_gemm.argtypes = [P, P, P, ctypes.c_int32, P, P, P, P, I64, I64, I64,
                                            I64, P, P, ctypes.c_int]
            lib.or_grouped_gemm_points.restype = None
            lib.or_grouped_gemm_points.argtypes = [P, P, P, ctypes.c_int32, P, P, P, P, I64, P, P,
                                                   I64, P, P]
            lib.or_dequant_weights.restype = None
            lib.or_dequant_weights.argtypes = [P, P, ctypes.c_float, ctypes.c_int, I64, I64, P]
            lib.or_dequant_acts.restype = None
            lib.or_dequant_acts.argtypes = [P, P, I64, I64, P]
            lib.or_swiglu.restype = None
            lib.or_swiglu.argtypes = [P, I64, I64, P, ctypes.c_float, P]
            lib.or_route_topk.restype = None
            lib.or_route_topk.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P, P]
            lib.or_route_pack.restype = None
            lib.or_route_pack.argtypes = [P, P, I64, I64, I64, P, P, P, P]
            lib.or_combine.restype = None
            lib.or_combine.argtypes = [P, I64, I64, P, P, I64, I64, P, P]
            lib.or_gather_rows.restype = None
            lib.or_gather_rows.argtypes = [P, P, I64, I64, P, I64, P, P]
            lib.or_e2m1_encode.restype = ctypes.c_uint
            lib.or_e2m1_encode.argtypes = [ctypes.c_float]
            lib.or_act_quant_fp4.restype = None
            lib.or_act_quant_fp4.argtypes = [P, I64, I64, ctypes.c_int, P, P, P]
            lib.or_dequant_acts_fp4.restype = None
            lib.or_dequant_acts_fp4.argtypes = [P, P, P, I64, I64, P]
            lib.or_loud_channels.restype = None
            lib.or_loud_channels.argtypes = [P, I64, I64, I64, P, P]
            lib.or_w4a4_gemm.restype = None
            lib.or_w4a4_gemm.argtypes = [P, P, P, P, P, ctypes.c_float, I64, I64, I64, P, P, I64, P, P, P, P]
            lib.or_cvt_bf16.restype = None
            lib.or_cvt_bf16.argtypes = [P, I64, P]
            lib.or_dequant_bf16.restype = None
            lib.or_dequant_bf16.argtypes = [P, P, ctypes.c_float, ctypes.c_int, I64, I64, P]
            lib.or_gemm_bf16.restype = None
            lib.or_gemm_bf16.argtypes = [P, P, I64, I64, I64, P, P]
            _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# --------------------------------------------------------------------------- element decoders
def e2m1_value(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes)
    return np.array([lib.or_e2m1_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_value(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes)
    return np.array([lib.or_e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e8m0_value(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes)
    return np.array([lib.or_e8m0_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_encode(x) -> np.ndarray:
    """f32 -> E4M3 byte (RNE, sign-preserving zero, saturating) for an array of any shape."""
    lib = _load()
    x, px = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.or_e4m3_encode_many(px, x.size, out.ctypes.data)
    return out


def pow2_ceil(p: float) -> np.float32:
    return np.float32(_load().or_pow2_ceil(float(np.float32(p))))


# --------------------------------------------------------------------------- act-quant
def act_quant(x) -> tuple[np.ndarray, np.ndarray]:
    """x f32 [rows, k] (k % 128 == 0) -> (codes u8 [rows, k], scales f32 [rows, k/128])."""
    lib = _load()
    x, px = _c(x, np.float32)
    rows, k = x.shape
    if k % 128:
        raise ValueError("k must be a multiple of 128")
    codes = np.empty((rows, k), dtype=np.uint8)
    scales = np.empty((rows, k // 128), dtype=np.float32)
    lib.or_act_quant(px, rows, k, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


# --------------------------------------------------------------------------- GEMM (f64 route)
def _check_expert(w, s, kind, n, k):
    gs = GROUP_SIZE[kind]
    if w.shape != (n, k // 2) or s.shape != (n, k // gs):
        raise ValueError(f"weight planes {w.shape}/{s.shape} do not match n={n} k={k} kind={kind}")


def expert_gemm(a_codes, a_scales, w, s, scale2, kind, threads=None):
    """Single expert, f64 quantized route: returns (ref f64 [g, n], absp f64 [g, n])."""
    lib = _load()
    a_codes, pa = _c(a_codes, np.uint8)
    a_scales, ps = _c(a_scales, np.float32)
    w, pw = _c(w, np.uint8)
    s, pss = _c(s, np.uint8)
    g, k = a_codes.shape
    n = w.shape[0]
    _check_expert(w, s, kind, n, k)
    out = np.empty((g, n), dtype=np.float64)
    absp = np.empty((g, n), dtype=np.float64)
    lib.or_expert_gemm(pa, ps, pw, pss, float(np.float32(scale2)), int(kind), g, n, k,
                       out.ctypes.data, absp.ctypes.data, int(threads or default_threads()))
    return out, absp


def expert_gemm_points(a_codes, a_scales, w, s, scale2, kind, rows, cols):
    lib = _load()
    a_codes, pa = _c(a_codes, np.uint8)
    a_scales, ps = _c(a_scales, np.float32)
    w, pw = _c(w, np.uint8)
    s, pss = _c(s, np.uint8)
    rows, pr = _c(rows, np.int64)
    cols, pc = _c(cols, np.int64)
    k = a_codes.shape[1]
    _check_expert(w, s, kind, w.shape[0], k)
    out = np.empty(rows.shape, dtype=np.float64)
    absp = np.empty(rows.shape, dtype=np.float64)
    lib.or_expert_gemm_points(pa, ps, pw, pss, float(np.float32(scale2)), int(kind), k, pr, pc,
                              rows.size, out.ctypes.data, absp.ctypes.data)
    return out, absp


def _expert_tables(weights, scales, kinds, scale2, n, k):
    E = len(weights)
    keep = []
    wp = np.empty(E, dtype=np.uint64)
    sp = np.empty(E, dtype=np.uint64)
    for e in range(E):
        w, pw = _c(weights[e], np.uint8)
        s, ps = _c(scales[e], np.uint8)
        _check_expert(w, s, int(kinds[e]), n, k)
        keep += [w, s]
        wp[e] = pw
        sp[e] = ps
    kinds_a, _ = _c(kinds, np.int32)
    s2, _ = _c(scale2, np.float32)
    return keep, wp, sp, kinds_a, s2


def grouped_gemm(a_codes, a_scales, offsets, weights, scales, kinds, scale2, n,
                 row0=0, row1=None, threads=None):
    """Grouped f64 route over packed rows [row0, row1): (ref, absp) f64 [row1-row0, n].

    weights[e]: u8 [n, k/2]; scales[e]: u8 [n, k/gs(kind[e])]; kinds, scale2: per expert."""
    lib = _load()
    a_codes, pa = _c(a_codes, np.uint8)
    a_scales, ps = _c(a_scales, np.float32)
    offsets, po = _c(offsets, np.int32)
    R, k = a_codes.shape
    row1 = R if row1 is None else row1
    keep, wp, sp, kinds_a, s2 = _expert_tables(weights, scales, kinds, scale2, n, k)
    out = np.full((row1 - row0, n), np.nan, dtype=np.float64)
    absp = np.full((row1 - row0, n), np.nan, dtype=np.float64)
    lib.or_grouped_gemm(pa, ps, po, len(weights), wp.ctypes.data, sp.ctypes.data,
                        kinds_a.ctypes.data, s2.ctypes.data, n, k, row0, row1,
                        out.ctypes.data, absp.ctypes.data, int(threads or default_threads()))
    del keep
    return out, absp


def grouped_gemm_points(a_codes, a_scales, offsets, weights, scales, kinds, scale2, n, rows, cols):
    lib = _load()
    a_codes, pa = _c(a_codes, np.uint8)
    a_scales, ps = _c(a_scales, np.float32)
    offsets, po = _c(offsets, np.int32)
    rows, pr = _c(rows, np.int64)
    cols, pc = _c(cols, np.int64)
    k = a_codes.shape[1]
    keep, wp, sp, kinds_a, s2 = _expert_tables(weights, scales, kinds, scale2, n, k)
    out = np.empty(rows.shape, dtype=np.float64)
    absp = np.empty(rows.shape, dtype=np.float64)
    lib.or_grouped_gemm_points(pa, ps, po, len(weights), wp.ctypes.data, sp.ctypes.data,
                               kinds_a.ctypes.data, s2.ctypes.data, k, pr, pc, rows.size,
                               out.ctypes.data, absp.ctypes.data)
    del keep
    return out, absp


# --------------------------------------------------------------------------- dequant route
def dequant_weights(w, s, scale2, kind) -> np.ndarray:
    lib = _load()
    w, pw = _c(w, np.uint8)
    s, ps = _c(s, np.uint8)
    n, k = w.shape[0], w.shape[1] * 2
    _check_expert(w, s, kind, n, k)
    wd = np.empty((n, k), dtype=np.float64)
    lib.or_dequant_weights(pw, ps, float(np.float32(scale2)), int(kind), n, k, wd.ctypes.data)
    return wd


def dequant_acts(a_codes, a_scales) -> np.ndarray:
    lib = _load()
    a_codes, pa = _c(a_codes, np.uint8)
    a_scales, ps = _c(a_scales, np.float32)
    g, k = a_codes.shape
    ad = np.empty((g, k), dtype=np.float64)
    lib.or_dequant_acts(pa, ps, g, k, ad.ctypes.data)
    return ad


def dense_route(a_codes, a_scales, w, s, scale2, kind) -> np.ndarray:
    """Dequantize both operands in f64 and multiply with numpy's f64 matmul."""
    return dequant_acts(a_codes, a_scales) @ dequant_weights(w, s, scale2, kind).T


# --------------------------------------------------------------------------- acceptance rule
U32 = 2.0 ** -24


def gemm_bound(absp, k) -> np.ndarray:
    """f32-accumulation error bound with the operation count taken as k: k * 2^-24 * sum|p|."""
    return float(k) * U32 * np.asarray(absp, dtype=np.float64)


def pages_op_count(kind, k) -> float:
    """The pages' own op count for their 128-thread kernel: (gs-1) + ceil(groups/128) + 7
    (reported as a diagnostic only)."""
    gs = GROUP_SIZE[kind]
    return (gs - 1) + np.ceil((k / gs) / 128.0) + 7


# --------------------------------------------------------------------------- expert activation

def swiglu(gu, inter: int, limit: float, weights=None) -> np.ndarray:
    """h = silu(min(gate, limit)) * clamp(up, -limit, limit) * weight per row, in f64.

    gu: f32 [rows, 2*inter] (gate columns first, then up); weights: f32 [rows] or None."""
    gu, pg = _c(gu, np.float32)
    rows = gu.shape[0]
    if gu.shape != (rows, 2 * inter):
        raise ValueError("gu must be [rows, 2*inter]")
    pw = None
    if weights is not None:
        weights, pw = _c(weights, np.float32)
        if weights.shape != (rows,):
            raise ValueError("weights must be [rows]")
    h = np.empty((rows, inter), dtype=np.float64)
    _load().or_swiglu(pg, rows, inter, pw, float(limit), h.ctypes.data)
    return h


# --------------------------------------------------------------------------- routing

def route_topk(logits, top_k: int, normalize: bool = False):
    """Top-k experts per token by logit (best first; equal logits by the lower id; NaN last) and
    their softmax weights in f64 (over all experts, or over the k selected with `normalize`).

    logits: f32 [T, E].  Returns (ids int32 [T, k], weights f64 [T, k])."""
    logits, pl = _c(logits, np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    taken = np.empty(max(E, 1), dtype=np.uint8)
    _load().or_route_topk(pl, T, E, top_k, int(bool(normalize)), taken.ctypes.data, ids.ctypes.data,
                          w.ctypes.data)
    return ids, w


def route_pack(ids, experts: int, weights=None):
    """Packs the pairs of ids int32 [T, k] per expert (ascending id, then ascending token).

    Returns (offsets int32 [E+1], row_ids int32 [R], pair_rows int32 [T, k], row_w f32 [R] or None),
    R = offsets[E]; pairs whose id is outside [0, E) are dropped (pair_rows -1)."""
    ids, pi = _c(ids, np.int32)
    T, k = ids.shape
    pw = None
    if weights is not None:
        weights, pw = _c(weights, np.float32)
        if weights.shape != (T, k):
            raise ValueError("weights must be [T, k]")
    offsets = np.empty(experts + 1, dtype=np.int32)
    row_ids = np.empty(T * k, dtype=np.int32)
    pair_rows = np.empty((T, k), dtype=np.int32)
    row_w = np.empty(T * k, dtype=np.float32) if weights is not None else None
    _load().or_route_pack(pi, pw, T, k, experts, offsets.ctypes.data, row_ids.ctypes.data,
                          pair_rows.ctypes.data, None if row_w is None else row_w.ctypes.data)
    R = int(offsets[-1])
    return offsets, row_ids[:R].copy(), pair_rows, None if row_w is None else row_w[:R].copy()


def combine(y, pair_rows, weights=None):
    """out[t] = sum_j weights[t, j] * y[pair_rows[t, j]] in f64 (weights 1 when None), and the
    matching sum of magnitudes.  y: f32 [R, n]; pair_rows int32 [T, k] (-1 = dropped pair)."""
    y, py = _c(y, np.float32)
    pair_rows, pp = _c(pair_rows, np.int32)
    T, k = pair_rows.shape
    n = y.shape[1]
    pw = None
    if weights is not None:
        weights, pw = _c(weights, np.float32)
        if weights.shape != (T, k):
            raise ValueError("weights must be [T, k]")
    out = np.empty((T, n), dtype=np.float64)
    absout = np.empty((T, n), dtype=np.float64)
    _load().or_combine(py, y.shape[0], n, pp, pw, T, k, out.ctypes.data, absout.ctypes.data)
    return out, absout


def gather_rows(codes, scales, row_ids):
    """Rows row_ids of the act-quant codes [a_rows, k] and scales [a_rows, k/128]; a row id
    outside [0, a_rows) gives zero codes and NaN scales."""
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.float32)
    row_ids, pr = _c(row_ids, np.int32)
    a_rows, k = codes.shape
    rows = row_ids.shape[0]
    oc = np.empty((rows, k), dtype=np.uint8)
    osc = np.empty((rows, k // 128), dtype=np.float32)
    _load().or_gather_rows(pc, ps, a_rows, k, pr, rows, oc.ctypes.data, osc.ctypes.data)
    return oc, osc


# --------------------------------------------------------------------------- the bf16-dequant rung

U_FP8 = 2.0 ** -4   # unit roundoff of E4M3 (3 mantissa bits, round to nearest)


def cvt_bf16(x) -> np.ndarray:
    """f32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    x, px = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().or_cvt_bf16(px, x.size, out.ctypes.data)
    return out


def bf16_value(b) -> np.ndarray:
    """Values (f64) of bf16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_bf16(w, s, scale2, kind) -> np.ndarray:
    """The rung's bf16 weights [n, k] (uint16 bit patterns): bf16(f32(E2M1 x ws))."""
    w, pw = _c(w, np.uint8)
    s, ps = _c(s, np.uint8)
    n, k = w.shape[0], w.shape[1] * 2
    _check_expert(w, s, kind, n, k)
    out = np.empty((n, k), dtype=np.uint16)
    _load().or_dequant_bf16(pw, ps, float(np.float32(scale2)), int(kind), n, k, out.ctypes.data)
    return out


def gemm_bf16(a, w):
    """out[r, c] = sum_k a[r, k] w[c, k] over bf16 bit patterns, in f64; and the magnitude sums."""
    a, pa = _c(a, np.uint16)
    w, pw = _c(w, np.uint16)
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("a and w must share k")
    out = np.empty((m, n), dtype=np.float64)
    absout = np.empty((m, n), dtype=np.float64)
    _load().or_gemm_bf16(pa, pw, m, n, k, out.ctypes.data, absout.ctypes.data)
    return out, absout


def class_shift_prediction(x, wd) -> np.ndarray:
    """(U_FP8 / sqrt(3)) * ||x (.) w||_2 per output: x f32 [m, k] (unquantized activations), wd f64
    [n, k] (dequantized weights).  The RMS of the shift that act-quant rounding errors, uniform in
    +-U_FP8 relative and independent across k, would cause."""
    x = np.asarray(x, dtype=np.float64)
    return U_FP8 / np.sqrt(3.0) * np.sqrt((x * x) @ (np.asarray(wd, dtype=np.float64) ** 2).T)


# --------------------------------------------------------------------------- W4A4 NVFP4 variant

def e2m1_encode(v) -> np.ndarray:
    """E2M1 codes of f32 values (nearest grid point, ties to the even code, magnitude capped at 6)."""
    lib = _load()
    v = np.asarray(v, dtype=np.float32)
    return np.array([lib.or_e2m1_encode(float(t)) for t in v.ravel()], dtype=np.uint8).reshape(v.shape)


def act_quant_fp4(x, two_level: bool = True):
    """W4A4 activations: (codes u8 [rows, k/2] nibble-packed, micro u8 [rows, k/16] UE4M3,
    row_scale f32 [rows]).  two_level=False is the sub-block-only quantizer (row scale 1)."""
    x, px = _c(x, np.float32)
    rows, k = x.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    codes = np.empty((rows, k // 2), dtype=np.uint8)
    micro = np.empty((rows, k // 16), dtype=np.uint8)
    rs = np.empty(rows, dtype=np.float32)
    _load().or_act_quant_fp4(px, rows, k, int(bool(two_level)), codes.ctypes.data, micro.ctypes.data,
                             rs.ctypes.data)
    return codes, micro, rs


def dequant_acts_fp4(codes, micro, row_scale) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    micro, pm = _c(micro, np.uint8)
    row_scale, pr = _c(row_scale, np.float32)
    rows, k = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, k), dtype=np.float64)
    _load().or_dequant_acts_fp4(pc, pm, pr, rows, k, out.ctypes.data)
    return out


def loud_channels(x, k_res: int) -> np.ndarray:
    """Indices of the k_res channels with the largest max |x| over tokens (ties to the lower index)."""
    x, px = _c(x, np.float32)
    rows, k = x.shape
    idx = np.empty(k_res, dtype=np.int32)
    taken = np.empty(k, dtype=np.uint8)
    _load().or_loud_channels(px, rows, k, int(k_res), taken.ctypes.data, idx.ctypes.data)
    return idx


def w4a4_gemm(codes, micro, row_scale, w, s, scale2, x=None, idx=None):
    """f64 W4A4 GEMM on the quantized operands (NVFP4 weights), plus the exact contribution of the
    kept channels idx of x when given.  Returns (out [g, n], sum of magnitudes)."""
    codes, pc = _c(codes, np.uint8)
    micro, pm = _c(micro, np.uint8)
    row_scale, prs = _c(row_scale, np.float32)
    w, pw = _c(w, np.uint8)
    s, ps = _c(s, np.uint8)
    g, k = codes.shape[0], codes.shape[1] * 2
    n = w.shape[0]
    _check_expert(w, s, NVFP4, n, k)
    k_res = 0 if idx is None else len(idx)
    px = pidx = None
    if k_res:
        x, px = _c(x, np.float32)
        idx, pidx = _c(idx, np.int32)
    ad = np.empty((g, k), dtype=np.float64)
    wd = np.empty((n, k), dtype=np.float64)
    out = np.empty((g, n), dtype=np.float64)
    absout = np.empty((g, n), dtype=np.float64)
    _load().or_w4a4_gemm(pc, pm, prs, pw, ps, float(np.float32(scale2)), g, n, k, px, pidx, k_res,
                         ad.ctypes.data, wd.ctypes.data, out.ctypes.data, absout.ctypes.data)
    return out, absout
