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
SWIZZLED = 2          # layout flag OR'ed into a kind: planes written by fp4_weight_swizzle
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
        L.fp4_grouped_gemm.argtypes = [P, P, P, I32, I32, P, P, P, P, P, I32, I32, P, ctypes.c_size_t, P]
        L.fp4_grouped_gemm.restype = ctypes.c_int
        L.fp4_grouped_gemm_workspace_size.argtypes = [I32, I32, I32, I32]
        L.fp4_grouped_gemm_workspace_size.restype = ctypes.c_size_t
        L.fp4_grouped_gemm_gather.argtypes = [P, P, I32, P, P, I32, I32, P, P, P, P, P, I32, I32, P]
        L.fp4_grouped_gemm_gather.restype = ctypes.c_int
        L.fp4moe_set_debug_checks.argtypes = [I32]
        L.fp4moe_set_debug_checks.restype = ctypes.c_int
        L.fp4_grouped_gemm_swiglu_quant.argtypes = [P, P, I32, P, P, I32, I32, P, P, P, P, I32, I32, P, F32,
                                                    P, P, P, P]
        L.fp4_grouped_gemm_swiglu_quant.restype = ctypes.c_int
        L.route_softmax_topk.argtypes = [P, I32, I32, I32, I32, P, P, P]
        L.route_softmax_topk.restype = ctypes.c_int
        L.route_pack_workspace_size.argtypes = [I32, I32]
        L.route_pack_workspace_size.restype = ctypes.c_int64
        L.route_pack.argtypes = [P, P, I32, I32, I32, P, P, P, P, P, P]
        L.route_pack.restype = ctypes.c_int
        L.route_pack_noalloc.argtypes = [P, P, I32, I32, I32, P, P, P, P, P]
        L.route_pack_noalloc.restype = ctypes.c_int
        L.gather_quant_rows.argtypes = [P, P, I32, I32, P, I32, P, P, P]
        L.gather_quant_rows.restype = ctypes.c_int
        L.moe_combine.argtypes = [P, I32, I32, P, P, I32, I32, P, P]
        L.moe_combine.restype = ctypes.c_int
        L.cvt_bf16.argtypes = [P, P, ctypes.c_int64, P]
        L.cvt_bf16.restype = ctypes.c_int
        L.fp4_dequant_bf16.argtypes = [P, P, F32, I32, I32, I32, P, P]
        L.fp4_dequant_bf16.restype = ctypes.c_int
        L.gemm_bf16.argtypes = [P, P, P, I32, I32, I32, P]
        L.gemm_bf16.restype = ctypes.c_int
        L.act_quant_fp4.argtypes = [P, P, I32, P, P, P, I32, I32, I32, P]
        L.act_quant_fp4.restype = ctypes.c_int
        L.loud_channels.argtypes = [P, I32, I32, I32, P, P]
        L.loud_channels.restype = ctypes.c_int
        L.w4a4_gemm.argtypes = [P, P, P, P, P, F32, P, P, I32, P, I32, I32, I32, P]
        L.w4a4_gemm.restype = ctypes.c_int
        L.fp4moe_last_error.argtypes = []
        L.fp4moe_last_error.restype = ctypes.c_char_p
        L.fp4moe_version.argtypes = []
        L.fp4moe_version.restype = ctypes.c_char_p
        L.fp4moe_set_gemm_schedule.argtypes = [I32]
        L.fp4moe_set_gemm_schedule.restype = ctypes.c_int
        L.fp4_swizzled_weight_bytes.restype = ctypes.c_size_t
        L.fp4_swizzled_weight_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.fp4_swizzled_scale_bytes.restype = ctypes.c_size_t
        L.fp4_swizzled_scale_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.fp4_weight_swizzle.restype = ctypes.c_int
        L.fp4_weight_swizzle.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def version() -> str:
    return lib().fp4moe_version().decode()


SCHEDULE_AUTO, SCHEDULE_ROWSTREAM, SCHEDULE_TILED, SCHEDULE_SPLITK = 0, 1, 2, 3


def set_gemm_schedule(schedule: int) -> None:
    """Force the GEMM kernel choice (0 automatic, 1 row-streaming, 2 tiled, 3 split-k for
    single-expert calls with g <= 16 and k <= 8192); a test hook."""
    _check(lib().fp4moe_set_gemm_schedule(int(schedule)), "fp4moe_set_gemm_schedule")


def set_debug_checks(on: bool) -> None:
    """Validate every grouped call's tables on the device first (synchronizes; FP4MOE_EDEVICE,
    raised as Fp4MoeError, when they break the CSR contract); a debugging aid."""
    _check(lib().fp4moe_set_debug_checks(1 if on else 0), "fp4moe_set_debug_checks")


OK, EINVAL, ELAUNCH, EDEVICE = 0, 1, 2, 3


class Fp4MoeCallError(Fp4MoeError):
    """A library call returned a nonzero code (rc: EINVAL, ELAUNCH or EDEVICE)."""

    def __init__(self, msg: str, rc: int):
        super().__init__(msg)
        self.rc = rc


def _check(rc: int, what: str):
    if rc != 0:
        raise Fp4MoeCallError(f"{what} failed (rc={rc}): {lib().fp4moe_last_error().decode()}", rc)


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


def swizzled_plane_bytes(kind: int, n: int, k: int):
    """(nibble bytes, scale bytes) of one expert's swizzled planes."""
    L = lib()
    wb, sb = L.fp4_swizzled_weight_bytes(int(n), int(k)), L.fp4_swizzled_scale_bytes(int(kind), int(n), int(k))
    if wb == 0 or sb == 0:
        raise ValueError(f"no swizzled layout for kind={kind} n={n} k={k}")
    return int(wb), int(sb)


def fp4_weight_swizzle(w_packed, w_scales, kind: int, w_out=None, s_out=None, stream=None):
    """One expert's plain planes (w_packed u8 [n, k/2], w_scales u8 [n, k/gs]) -> the swizzled
    planes (u8 1-D tensors) that the GEMMs read with kind | SWIZZLED."""
    _dev(w_packed, torch.uint8, "w_packed", 2)
    _dev(w_scales, torch.uint8, "w_scales", 2)
    if kind not in GROUP_SIZE:
        raise ValueError(f"kind must be 0 (NVFP4) or 1 (MXFP4), got {kind}")
    n, k = w_packed.shape[0], 2 * w_packed.shape[1]
    if w_scales.shape != (n, k // GROUP_SIZE[kind]):
        raise ValueError("w_scales shape does not match w_packed")
    wb, sb = swizzled_plane_bytes(kind, n, k)
    if w_out is None:
        w_out = torch.empty(wb, dtype=torch.uint8, device=w_packed.device)
    if s_out is None:
        s_out = torch.empty(sb, dtype=torch.uint8, device=w_packed.device)
    _dev(w_out, torch.uint8, "w_out")
    _dev(s_out, torch.uint8, "s_out")
    if w_out.numel() != wb or s_out.numel() != sb:
        raise ValueError(f"swizzled planes must hold {wb} and {sb} bytes")
    _check(lib().fp4_weight_swizzle(_ptr(w_packed), _ptr(w_scales), int(kind), n, k, _ptr(w_out), _ptr(s_out),
                                    _stream(stream)), "fp4_weight_swizzle")
    return w_out, s_out


def fp4_expert_gemm(a_codes, a_scales, w_packed, w_scales, scale2: float, kind: int, out=None,
                    stream=None, n=None):
    """One expert: a_codes u8 [g, k], a_scales f32 [g, k/128], w_packed u8 [n, k/2],
    w_scales u8 [n, k/gs] -> out f32 [g, n].  With kind | SWIZZLED the planes are the 1-D
    tensors of fp4_weight_swizzle and n must be given."""
    _dev(a_codes, torch.uint8, "a_codes", 2)
    _dev(a_scales, torch.float32, "a_scales", 2)
    g, k = a_codes.shape
    kind = int(kind)
    base = kind & ~SWIZZLED if kind >= 0 else kind
    if base not in GROUP_SIZE or kind > (MXFP4 | SWIZZLED):
        raise ValueError(f"kind must be 0/1 (NVFP4/MXFP4), or 2/3 for swizzled planes, got {kind}")
    if kind & SWIZZLED:
        _dev(w_packed, torch.uint8, "w_packed", 1)
        _dev(w_scales, torch.uint8, "w_scales", 1)
        if n is None:
            raise ValueError("n must be given with swizzled planes")
        n = int(n)
        if (w_packed.numel(), w_scales.numel()) != swizzled_plane_bytes(base, n, k):
            raise ValueError("swizzled plane sizes do not match n and k")
        if a_scales.shape != (g, k // 128):
            raise ValueError("operand shapes do not match")
    else:
        _dev(w_packed, torch.uint8, "w_packed", 2)
        _dev(w_scales, torch.uint8, "w_scales", 2)
        n = w_packed.shape[0]
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


def _grouped_tables(offsets, w_ptrs, s_ptrs, kinds, scale2):
    _dev(offsets, torch.int32, "offsets", 1)
    _dev(w_ptrs, torch.int64, "w_ptrs", 1)
    _dev(s_ptrs, torch.int64, "s_ptrs", 1)
    _dev(kinds, torch.int32, "kinds", 1)
    _dev(scale2, torch.float32, "scale2", 1)
    E = offsets.shape[0] - 1
    if not (w_ptrs.shape[0] == s_ptrs.shape[0] == kinds.shape[0] == scale2.shape[0] == E):
        raise ValueError("per-expert tables must all have num_experts entries")
    return E


def _act_operands(a_codes, a_scales):
    _dev(a_codes, torch.uint8, "a_codes", 2)
    _dev(a_scales, torch.float32, "a_scales", 2)
    a_rows, k = a_codes.shape
    if k % 128 or a_scales.shape != (a_rows, k // 128):
        raise ValueError("a_codes must be [rows, k] with k % 128 == 0 and a_scales [rows, k/128]")
    return a_rows, k


def grouped_gemm_workspace_size(num_experts: int, total_rows: int, n: int, k: int) -> int:
    return int(lib().fp4_grouped_gemm_workspace_size(int(num_experts), int(total_rows), int(n), int(k)))


def fp4_grouped_gemm(a_codes, a_scales, offsets, w_ptrs, s_ptrs, kinds, scale2, n: int, out=None,
                     workspace=None, stream=None):
    """Routed rows packed per expert (the C ABI's fp4_grouped_gemm).  a_codes u8 [R, k] and
    a_scales f32 [R, k/128] in packed order, offsets int32 [E+1], w_ptrs/s_ptrs int64 [E] (device
    addresses), kinds int32 [E] (0/1 NVFP4/MXFP4, | SWIZZLED for swizzled planes), scale2 f32 [E]
    -> out f32 [R, n].  workspace: a uint8 device tensor of at least grouped_gemm_workspace_size()
    bytes, or None when that size is 0."""
    R, k = _act_operands(a_codes, a_scales)
    E = _grouped_tables(offsets, w_ptrs, s_ptrs, kinds, scale2)
    if out is None:
        out = torch.empty((R, n), dtype=torch.float32, device=a_codes.device)
    _dev(out, torch.float32, "out", 2)
    if out.shape != (R, n):
        raise ValueError("out shape must be [total_rows, n]")
    wbytes = 0
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace", 1)
        wbytes = workspace.numel()
    _check(lib().fp4_grouped_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(offsets), E, R, _ptr(w_ptrs),
                                  _ptr(s_ptrs), _ptr(kinds), _ptr(scale2), _ptr(out), int(n), k,
                                  _ptr(workspace), wbytes, _stream(stream)),
           "fp4_grouped_gemm")
    return out


def fp4_grouped_gemm_gather(a_codes, a_scales, row_ids, offsets, w_ptrs, s_ptrs, kinds, scale2, n: int,
                            out=None, stream=None):
    """fp4_grouped_gemm with the activations read through a gather table.  a_codes u8 [a_rows, k],
    a_scales f32 [a_rows, k/128] (e.g. one row per token), row_ids int32 [R] or None, offsets int32
    [E+1], the per-expert tables as for fp4_grouped_gemm -> out f32 [R, n] with R = offsets[-1]
    (taken on the host from `out`'s shape when out is given, otherwise from row_ids' length)."""
    a_rows, k = _act_operands(a_codes, a_scales)
    E = _grouped_tables(offsets, w_ptrs, s_ptrs, kinds, scale2)
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
    _check(lib().fp4_grouped_gemm_gather(_ptr(a_codes), _ptr(a_scales), a_rows, _ptr(row_ids),
                                         _ptr(offsets), E, R, _ptr(w_ptrs), _ptr(s_ptrs), _ptr(kinds),
                                         _ptr(scale2), _ptr(out), int(n), k, _stream(stream)),
           "fp4_grouped_gemm_gather")
    return out


def fp4_grouped_gemm_swiglu_quant(a_codes, a_scales, row_ids, offsets, w_ptrs, s_ptrs, kinds, scale2,
                                  inter: int, limit: float, row_weights=None, h_codes=None, h_scales=None,
                                  h_out=None, stream=None):
    """The gate/up projection fused with the expert activation and its FP8 quantization: the
    arguments of fp4_grouped_gemm_gather (expert planes [2*inter, k/2], gate columns first) plus those of
    swiglu_quant_fp8 -> (h_codes u8 [R, inter], h_scales f32 [R, inter/128]), R = len(row_ids)
    (or h_codes' rows when row_ids is None).  h_out (f32 [R, inter]) receives h when given."""
    a_rows, k = _act_operands(a_codes, a_scales)
    E = _grouped_tables(offsets, w_ptrs, s_ptrs, kinds, scale2)
    inter = int(inter)
    if inter <= 0 or inter % 128:
        raise ValueError("inter must be a positive multiple of 128")
    if row_ids is not None:
        _dev(row_ids, torch.int32, "row_ids", 1)
        R = row_ids.shape[0]
    elif h_codes is not None:
        R = h_codes.shape[0]
    else:
        raise ValueError("give row_ids or h_codes so that the number of packed rows is known")
    if h_codes is None:
        h_codes = torch.empty((R, inter), dtype=torch.uint8, device=a_codes.device)
    if h_scales is None:
        h_scales = torch.empty((R, inter // 128), dtype=torch.float32, device=a_codes.device)
    _dev(h_codes, torch.uint8, "h_codes", 2)
    _dev(h_scales, torch.float32, "h_scales", 2)
    if h_codes.shape != (R, inter) or h_scales.shape != (R, inter // 128):
        raise ValueError("h_codes/h_scales shapes must be [R, inter] and [R, inter/128]")
    if row_weights is not None:
        _dev(row_weights, torch.float32, "row_weights", 1)
        if row_weights.shape != (R,):
            raise ValueError("row_weights must be [R]")
    if h_out is not None:
        _dev(h_out, torch.float32, "h_out", 2)
        if h_out.shape != (R, inter):
            raise ValueError("h_out must be [R, inter]")
    _check(lib().fp4_grouped_gemm_swiglu_quant(_ptr(a_codes), _ptr(a_scales), a_rows, _ptr(row_ids), _ptr(offsets),
                                               E, R, _ptr(w_ptrs), _ptr(s_ptrs), _ptr(kinds), _ptr(scale2), inter,
                                               k, _ptr(row_weights), float(limit), _ptr(h_codes), _ptr(h_scales),
                                               _ptr(h_out), _stream(stream)),
           "fp4_grouped_gemm_swiglu_quant")
    return h_codes, h_scales


# --------------------------------------------------------------------------- routing

def route_softmax_topk(logits, top_k: int, normalize: bool = False, ids=None, weights=None, stream=None):
    """logits f32 [T, E] -> (ids int32 [T, top_k], weights f32 [T, top_k]): the top_k experts per
    token, best first (equal logits by the lower id), with their softmax weights (over all experts,
    or over the selection with normalize)."""
    _dev(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _dev(ids, torch.int32, "ids", 2)
    _dev(weights, torch.float32, "weights", 2)
    if ids.shape != (T, top_k) or weights.shape != (T, top_k):
        raise ValueError("ids/weights must be [T, top_k]")
    _check(lib().route_softmax_topk(_ptr(logits), T, E, int(top_k), int(bool(normalize)), _ptr(ids),
                                    _ptr(weights), _stream(stream)), "route_softmax_topk")
    return ids, weights


def route_pack_workspace_size(tokens: int, experts: int) -> int:
    return int(lib().route_pack_workspace_size(int(tokens), int(experts)))


def route_pack(topk_ids, experts: int, topk_weights=None, offsets=None, row_ids=None, pair_rows=None,
               row_weights=None, workspace=None, stream=None):
    """topk_ids int32 [T, k] -> (offsets int32 [E+1], row_ids int32 [T*k], pair_rows int32 [T, k],
    row_weights f32 [T*k] or None).  Rows 0 .. offsets[E]-1 of row_ids/row_weights are written."""
    _dev(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    if topk_weights is not None:
        _dev(topk_weights, torch.float32, "topk_weights", 2)
        if topk_weights.shape != (T, k):
            raise ValueError("topk_weights must be [T, k]")
        if row_weights is None:
            row_weights = torch.empty(T * k, dtype=torch.float32, device=dev)
        _dev(row_weights, torch.float32, "row_weights", 1)
    if offsets is None:
        offsets = torch.empty(experts + 1, dtype=torch.int32, device=dev)
    if row_ids is None:
        row_ids = torch.empty(T * k, dtype=torch.int32, device=dev)
    if pair_rows is None:
        pair_rows = torch.empty((T, k), dtype=torch.int32, device=dev)
    _dev(offsets, torch.int32, "offsets", 1)
    _dev(row_ids, torch.int32, "row_ids", 1)
    _dev(pair_rows, torch.int32, "pair_rows", 2)
    if offsets.shape != (experts + 1,) or row_ids.shape != (T * k,) or pair_rows.shape != (T, k):
        raise ValueError("offsets must be [E+1], row_ids [T*k], pair_rows [T, k]")
    if row_weights is not None and row_weights.shape != (T * k,):
        raise ValueError("row_weights must be [T*k]")
    need = route_pack_workspace_size(T, experts)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _dev(workspace, torch.uint8, "workspace")
    if workspace.numel() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(lib().route_pack(_ptr(topk_ids), _ptr(topk_weights), T, k, int(experts), _ptr(offsets),
                            _ptr(row_ids), _ptr(pair_rows), _ptr(row_weights), _ptr(workspace),
                            _stream(stream)), "route_pack")
    return offsets, row_ids, pair_rows, row_weights


def gather_quant_rows(codes, scales, row_ids, out_codes=None, out_scales=None, stream=None):
    """codes u8 [a_rows, k], scales f32 [a_rows, k/128], row_ids int32 [rows] -> the rows row_ids
    (zero codes and NaN scales for ids outside [0, a_rows))."""
    _dev(codes, torch.uint8, "codes", 2)
    _dev(scales, torch.float32, "scales", 2)
    _dev(row_ids, torch.int32, "row_ids", 1)
    a_rows, k = codes.shape
    rows = row_ids.shape[0]
    if out_codes is None:
        out_codes = torch.empty((rows, k), dtype=torch.uint8, device=codes.device)
    if out_scales is None:
        out_scales = torch.empty((rows, k // 128), dtype=torch.float32, device=codes.device)
    _dev(out_codes, torch.uint8, "out_codes", 2)
    _dev(out_scales, torch.float32, "out_scales", 2)
    if scales.shape != (a_rows, k // 128) or out_codes.shape != (rows, k) or out_scales.shape != (rows, k // 128):
        raise ValueError("shape mismatch between codes/scales and the outputs")
    _check(lib().gather_quant_rows(_ptr(codes), _ptr(scales), a_rows, k, _ptr(row_ids), rows, _ptr(out_codes),
                                   _ptr(out_scales), _stream(stream)), "gather_quant_rows")
    return out_codes, out_scales


def moe_combine(y, pair_rows, pair_weights=None, out=None, stream=None):
    """y f32 [R, n] (packed expert outputs), pair_rows int32 [T, k] -> out f32 [T, n] with
    out[t] = sum_j pair_weights[t, j] * y[pair_rows[t, j]] (weights 1 when None; rows < 0 skipped)."""
    _dev(y, torch.float32, "y", 2)
    _dev(pair_rows, torch.int32, "pair_rows", 2)
    T, k = pair_rows.shape
    y_rows, n = y.shape
    if pair_weights is not None:
        _dev(pair_weights, torch.float32, "pair_weights", 2)
        if pair_weights.shape != (T, k):
            raise ValueError("pair_weights must be [T, k]")
    if out is None:
        out = torch.empty((T, n), dtype=torch.float32, device=y.device)
    _dev(out, torch.float32, "out", 2)
    if out.shape != (T, n):
        raise ValueError("out must be [T, n]")
    _check(lib().moe_combine(_ptr(y), y_rows, n, _ptr(pair_rows), _ptr(pair_weights), T, k, _ptr(out),
                             _stream(stream)), "moe_combine")
    return out


# --------------------------------------------------------------------------- the bf16-dequant rung

def cvt_bf16(x, out=None, stream=None):
    """f32 tensor -> bf16 tensor of the same shape (round to nearest even)."""
    _dev(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out")
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    _check(lib().cvt_bf16(_ptr(x), _ptr(out), x.numel(), _stream(stream)), "cvt_bf16")
    return out


def fp4_dequant_bf16(w_packed, w_scales, scale2: float, kind: int, out=None, stream=None):
    """Expert weights u8 [n, k/2] + scales u8 [n, k/gs] -> bf16 [n, k] (the rung's weights)."""
    _dev(w_packed, torch.uint8, "w_packed", 2)
    _dev(w_scales, torch.uint8, "w_scales", 2)
    n, k = w_packed.shape[0], w_packed.shape[1] * 2
    if w_scales.shape != (n, k // GROUP_SIZE[int(kind)]):
        raise ValueError("w_scales shape does not match w_packed and kind")
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=w_packed.device)
    _dev(out, torch.bfloat16, "out", 2)
    if out.shape != (n, k):
        raise ValueError("out must be [n, k]")
    _check(lib().fp4_dequant_bf16(_ptr(w_packed), _ptr(w_scales), float(scale2), int(kind), n, k, _ptr(out),
                                  _stream(stream)), "fp4_dequant_bf16")
    return out


def gemm_bf16(a, w, out=None, stream=None):
    """a bf16 [m, k], w bf16 [n, k] -> out f32 [m, n] = a w^T (f32 accumulation)."""
    _dev(a, torch.bfloat16, "a", 2)
    _dev(w, torch.bfloat16, "w", 2)
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("a and w must share k")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _dev(out, torch.float32, "out", 2)
    if out.shape != (m, n):
        raise ValueError("out must be [m, n]")
    _check(lib().gemm_bf16(_ptr(a), _ptr(w), _ptr(out), m, n, k, _stream(stream)), "gemm_bf16")
    return out


# --------------------------------------------------------------------------- W4A4 NVFP4 variant

def act_quant_fp4(x, two_level: bool = True, skip_channels=None, codes=None, micro=None, row_scale=None,
                  stream=None):
    """x f32 [rows, k] -> (codes u8 [rows, k/2], micro u8 [rows, k/16] UE4M3, row_scale f32 [rows]);
    channels in skip_channels (int32 [n]) count as zero."""
    _dev(x, torch.float32, "x", 2)
    rows, k = x.shape
    n_skip = 0
    if skip_channels is not None:
        _dev(skip_channels, torch.int32, "skip_channels", 1)
        n_skip = skip_channels.shape[0]
    if codes is None:
        codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if micro is None:
        micro = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    if row_scale is None:
        row_scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _dev(codes, torch.uint8, "codes", 2)
    _dev(micro, torch.uint8, "micro", 2)
    _dev(row_scale, torch.float32, "row_scale", 1)
    if codes.shape != (rows, k // 2) or micro.shape != (rows, k // 16) or row_scale.shape != (rows,):
        raise ValueError("output shapes do not match x")
    _check(lib().act_quant_fp4(_ptr(x), _ptr(skip_channels), n_skip, _ptr(codes), _ptr(micro), _ptr(row_scale),
                               rows, k, int(bool(two_level)), _stream(stream)), "act_quant_fp4")
    return codes, micro, row_scale


def loud_channels(x, k_res: int, idx=None, stream=None):
    """The k_res channels of x f32 [rows, k] with the largest max |x|, loudest first (int32)."""
    _dev(x, torch.float32, "x", 2)
    rows, k = x.shape
    if idx is None:
        idx = torch.empty(k_res, dtype=torch.int32, device=x.device)
    _dev(idx, torch.int32, "idx", 1)
    if idx.shape != (k_res,):
        raise ValueError("idx must be [k_res]")
    _check(lib().loud_channels(_ptr(x), rows, k, int(k_res), _ptr(idx), _stream(stream)), "loud_channels")
    return idx


def w4a4_gemm(codes, micro, row_scale, w_packed, w_scales, scale2: float, x=None, res_idx=None, out=None,
              stream=None):
    """W4A4 GEMM with NVFP4 weights -> out f32 [g, n]; res_idx (int32 [k_res]) adds the kept channels of
    x f32 [g, k] exactly."""
    _dev(codes, torch.uint8, "codes", 2)
    _dev(micro, torch.uint8, "micro", 2)
    _dev(row_scale, torch.float32, "row_scale", 1)
    _dev(w_packed, torch.uint8, "w_packed", 2)
    _dev(w_scales, torch.uint8, "w_scales", 2)
    g, k = codes.shape[0], codes.shape[1] * 2
    n = w_packed.shape[0]
    if w_packed.shape != (n, k // 2) or w_scales.shape != (n, k // 16) or micro.shape != (g, k // 16):
        raise ValueError("operand shapes do not match")
    k_res = 0
    if res_idx is not None:
        _dev(res_idx, torch.int32, "res_idx", 1)
        _dev(x, torch.float32, "x", 2)
        k_res = res_idx.shape[0]
    if out is None:
        out = torch.empty((g, n), dtype=torch.float32, device=codes.device)
    _dev(out, torch.float32, "out", 2)
    _check(lib().w4a4_gemm(_ptr(codes), _ptr(micro), _ptr(row_scale), _ptr(w_packed), _ptr(w_scales),
                           float(scale2), _ptr(x) if k_res else None, _ptr(res_idx), k_res, _ptr(out), g, n, k,
                           _stream(stream)), "w4a4_gemm")
    return out
