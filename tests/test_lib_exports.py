"""The C-ABI library loads, exports every function include/*.h declares, and rejects invalid
arguments on the host (these calls enqueue nothing, so no GPU is needed)."""
import ctypes
import glob
import os
import re

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "block_scaled_fp4_quant_amd", "libfp4moe.so")


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"FP4MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    import block_scaled_fp4_quant_amd as m
    return m.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("act_quant_fp8", "swiglu_quant_fp8", "fp4_expert_gemm", "fp4_grouped_gemm",
               "fp4_grouped_gemm_workspace_size", "fp4_grouped_gemm_gather", "fp4_grouped_gemm_swiglu_quant",
               "fp4moe_set_debug_checks", "fp4moe_last_error", "fp4moe_version"):
        assert fn in names


def test_header_return_codes():
    text = open(os.path.join(ROOT, "include", "fp4moe.h")).read()
    m = re.search(r"enum\s*\{\s*FP4MOE_OK\s*=\s*0\s*,\s*FP4MOE_EINVAL\s*=\s*1\s*,\s*FP4MOE_ELAUNCH\s*=\s*2\s*,"
                  r"\s*FP4MOE_EDEVICE\s*=\s*3\s*\}", text)
    assert m, "return codes OK=0, EINVAL=1, ELAUNCH=2, EDEVICE=3"
    import block_scaled_fp4_quant_amd as fp4
    assert (fp4.OK, fp4.EINVAL, fp4.ELAUNCH, fp4.EDEVICE) == (0, 1, 2, 3)


def test_every_declared_symbol_is_exported(lib):
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


def test_version(lib):
    import block_scaled_fp4_quant_amd as m
    assert "gfx950" in m.version()


NULL = None
BAD = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("rows,k", [(-1, 128), (4, 0), (4, 100), (4, 129)])
def test_act_quant_rejects(lib, rows, k):
    assert lib.act_quant_fp8(BAD, BAD, BAD, rows, k, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("act_quant_fp8")


def test_act_quant_null_and_noop(lib):
    assert lib.act_quant_fp8(NULL, BAD, BAD, 4, 128, NULL) == 1
    assert lib.act_quant_fp8(NULL, NULL, NULL, 0, 128, NULL) == 0      # rows == 0: no-op
    assert lib.fp4moe_last_error().decode() == ""


@pytest.mark.parametrize("rows,inter,limit", [(-1, 128, 7.0), (4, 0, 7.0), (4, 96, 7.0), (4, 200, 7.0),
                                              (4, 128, 0.0), (4, 128, -1.0), (4, 128, float("nan"))])
def test_swiglu_quant_rejects(lib, rows, inter, limit):
    assert lib.swiglu_quant_fp8(BAD, NULL, limit, BAD, BAD, NULL, rows, inter, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("swiglu_quant_fp8")


def test_swiglu_quant_null_and_noop(lib):
    assert lib.swiglu_quant_fp8(NULL, NULL, 7.0, BAD, BAD, NULL, 4, 128, NULL) == 1
    assert lib.swiglu_quant_fp8(BAD, NULL, 7.0, BAD, NULL, NULL, 4, 128, NULL) == 1
    assert lib.swiglu_quant_fp8(NULL, NULL, 7.0, NULL, NULL, NULL, 0, 128, NULL) == 0   # no-op
    assert lib.fp4moe_last_error().decode() == ""


@pytest.mark.parametrize("g,n,k,kind", [(-1, 16, 128, 0), (4, 0, 128, 0), (4, 16, 96, 0),
                                        (4, 16, 128, 4), (4, 16, 128, -1), (1 << 24, 16, 256, 0),
                                        (4, 1 << 20, 8192, 1)])
def test_expert_gemm_rejects(lib, g, n, k, kind):
    assert lib.fp4_expert_gemm(BAD, BAD, BAD, BAD, 1.0, kind, BAD, g, n, k, NULL) == 1
    assert "fp4_expert_gemm" in lib.fp4moe_last_error().decode()


def test_expert_gemm_null_and_noop(lib):
    assert lib.fp4_expert_gemm(BAD, BAD, NULL, BAD, 1.0, 0, BAD, 4, 16, 128, NULL) == 1
    assert lib.fp4_expert_gemm(NULL, NULL, NULL, NULL, 1.0, 1, NULL, 0, 16, 128, NULL) == 0


@pytest.mark.parametrize("a_rows,row_ids,E,R,n,k", [(-1, BAD, 4, 8, 16, 128), (8, BAD, 4, -1, 16, 128),
                                                    (8, BAD, 0, 8, 16, 128), (8, BAD, 4, 8, 0, 128),
                                                    (8, BAD, 4, 8, 16, 200), (4, NULL, 4, 8, 16, 128)])
def test_grouped_gemm_gather_rejects(lib, a_rows, row_ids, E, R, n, k):
    assert lib.fp4_grouped_gemm_gather(BAD, BAD, a_rows, row_ids, BAD, E, R, BAD, BAD, BAD, BAD, BAD,
                                       n, k, NULL) == 1
    assert "fp4_grouped_gemm_gather" in lib.fp4moe_last_error().decode()


def test_grouped_gemm_gather_null_and_noop(lib):
    assert lib.fp4_grouped_gemm_gather(BAD, BAD, 8, BAD, NULL, 4, 8, BAD, BAD, BAD, BAD, BAD, 16, 128, NULL) == 1
    assert lib.fp4_grouped_gemm_gather(NULL, NULL, 0, NULL, NULL, 4, 0, NULL, NULL, NULL, NULL, NULL,
                                       16, 128, NULL) == 0


def test_grouped_gemm_workspace_size(lib):
    # the packed-rows grouped GEMM needs no scratch: every kernel finds its tiles from the offsets
    for E, R, n, k in [(1, 1, 16, 128), (256, 4096, 2048, 7168), (256, 65536, 4096, 7168), (4, 0, 16, 128)]:
        assert lib.fp4_grouped_gemm_workspace_size(E, R, n, k) == 0


@pytest.mark.parametrize("E,R,n,k", [(4, -1, 16, 128), (0, 8, 16, 128), (4, 8, 0, 128), (4, 8, 16, 200),
                                     (4, 8, 16, 0), (4, 1 << 24, 16, 256)])
def test_grouped_gemm_rejects(lib, E, R, n, k):
    assert lib.fp4_grouped_gemm(BAD, BAD, BAD, E, R, BAD, BAD, BAD, BAD, BAD, n, k, NULL, 0, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("fp4_grouped_gemm:")


def test_grouped_gemm_workspace_and_null_checks(lib):
    f = lib.fp4_grouped_gemm
    # a NULL workspace with a nonzero size
    assert f(BAD, BAD, BAD, 4, 8, BAD, BAD, BAD, BAD, BAD, 16, 128, NULL, 64, NULL) == 1
    assert "workspace" in lib.fp4moe_last_error().decode()
    # a NULL operand with rows to compute
    assert f(BAD, NULL, BAD, 4, 8, BAD, BAD, BAD, BAD, BAD, 16, 128, NULL, 0, NULL) == 1
    assert "NULL" in lib.fp4moe_last_error().decode()
    # total_rows == 0 is a no-op, with or without a (never touched) workspace
    assert f(NULL, NULL, NULL, 4, 0, NULL, NULL, NULL, NULL, NULL, 16, 128, NULL, 0, NULL) == 0
    assert f(NULL, NULL, NULL, 4, 0, NULL, NULL, NULL, NULL, NULL, 16, 128, BAD, 256, NULL) == 0
    assert lib.fp4moe_last_error().decode() == ""


def test_debug_checks_switch(lib):
    assert lib.fp4moe_set_debug_checks(2) == 1
    assert "fp4moe_set_debug_checks" in lib.fp4moe_last_error().decode()
    assert lib.fp4moe_set_debug_checks(1) == 0
    # argument validation still comes first: nothing reaches the device check
    assert lib.fp4_grouped_gemm(BAD, BAD, BAD, 0, 8, BAD, BAD, BAD, BAD, BAD, 16, 128, NULL, 0, NULL) == 1
    assert lib.fp4moe_set_debug_checks(0) == 0


@pytest.mark.parametrize("a_rows,E,R,inter,k,limit", [
    (-1, 4, 8, 128, 128, 1.0), (8, 0, 8, 128, 128, 1.0), (8, 4, 8, 0, 128, 1.0), (8, 4, 8, 192, 128, 1.0),
    (8, 4, 8, 128, 96, 1.0), (8, 4, 8, 128, 128, 0.0), (8, 4, 8, 128, 128, float("nan")),
    (1 << 20, 4, 8, 128, 4096, 1.0)])
def test_fused_gate_up_rejects(lib, a_rows, E, R, inter, k, limit):
    assert lib.fp4_grouped_gemm_swiglu_quant(BAD, BAD, a_rows, BAD, BAD, E, R, BAD, BAD, BAD, BAD, inter, k, NULL,
                                             limit, BAD, BAD, NULL, NULL) == 1
    assert "fp4_grouped_gemm_swiglu_quant" in lib.fp4moe_last_error().decode()


def test_fused_gate_up_null_alignment_and_noop(lib):
    f = lib.fp4_grouped_gemm_swiglu_quant
    assert f(BAD, BAD, 8, BAD, BAD, 4, 8, BAD, BAD, BAD, BAD, 128, 128, NULL, 1.0, NULL, BAD, NULL, NULL) == 1
    assert f(BAD, BAD, 8, BAD, BAD, 4, 8, BAD, BAD, BAD, BAD, 128, 128, NULL, 1.0, ctypes.c_void_p(0x1008), BAD, NULL, NULL) == 1
    assert "aligned" in lib.fp4moe_last_error().decode()
    assert f(NULL, NULL, 0, NULL, NULL, 4, 0, NULL, NULL, NULL, NULL, 128, 128, NULL, 1.0, NULL, NULL, NULL,
             NULL) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_scaled_fp4_quant_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(m.Fp4MoeError):
        m.lib()


def test_routing_is_declared():
    names = declared_functions()
    for fn in ("route_softmax_topk", "route_pack_workspace_size", "route_pack", "gather_quant_rows",
               "moe_combine"):
        assert fn in names


@pytest.mark.parametrize("tokens,experts,top_k,normalize", [(-1, 8, 2, 0), (4, 0, 1, 0), (4, 1025, 8, 0),
                                                            (4, 8, 0, 0), (4, 8, 9, 0), (4, 100, 65, 0),
                                                            (4, 8, 2, 2), (1 << 22, 1024, 8, 0)])
def test_route_topk_rejects(lib, tokens, experts, top_k, normalize):
    assert lib.route_softmax_topk(BAD, tokens, experts, top_k, normalize, BAD, BAD, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("route_softmax_topk")


def test_route_topk_null_and_noop(lib):
    assert lib.route_softmax_topk(NULL, 4, 8, 2, 0, BAD, BAD, NULL) == 1
    assert lib.route_softmax_topk(NULL, 0, 8, 2, 0, NULL, NULL, NULL) == 0


def test_route_pack_workspace_size(lib):
    assert lib.route_pack_workspace_size(-1, 256) == 0
    assert lib.route_pack_workspace_size(0, 256) == 4 * 256
    assert lib.route_pack_workspace_size(1, 256) == 4 * 256 * 2
    assert lib.route_pack_workspace_size(64, 256) == 4 * 256 * 2
    assert lib.route_pack_workspace_size(65, 256) == 4 * 256 * 3
    assert lib.route_pack_workspace_size(8192, 256) == 4 * 256 * 129


@pytest.mark.parametrize("tokens,top_k,experts", [(-1, 8, 256), (4, 0, 256), (4, 65, 256), (4, 8, 0),
                                                  (4, 8, 1025), (1 << 26, 64, 8)])
def test_route_pack_rejects(lib, tokens, top_k, experts):
    assert lib.route_pack(BAD, NULL, tokens, top_k, experts, BAD, BAD, BAD, NULL, BAD, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("route_pack")


def test_route_pack_null_and_alignment(lib):
    assert lib.route_pack(BAD, NULL, 4, 2, 8, NULL, BAD, BAD, NULL, BAD, NULL) == 1      # offsets
    assert lib.route_pack(BAD, NULL, 4, 2, 8, BAD, BAD, BAD, NULL, NULL, NULL) == 1      # workspace
    assert lib.route_pack(NULL, NULL, 0, 2, 8, BAD, NULL, NULL, NULL, NULL, NULL) == 1   # even empty
    assert lib.route_pack(BAD, NULL, 4, 2, 8, BAD, BAD, BAD, NULL, ctypes.c_void_p(0x1002), NULL) == 1


@pytest.mark.parametrize("a_rows,k,rows", [(-1, 128, 4), (4, 100, 4), (4, 128, -1), (1 << 24, 256, 4)])
def test_gather_rejects(lib, a_rows, k, rows):
    assert lib.gather_quant_rows(BAD, BAD, a_rows, k, BAD, rows, BAD, BAD, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("gather_quant_rows")


def test_gather_null_alignment_noop(lib):
    assert lib.gather_quant_rows(BAD, BAD, 4, 128, NULL, 2, BAD, BAD, NULL) == 1
    assert lib.gather_quant_rows(ctypes.c_void_p(0x1008), BAD, 4, 128, BAD, 2, BAD, BAD, NULL) == 1
    assert lib.gather_quant_rows(NULL, NULL, 4, 128, NULL, 0, NULL, NULL, NULL) == 0


@pytest.mark.parametrize("y_rows,n,tokens,top_k", [(-1, 16, 4, 2), (8, 0, 4, 2), (8, 16, -1, 2),
                                                   (8, 16, 4, 0), (8, 16, 4, 65), (1 << 20, 4096, 4, 2)])
def test_combine_rejects(lib, y_rows, n, tokens, top_k):
    assert lib.moe_combine(BAD, y_rows, n, BAD, NULL, tokens, top_k, BAD, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("moe_combine")


def test_combine_null_and_noop(lib):
    assert lib.moe_combine(BAD, 8, 16, NULL, NULL, 4, 2, BAD, NULL) == 1
    assert lib.moe_combine(NULL, 0, 16, NULL, NULL, 0, 2, NULL, NULL) == 0


def test_rung_rejects(lib):
    assert lib.cvt_bf16(BAD, BAD, -1, NULL) == 1
    assert lib.cvt_bf16(NULL, BAD, 4, NULL) == 1
    assert lib.cvt_bf16(NULL, NULL, 0, NULL) == 0
    assert lib.fp4_dequant_bf16(BAD, BAD, ctypes.c_float(1.0), 0, 8, 100, BAD, NULL) == 1     # k % 128
    assert lib.fp4_dequant_bf16(BAD, BAD, ctypes.c_float(1.0), 2, 8, 128, BAD, NULL) == 1     # kind
    assert lib.fp4_dequant_bf16(BAD, BAD, ctypes.c_float(1.0), 0, 8, 128, ctypes.c_void_p(0x1008), NULL) == 1
    assert lib.fp4_dequant_bf16(NULL, NULL, ctypes.c_float(1.0), 0, 0, 128, NULL, NULL) == 0
    assert lib.gemm_bf16(BAD, BAD, BAD, 4, 4, 24, NULL) == 1                                # k % 16
    assert lib.gemm_bf16(BAD, BAD, BAD, 4, 0, 32, NULL) == 1
    assert lib.gemm_bf16(NULL, BAD, BAD, 4, 4, 32, NULL) == 1
    assert lib.gemm_bf16(NULL, NULL, NULL, 0, 4, 32, NULL) == 0
    for fn in ("cvt_bf16", "fp4_dequant_bf16", "gemm_bf16"):
        assert fn in declared_functions()


def test_w4a4_rejects(lib):
    assert lib.act_quant_fp4(BAD, NULL, 0, BAD, BAD, BAD, 4, 100, 1, NULL) == 1          # k % 128
    assert lib.act_quant_fp4(BAD, NULL, 65, BAD, BAD, BAD, 4, 128, 1, NULL) == 1         # n_skip
    assert lib.act_quant_fp4(BAD, NULL, 2, BAD, BAD, BAD, 4, 128, 1, NULL) == 1          # skip NULL
    assert lib.act_quant_fp4(BAD, NULL, 0, BAD, BAD, BAD, 4, 128, 2, NULL) == 1          # two_level
    assert lib.act_quant_fp4(NULL, NULL, 0, NULL, NULL, NULL, 0, 128, 1, NULL) == 0
    assert lib.loud_channels(BAD, 4, 8193, 1, BAD, NULL) == 1
    assert lib.loud_channels(BAD, 4, 16, 17, BAD, NULL) == 1
    assert lib.loud_channels(BAD, 4, 128, 65, BAD, NULL) == 1
    assert lib.loud_channels(NULL, 4, 128, 0, NULL, NULL) == 0
    assert lib.w4a4_gemm(BAD, BAD, BAD, BAD, BAD, ctypes.c_float(1.0), NULL, NULL, 0, BAD, 4, 8, 100, NULL) == 1
    assert lib.w4a4_gemm(BAD, BAD, BAD, BAD, BAD, ctypes.c_float(1.0), NULL, NULL, 4, BAD, 4, 8, 128, NULL) == 1
    assert lib.w4a4_gemm(BAD, BAD, BAD, BAD, BAD, ctypes.c_float(1.0), NULL, NULL, 65, BAD, 4, 8, 128, NULL) == 1
    assert lib.w4a4_gemm(NULL, NULL, NULL, NULL, NULL, ctypes.c_float(1.0), NULL, NULL, 0, NULL, 0, 8, 128, NULL) == 0
    for fn in ("act_quant_fp4", "loud_channels", "w4a4_gemm"):
        assert fn in declared_functions()


def test_swizzle_sizes_and_rejects(lib):
    # sizes: n rounded up to 16 columns; scales per chunk of 4 blocks (NVFP4 8 B, MXFP4 4 B per lane piece)
    assert lib.fp4_swizzled_weight_bytes(2048, 7168) == 2048 * 3584
    assert lib.fp4_swizzled_weight_bytes(20, 256) == 32 * 128
    assert lib.fp4_swizzled_scale_bytes(0, 2048, 7168) == 2048 * 7168 // 16
    assert lib.fp4_swizzled_scale_bytes(1, 2048, 7168) == 2048 * 7168 // 32
    assert lib.fp4_swizzled_scale_bytes(0, 16, 128) == 1 * 1 * 64 * 8          # one partial chunk
    assert lib.fp4_swizzled_scale_bytes(2, 16, 128) == 0                       # kind must be 0/1
    assert lib.fp4_swizzled_weight_bytes(16, 100) == 0
    A = ctypes.c_void_p(0x10000)
    assert lib.fp4_weight_swizzle(A, A, 0, 16, 100, A, A, NULL) == 1          # k % 128
    assert lib.fp4_weight_swizzle(A, A, 2, 16, 128, A, A, NULL) == 1          # kind
    assert lib.fp4_weight_swizzle(A, A, 0, 0, 128, A, A, NULL) == 1           # n
    assert lib.fp4_weight_swizzle(ctypes.c_void_p(0x10008), A, 0, 16, 128, A, A, NULL) == 1   # alignment
    assert lib.fp4_weight_swizzle(NULL, A, 0, 16, 128, A, A, NULL) == 1
    assert lib.fp4moe_last_error().decode().startswith("fp4_weight_swizzle")
    # the GEMM takes kinds 0..3 and rejects others before any launch
    assert lib.fp4_expert_gemm(A, A, A, A, ctypes.c_float(1.0), 4, A, 1, 16, 128, NULL) == 1
