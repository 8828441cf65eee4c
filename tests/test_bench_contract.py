"""Host-side pieces of bench.py's output contract: a recorded HBM-traffic figure is reported only for
the exact kernel sources and weight layout it was measured with, the algorithmic-byte count of the
decode step adds up, and asking for more than one GPU exits with a message."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_recorded_traffic_matches_sources_and_layout(tmp_path, monkeypatch):
    sha = bench.sources_sha("config3")
    rec = {"config3": {"layout": "swizzled", "gemm_sources_sha": sha, "hbm_bytes_per_launch": 123}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("config3", "swizzled") == 123
    assert bench.recorded_traffic("config3", "plain") is None          # other layout
    assert bench.recorded_traffic("config4", "swizzled") is None       # no record
    rec["config3"]["gemm_sources_sha"] = "0" * 16                      # sources changed since
    f.write_text(json.dumps(rec))
    assert bench.recorded_traffic("config3", "swizzled") is None


def test_decode_step_algorithmic_bytes():
    wl = workloads.config3()
    alg = bench.algorithmic_bytes(wl)
    assert alg["weights"] == 256 * (2048 * 7168 // 2 + 2048 * 7168 // 16 + 4) == 2_113_930_240
    assert alg["acts"] == 512 * 7168 + 512 * 56 * 4
    assert alg["out"] == 4096 * 2048 * 4
    assert alg["total"] == 2_151_292_932


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.fixture(scope="module")
def config4_wl():
    return workloads.config4()


def test_prefill_step_algorithmic_bytes_and_flops(config4_wl):
    wl = config4_wl
    alg = bench.algorithmic_bytes(wl)
    # 255 NVFP4 experts of [4096, 7168/2] nibbles + [4096, 7168/16] E4M3 scales + scale2, and one
    # MXFP4 expert with [4096, 7168/32] E8M0 scales
    assert alg["weights"] == 255 * (4096 * 3584 + 4096 * 448 + 4) + (4096 * 3584 + 4096 * 224) == 4_226_941_948
    assert wl.R == 65536 and 2.0 * wl.R * wl.k * wl.n == pytest.approx(3.848e12, rel=1e-3)


def _fake_measure(gemm_ms, step_ms):
    return {"step_ms": step_ms, "wall_ms": step_ms, "aq_ms": 0.01, "gemm_ms": gemm_ms, "gemm_ms_min": gemm_ms,
            "gemm_pct": {"p10": gemm_ms * 1e3, "p50": gemm_ms * 1e3, "p90": gemm_ms * 1e3}}


class _Args:
    tokens = 0
    layout = "swizzled"
    steps = 20


def test_half_results(config4_wl):
    """Each half's roofline: achieved = algorithmic bytes (decode) or flops (prefill) over the GEMM's
    mean event time, frac = achieved / the published peak; the prefill half also against 5 PFLOP/s."""
    wl3 = workloads.config3()
    d = bench.half_result("config3", wl3, _fake_measure(0.35, 0.36), _Args, {"x": "0"})
    assert d["unit"] == "TB/s" and d["roofline"]["bound"] == "hbm"
    assert d["roofline"]["achieved"] == pytest.approx(2_151_292_932 / 0.35e-3 / 1e9, abs=0.1)
    assert d["roofline"]["frac"] == pytest.approx(d["roofline"]["achieved"] / 8000.0, abs=1e-4)
    assert d["value"] == pytest.approx(2_113_930_240 / 0.36e-3 / 1e12, abs=1e-4)
    p = bench.half_result("config4", config4_wl, _fake_measure(3.8, 3.9), _Args, {"x": "0"})
    tf = 2.0 * 65536 * 7168 * 4096 / 3.8e-3 / 1e12
    assert p["unit"] == "TFLOP/s" and p["roofline"]["bound"] == "mfma"
    assert p["roofline"]["achieved"] == pytest.approx(tf, abs=0.1)
    assert p["roofline"]["frac"] == pytest.approx(tf / 2500.0, abs=1e-4)
    assert p["roofline_fp8"]["frac"] == pytest.approx(tf / 5000.0, abs=1e-4)


def test_input_hashes_are_stable():
    a, b = workloads.config0(), workloads.config0()
    wl = workloads.grouped_random(3, 20, 4, 2, 32, 128)
    h1 = bench.input_hashes(wl)
    h2 = bench.input_hashes(workloads.grouped_random(3, 20, 4, 2, 32, 128))
    assert h1 == h2 and set(h1) >= {"x", "row_ids", "offsets", "w_bank", "s_bank"}
    assert all(len(v) == 64 for v in h1.values())
    assert a.x.tobytes() == b.x.tobytes()


def test_cpu_model_names_the_host():
    m = bench.cpu_model()
    assert "logical CPUs available" in m and "family" in m


PROBE_LIB = os.path.join(ROOT, "block_scaled_fp4_quant_amd", "libfp4moe_probe.so")


def _probe():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        pytest.fail(f"{PROBE_LIB} is missing: build the package first")
    L = ctypes.CDLL(PROBE_LIB)
    fn = L.fp4moe_probe_mfma_loop
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def test_mfma_probe_library_rejects_bad_arguments():
    # the measurement probe behind --workload peaks: it loads, and it rejects invalid arguments on
    # the host before any HIP call (no GPU needed)
    import ctypes
    fn = _probe()
    dummy = ctypes.c_void_p(16)
    assert fn(0, 1, 8, dummy, dummy, None) == 1          # iters <= 0
    assert fn(10, 1, 0, dummy, dummy, None) == 1         # no workgroups
    assert fn(10, 1, 8, None, dummy, None) == 1          # null sink
    assert fn(10, 1, 8, dummy, None, None) == 1          # null clocks


@pytest.mark.gpu
def test_mfma_probe_runs_and_stamps_clocks():
    import ctypes
    import numpy as np
    import torch
    fn = _probe()
    nblocks, iters = 16, 200
    sink = torch.empty(nblocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(nblocks * 4, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    for toggle in (0, 1):
        rc = fn(iters, toggle, nblocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0
        torch.cuda.synchronize()
        c = clocks.cpu().numpy().view(np.uint64).reshape(nblocks, 4)
        assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] > c[:, 2]).all()
        mhz = (c[:, 1] - c[:, 0]).astype(np.float64) / (c[:, 3] - c[:, 2]).astype(np.float64) * 100.0
        assert 100.0 < float(np.median(mhz)) < 5000.0     # a core clock, in MHz
        assert bool(torch.isfinite(sink).all())           # operands in [0.5, 1): sums stay finite


def test_source_hash_ignores_comments_and_layout_only():
    # a recorded traffic figure stays valid across comment and whitespace edits, not code edits
    base = 'int f(int x) {\n  // twice\n  return 2 * x; /* done */\n}\nconst char* s = "// not a comment";\n'
    same = 'int f(int x) {   return 2 * x;\n\n}\n// new note\nconst char* s = "// not a comment"; /* x */\n'
    code = 'int f(int x) {\n  return 3 * x;\n}\nconst char* s = "// not a comment";\n'
    lit = 'int f(int x) {\n  return 2 * x;\n}\nconst char* s = "//  not a comment";\n'
    assert bench.code_text(base) == bench.code_text(same)
    assert bench.code_text(base) != bench.code_text(code)
    assert bench.code_text(base) != bench.code_text(lit)            # string literals are kept whole
    assert bench.code_text("char c = '\"'; // q\nint y;") == "char c = '\"'; int y;"
