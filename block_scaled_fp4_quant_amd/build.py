"""Build libfp4moe.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc, and beside it
libfp4moe_probe.so (the benchmark's matrix-core rate probe, not part of the method).

Usage: python -m block_scaled_fp4_quant_amd.build  (or call build()).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp4moe.so")
PROBE_LIB = os.path.join(PKG, "libfp4moe_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
SOURCES = ["act_quant.hip", "swiglu_quant.hip", "route.hip", "rung.hip", "w4a4.hip", "swizzle.hip", "gemm_decode.hip", "gemm_skinny.hip", "gemm_prefill.hip", "table_check.hip", "capi.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed-f32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels whose leading arguments are scalars get up to 16 of their dwords in SGPRs before the
    # first instruction (the compiler keeps a loading prologue for firmware without the feature)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-fvisibility=hidden", "-Wall",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, jobs: int = 4) -> str:
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose, jobs)
    return _build_lib(SOURCES, LIB, verbose, jobs)


def _build_lib(sources, lib_path: str, verbose: bool, jobs: int) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="fp4moe_build_") as tmp:
        objs, procs = [], []
        for src in sources:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        while procs:
            _wait(procs.pop(0))
        tmp_lib = lib_path + ".tmp%d" % os.getpid()
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, lib_path)
    return lib_path


def _wait(item):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    if text.strip():
        print(text, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
