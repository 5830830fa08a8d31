"""Builds the gfx950 shared library libmoe_nvfp4.so in-tree with hipcc.

    python -m nvfp4_expert_layer_amd.build        (or build() from Python)

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (the compiler must not form v_pk_*_f32), and linked into
nvfp4_expert_layer_amd/libmoe_nvfp4.so next to this file.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_nvfp4.so")
SOURCES = ["router.hip", "quant.hip", "gemm.hip", "prefill.hip", "decode.hip", "mid.hip", "engine.cpp"]
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the library needs ROCm's hipcc to build")
    return path


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Per-source compiler options.  The tiled GEMMs are scheduled for instruction
# level parallelism (LLVM's max-ilp machine scheduler): measured 4% faster on
# the T=8192 W4A4 layer's GEMMs (GEMM1 1229 against 1284 us, GEMM2 634 against
# 672 us), 1% on the T=16384 W4A16 shard; the other sources measured equal or
# slower with it.
EXTRA_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + EXTRA_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    sources = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        results = list(ex.map(_compile, sources))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
