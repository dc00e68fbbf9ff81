"""Compile libbitlinear (and the synthetic-input and measured-ceiling helper libraries) for
gfx950 with hipcc.

    python ternary_weight_linear_amd/build.py        # builds both .so files in-tree

Run it as a script (or load it by path): importing the package first would dlopen the
library that is about to be rebuilt.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libbitlinear.so")
SYNTH_DIR = os.path.join(ROOT, "synth")
SYNTH_LIB_PATH = os.path.join(SYNTH_DIR, "libblsynth.so")
# measured ceilings (streaming read, int8 matrix-core loop) for the benchmark's rooflines
CEIL_LIB_PATH = os.path.join(PKG, "libblceil.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("BL_OFFLOAD_ARCH", "gfx950")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed fp32 VALU instructions are kept out of every kernel (-packed-fp32-ops); fp32
# division stays IEEE (no fast-math): the quantisers decide integer codes with it.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-result"]

# Per-source extras. mf_decode.hip: matrix-core accumulators in ordinary VGPRs (with the
# default AGPR form the compiler copies them between register files around the loop's
# uniform branches, ~20 extra ops per batch of tiles).
EXTRA = {"mf_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

SOURCES = ["api.hip", "pack.hip", "quant.hip", "gemv.hip", "gemm.hip", "onebit.hip", "svid.hip",
           "stack.hip",
           "residual.hip", "tern_mfma.hip", "mf_decode.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _compile(src, obj, includes, extra=()):
    _run([HIPCC, *COMMON, *extra, *[f"-I{i}" for i in includes], "-c", src, "-o", obj])
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbitlinear.so and libblsynth.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        for s in SOURCES:
            # hidden by default: only the entry points include/libbitlinear.h declares are
            # exported (the header marks them visible)
            jobs.append(ex.submit(_compile, os.path.join(CSRC, s),
                                  os.path.join(BUILD_DIR, s.replace(".hip", ".o")), [CSRC, INCLUDE],
                                  ["-fvisibility=hidden", *EXTRA.get(s, [])]))
        jsyn = ex.submit(_compile, os.path.join(SYNTH_DIR, "csrc", "synth.hip"),
                         os.path.join(BUILD_DIR, "synth.o"), [])
        jceil = ex.submit(_compile, os.path.join(CSRC, "ceilings.hip"),
                          os.path.join(BUILD_DIR, "ceilings.o"), [],
                          ["-fvisibility=hidden", "-mllvm", "-amdgpu-mfma-vgpr-form"])
        objs = [j.result() for j in jobs]
        syn_obj = jsyn.result()
        ceil_obj = jceil.result()
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    tmp = SYNTH_LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", syn_obj, "-o", tmp])
    os.replace(tmp, SYNTH_LIB_PATH)
    tmp = CEIL_LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", ceil_obj, "-o", tmp])
    os.replace(tmp, CEIL_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, SYNTH_LIB_PATH, "and", CEIL_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
