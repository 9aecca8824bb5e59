"""Build libqkvfa.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python quantized_kv_flashattention_amd/build.py`` (or call ``build()``).
Run it by path: importing the package loads the library it builds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libqkvfa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "quantize.hip", "decode.hip", "prefill.hip", "prefill_short.hip"]
# measurement helper (achievable-HBM streaming read), a library of its own
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libqkvfa_bench.so")
BENCH_SOURCES = ["bench_read.hip"]
# measurement build: the same sources with decode phase timestamps
TRACE_LIB_PATH = os.path.join(PKG_DIR, "libqkvfa_trace.so")

# No fast-math: the quantizer needs IEEE fp32 division and round-half-even.
# Packed fp32 VALU ops are disabled (-packed-fp32-ops) for every device file.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the online-softmax rescale
    # touches them with VALU ops, which cannot read AGPRs directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _link(sources, path, verbose, extra=()):
    tmp = path + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, path)


def build(verbose: bool = False, trace: bool = True) -> str:
    """Compile ``libqkvfa.so`` and the measurement libraries (``libqkvfa_bench.so``,
    and unless ``trace`` is false ``libqkvfa_trace.so``) next to this file;
    return the path of ``libqkvfa.so``."""
    _link(SOURCES, LIB_PATH, verbose)
    _link(BENCH_SOURCES, BENCH_LIB_PATH, verbose)
    if trace:
        _link(SOURCES, TRACE_LIB_PATH, verbose, extra=["-DQKVFA_PHASE_TRACE"])
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--no-trace" not in sys.argv))
