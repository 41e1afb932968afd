"""Build the HIP library ``libbcjr.so`` for gfx950 in-tree (no JIT cache).

    python -m bcjr_soft_decoding_amd.build

Every source under ``csrc/`` is compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled, and linked into ``bcjr_soft_decoding_amd/_lib/libbcjr.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libbcjr.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["host.cpp", "sparse_kernels.hip", "viterbi_kernels.hip", "dense_kernels.hip", "code_kernels.hip",
           "scan_kernels.hip", "noalloc.hip"]
# Second translation units: (source, object name, extra options). sparse_kernels.hip is built a
# second time with only the shapes whose fp32-message kernels run faster under the machine
# scheduler that maximises instruction-level parallelism (see ilp_fwd_shape / ilp_bwd_shape).
ILP_FLAGS = ["-DBCJR_ILP_TU", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA_UNITS = [("sparse_kernels.hip", "sparse_kernels_ilp", ILP_FLAGS)]
# The forward-backward kernels' max reductions need no NaN canonicalisation: a NaN or Inf input
# still reaches the outputs through the exponentials and sums that follow every max (the
# propagation the C ABI documents is tested); the Viterbi decoder keeps strict IEEE semantics
# for its bit-exact contract.
EXTRA_FLAGS = {"sparse_kernels.hip": ["-fno-honor-nans"], "dense_kernels.hip": ["-fno-honor-nans"]}


# The CPU sanitizer run (tests/run_sanitizers.py) builds a second library whose host code (the
# validation, size arithmetic and launch set-up) carries AddressSanitizer and
# UndefinedBehaviorSanitizer; every option applies to the host pass only (the device code is
# the same as in the ordinary build).
SAN_LIB = os.path.join(OUT_DIR, "libbcjr_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def _compile(unit, sanitize: bool = False) -> str:
    src, name, extra = unit if isinstance(unit, tuple) else (unit, unit, [])
    bdir = os.path.join(BUILD_DIR, "san") if sanitize else BUILD_DIR
    obj = os.path.join(bdir, os.path.basename(name) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), *extra, *(SAN_FLAGS if sanitize else []), *lang,
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    # the host pass does not know the gfx950 target feature; that warning is expected
    errs = [ln for ln in r.stderr.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link _lib/libbcjr.so (with sanitize: the
    host-sanitized _lib/libbcjr_san.so, for the CPU sanitizer run only)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(os.path.join(BUILD_DIR, "san") if sanitize else BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda unit: _compile(unit, sanitize), [*SOURCES, *EXTRA_UNITS]))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_FLAGS if sanitize else []), "-o",
           tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
