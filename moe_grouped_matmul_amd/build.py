"""Ahead-of-time build of the gfx950 library ``libdg_mi355x.so`` (in-tree).

Compiles every HIP source under ``csrc/`` with hipcc for gfx950 and links one
shared library next to this file.  Kernel register/scratch usage reported by
the compiler is kept in ``_build/resource_usage.txt`` (read by a test that
requires zero scratch, i.e. no register spills).

Usage: python -m moe_grouped_matmul_amd.build   (or build() from Python)
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB_NAME = "libdg_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["quant.hip", "gemm_skinny.hip", "gemm_persist.hip", "gemm_wide.hip", "noalloc.hip", "api.cpp"]
# per-source flags: the persistent kernels need the iterative ILP scheduler to
# stay within 256 VGPRs (two waves per SIMD) without spilling
SOURCE_FLAGS = {"gemm_persist.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
                "gemm_wide.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}
COMMON = [
    "-O3",
    "--offload-arch=gfx950",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the promotion FMAs read them without
    # v_accvgpr_read copies and consecutive MFMAs get distinct destinations
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _compile(src, build_dir, extra):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, out_path=None, extra_flags=()):
    """Compile and link; out_path/extra_flags serve experiments with compile-time
    tuning macros (the default build is what the package loads)."""
    lib_path = out_path or LIB_PATH
    build_dir = BUILD if out_path is None else os.path.join(os.path.dirname(out_path), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir, list(extra_flags)), SOURCES))
    report = []
    for (obj, log), src in zip(results, SOURCES):
        lines = [l for l in log.splitlines() if "remark" in l or "Function Name" in l or ":" in l]
        report.append(f"== {src}\n" + "\n".join(l for l in log.splitlines() if "remark:" in l))
    with open(os.path.join(build_dir, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report) + "\n")
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
