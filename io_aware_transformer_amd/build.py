"""Build the HIP attention library (libfa.so) in-tree for gfx950.

Usage: ``python -m io_aware_transformer_amd.build`` (or ``build()`` from
Python).  Every call recompiles.  Objects go to ``_build/``; the compiler's
per-kernel resource report (VGPRs, AGPRs, LDS, scratch, occupancy) is kept in
``_build/resource_usage.txt``.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_host.cpp", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip", "fa_split_bf16.hip"]
ARCH = "gfx950"


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-fPIC",
        "-std=c++17",
        # keep the compiler from emitting packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Wall",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, out=None):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for src, (_, log) in zip(SOURCES, results):
            f.write(f"==== {src}\n")
            f.write("\n".join(line for line in log.splitlines() if "remark" in line or "warning" in line.lower()))
            f.write("\n")
    target = out or LIB
    tmp = target + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target}")
    return target


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
