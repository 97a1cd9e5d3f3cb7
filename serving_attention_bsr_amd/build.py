"""Build libbsr_attn.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instruction selection disabled.
The host-side sources (planner, C ABI) go through hipcc as well, since the ABI
launches kernels through the HIP runtime.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libbsr_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIP_SOURCES = ["kernels_d64.hip", "kernels_d128.hip", "kernels_d256.hip", "kernels_d64_var.hip",
               "kernels_d128_var.hip", "kernels_d256_var.hip", "merge_states.hip", "append_kv.hip", "run_static.hip",
               "quest.hip"]
HOST_SOURCES = ["api.cpp", "plan.cpp"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Matrix-core results and accumulators in ordinary vector registers: with more than
# 256 registers per lane available (one workgroup per CU) the compiler would
# otherwise place them in accumulation registers and copy every value the softmax
# reads or writes (measured: the shared-prefix batch 118 -> 110 us).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l]
    return proc.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int = 8, out_path: str = OUT, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    jobs_list = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        jobs_list.append([hipcc, *COMMON, *extra, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(build_dir, src.replace(".cpp", ".o"))
        jobs_list.append([hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(_run, jobs_list))
    failed = False
    for cmd, (rc, out) in zip(jobs_list, results):
        if verbose or rc != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        failed |= rc != 0
    if failed:
        raise RuntimeError("HIP build failed")
    objs = [c[-1] for c in jobs_list]
    tmp = out_path + ".tmp"
    rc, out = _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("link failed")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
