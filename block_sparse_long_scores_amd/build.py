"""Build libfp2.so (HIP for gfx950) in-tree: ``python -m block_sparse_long_scores_amd.build``.
Also builds libfp2_microbench.so, the MFMA-peak microbenchmark bench.py reports.

Every source is compiled with hipcc for gfx950 only, with packed fp32 VALU
instructions disabled (the kernels never rely on them), and linked into one
shared library next to this file.  The library is rebuilt on every call.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp2.so")
# the MFMA microbenchmark the benchmark report measures the part's matrix
# peak with (not part of the library's interface)
MICRO_SRC = os.path.join(PKG, "microbench", "mfma_peak.hip")
MICRO_LIB = os.path.join(PKG, "libfp2_microbench.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


# Per-source code-generation options.  The bf16 attention kernel asks for the
# VGPR form of the MFMA results (S then stays in VGPRs for the softmax instead
# of being read back from AGPRs one value at a time); the fp8 one keeps the
# default selection.
EXTRA = {
    "attention_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    tmp = MICRO_LIB + ".tmp"
    cmd = [hipcc()] + COMMON + ["-shared", MICRO_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("microbenchmark build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, MICRO_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
