"""Build libw4a16q.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m w4a16_group_wise_amd.build

compiles every csrc/*.hip with --offload-arch=gfx950 and links them into
w4a16_group_wise_amd/libw4a16q.so.  Packed-FP32 instructions are disabled for all device code
and fp32 division / square root stay correctly rounded (the candidate scales divide by 7).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16q.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# per-source additions: the scale search and the few-row W4A16 product read their matrix-core
# results with vector instructions right after each product, so those stay in ordinary VGPRs
# (no accvgpr copies)
FILE_FLAGS = {
    "scale_search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libw4a16q")
    return p


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OUT, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stderr.strip() or r.stdout.strip()):
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, sources()))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
