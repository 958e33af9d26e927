"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32
instructions disabled and IEEE-correct fp32 division and square root (the
quantizer's scale and reciprocal must round exactly as the fixed formula says).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["kvq_api.hip", "kvq_quant.hip", "kvq_attn.hip", "kvq_attn_kivi.hip", "kvq_attn_rope.hip",
           "kvq_attn_cb.hip", "kvq_attn_sparse.hip", "kvq_attn_8bit.hip"]
ATTN_KERNEL_SOURCES = ["kvq_attn_kivi.hip", "kvq_attn_rope.hip", "kvq_attn_cb.hip", "kvq_attn_sparse.hip",
                       "kvq_attn_8bit.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # matrix-core accumulators in ordinary VGPRs: no copies between register
    # files around the softmax, and a smaller footprint (higher occupancy)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  The attention kernels never produce or test for NaN
# (masked slots are removed by selects, not arithmetic), so their max/min need
# no NaN-quieting operand canonicalization; their resource usage is reported
# so that the build can reject any that spills to scratch.
SOURCE_FLAGS = {src: ["-fno-honor-nans", "-Rpass-analysis=kernel-resource-usage"]
                for src in ["kvq_attn.hip"] + ATTN_KERNEL_SOURCES}
# The quantizer's inputs are finite (a documented precondition), so its
# min/max need no NaN quieting either.
SOURCE_FLAGS["kvq_quant.hip"] = ["-fno-honor-nans"]
NO_SCRATCH = {src: "attn_kernel" for src in ATTN_KERNEL_SOURCES}


def scratch_users(remarks: str, name_part: str):
    """Kernels whose name contains name_part and whose resource-usage remark
    reports a nonzero ScratchSize."""
    bad, current = [], None
    for line in remarks.splitlines():
        if "remark: Function Name:" in line:
            current = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line and current and name_part in current:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if n:
                bad.append((current, n))
    return bad


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
        if src in NO_SCRATCH:
            bad = scratch_users(r.stderr, NO_SCRATCH[src])
            if bad:
                raise RuntimeError("%s: kernels spill to scratch (lower their waves-per-SIMD target): %s"
                                   % (src, ", ".join("%s (%d B/lane)" % x for x in bad)))
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
